/*
 * Seeded synthetic inputs shared by the CPU oracle and the GPU tests/bench.
 *
 * This file holds no arithmetic of the decoder forward pass: it only turns
 * (seed, tensor name, element index) into numbers.  Every value is a pure
 * function of that triple, so any slice of any tensor can be regenerated
 * independently and in parallel.
 *
 * Counter-based stream (SplitMix64 finaliser, Steele/Lea/Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014):
 *   key(seed, name) = mix(fnv1a64(name) ^ mix(seed))
 *   word(key, i)    = mix(key + (i + 1) * 0x9E3779B97F4A7C15)
 * Normals: Box-Muller (1958) in double on the pair of words (2j, 2j+1);
 *   r = sqrt(-2 ln u1), u1 in (0,1];  phi = 2*pi*u2, u2 in [0,1)
 *   element 2j = r cos(phi), element 2j+1 = r sin(phi)
 * then scaled by the requested standard deviation, rounded to fp32 (RNE)
 * and, for bf16 outputs, from fp32 to bf16 (RNE).
 * Integers in [lo, hi]: Lemire's multiply-shift with rejection
 * ("Fast random integer generation in an interval", TOMACS 2019); a
 * rejected draw moves to a fresh sub-stream key' = mix(key + attempt).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t word_at(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * GOLDEN);
}

uint64_t tdfs_fnv1a64(const char *s) {
  uint64_t h = 0xCBF29CE484222325ULL;
  for (; *s; ++s) {
    h ^= (uint8_t)*s;
    h *= 0x100000001B3ULL;
  }
  return h;
}

uint64_t tdfs_stream_key(uint64_t seed, const char *name) {
  return mix64(tdfs_fnv1a64(name) ^ mix64(seed));
}

uint64_t tdfs_word(uint64_t key, uint64_t i) { return word_at(key, i); }

/* Both normals of pair j: out2[0] = element 2j, out2[1] = element 2j+1. */
static inline void normal_pair(uint64_t key, uint64_t j, double out2[2]) {
  uint64_t a = word_at(key, 2 * j), b = word_at(key, 2 * j + 1);
  double u1 = (double)((a >> 11) + 1) * 0x1.0p-53; /* (0, 1] */
  double u2 = (double)(b >> 11) * 0x1.0p-53;       /* [0, 1) */
  double r = sqrt(-2.0 * log(u1));
  double phi = 6.283185307179586476925286766559 * u2;
  out2[0] = r * cos(phi);
  out2[1] = r * sin(phi);
}

/* Calls emit(idx_in_out, value) for elements [first, first+n) pair by pair. */
#define FOR_EACH_NORMAL(key, first, n, EMIT)                                   \
  do {                                                                         \
    uint64_t j0 = (first) >> 1, j1 = ((first) + (uint64_t)(n) + 1) >> 1;       \
    _Pragma("omp parallel for schedule(static)")                               \
    for (int64_t jj = (int64_t)j0; jj < (int64_t)j1; ++jj) {                   \
      double v[2];                                                             \
      normal_pair((key), (uint64_t)jj, v);                                     \
      for (int e = 0; e < 2; ++e) {                                            \
        uint64_t g = 2 * (uint64_t)jj + (uint64_t)e;                           \
        if (g >= (first) && g < (first) + (uint64_t)(n)) {                     \
          int64_t i = (int64_t)(g - (first));                                  \
          EMIT;                                                                \
        }                                                                      \
      }                                                                        \
    }                                                                          \
  } while (0)

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* out[i] = fp32(std * N(0,1)) for i in [first, first + n) of stream `key`. */
void tdfs_normal_f32(uint64_t key, uint64_t first, int64_t n, double std, float *out) {
  FOR_EACH_NORMAL(key, first, n, out[i] = (float)(std * v[e]));
}

/* As tdfs_normal_f32, then fp32 -> bf16 (RNE); out holds bf16 bit patterns. */
void tdfs_normal_bf16(uint64_t key, uint64_t first, int64_t n, double std, uint16_t *out) {
  FOR_EACH_NORMAL(key, first, n, out[i] = f32_to_bf16_rne((float)(std * v[e])));
}

static inline uint16_t f32_to_f16_rne(float f) {
  /* normal and subnormal halves; values past the half range saturate to inf */
  uint32_t u;
  memcpy(&u, &f, 4);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t absu = u & 0x7FFFFFFFu;
  if (absu >= 0x47800000u) return (uint16_t)(sign | 0x7C00u); /* >= 65536: inf */
  if (absu < 0x33000000u) return (uint16_t)sign;              /* < 2^-25: zero */
  int32_t exp = (int32_t)(absu >> 23) - 127;
  uint32_t mant = (absu & 0x7FFFFFu) | 0x800000u;
  int32_t shift = exp < -14 ? 13 + (-14 - exp) : 13; /* bits dropped from the 24-bit mantissa */
  uint32_t half = mant >> shift, rem = mant & ((1u << shift) - 1u), mid = 1u << (shift - 1);
  if (rem > mid || (rem == mid && (half & 1u))) ++half;
  if (exp < -14) return (uint16_t)(sign | half);             /* subnormal (may round up to the min normal) */
  return (uint16_t)(sign | (((uint32_t)(exp + 15) << 10) + (half - 0x400u)));
}

static inline float f16_to_f32(uint16_t h) {
  const uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
  float v;
  if (e == 0) v = (float)m * 5.9604644775390625e-08f; /* m * 2^-24 */
  else {
    uint32_t u = ((e + 112u) << 23) | (m << 13);
    memcpy(&v, &u, 4);
  }
  uint32_t b;
  memcpy(&b, &v, 4);
  b |= sign;
  memcpy(&v, &b, 4);
  return v;
}

/* Q8_0 blocks of a row-major [rows][K] matrix (K a multiple of 32) whose
 * element (r, k) is draw r*K + k of stream `key`, fp32(std * N(0,1)): per
 * block of 32 consecutive elements of a row, scale d = fp16(max|w| / 127)
 * and q = round-to-nearest-even(w / d) clamped to [-127, 127] (0 when d is
 * 0).  q: [rows][K] int8; d: [rows][K/32] fp16 bit patterns. */
void tdfs_normal_q8_0(uint64_t key, int64_t rows, int64_t K, double std, int8_t *q, uint16_t *d) {
  const int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t blk = 0; blk < rows * nb; ++blk) {
    const int64_t r = blk / nb, b = blk % nb;
    const uint64_t first = (uint64_t)(r * K + b * 32);
    float w[32];
    /* draws come in pairs (Box-Muller); first is even */
    for (int j = 0; j < 32; j += 2) {
      double v[2];
      normal_pair(key, (first + (uint64_t)j) / 2, v);
      w[j] = (float)(std * v[0]);
      w[j + 1] = (float)(std * v[1]);
    }
    float amax = 0.f;
    for (int j = 0; j < 32; ++j) amax = fabsf(w[j]) > amax ? fabsf(w[j]) : amax;
    const uint16_t dh = f32_to_f16_rne(amax / 127.0f);
    const float dv = f16_to_f32(dh);
    d[blk] = dh;
    for (int j = 0; j < 32; ++j) {
      float x = dv > 0.f ? nearbyintf(w[j] / dv) : 0.f;
      if (x > 127.f) x = 127.f;
      if (x < -127.f) x = -127.f;
      q[r * K + b * 32 + j] = (int8_t)x;
    }
  }
}

static inline int64_t uniform_at(uint64_t key, uint64_t i, uint64_t range) {
  /* integer in [0, range) */
  uint64_t k = key;
  for (uint64_t attempt = 0;; ++attempt) {
    uint64_t x = word_at(k, i);
    unsigned __int128 m = (unsigned __int128)x * range;
    uint64_t l = (uint64_t)m;
    if (l >= range || l >= (uint64_t)(-range) % range) return (int64_t)(m >> 64);
    k = mix64(key + attempt + 1);
  }
}

/* out[i] uniform integer in [lo, hi] for i in [first, first + n). */
void tdfs_uniform_i32(uint64_t key, uint64_t first, int64_t n, int64_t lo, int64_t hi, int32_t *out) {
  uint64_t range = (uint64_t)(hi - lo) + 1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (int32_t)(lo + uniform_at(key, first + (uint64_t)i, range));
}

/* fp32 -> bf16 (RNE), the rounding used for every bf16 tensor above. */
void tdfs_f32_to_bf16(const float *in, int64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}
