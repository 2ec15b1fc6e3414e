// Device helpers shared by the gfx950 kernels: storage conversions and
// wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tdf {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---- storage types -----------------------------------------------------
// bf16 and fp16 values are carried as uint16_t bit patterns in memory.

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// round to nearest even (inputs here are finite)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Cache element types: KvT = float, or a tag for 16-bit formats.
struct kv_bf16 {};
struct kv_f16 {};
struct kv_q8 {};  // Q8_0 blocks of 32 (int8 codes + fp16 scales, read by the vector attention)

template <typename KvT> struct KvStore;
template <> struct KvStore<float> {
  typedef float T;
  __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct KvStore<kv_bf16> {
  typedef uint16_t T;
  __device__ __forceinline__ static float load(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void store(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};
template <> struct KvStore<kv_q8> {
  typedef int8_t T;  // codes; blocks are written whole by kv_quantize
};
template <> struct KvStore<kv_f16> {
  typedef uint16_t T;
  __device__ __forceinline__ static float load(const uint16_t* p, int64_t i) { return f16_to_f32(p[i]); }
  __device__ __forceinline__ static void store(uint16_t* p, int64_t i, float v) { p[i] = f32_to_f16(v); }
};

// ---- wave64 reductions ---------------------------------------------------

// All 64 lanes must be active.  Inside each row of 16 lanes: xor 1 and xor 2
// (quad permutes), then the half-row and row mirrors (lane i <-> 7-i and
// i <-> 15-i), after which every lane holds its row's result; the four rows
// are then read out with readlane.
template <int CTRL>
__device__ __forceinline__ float dpp_read(float v, float ident) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, ident),
                                                               __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_read(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_read<0xB1>(v, 0.f);
  v += dpp_read<0x4E>(v, 0.f);
  v += dpp_read<0x141>(v, 0.f);
  v += dpp_read<0x140>(v, 0.f);
  return (lane_read(v, 0) + lane_read(v, 16)) + (lane_read(v, 32) + lane_read(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_read<0xB1>(v, -INFINITY));
  v = fmaxf(v, dpp_read<0x4E>(v, -INFINITY));
  v = fmaxf(v, dpp_read<0x141>(v, -INFINITY));
  v = fmaxf(v, dpp_read<0x140>(v, -INFINITY));
  return fmaxf(fmaxf(lane_read(v, 0), lane_read(v, 16)), fmaxf(lane_read(v, 32), lane_read(v, 48)));
}

// (value, index) max with the lowest index winning ties
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

// (value, index) max over the wave (all 64 lanes active), same pattern as
// wave_max; every lane receives the winner
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float v2 = dpp_read<CTRL>(v, -INFINITY);
  const int i2 = __builtin_amdgcn_update_dpp(0x7FFFFFFF, i, CTRL, 0xF, 0xF, false);
  argmax_merge(v, i, v2, i2);
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_step<0xB1>(v, i);
  argmax_step<0x4E>(v, i);
  argmax_step<0x141>(v, i);
  argmax_step<0x140>(v, i);
  float bv = lane_read(v, 0);
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) argmax_merge(bv, bi, lane_read(v, r), __builtin_amdgcn_readlane(i, r));
  v = bv;
  i = bi;
}

// x ~= hi + lo with hi = bf16(x), lo = bf16(x - hi): about 16 significant bits
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Q8_0 block rule, in float32: the scale is fp16(max|x| / 127); a code is
// x / d rounded half-even and clamped to [-127, 127], or 0 when d is 0
__device__ __forceinline__ uint16_t q8_scale_bits(float amax) { return f32_to_f16(amax / 127.f); }
__device__ __forceinline__ int8_t q8_code(float x, float d) {
  const float r = d > 0.f ? rintf(x / d) : 0.f;
  return (int8_t)fminf(fmaxf(r, -127.f), 127.f);
}

}  // namespace tdf
