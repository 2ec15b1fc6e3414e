// Token sampling chain on the GPU (Ollama engine page, "Token sampling
// pipeline"): Top-K -> temperature -> softmax -> Top-P -> Min-P -> weighted
// draw, one block of 1024 threads per logits row.
//
// Ranking: larger logit first, ties to the lower token id.  Each element is
// represented by a 64-bit candidate key (order-preserving 32-bit key of the
// float above, the complement of the token id below), so that the ranking
// is the descending order of the keys.
//
// Top-K: a strided sample of 1024 logits is sorted, and the sample's key at
// the rank where about 3K elements of the row are expected to lie above it
// becomes the collection threshold; one pass over the row then gathers every
// element at or above it into LDS (at most 8192).  If the gather holds fewer
// than K elements or overflows (ties, adversarial layouts), the exact K-th
// largest key is found instead by a radix select (four 8-bit histogram
// passes) and exactly the K top-ranked elements are gathered.  The gathered
// keys are sorted (bitonic: registers, lane exchanges, LDS); the first K are the Top-K.  They are
// divided by the temperature and turned into probabilities; an inclusive scan
// gives the cumulative probabilities that the Top-P cut (the first rank past
// the first whose cumulative exceeds p; p >= 1 keeps all), the Min-P cut
// (probability >= min_p times the largest) and the inverse-CDF draw (first
// cumulative above u times the survivors' total) read.  The uniform number u
// of each row is an input.
#include "k_common.hpp"
#include "kernels.hpp"
#include "tdf.h"

namespace tdf {

constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / 64;
constexpr int kCandCap = 8192;   // gathered candidates held in LDS
constexpr int kGatherBatch = 16; // row elements per thread per round of loads
constexpr int kGatherBatch4 = 8;  // 16-byte row pieces per thread per round of loads

// larger float -> larger unsigned key (-0 and +0 share the key of +0)
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = x == 0.f ? 0u : __builtin_bit_cast(uint32_t, x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t cand_key(uint32_t key, int id) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}
__device__ __forceinline__ float cand_value(uint64_t c) {
  const uint32_t k = (uint32_t)(c >> 32);
  return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ int cand_id(uint64_t c) { return (int)(0xFFFFFFFFu - (uint32_t)c); }

// number of set bits of the wave mask m held by lanes below this one
__device__ __forceinline__ uint32_t count_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Append c to list[0 .. cap) for every lane with hit: one LDS atomic per wave
// (all 64 lanes must be active).  Slots at or past cap are counted, not
// written.
__device__ __forceinline__ void wave_append(bool hit, uint64_t c, uint32_t* n, uint64_t* list, uint32_t cap) {
  const uint64_t m = __ballot(hit);
  if (m == 0) return;
  uint32_t base = 0;
  if (hit && count_below(m) == 0) base = atomicAdd(n, (uint32_t)__popcll(m));
  base = __builtin_amdgcn_readlane(base, __builtin_ctzll(m));
  if (hit) {
    const uint32_t slot = base + count_below(m);
    if (slot < cap) list[slot] = c;
  }
}

__device__ __forceinline__ float block_sum1024(float v, float* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kSampleWaves; ++w) t += red[w];
  return t;
}

__device__ __forceinline__ int block_min1024(int v, int* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = red[0];
#pragma unroll
  for (int w = 1; w < kSampleWaves; ++w) t = min(t, red[w]);
  return t;
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, kWave);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, kWave);
  return ((uint64_t)hi << 32) | lo;
}

// compare-exchange of the register pairs (e, e ^ S) of a descending bitonic
// stage over runs of `size` (element index tid * E + e)
template <int E, int S>
__device__ __forceinline__ void cx_regs(uint64_t (&v)[E], int tid, int size) {
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if constexpr (S < E) {
      const int f = e ^ S;
      if (f > e) {
        const bool desc = ((tid * E + e) & size) == 0;
        const uint64_t x = v[e], y = v[f];
        if ((x < y) == desc) {
          v[e] = y;
          v[f] = x;
        }
      }
    }
  }
}

// Descending bitonic sort of 1024 * E keys held E per thread (element
// tid * E + e in v[e]).  Compare-exchange partners closer than E are in the
// same thread (registers), closer than 64 E in the same wave (lane exchange),
// the rest go through lds (>= 1024 E entries, free for the sort's use).  The
// stage loops stay rolled: every stage touches each register at the same
// index, so no register is indexed at run time.
template <int E>
__device__ __forceinline__ void sort_desc_regs(uint64_t (&v)[E], uint64_t* lds) {
  static_assert(E == 1 || E == 2 || E == 4 || E == 8, "E must be 1, 2, 4 or 8");
  const int tid = threadIdx.x;
  for (int size = 2; size <= kSampleThreads * E; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride < E) {
        if (stride == 4)
          cx_regs<E, 4>(v, tid, size);
        else if (stride == 2)
          cx_regs<E, 2>(v, tid, size);
        else
          cx_regs<E, 1>(v, tid, size);
        continue;
      }
      uint64_t o[E];
      if (stride < 64 * E) {
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = shfl_xor64(v[e], stride / E);
      } else {
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) lds[tid * E + e] = v[e];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = lds[(tid * E + e) ^ stride];
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        // the lower index of a pair keeps the larger key in a descending
        // run, the upper index in an ascending one
        const int i = tid * E + e;
        const bool keep_max = ((i & stride) == 0) == ((i & size) == 0);
        const uint64_t hi = v[e] > o[e] ? v[e] : o[e], lo = v[e] > o[e] ? o[e] : v[e];
        v[e] = keep_max ? hi : lo;
      }
    }
  }
}

// Sort list[0 .. C) (C <= 1024 E) descending in place; entries from C up to
// 1024 E are scratch.
template <int E>
__device__ void sort_list(uint64_t* list, uint32_t C) {
  const int tid = threadIdx.x;
  uint64_t v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t i = (uint32_t)(tid * E + e);
    v[e] = i < C ? list[i] : 0ull;
  }
  sort_desc_regs<E>(v, list);
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) list[tid * E + e] = v[e];
  __syncthreads();
}

// Append every element of ids [first, last) whose key is >= tkey to
// cand[0 .. kCandCap) (n_cand counts them all, also past the capacity).  VEC:
// 16-byte loads (row 16-byte aligned, first = 0, last a multiple of 4).  Each
// thread counts its hits of a batch, a wave scan places them, and one LDS
// atomic per wave reserves the wave's slots.
#define GATHER_ID(e) (VEC ? b + 4 * (((e) >> 2) * kSampleThreads + tid) + ((e) & 3) : b + (e) * kSampleThreads + tid)
template <bool VEC>
__device__ __forceinline__ void gather_pass(const float* __restrict__ row, int first, int last, uint32_t tkey,
                                            uint32_t* n_cand, uint64_t* cand) {
  constexpr int NE = VEC ? 4 * kGatherBatch4 : kGatherBatch;
  const int tid = threadIdx.x, lane = tid & 63;
  for (int b = first; b < last; b += NE * kSampleThreads) {
    float xe[NE];
    if constexpr (VEC) {
      const float4* r4 = reinterpret_cast<const float4*>(row);
      const int n4 = last >> 2;
#pragma unroll
      for (int k = 0; k < kGatherBatch4; ++k) {
        const float4 t = r4[min((b >> 2) + k * kSampleThreads + tid, n4 - 1)];
        xe[4 * k] = t.x;
        xe[4 * k + 1] = t.y;
        xe[4 * k + 2] = t.z;
        xe[4 * k + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int k = 0; k < kGatherBatch; ++k) xe[k] = row[min(b + k * kSampleThreads + tid, last - 1)];
    }
    uint32_t cnt = 0;
#pragma unroll
    for (int e = 0; e < NE; ++e) cnt += (GATHER_ID(e) < last && order_key(xe[e]) >= tkey) ? 1u : 0u;
    if (__ballot(cnt != 0) == 0) continue;
    uint32_t incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t t = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += t;
    }
    const uint32_t tot = __builtin_amdgcn_readlane(incl, 63);
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(n_cand, tot);
    uint32_t pos = __builtin_amdgcn_readfirstlane(base) + incl - cnt;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const uint32_t key = order_key(xe[e]);
      if (GATHER_ID(e) < last && key >= tkey) {
        if (pos < (uint32_t)kCandCap) cand[pos] = cand_key(key, GATHER_ID(e));
        ++pos;
      }
    }
  }
}
#undef GATHER_ID

__global__ void __launch_bounds__(kSampleThreads) sample_kernel(const float* __restrict__ logits, int V,
                                                                SampleParams sp, const float* __restrict__ u_row,
                                                                int32_t* __restrict__ tok) {
  __shared__ uint64_t cand[kCandCap];
  __shared__ float cum[kMaxTopK];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t n_cand, sel_prefix, sel_krem;
  __shared__ uint32_t eq_wave[kSampleWaves];
  __shared__ float red[kSampleWaves];
  __shared__ int redi[kSampleWaves];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float* row = logits + (int64_t)r * V;
  const int K = min(sp.top_k, V);

  // ---- collection threshold from a strided sample (rows that fit the
  // candidate list whole take every element)
  uint32_t tkey = 0;
  if (V > kCandCap) {
    const int i = (int)(((int64_t)tid * V) / kSampleThreads);
    uint64_t sv[1] = {cand_key(order_key(row[i]), i)};
    sort_desc_regs<1>(sv, cand);
    // about (j + 1) V / 1024 elements of the row lie at or above sample rank j
    const int j = min(kSampleThreads - 1, (int)((3LL * K * kSampleThreads + V - 1) / V));
    if (tid == j) sel_prefix = (uint32_t)(sv[0] >> 32);
    __syncthreads();
    tkey = sel_prefix;
  }
  if (tid == 0) n_cand = 0;
  __syncthreads();
  {
    const int v4 = ((reinterpret_cast<uintptr_t>(row) & 15) == 0) ? (V & ~3) : 0;
    gather_pass<true>(row, 0, v4, tkey, &n_cand, cand);
    gather_pass<false>(row, v4, V, tkey, &n_cand, cand);
  }
  __syncthreads();
  uint32_t C = n_cand;

  if (C < (uint32_t)K || C > (uint32_t)kCandCap) {
    // ---- exact K-th largest key: radix select over 8-bit digits
    uint32_t prefix = 0, pmask = 0, krem = (uint32_t)K;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int b = 0; b < V; b += kGatherBatch * kSampleThreads) {
        float x[kGatherBatch];
#pragma unroll
        for (int k = 0; k < kGatherBatch; ++k) x[k] = row[min(b + k * kSampleThreads + tid, V - 1)];
#pragma unroll
        for (int k = 0; k < kGatherBatch; ++k) {
          const uint32_t key = order_key(x[k]);
          if (b + k * kSampleThreads + tid < V && (key & pmask) == prefix)
            atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
      }
      __syncthreads();
      if (tid == 0) {
        // bins from the top: the bin holding the krem-th largest of the matches
        uint32_t above = 0;
        int bin = 255;
        for (; bin > 0; --bin) {
          if (above + hist[bin] >= krem) break;
          above += hist[bin];
        }
        sel_prefix = prefix | ((uint32_t)bin << shift);
        sel_krem = krem - above;
      }
      __syncthreads();
      prefix = sel_prefix;
      krem = sel_krem;
      pmask |= 255u << shift;
    }
    // prefix = key of the K-th largest: gather the K - krem keys above it and,
    // of the keys equal to it, the krem lowest ids (each thread owns a run of
    // kGatherBatch consecutive ids; an exclusive scan over threads orders
    // the equal keys by id)
    const uint32_t n_gt = (uint32_t)K - krem;
    if (tid == 0) n_cand = 0;
    __syncthreads();
    uint32_t eq_before = 0;
    for (int b = 0; b < V; b += kGatherBatch * kSampleThreads) {
      const int i0 = b + tid * kGatherBatch;
      uint32_t key[kGatherBatch];
#pragma unroll
      for (int k = 0; k < kGatherBatch; ++k) key[k] = order_key(row[min(i0 + k, V - 1)]);
      uint32_t n_eq = 0;
#pragma unroll
      for (int k = 0; k < kGatherBatch; ++k) {
        const bool ok = i0 + k < V;
        n_eq += (ok && key[k] == prefix) ? 1u : 0u;
        wave_append(ok && key[k] > prefix, cand_key(key[k], i0 + k), &n_cand, cand, n_gt);
      }
      // exclusive scan of n_eq over the block
      uint32_t incl = n_eq;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += v;
      }
      __syncthreads();
      if (lane == 63) eq_wave[wv] = incl;
      __syncthreads();
      uint32_t rank = eq_before + incl - n_eq, total = 0;
#pragma unroll
      for (int w = 0; w < kSampleWaves; ++w) {
        const uint32_t t = eq_wave[w];
        rank += w < wv ? t : 0u;
        total += t;
      }
#pragma unroll
      for (int k = 0; k < kGatherBatch; ++k) {
        if (i0 + k < V && key[k] == prefix) {
          if (rank < krem) cand[n_gt + rank] = cand_key(key[k], i0 + k);
          ++rank;
        }
      }
      eq_before += total;
    }
    __syncthreads();
    C = (uint32_t)K;
  }

  // ---- sort the gathered keys; the first K are the Top-K in ranking order
  if (C <= 1024u)
    sort_list<1>(cand, C);
  else if (C <= 2048u)
    sort_list<2>(cand, C);
  else if (C <= 4096u)
    sort_list<4>(cand, C);
  else
    sort_list<8>(cand, C);

  // ---- temperature, softmax, cumulative probabilities
  const float inv_t = 1.0f / sp.temperature;
  const float m = cand_value(cand[0]) * inv_t;
  float e = 0.f;
  if (tid < K) e = __expf(cand_value(cand[tid]) * inv_t - m);
  const float total = block_sum1024(e, red);
  const float p = e / total;
  // inclusive scan of p over the ranking (wave scan + wave totals)
  float c = p;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float v = __shfl_up(c, o, kWave);
    if (lane >= o) c += v;
  }
  __syncthreads();
  if (lane == 63) red[wv] = c;
  __syncthreads();
  float base = 0.f;
  for (int w = 0; w < wv; ++w) base += red[w];
  c += base;
  if (tid < K) cum[tid] = c;

  // ---- cuts: n = the first rank >= 1 past the Top-P cut (cumulative > p,
  // unless p >= 1) or past the Min-P cut (probability below min_p times the
  // largest, which is 1 / total); survivors are the ranks below n
  const float thr = sp.min_p / total;
  int cut = K;
  if (tid >= 1 && tid < K && ((sp.top_p < 1.f && c > sp.top_p) || p < thr)) cut = tid;
  const int n = block_min1024(cut, redi);
  // ---- draw: the first survivor whose cumulative exceeds u times the
  // survivors' total, else the last survivor
  const float target = u_row[r] * cum[n - 1];
  const int hit = (tid < n && c > target) ? tid : n - 1;
  const int pick = block_min1024(hit, redi);
  if (tid == 0) tok[r] = cand_id(cand[pick]);
}

hipError_t launch_sample(const float* logits, int R, int V, const SampleParams& sp, const float* u,
                         int32_t* tok, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  if (sp.top_k < 1 || sp.top_k > kMaxTopK || V <= 0 || !(sp.temperature > 0.f)) return hipErrorInvalidValue;
  sample_kernel<<<R, kSampleThreads, 0, s>>>(logits, V, sp, u, tok);
  return hipGetLastError();
}

}  // namespace tdf
