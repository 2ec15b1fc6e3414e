// Token sampling chain on the GPU (Ollama engine page, "Token sampling
// pipeline"): Top-K -> temperature -> softmax -> Top-P -> Min-P -> weighted
// draw, one block of 1024 threads per logits row.
//
// Top-K: the K-th largest logit is found by a radix select on the 32-bit
// order-preserving key of each float (four 8-bit passes, each a histogram of
// the elements that match the key prefix found so far); every element above
// that key is a candidate, and of the elements equal to it the lowest token
// ids fill the remaining places (ranking: larger logit first, ties to the
// lower id).  The <= 1024 candidates are sorted in LDS (bitonic), divided by
// the temperature and turned into probabilities; an inclusive scan gives the
// cumulative probabilities that the Top-P cut (cumulative <= p, the first
// token always kept, p >= 1 keeps all), the Min-P cut (probability >= min_p times the largest)
// and the inverse-CDF draw (first cumulative above u times the survivors'
// total) read.  The uniform number u of each row is an input.
#include "k_common.hpp"
#include "kernels.hpp"
#include "tdf.h"

namespace tdf {

constexpr int kSampleThreads = 1024;

// larger float -> larger unsigned key
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float block_sum1024(float v, float* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kSampleThreads / 64; ++w) t += red[w];
  return t;
}

__global__ void __launch_bounds__(kSampleThreads) sample_kernel(const float* __restrict__ logits, int V,
                                                                SampleParams sp, const float* __restrict__ u_row,
                                                                int32_t* __restrict__ tok) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sel_prefix, sel_krem;
  __shared__ float cv[kMaxTopK];
  __shared__ int32_t ci[kMaxTopK];
  __shared__ uint32_t n_above;
  __shared__ uint32_t eq_base[kSampleThreads / 64];
  __shared__ float red[kSampleThreads / 64];
  __shared__ float cum[kMaxTopK];
  __shared__ float pr[kMaxTopK];
  const int r = blockIdx.x, tid = threadIdx.x;
  const float* row = logits + (int64_t)r * V;
  const int K = min(sp.top_k, V);

  // ---- radix select of the K-th largest key
  uint32_t prefix = 0, pmask = 0, krem = (uint32_t)K;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < V; i += kSampleThreads) {
      const uint32_t key = order_key(row[i]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      // bins from the top: the bin holding the krem-th largest of the matches
      uint32_t above = 0;
      int b = 255;
      for (; b > 0; --b) {
        if (above + hist[b] >= krem) break;
        above += hist[b];
      }
      sel_prefix = prefix | ((uint32_t)b << shift);
      sel_krem = krem - above;
    }
    __syncthreads();
    prefix = sel_prefix;
    krem = sel_krem;
    pmask |= 255u << shift;
  }
  // prefix = key of the K-th largest; krem of the elements equal to it are
  // taken (lowest ids first); K - krem elements are strictly larger

  // ---- collect: contiguous chunks per thread, so that a scan over threads
  // orders the equal keys by token id
  const int chunk = (V + kSampleThreads - 1) / kSampleThreads;
  const int i0 = tid * chunk, i1 = min(V, i0 + chunk);
  uint32_t my_eq = 0;
  for (int i = i0; i < i1; ++i) my_eq += order_key(row[i]) == prefix ? 1u : 0u;
  // exclusive scan of my_eq over threads (wave scan, then wave totals)
  uint32_t incl = my_eq;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t v = __shfl_up(incl, o, kWave);
    if ((tid & 63) >= o) incl += v;
  }
  if (tid == 0) n_above = 0;
  if ((tid & 63) == 63) eq_base[tid >> 6] = incl;
  __syncthreads();
  if (tid == 0) {
    uint32_t run = 0;
    for (int w = 0; w < kSampleThreads / 64; ++w) {
      const uint32_t t = eq_base[w];
      eq_base[w] = run;
      run += t;
    }
  }
  __syncthreads();
  uint32_t eq_rank = eq_base[tid >> 6] + incl - my_eq;
  const uint32_t n_gt = (uint32_t)K - krem;
  for (int i = i0; i < i1; ++i) {
    const float x = row[i];
    const uint32_t key = order_key(x);
    if (key > prefix) {
      const uint32_t slot = atomicAdd(&n_above, 1u);
      cv[slot] = x;
      ci[slot] = i;
    } else if (key == prefix) {
      if (eq_rank < krem) {
        cv[n_gt + eq_rank] = x;
        ci[n_gt + eq_rank] = i;
      }
      ++eq_rank;
    }
  }
  // pad to a power of two for the sort
  int P = 1;
  while (P < K) P <<= 1;
  for (int i = K + tid; i < P; i += kSampleThreads) {
    cv[i] = -INFINITY;
    ci[i] = 0x7FFFFFFF;
  }
  __syncthreads();

  // ---- bitonic sort: larger value first, ties to the lower id
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < P; i += kSampleThreads) {
        const int j = i ^ stride;
        if (j > i) {
          const bool desc = (i & size) == 0;
          const float a = cv[i], b = cv[j];
          const int ia = ci[i], ib = ci[j];
          const bool a_first = a > b || (a == b && ia < ib);
          if (desc != a_first) {
            cv[i] = b; cv[j] = a;
            ci[i] = ib; ci[j] = ia;
          }
        }
      }
      __syncthreads();
    }
  }

  // ---- temperature, softmax, cumulative probabilities
  const float inv_t = 1.0f / sp.temperature;
  const float m = cv[0] * inv_t;
  float e = 0.f;
  if (tid < K) e = __expf(cv[tid] * inv_t - m);
  const float total = block_sum1024(e, red);
  const float p = e / total;
  // inclusive scan of p over the ranking (wave scan + wave totals)
  float c = p;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float v = __shfl_up(c, o, kWave);
    if ((tid & 63) >= o) c += v;
  }
  __syncthreads();
  if ((tid & 63) == 63) red[tid >> 6] = c;
  __syncthreads();
  float base = 0.f;
  for (int w = 0; w < (tid >> 6); ++w) base += red[w];
  c += base;
  if (tid < K) {
    cum[tid] = c;
    pr[tid] = p;
  }
  __syncthreads();
  if (tid == 0) {
    // Top-P: the first token, then tokens while the cumulative is <= p
    int n = 1;
    if (sp.top_p >= 1.f) n = K;  // the cumulative never exceeds 1
    while (n < K && cum[n] <= sp.top_p) ++n;
    // Min-P: probability >= min_p times the largest (a prefix of the ranking)
    int nm = 1;
    const float thr = sp.min_p * pr[0];
    while (nm < K && pr[nm] >= thr) ++nm;
    n = min(n, nm);
    // inverse-CDF draw over the survivors
    const float target = u_row[r] * cum[n - 1];
    int pick = n - 1;
    for (int i = 0; i < n; ++i)
      if (cum[i] > target) {
        pick = i;
        break;
      }
    tok[r] = ci[pick];
  }
}

hipError_t launch_sample(const float* logits, int R, int V, const SampleParams& sp, const float* u,
                         int32_t* tok, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  if (sp.top_k < 1 || sp.top_k > kMaxTopK || V <= 0 || !(sp.temperature > 0.f)) return hipErrorInvalidValue;
  sample_kernel<<<R, kSampleThreads, 0, s>>>(logits, V, sp, u, tok);
  return hipGetLastError();
}

}  // namespace tdf
