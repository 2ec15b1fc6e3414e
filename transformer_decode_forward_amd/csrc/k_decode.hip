// Decode-side kernels for gfx950: embedding gather, RMSNorm, GEMV with fused
// epilogues (RoPE + KV write, SwiGLU, residual add), row gather, greedy
// argmax and the cache shift's key rotation (the decode attention is in
// k_attn_decode.hip).
//
// The math of each step is the Llama layer of the Ollama engine page ("Deep
// dive: the Llama forward pass in Go"): RMSNorm, Q/K/V projections, RoPE,
// scaled dot-product attention over cached K/V with fewer KV heads than
// query heads, output projection + residual, RMSNorm, SILU(gate) * up, down
// projection + residual.  Decode is bound by HBM (llama.cpp walkthrough,
// "KV-cache and the Prefill / Decode stages": decode is memory-bound), so the
// GEMV streams each weight row once with 16-byte loads per lane and keeps the
// activations in float32.
#include <algorithm>
#include <type_traits>

#include "k_common.hpp"
#include "kernels.hpp"
#include "tdf.h"

namespace tdf {

// ---------------------------------------------------------------------------
// small kernels

// block sum of 256 threads (4 waves); every thread gets the total
__device__ __forceinline__ float block_sum256(float v, float* red4) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = v;
  __syncthreads();
  return red4[0] + red4[1] + red4[2] + red4[3];
}

// Storage of the weight matrices and the embedding table.  A Q8_0 matrix
// [rows][K] is rows*K int8 values q followed by its fp16 block scales
// [rows][K/32]; element (r, k) is scale[(r*K + k) / 32] * q[r*K + k].
enum WeightKind : int { W_F32 = 0, W_BF16 = 1, W_Q8 = 2 };

__host__ __device__ __forceinline__ constexpr int weight_kind(int dtype) {
  return dtype == TDF_BF16 ? W_BF16 : dtype == TDF_Q8_0 ? W_Q8 : W_F32;
}

// fp16 block scales of a Q8_0 matrix of `rows` rows of K elements
__device__ __forceinline__ const uint16_t* q8_scales(const void* w, int64_t rows, int K) {
  return (const uint16_t*)((const int8_t*)w + rows * K);
}

// signed byte b (0..3) of a 32-bit word, as float
__device__ __forceinline__ float sbyte(uint32_t v, int b) {
  return (float)((int32_t)(v << (24 - 8 * b)) >> 24);
}

template <int WT>
__global__ void __launch_bounds__(256) embed_kernel(const void* __restrict__ table, int64_t n_rows,
                                                    const int32_t* __restrict__ tokens, int d,
                                                    float* __restrict__ x, const float* __restrict__ g,
                                                    float* __restrict__ u, float* __restrict__ ssp,
                                                    int stride) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int64_t row = (int64_t)tokens[t] * d;
  float* xr = x + (int64_t)t * d;
  float* ur = u ? u + (int64_t)t * d : nullptr;
  float ss = 0.f;
  if ((d & 3) == 0) {
#pragma unroll 4
    for (int k = threadIdx.x * 4; k < d; k += 1024) {
      float4 v;
      if (WT == W_BF16) {
        const uint2 q = *(const uint2*)((const uint16_t*)table + row + k);
        v = make_float4(__builtin_bit_cast(float, q.x << 16), __builtin_bit_cast(float, q.x & 0xFFFF0000u),
                        __builtin_bit_cast(float, q.y << 16), __builtin_bit_cast(float, q.y & 0xFFFF0000u));
      } else if (WT == W_Q8) {
        // four int8 of one 32-element block (d is a multiple of 32)
        const uint32_t q = *(const uint32_t*)((const int8_t*)table + row + k);
        const float sc = f16_to_f32(q8_scales(table, n_rows, d)[(row + k) >> 5]);
        v = make_float4(sc * sbyte(q, 0), sc * sbyte(q, 1), sc * sbyte(q, 2), sc * sbyte(q, 3));
      } else {
        v = *(const float4*)((const float*)table + row + k);
      }
      *(float4*)(xr + k) = v;
      if (g) {
        const float4 gv = *(const float4*)(g + k);
        *(float4*)(ur + k) = make_float4(gv.x * v.x, gv.y * v.y, gv.z * v.z, gv.w * v.w);
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
    }
  } else {
    for (int k = threadIdx.x; k < d; k += 256) {
      const float v = WT == W_BF16 ? bf16_to_f32(((const uint16_t*)table)[row + k]) : ((const float*)table)[row + k];
      xr[k] = v;
      if (g) {
        ur[k] = g[k] * v;
        ss += v * v;
      }
    }
  }
  if (g) {
    ss = block_sum256(ss, red);
    if (threadIdx.x == 0) ssp[(int64_t)t * stride] = ss;
  }
}

hipError_t launch_embed(const void* table, int weight_dtype, int n_rows, const int32_t* tokens, int T, int d,
                        float* x, const float* g, float* u, float* ssp, int stride, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int wk = weight_kind(weight_dtype);
  if (wk == W_Q8 && d % 32 != 0) return hipErrorInvalidValue;
  if (wk == W_BF16)
    embed_kernel<W_BF16><<<T, 256, 0, s>>>(table, n_rows, tokens, d, x, g, u, ssp, stride);
  else if (wk == W_Q8)
    embed_kernel<W_Q8><<<T, 256, 0, s>>>(table, n_rows, tokens, d, x, g, u, ssp, stride);
  else
    embed_kernel<W_F32><<<T, 256, 0, s>>>(table, n_rows, tokens, d, x, g, u, ssp, stride);
  return hipGetLastError();
}

template <int P>
__global__ void __launch_bounds__(256) rmsnorm_kernel(const float* __restrict__ x,
                                                      const float* __restrict__ g, int d, float eps,
                                                      float* __restrict__ out_f32,
                                                      uint16_t* __restrict__ out_hi,
                                                      uint16_t* __restrict__ out_lo) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const float* xr = x + (int64_t)t * d;
  const int64_t ro = (int64_t)t * d;
  if ((d & 3) == 0 && d <= P * 1024) {
    // rows of up to 1024 P: the row stays in registers between the two
    // passes, and the gains are requested with it; loads are clamped and
    // masked by a multiply (no loads under branches)
    float4 xv[P], gv[P];
    float ss = 0.f;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int k = threadIdx.x * 4 + p * 1024;
      const float4 v = *(const float4*)(xr + min(k, d - 4));
      gv[p] = *(const float4*)(g + min(k, d - 4));
      const float on = k < d ? 1.f : 0.f;
      xv[p] = make_float4(v.x * on, v.y * on, v.z * on, v.w * on);
      ss += xv[p].x * xv[p].x + xv[p].y * xv[p].y + xv[p].z * xv[p].z + xv[p].w * xv[p].w;
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    ss = (red[0] + red[1]) + (red[2] + red[3]);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int k = threadIdx.x * 4 + p * 1024;
      if (k >= d) break;
      const float v[4] = {xv[p].x * r * gv[p].x, xv[p].y * r * gv[p].y, xv[p].z * r * gv[p].z, xv[p].w * r * gv[p].w};
      if (out_f32) *(float4*)(out_f32 + ro + k) = make_float4(v[0], v[1], v[2], v[3]);
      if (out_hi) {
        uint16_t h[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split_bf16(v[e], h[e], l[e]);
        *(uint2*)(out_hi + ro + k) = make_uint2(h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16);
        *(uint2*)(out_lo + ro + k) = make_uint2(l[0] | (uint32_t)l[1] << 16, l[2] | (uint32_t)l[3] << 16);
      }
    }
    return;
  }
  float ss = 0.f;
  for (int k = threadIdx.x; k < d; k += 256) ss += xr[k] * xr[k];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  ss = red[0] + red[1] + red[2] + red[3];
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  for (int k = threadIdx.x; k < d; k += 256) {
    float v = xr[k] * r * g[k];
    if (out_f32) out_f32[ro + k] = v;
    if (out_hi) split_bf16(v, out_hi[ro + k], out_lo[ro + k]);
  }
}

hipError_t launch_rmsnorm(const float* x, const float* g, int T, int d, float eps, float* out_f32,
                          uint16_t* out_hi, uint16_t* out_lo, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if ((out_hi == nullptr) != (out_lo == nullptr)) return hipErrorInvalidValue;
  // float4 per thread: 4 for rows of up to 4096 (no clamped duplicate
  // requests), else 8
  if (d <= 4 * 1024) rmsnorm_kernel<4><<<T, 256, 0, s>>>(x, g, d, eps, out_f32, out_hi, out_lo);
  else rmsnorm_kernel<8><<<T, 256, 0, s>>>(x, g, d, eps, out_f32, out_hi, out_lo);
  return hipGetLastError();
}

__global__ void scatter_kernel(int32_t* __restrict__ dst, const int64_t* __restrict__ pairs, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[pairs[2 * i]] = (int32_t)pairs[2 * i + 1];
}

hipError_t launch_scatter(int32_t* dst, const int64_t* pairs, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  scatter_kernel<<<(n + 255) / 256, 256, 0, s>>>(dst, pairs, n);
  return hipGetLastError();
}

// cs[t][i] = (cos, sin)(pos[t] * theta^(-2i/hd)), angles in double
__global__ void rope_table_kernel(const int32_t* __restrict__ pos, const double* __restrict__ inv_freq,
                                  int half, int n, float2* __restrict__ cs) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int t = i / half, j = i % half;
  double sn, c;
  sincos((double)pos[t] * inv_freq[j], &sn, &c);
  cs[i] = make_float2((float)c, (float)sn);
}

hipError_t launch_rope_table(const int32_t* pos, const double* inv_freq, int T, int half, float2* cs,
                             hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int n = T * half;
  rope_table_kernel<<<(n + 255) / 256, 256, 0, s>>>(pos, inv_freq, half, n, cs);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) gather_rows_kernel(const float* __restrict__ src,
                                                          const int32_t* __restrict__ rows, int d,
                                                          float* __restrict__ dst, const float* __restrict__ g,
                                                          float* __restrict__ u, float* __restrict__ ssp,
                                                          int stride) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  const float* sr = src + (int64_t)(rows ? rows[r] : r) * d;
  float ss = 0.f;
  for (int k = threadIdx.x; k < d; k += 256) {
    const float v = sr[k];
    if (dst) dst[(int64_t)r * d + k] = v;
    if (g) {
      u[(int64_t)r * d + k] = g[k] * v;
      ss += v * v;
    }
  }
  if (g) {
    ss = block_sum256(ss, red);
    if (threadIdx.x == 0) ssp[(int64_t)r * stride] = ss;
  }
}

hipError_t launch_gather_rows(const float* src, const int32_t* rows, int R, int d, float* dst,
                              const float* g, float* u, float* ssp, int stride, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  gather_rows_kernel<<<R, 256, 0, s>>>(src, rows, d, dst, g, u, ssp, stride);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// cache shift: re-rotate the stored keys of some cells (see launch_kv_rotate)

template <typename KvT>
__global__ void __launch_bounds__(256) kv_rotate_kernel(char* kv, size_t layer_stride_bytes, int Hkv,
                                                        int n_ctx, int hd, const int32_t* __restrict__ cells,
                                                        int n_cells, const double2* __restrict__ cs) {
  typedef typename KvStore<KvT>::T ST;
  const int half = hd / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)n_cells * Hkv * half) return;
  const int i = (int)(idx % half);
  const int h = (int)((idx / half) % Hkv);
  const int c = cells[idx / half / Hkv];
  ST* k = (ST*)(kv + (size_t)blockIdx.y * layer_stride_bytes);
  const int64_t e = ((int64_t)h * n_ctx + c) * hd + 2 * i;
  const double y0 = KvStore<KvT>::load(k, e), y1 = KvStore<KvT>::load(k, e + 1);
  const double2 r = cs[i];
  KvStore<KvT>::store(k, e, (float)(y0 * r.x - y1 * r.y));
  KvStore<KvT>::store(k, e + 1, (float)(y0 * r.y + y1 * r.x));
}

hipError_t launch_kv_rotate(void* kv, int kv_dtype, size_t layer_stride_bytes, int L, int Hkv, int n_ctx, int hd,
                            const int32_t* cells, int n_cells, const double2* cs, hipStream_t s) {
  if (n_cells <= 0 || L <= 0) return hipSuccess;
  const int64_t n = (int64_t)n_cells * Hkv * (hd / 2);
  const dim3 grid((unsigned)((n + 255) / 256), (unsigned)L);
  if (kv_dtype == TDF_BF16)
    kv_rotate_kernel<kv_bf16><<<grid, 256, 0, s>>>((char*)kv, layer_stride_bytes, Hkv, n_ctx, hd, cells, n_cells, cs);
  else if (kv_dtype == TDF_F16)
    kv_rotate_kernel<kv_f16><<<grid, 256, 0, s>>>((char*)kv, layer_stride_bytes, Hkv, n_ctx, hd, cells, n_cells, cs);
  else
    kv_rotate_kernel<float><<<grid, 256, 0, s>>>((char*)kv, layer_stride_bytes, Hkv, n_ctx, hd, cells, n_cells, cs);
  return hipGetLastError();
}

// Greedy token: two passes.  Pass 1, block (split j, row r), reduces the
// columns [j*L, j*L + L) of a row to (max, lowest index of the max); pass 2,
// one block per row, reduces the splits.  L = 2048 * m with m the smallest
// multiple that keeps the splits within kArgmaxMaxSplits.  Every thread
// issues its loads up front; masked columns add -inf (an add, not a select,
// so the loads stay out of branches).
constexpr int kArgmaxCols = 2048;  // columns per split and multiple m (256 threads x 2 float4)

__global__ void __launch_bounds__(256) argmax_split_kernel(const float* __restrict__ logits, int V, int m,
                                                           float* __restrict__ pv, int32_t* __restrict__ pi,
                                                           int n_split) {
  const int j = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const float* row = logits + (int64_t)r * V;
  const int lo = j * kArgmaxCols * m, hi = min(V, lo + kArgmaxCols * m);
  float best = -INFINITY;
  int bi = 0x7FFFFFFF;
  if ((V & 3) == 0) {
    for (int c = 0; c < m; ++c) {
      const int n0 = lo + c * kArgmaxCols + tid * 4, n1 = n0 + 1024;
      const float4 a = *(const float4*)(row + min(n0, V - 4));
      const float4 b = *(const float4*)(row + min(n1, V - 4));
      const float ma = n0 < hi ? 0.f : -INFINITY, mb = n1 < hi ? 0.f : -INFINITY;
      argmax_merge(best, bi, a.x + ma, n0);
      argmax_merge(best, bi, a.y + ma, n0 + 1);
      argmax_merge(best, bi, a.z + ma, n0 + 2);
      argmax_merge(best, bi, a.w + ma, n0 + 3);
      argmax_merge(best, bi, b.x + mb, n1);
      argmax_merge(best, bi, b.y + mb, n1 + 1);
      argmax_merge(best, bi, b.z + mb, n1 + 2);
      argmax_merge(best, bi, b.w + mb, n1 + 3);
    }
  } else {
    for (int n = lo + tid; n < hi; n += 256) argmax_merge(best, bi, row[n], n);
  }
  // a masked column can only win with best = -inf everywhere; keep its index valid
  if (best == -INFINITY) bi = 0x7FFFFFFF;
  __shared__ float sv[4];
  __shared__ int si[4];
  wave_argmax(best, bi);
  if ((tid & 63) == 0) {
    sv[tid >> 6] = best;
    si[tid >> 6] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w) argmax_merge(best, bi, sv[w], si[w]);
    pv[(int64_t)r * n_split + j] = best;
    pi[(int64_t)r * n_split + j] = bi;
  }
}

__global__ void __launch_bounds__(256) argmax_final_kernel(const float* __restrict__ pv,
                                                           const int32_t* __restrict__ pi, int n_split,
                                                           int32_t* __restrict__ tok) {
  const int r = blockIdx.x, tid = threadIdx.x;
  const int k = min(tid, n_split - 1);
  const float v = pv[(int64_t)r * n_split + k];
  const int i = pi[(int64_t)r * n_split + k];
  float best = v + (tid < n_split ? 0.f : -INFINITY);
  int bi = tid < n_split ? i : 0x7FFFFFFF;
  __shared__ float sv[4];
  __shared__ int si[4];
  wave_argmax(best, bi);
  if ((tid & 63) == 0) {
    sv[tid >> 6] = best;
    si[tid >> 6] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w) argmax_merge(best, bi, sv[w], si[w]);
    // every logit -inf or NaN: fall back to token 0
    tok[r] = bi == 0x7FFFFFFF ? 0 : bi;
  }
}

int argmax_splits(int V) {
  int m = 1;
  while ((V + kArgmaxCols * m - 1) / (kArgmaxCols * m) > kArgmaxMaxSplits) ++m;
  return (V + kArgmaxCols * m - 1) / (kArgmaxCols * m);
}

hipError_t launch_argmax(const float* logits, int R, int V, int32_t* tok, float* part_v, int32_t* part_i,
                         hipStream_t s) {
  if (R <= 0) return hipSuccess;
  if (V <= 0) return hipErrorInvalidValue;
  int m = 1;
  while ((V + kArgmaxCols * m - 1) / (kArgmaxCols * m) > kArgmaxMaxSplits) ++m;
  const int n_split = (V + kArgmaxCols * m - 1) / (kArgmaxCols * m);
  argmax_split_kernel<<<dim3(n_split, R), 256, 0, s>>>(logits, V, m, part_v, part_i, n_split);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  argmax_final_kernel<<<R, 256, 0, s>>>(part_v, part_i, n_split, tok);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// GEMV: one wave per R/2 output pairs (R = 2 or 4 rows).  For EPI_SWIGLU a
// pair is (gate row n, up row n); otherwise rows (2p, 2p+1), so that a RoPE
// pair (2i, 2i+1) of a head lands in one wave.  Lanes stride the rows in
// chunks of 16 bytes per lane, all NT tokens reuse each weight chunk from
// registers and the R rows share each activation chunk.

// EPL weights of one lane from raw 16-byte vectors: 8 bf16 (one vector), 8
// float32 (two vectors) or 16 int8 of a Q8_0 block half (one vector; the
// block scale is applied to the partial dot product by the caller)
template <int WT>
__device__ __forceinline__ void unpack_w(const uint4* raw, float* w) {
  if (WT == W_BF16) {
    const uint32_t p[4] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[2 * j] = __builtin_bit_cast(float, p[j] << 16);
      w[2 * j + 1] = __builtin_bit_cast(float, p[j] & 0xFFFF0000u);
    }
  } else if (WT == W_Q8) {
    const uint32_t p[4] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) w[4 * j + b] = sbyte(p[j], b);
  } else {
    const uint32_t p[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = __builtin_bit_cast(float, p[j]);
  }
}

// 16 bytes of streamed weights; NT: with the non-temporal hint (the rows are
// read once, so they need not displace the activations in the caches)
template <bool NT>
__device__ __forceinline__ uint4 load_w16(const void* p) {
  if constexpr (NT) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
    return make_uint4(v[0], v[1], v[2], v[3]);
  } else {
    return *(const uint4*)p;
  }
}

// one weight (rows whose length is not a multiple of 8; never Q8_0)
template <int WT>
__device__ __forceinline__ float load1(const void* base, int64_t idx) {
  return WT == W_BF16 ? bf16_to_f32(((const uint16_t*)base)[idx]) : ((const float*)base)[idx];
}

template <typename KvT>
__device__ __forceinline__ void kv_put(void* cache, int64_t idx, float v) {
  KvStore<KvT>::store((typename KvStore<KvT>::T*)cache, idx, v);
}

// Waves per GEMV block: 4, or 32 / R when the epilogue stores K/V rows in a
// Q8_0 cache.  Then a block's 32 rows are exactly one 32-value block of one
// head's K or V row, so the block decides its scale and codes itself.
template <typename KvT, int R> struct GemvWaves { static constexpr int n = 4; };
template <int R> struct GemvWaves<kv_q8, R> { static constexpr int n = 32 / R; };

// sum of r[0..BW)[t] as a pairwise tree ((r0 + r1) + (r2 + r3)) ...
template <int BW, int NT>
__device__ __forceinline__ float block_tree_sum(const float (&r)[BW][NT], int t) {
  float v[BW];
#pragma unroll
  for (int i = 0; i < BW; ++i) v[i] = r[i][t];
#pragma unroll
  for (int w = BW / 2; w >= 1; w /= 2)
#pragma unroll
    for (int i = 0; i < w; ++i) v[i] = v[2 * i] + v[2 * i + 1];
  return v[0];
}

template <int WT, int NT, int EPI, typename KvT, bool NORM, int U, int R>
__global__ void __launch_bounds__((64 * GemvWaves<KvT, R>::n)) gemv_kernel(LinearArgs a, int t0, int nt) {
  static_assert(R == 2 || R == 4, "rows per wave");
  constexpr int BW = GemvWaves<KvT, R>::n, BT = 64 * BW;  // waves and threads per block
  constexpr bool KVQ8 = std::is_same<KvT, kv_q8>::value;
  static_assert(!KVQ8 || (EPI == EPI_QKV && NT == 1), "Q8_0 cache rows: single-token QKV");
  constexpr int P = R / 2;  // output pairs per wave
  __shared__ float red[BW][NT];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wave = blockIdx.x * BW + wid;
  const int N = a.n0 + a.n1 + a.n2;
  const int K = a.K;
  // The R rows of this wave.  Rows past the end are clamped to the last row
  // for the loads (all in bounds) and their outputs dropped: rv[i] = 0.
  // sc[i]: block scales of row i's matrix (Q8_0).  Inactive waves (no valid
  // row) still join the block reductions.
  int row[R];
  bool rv[R];
  const void* p[R];
  const uint16_t* sc[R];
  int64_t off[R];
  if (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int n = wave * P + j;
      rv[2 * j] = rv[2 * j + 1] = n < a.n0;
      const int nc = min(n, a.n0 - 1);
      row[2 * j] = row[2 * j + 1] = n;
      p[2 * j] = a.w0;
      p[2 * j + 1] = a.w1;
      off[2 * j] = off[2 * j + 1] = (int64_t)nc * K;
      sc[2 * j] = WT == W_Q8 ? q8_scales(a.w0, a.n0, K) : nullptr;
      sc[2 * j + 1] = WT == W_Q8 ? q8_scales(a.w1, a.n0, K) : nullptr;
    }
  } else {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int r = R * wave + i;
      rv[i] = r < N;
      row[i] = r;
      const int rc = min(r, N - 1);
      if (rc < a.n0) {
        p[i] = a.w0; off[i] = (int64_t)rc * K;
        sc[i] = WT == W_Q8 ? q8_scales(a.w0, a.n0, K) : nullptr;
      } else if (rc < a.n0 + a.n1) {
        p[i] = a.w1; off[i] = (int64_t)(rc - a.n0) * K;
        sc[i] = WT == W_Q8 ? q8_scales(a.w1, a.n1, K) : nullptr;
      } else {
        p[i] = a.w2; off[i] = (int64_t)(rc - a.n0 - a.n1) * K;
        sc[i] = WT == W_Q8 ? q8_scales(a.w2, a.n2, K) : nullptr;
      }
    }
  }
  const bool active = rv[0];
  const float* act = a.act_f32 + (int64_t)t0 * K;

  // RMSNorm consumer: the block's threads fetch the producer's partial
  // sums of x^2 together with the first batch of weights (same memory round
  // trip) and add them up once per block after the row loop.  The loads use
  // clamped indices and are masked by a multiply: a load under a divergent
  // branch (or a select of a load, which becomes one) makes the compiler wait
  // for every load in flight.
  constexpr int kNormPer = 4;  // partials per thread fetched with the weights (4 * BT per block)
  float nss[NORM ? NT : 1][kNormPer];
#pragma unroll
  for (int t = 0; t < (NORM ? NT : 1); ++t)
#pragma unroll
    for (int q = 0; q < kNormPer; ++q) nss[t][q] = 0.f;
  auto norm_fetch = [&](float on) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < kNormPer; ++q) {
        const int pidx = threadIdx.x + q * BT;
        const int tc = t < nt ? t : nt - 1;
        const float v = a.norm_ssp[(int64_t)(t0 + tc) * a.norm_stride + min(pidx, a.norm_nparts - 1)];
        nss[t][q] += v * ((t < nt && pidx < a.norm_nparts) ? on : 0.f);
      }
  };
  bool norm_fetched = false;

  float acc[R][NT];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = 0.f;

  // Each lane takes EPL consecutive elements of a chunk of 64 * EPL: 8 bf16
  // or float32, or 16 int8 (half a Q8_0 block, one scale per lane)
  constexpr int EPL = WT == W_Q8 ? 16 : 8;
  constexpr int CH = 64 * EPL;
  constexpr int WV = WT == W_F32 ? 2 : 1;                      // 16-byte vectors per lane and chunk
  constexpr int ESZ = WT == W_F32 ? 4 : WT == W_BF16 ? 2 : 1;  // bytes per weight
  constexpr int XV = EPL / 4;                                  // float4 activations per lane and chunk
  // non-temporal weight loads: measured faster for bf16 weights (LM head
  // 152 vs 166 us at 8B widths) and for four Q8_0 rows per wave, slower for
  // two Q8_0 rows per wave
  constexpr bool NTW = WT != W_Q8 || R == 4;
  // the R rows' partial dot products of one chunk (weights W[R][EPL], one
  // token's activations XV4) into their accumulators, the rows' FMA chains
  // interleaved (Q8_0: the int8 dot products times the block scales S[R])
#define TDF_GEMV_CHUNK(W, S, XV4, T)                                                    \
  {                                                                                     \
    const float* x_ = (const float*)(XV4);                                              \
    if (WT == W_Q8) {                                                                   \
      float d_[R];                                                                      \
      _Pragma("unroll") for (int i_ = 0; i_ < R; ++i_) d_[i_] = 0.f;                    \
      _Pragma("unroll") for (int j_ = 0; j_ < EPL; ++j_)                                \
        _Pragma("unroll") for (int i_ = 0; i_ < R; ++i_) d_[i_] = fmaf(W[i_][j_], x_[j_], d_[i_]); \
      _Pragma("unroll") for (int i_ = 0; i_ < R; ++i_) acc[i_][T] = fmaf(S[i_], d_[i_], acc[i_][T]); \
    } else {                                                                            \
      _Pragma("unroll") for (int j_ = 0; j_ < EPL; ++j_)                                \
        _Pragma("unroll") for (int i_ = 0; i_ < R; ++i_)                                \
          acc[i_][T] = fmaf(W[i_][j_], x_[j_], acc[i_][T]);                             \
    }                                                                                   \
  }

  if (active) {
    if ((K & (EPL - 1)) == 0) {
      // Batches of U chunks: every lane issues all R*U weight loads (16 bytes
      // of bf16 or int8, or 2x16 of float32, each) and the activation loads
      // of the batch before it waits, so each wave keeps R*U*16 bytes per
      // lane of weights in flight.  The last batch may be partial: its loads
      // are clamped to the last chunk and the surplus chunks skipped (a
      // wave-uniform test).
      const int n_full = K / CH;
      for (int it = 0; it < n_full; it += U) {
        uint4 raw[U][R][WV];
        float sw[U][R];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t k = (int64_t)min(it + u, n_full - 1) * CH + lane * EPL;
#pragma unroll
          for (int i = 0; i < R; ++i) {
#pragma unroll
            for (int v = 0; v < WV; ++v)
              raw[u][i][v] = load_w16<NTW>((const char*)p[i] + (off[i] + k) * ESZ + 16 * v);
            sw[u][i] = WT == W_Q8 ? f16_to_f32(sc[i][(off[i] + k) >> 5]) : 1.f;
          }
        }
        // the norm partials ride with the first batch (counted once)
        if (NORM) norm_fetch(it == 0 ? 1.f : 0.f);
        float4 xv[NT][U][XV];
#pragma unroll
        for (int t = 0; t < NT; ++t)
          if (t < nt) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
              const int k = min(it + u, n_full - 1) * CH + lane * EPL;
#pragma unroll
              for (int v = 0; v < XV; ++v) xv[t][u][v] = *(const float4*)(act + (int64_t)t * K + k + 4 * v);
            }
          }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (it + u >= n_full) break;
          float w[R][EPL];
#pragma unroll
          for (int i = 0; i < R; ++i) unpack_w<WT>(raw[u][i], w[i]);
#pragma unroll
          for (int t = 0; t < NT; ++t)
            if (t < nt) TDF_GEMV_CHUNK(w, sw[u], xv[t][u], t)
        }
      }
      norm_fetched = n_full > 0;
      // the ragged end of the row (K not a multiple of the chunk)
      for (int k = n_full * CH + lane * EPL; k < K; k += CH) {
        uint4 raw[R][WV];
        float sw[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
#pragma unroll
          for (int v = 0; v < WV; ++v) raw[i][v] = load_w16<NTW>((const char*)p[i] + (off[i] + k) * ESZ + 16 * v);
          sw[i] = WT == W_Q8 ? f16_to_f32(sc[i][(off[i] + k) >> 5]) : 1.f;
        }
        float w[R][EPL];
#pragma unroll
        for (int i = 0; i < R; ++i) unpack_w<WT>(raw[i], w[i]);
#pragma unroll
        for (int t = 0; t < NT; ++t)
          if (t < nt) {
            float4 xv[XV];
#pragma unroll
            for (int v = 0; v < XV; ++v) xv[v] = *(const float4*)(act + (int64_t)t * K + k + 4 * v);
            TDF_GEMV_CHUNK(w, sw, xv, t)
          }
      }
    } else if (WT != W_Q8) {
      for (int k = lane; k < K; k += 64) {
        float w[R];
#pragma unroll
        for (int i = 0; i < R; ++i) w[i] = load1<WT>(p[i], off[i] + k);
#pragma unroll
        for (int t = 0; t < NT; ++t)
          if (t < nt) {
            const float x = act[(int64_t)t * K + k];
#pragma unroll
            for (int i = 0; i < R; ++i) acc[i][t] = fmaf(w[i], x, acc[i][t]);
          }
      }
    }
  }
#undef TDF_GEMV_CHUNK
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = wave_sum(acc[i][t]);
  if (NORM) {
    // RMS scale 1/sqrt(ss/K + eps), ss = sum of the producer's partials
    if (!norm_fetched) norm_fetch(1.f);  // short or ragged rows, inactive waves
    __shared__ float red_n[BW][NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float ss = 0.f;
#pragma unroll
      for (int q = 0; q < kNormPer; ++q) ss += nss[t][q];
      if (t < nt)
        for (int pi = threadIdx.x + kNormPer * BT; pi < a.norm_nparts; pi += BT)
          ss += a.norm_ssp[(int64_t)(t0 + t) * a.norm_stride + pi];
      ss = wave_sum(ss);
      if (lane == 0) red_n[wid][t] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float ss = block_tree_sum<BW, NT>(red_n, t);
      const float r = 1.0f / sqrtf(ss / (float)K + a.norm_eps);
#pragma unroll
      for (int i = 0; i < R; ++i) acc[i][t] *= r;
    }
  }
  // lane t writes token t; pair j covers rows 2j and 2j+1 of the wave (r1 ==
  // r0: a single row at the end of the matrix stack)
  const bool produce = EPI == EPI_RESIDUAL && a.next_g != nullptr;
  // Q8_0 cache: the block's 32 K or V values (row r at [r % 32])
  __shared__ float kvq[KVQ8 ? 32 : 1];
  float sq[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    sq[t] = 0.f;
    if (lane != t || t >= nt) continue;
    const int tg = t0 + t;
#pragma unroll
    for (int j = 0; j < P; ++j) {
      if (!rv[2 * j]) continue;
      const int r0 = row[2 * j];
      const int r1 = rv[2 * j + 1] ? row[2 * j + 1] : r0;
      const float y0 = acc[2 * j][t], y1 = acc[2 * j + 1][t];
      if (EPI == EPI_STORE) {
        a.out[(int64_t)tg * a.ldo + r0] = y0;
        if (r1 != r0) a.out[(int64_t)tg * a.ldo + r1] = y1;
      } else if (EPI == EPI_RESIDUAL) {
        float* xo = a.out + (int64_t)tg * a.ldo;
        const float x0 = xo[r0] + y0;
        xo[r0] = x0;
        if (produce) {
          a.next_u[(int64_t)tg * a.ldo + r0] = a.next_g[r0] * x0;
          sq[t] += x0 * x0;
        }
        if (r1 != r0) {
          const float x1 = xo[r1] + y1;
          xo[r1] = x1;
          if (produce) {
            a.next_u[(int64_t)tg * a.ldo + r1] = a.next_g[r1] * x1;
            sq[t] += x1 * x1;
          }
        }
      } else if (EPI == EPI_SWIGLU) {
        a.out[(int64_t)tg * a.ldo + r0] = silu(y0) * y1;
      } else if (EPI == EPI_QKV) {
        const int hd = a.head_dim;
        if (r0 < a.n0 + a.n1) {
          // q or k row pair (2i, 2i+1) of one head: rotate by pos * theta^(-2i/hd)
          const int lr = r0 < a.n0 ? r0 : r0 - a.n0;
          const int i = (lr % hd) >> 1;
          const float2 cs = a.rope_cs[(int64_t)tg * (hd >> 1) + i];
          const float z0 = y0 * cs.x - y1 * cs.y, z1 = y0 * cs.y + y1 * cs.x;
          if (r0 < a.n0) {
            a.q_out[(int64_t)tg * a.n0 + lr] = z0;
            a.q_out[(int64_t)tg * a.n0 + lr + 1] = z1;
          } else if constexpr (KVQ8) {
            kvq[r0 & 31] = z0;
            kvq[(r0 & 31) + 1] = z1;
          } else {
            const int64_t ci = ((int64_t)(lr / hd) * a.n_ctx + a.slots[tg]) * hd + (lr % hd);
            kv_put<KvT>(a.k_cache, ci, z0);
            kv_put<KvT>(a.k_cache, ci + 1, z1);
          }
        } else if constexpr (KVQ8) {
          kvq[r0 & 31] = y0;
          kvq[(r0 & 31) + 1] = y1;
        } else {
          const int lr = r0 - a.n0 - a.n1;
          const int64_t ci = ((int64_t)(lr / hd) * a.n_ctx + a.slots[tg]) * hd + (lr % hd);
          kv_put<KvT>(a.v_cache, ci, y0);
          if (r1 != r0) kv_put<KvT>(a.v_cache, ci + 1, y1);
        }
      }
    }
  }
  if (produce) {
    // per-block partial sums of x_new^2, one per token
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float v = __shfl(sq[t], t, kWave);
      if (lane == 0) red[wid][t] = v;
    }
    __syncthreads();
    if (threadIdx.x < nt) {
      float v = red[0][threadIdx.x];
#pragma unroll
      for (int w = 1; w < BW; ++w) v += red[w][threadIdx.x];
      a.next_ssp[(int64_t)(t0 + threadIdx.x) * a.next_stride + blockIdx.x] = v;
    }
  }
  if constexpr (KVQ8) {
    // A K or V block (rows n0 .. N; the row counts and head_dim are multiples
    // of 32, checked by the launcher): wave 0 quantizes the 32 values into
    // their cell, one code per lane, with the rule of kv_quantize.
    const int rb = blockIdx.x * 32;
    if (rb >= a.n0 && rb < N) {
      __syncthreads();
      if (wid == 0) {
        const bool is_v = rb >= a.n0 + a.n1;
        const int lr = rb - a.n0 - (is_v ? a.n1 : 0);
        const int hd = a.head_dim, Hkv = a.n1 / hd;
        const float x = lane < 32 ? kvq[lane] : 0.f;
        const uint16_t dbits = q8_scale_bits(wave_max(fabsf(x)));
        const float d = f16_to_f32(dbits);
        const int64_t crow = (int64_t)(lr / hd) * a.n_ctx + a.slots[t0];
        int8_t* codes = (int8_t*)(is_v ? a.v_cache : a.k_cache);
        if (lane < 32) codes[crow * hd + (lr % hd) + lane] = q8_code(x, d);
        if (lane == 0) {
          uint16_t* scales = (uint16_t*)(codes + (int64_t)Hkv * a.n_ctx * hd);
          scales[crow * (hd / 32) + (lr % hd) / 32] = dbits;
        }
      }
    }
  }
}

// Residual GEMVs always take two rows per wave: their per-block partial sums
// of x^2 (8 rows per block) feed the next RMSNorm.
int gemv_residual_parts(int N) { return ((N + 1) / 2 + 3) / 4; }

template <int WT, int NT, int EPI, typename KvT, int R>
static hipError_t gemv_launch_r(const LinearArgs& a, hipStream_t s) {
  const int N = a.n0 + a.n1 + a.n2;
  constexpr int P = R / 2;
  constexpr int BW = GemvWaves<KvT, R>::n;
  const int waves = EPI == EPI_SWIGLU ? (a.n0 + P - 1) / P : (N + R - 1) / R;
  const int blocks = (waves + BW - 1) / BW;
  // chunks per batch at two rows per wave: 8 for a single token on grids of
  // at least 8192 rows (the large matrices), else 4 (2 for float32 weights);
  // a Q8_0 chunk holds twice the elements of a bf16 one, so half as many per
  // batch (one when several tokens' activations share the registers).  Four
  // rows per wave take half as many chunks per batch.
  constexpr int U_MANY2 = WT == W_BF16 ? 4 : WT == W_Q8 ? (NT == 1 ? 2 : 1) : 2;
  constexpr int U_BIG2 = NT == 1 ? (WT == W_BF16 ? 8 : WT == W_Q8 ? 4 : U_MANY2) : U_MANY2;
  constexpr int U_MANY = R == 2 ? U_MANY2 : (U_MANY2 > 1 ? U_MANY2 / 2 : 1);
  constexpr int U_BIG = R == 2 ? U_BIG2 : (U_BIG2 > 1 ? U_BIG2 / 2 : 1);
  const bool big = (int64_t)waves * R >= 8 * 1024;
  for (int t0 = 0; t0 < a.T; t0 += NT) {
    const int nt = a.T - t0 < NT ? a.T - t0 : NT;
    if (a.norm_ssp) {
      if (big) gemv_kernel<WT, NT, EPI, KvT, true, U_BIG, R><<<blocks, 64 * BW, 0, s>>>(a, t0, nt);
      else gemv_kernel<WT, NT, EPI, KvT, true, U_MANY, R><<<blocks, 64 * BW, 0, s>>>(a, t0, nt);
    } else {
      if (big) gemv_kernel<WT, NT, EPI, KvT, false, U_BIG, R><<<blocks, 64 * BW, 0, s>>>(a, t0, nt);
      else gemv_kernel<WT, NT, EPI, KvT, false, U_MANY, R><<<blocks, 64 * BW, 0, s>>>(a, t0, nt);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Single-token QKV into a Q8_0 cache: one block per 32 rows (every row count
// is a multiple of 32), R rows per wave, U chunks per batch.
template <int WT, int R, int U>
static hipError_t gemv_launch_kvq8(const LinearArgs& a, hipStream_t s) {
  constexpr int BT = 64 * GemvWaves<kv_q8, R>::n;
  const int blocks = (a.n0 + a.n1 + a.n2) / 32;
  if (a.norm_ssp) gemv_kernel<WT, 1, EPI_QKV, kv_q8, true, U, R><<<blocks, BT, 0, s>>>(a, 0, 1);
  else gemv_kernel<WT, 1, EPI_QKV, kv_q8, false, U, R><<<blocks, BT, 0, s>>>(a, 0, 1);
  return hipGetLastError();
}

// rows per wave: 4 for the single-token Q8_0 GEMV of matrices with at least
// 16384 rows (so that each wave still carries 16 bytes per lane and row for
// each chunk of a bf16 wave), else 2
template <int WT, int NT, int EPI, typename KvT>
static hipError_t gemv_launch_t(const LinearArgs& a, hipStream_t s) {
  if constexpr (WT == W_Q8 && NT == 1 && EPI != EPI_RESIDUAL) {
    const int rows = EPI == EPI_SWIGLU ? 2 * a.n0 : a.n0 + a.n1 + a.n2;
    if (rows >= 16 * 1024) return gemv_launch_r<WT, NT, EPI, KvT, 4>(a, s);
  }
  return gemv_launch_r<WT, NT, EPI, KvT, 2>(a, s);
}

template <int WT, int NT>
static hipError_t gemv_dispatch_epi(const LinearArgs& a, hipStream_t s) {
  switch (a.epi) {
    case EPI_STORE: return gemv_launch_t<WT, NT, EPI_STORE, float>(a, s);
    case EPI_RESIDUAL: return gemv_launch_t<WT, NT, EPI_RESIDUAL, float>(a, s);
    case EPI_SWIGLU: return gemv_launch_t<WT, NT, EPI_SWIGLU, float>(a, s);
    case EPI_QKV:
      if (a.kv_dtype == TDF_Q8_0) {
        // single token only; whole 32-value blocks of K/V rows per GEMV block
        if constexpr (NT == 1) {
          if (a.T != 1 || a.head_dim % 32 || a.n0 % 32 || a.n1 % 32 || a.n2 % 32 || a.n1 != a.n2)
            return hipErrorInvalidValue;
          return gemv_launch_kvq8<WT, 2, WT == W_Q8 ? 2 : 4>(a, s);
        }
        return hipErrorInvalidValue;
      }
      if (a.kv_dtype == TDF_BF16) return gemv_launch_t<WT, NT, EPI_QKV, kv_bf16>(a, s);
      if (a.kv_dtype == TDF_F16) return gemv_launch_t<WT, NT, EPI_QKV, kv_f16>(a, s);
      return gemv_launch_t<WT, NT, EPI_QKV, float>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int WT>
static hipError_t gemv_dispatch_tokens(const LinearArgs& a, hipStream_t s) {
  // tokens per pass: 1 for the latency-critical single-token step, else 8
  if (a.T == 1) return gemv_dispatch_epi<WT, 1>(a, s);
  if (a.T <= 4) return gemv_dispatch_epi<WT, 4>(a, s);
  return gemv_dispatch_epi<WT, 8>(a, s);
}

hipError_t launch_linear_gemv(const LinearArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  switch (weight_kind(a.weight_dtype)) {
    case W_BF16: return gemv_dispatch_tokens<W_BF16>(a, s);
    case W_Q8:
      if (a.K % 32 != 0) return hipErrorInvalidValue;
      return gemv_dispatch_tokens<W_Q8>(a, s);
    default: return gemv_dispatch_tokens<W_F32>(a, s);
  }
}

}  // namespace tdf
