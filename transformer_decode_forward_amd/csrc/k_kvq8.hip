// Q8_0 KV cache (a quantized cache type: the Ollama backends chapter and the
// llama.cpp walkthrough's KV-cache section name quantized cache types without
// defining them).  A cached K or V row of head_dim values is stored as blocks
// of 32: one fp16 scale d = fp16(max|x| / 127) and 32 int8 codes
// q = round-half-even(x / d) clamped to [-127, 127] (all zero when d is 0),
// decided in float32; the value read back is d * q.
//
// Layout of one layer's K (or V) array: the codes [Hkv][n_ctx][hd] int8, then
// the scales [Hkv][n_ctx][hd / 32] fp16.
//
// A single-token projection quantizes its K/V blocks in its own epilogue
// (the decode GEMV); the others write float32 K/V rows into a staging area,
// and kv_quantize then stores each 32-element block of a row in its cell.  The cache shift
// rotates the stored keys in double and re-quantizes them.
#include "k_common.hpp"
#include "kernels.hpp"
#include "tdf.h"

namespace tdf {

// one block: codes and scale of 32 float32 values
__device__ __forceinline__ void q8_block(const float* x, int8_t* q, uint16_t& dbits) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  dbits = q8_scale_bits(amax);
  const float d = f16_to_f32(dbits);
#pragma unroll
  for (int i = 0; i < 32; ++i) q[i] = q8_code(x[i], d);
}

// src row (t, h) at src + t * ts + h * hs (float32, hd values); destination
// cell cells[t] of head h.  One thread per (t, h, block, K|V).
__global__ void __launch_bounds__(256) kv_quantize_kernel(const float* __restrict__ sk, const float* __restrict__ sv,
                                                          int64_t ts, int64_t hs, int T, int Hkv, int hd,
                                                          const int32_t* __restrict__ cells, int8_t* dk, int8_t* dv,
                                                          int n_ctx) {
  const int nb = hd / 32;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)2 * T * Hkv * nb) return;
  const int b = (int)(idx % nb);
  const int h = (int)((idx / nb) % Hkv);
  const int t = (int)((idx / nb / Hkv) % T);
  const bool is_v = idx >= (int64_t)T * Hkv * nb;
  const float* src = (is_v ? sv : sk) + t * ts + h * hs + b * 32;
  int8_t* dst = is_v ? dv : dk;
  float x[32];
#pragma unroll
  for (int i = 0; i < 32; i += 4) {
    const float4 v = *(const float4*)(src + i);
    x[i] = v.x; x[i + 1] = v.y; x[i + 2] = v.z; x[i + 3] = v.w;
  }
  int8_t q[32];
  uint16_t dbits;
  q8_block(x, q, dbits);
  const int64_t row = (int64_t)h * n_ctx + cells[t];
  uint32_t w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    w[j] = (uint32_t)(uint8_t)q[4 * j] | ((uint32_t)(uint8_t)q[4 * j + 1] << 8) |
           ((uint32_t)(uint8_t)q[4 * j + 2] << 16) | ((uint32_t)(uint8_t)q[4 * j + 3] << 24);
  uint4* out = (uint4*)(dst + row * hd + b * 32);
  out[0] = make_uint4(w[0], w[1], w[2], w[3]);
  out[1] = make_uint4(w[4], w[5], w[6], w[7]);
  uint16_t* scales = (uint16_t*)(dst + (int64_t)Hkv * n_ctx * hd);
  scales[row * nb + b] = dbits;
}

hipError_t launch_kv_quantize(const float* src_k, const float* src_v, int64_t t_stride, int64_t h_stride, int T,
                              int Hkv, int hd, const int32_t* cells, void* k_dst, void* v_dst, int n_ctx,
                              hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (hd % 32 != 0) return hipErrorInvalidValue;
  const int64_t n = (int64_t)2 * T * Hkv * (hd / 32);
  kv_quantize_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(src_k, src_v, t_stride, h_stride, T, Hkv, hd,
                                                                  cells, (int8_t*)k_dst, (int8_t*)v_dst, n_ctx);
  return hipGetLastError();
}

// Rotation of the stored keys of n_cells cells by the per-pair angles cs:
// one thread per (cell, head, block) and layer (grid.y): dequantize the 32
// values, rotate each pair (2i, 2i+1) in double, round to float32 and store
// the block again.
__global__ void __launch_bounds__(256) kv_rotate_q8_kernel(char* kv, size_t layer_stride_bytes, int Hkv, int n_ctx,
                                                           int hd, const int32_t* __restrict__ cells, int n_cells,
                                                           const double2* __restrict__ cs) {
  const int nb = hd / 32;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)n_cells * Hkv * nb) return;
  const int b = (int)(idx % nb);
  const int h = (int)((idx / nb) % Hkv);
  const int c = cells[idx / nb / Hkv];
  int8_t* k = (int8_t*)(kv + (size_t)blockIdx.y * layer_stride_bytes);
  uint16_t* scales = (uint16_t*)(k + (int64_t)Hkv * n_ctx * hd);
  const int64_t row = (int64_t)h * n_ctx + c;
  const float d = f16_to_f32(scales[row * nb + b]);
  int8_t* q = k + row * hd + b * 32;
  float x[32];
#pragma unroll
  for (int i = 0; i < 32; i += 2) {
    const double y0 = (double)(d * (float)q[i]), y1 = (double)(d * (float)q[i + 1]);
    const double2 r = cs[(b * 32 + i) / 2];
    x[i] = (float)(y0 * r.x - y1 * r.y);
    x[i + 1] = (float)(y0 * r.y + y1 * r.x);
  }
  int8_t qn[32];
  uint16_t dbits;
  q8_block(x, qn, dbits);
#pragma unroll
  for (int i = 0; i < 32; ++i) q[i] = qn[i];
  scales[row * nb + b] = dbits;
}

hipError_t launch_kv_rotate_q8(void* kv, size_t layer_stride_bytes, int L, int Hkv, int n_ctx, int hd,
                               const int32_t* cells, int n_cells, const double2* cs, hipStream_t s) {
  if (n_cells <= 0 || L <= 0) return hipSuccess;
  if (hd % 32 != 0) return hipErrorInvalidValue;
  const int64_t n = (int64_t)n_cells * Hkv * (hd / 32);
  const dim3 grid((unsigned)((n + 255) / 256), (unsigned)L);
  kv_rotate_q8_kernel<<<grid, 256, 0, s>>>((char*)kv, layer_stride_bytes, Hkv, n_ctx, hd, cells, n_cells, cs);
  return hipGetLastError();
}

}  // namespace tdf
