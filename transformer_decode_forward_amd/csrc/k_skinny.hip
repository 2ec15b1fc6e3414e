// Linear layers of ubatches of 9..32 tokens (decode steps of several
// sequences): the weights are streamed once, so the kernel is built like a
// GEMV with the matrix cores doing the dot products.
//
// Pass 1 (skinny_kernel): block = 4 waves = 128 weight rows x one slice of K.
// A wave computes out[32 tokens][32 rows] on v_mfma_f32_32x32x16_bf16, the
// activations (the hi/lo bf16 pair of the producers, as in the prefill GEMM)
// staged per 128-wide K chunk in LDS and shared by the 4 waves, the weights
// requested row-contiguously (each load covers whole 256-byte segments of
// four rows) and passed through the wave's LDS tile into the B operand
// layout (lane = row, 16 contiguous bytes of it).  Every lane requests the
// next chunk before the current chunk's MFMAs.  Partial sums of each K slice go to a float32
// workspace [slice][32][N].
// Q8_0 weights: a row's 128-wide chunk is 128 int8 (8 lanes of 16 bytes),
// widened exactly to bf16 on its way into the LDS tile; each 32-deep block's
// products collect in a temporary tile that is added to the accumulator
// times the row's block scale (the lane's row: one scale per lane and block).
// Pass 2 (skinny_epilogue_kernel): sums the slices and applies the epilogue
// of the layer (store, residual add, SwiGLU as a hi/lo pair, or RoPE with
// the K/V cache write), as the other linear kernels do.
#include <type_traits>

#include "k_common.hpp"
#include "kernels.hpp"
#include "tdf.h"

namespace tdf {

constexpr int kSkU = 8;              // 16-wide K steps per chunk
constexpr int kSkChunk = 16 * kSkU;  // 128
constexpr int kSkPitch = kSkChunk + 8;

struct SkinnyArgs {
  LinearArgs a;
  int N = 0;        // stacked rows (SwiGLU: gate rows then up rows)
  int ksplit = 1, kslice = 0;
  float* part = nullptr;  // [ksplit][tstride][N]
  int tstride = 32;       // rows of one K slice's partials
};

// stacked row r: its matrix, row index in it and the matrix's row count
__device__ __forceinline__ void sk_locate(const LinearArgs& a, bool swiglu, int r, const void*& w, int64_t& row,
                                          int& rows) {
  if (swiglu) {
    w = r < a.n0 ? a.w0 : a.w1; row = r < a.n0 ? r : r - a.n0; rows = a.n0;
  } else if (r < a.n0) {
    w = a.w0; row = r; rows = a.n0;
  } else if (r < a.n0 + a.n1) {
    w = a.w1; row = r - a.n0; rows = a.n1;
  } else {
    w = a.w2; row = r - a.n0 - a.n1; rows = a.n2;
  }
}

__device__ __forceinline__ const uint16_t* sk_row(const LinearArgs& a, bool swiglu, int r) {
  const void* w;
  int64_t row;
  int rows;
  sk_locate(a, swiglu, r, w, row, rows);
  return (const uint16_t*)w + row * a.K;
}

// Q8_0: the int8 values of row r, and its fp16 block scales
__device__ __forceinline__ const int8_t* sk_row_q8(const LinearArgs& a, bool swiglu, int r) {
  const void* w;
  int64_t row;
  int rows;
  sk_locate(a, swiglu, r, w, row, rows);
  return (const int8_t*)w + row * a.K;
}
__device__ __forceinline__ const uint16_t* sk_scales_q8(const LinearArgs& a, bool swiglu, int r) {
  const void* w;
  int64_t row;
  int rows;
  sk_locate(a, swiglu, r, w, row, rows);
  return (const uint16_t*)((const int8_t*)w + (int64_t)rows * a.K) + row * (a.K / 32);
}

// 16 int8 -> 16 bf16 (exact) as two 8-element vectors
__device__ __forceinline__ void widen_i8x16(uint4 q, bf16x8& lo8, bf16x8& hi8) {
  const uint32_t p[4] = {q.x, q.y, q.z, q.w};
  uint32_t o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t v = p[j >> 1];
    const int b = (j & 1) * 2;
    const uint32_t f0 = __builtin_bit_cast(uint32_t, (float)((int32_t)(v << (24 - 8 * b)) >> 24));
    const uint32_t f1 = __builtin_bit_cast(uint32_t, (float)((int32_t)(v << (16 - 8 * b)) >> 24));
    o[j] = (f0 >> 16) | (f1 & 0xFFFF0000u);
  }
  lo8 = __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
  hi8 = __builtin_bit_cast(bf16x8, make_uint4(o[4], o[5], o[6], o[7]));
}

template <bool SWIGLU, bool Q8>
__global__ void __launch_bounds__(256) skinny_kernel(SkinnyArgs s) {
  const LinearArgs& a = s.a;
  __shared__ __attribute__((aligned(16))) uint16_t Ah[32 * kSkPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Al[32 * kSkPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[4][32 * kSkPitch];
  const int nrt = (s.N + 127) / 128;
  const int rt = blockIdx.x % nrt, ks = blockIdx.x / nrt;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int K = a.K, T = a.T;
  const int k0 = ks * s.kslice, k1 = min(K, k0 + s.kslice);
  // Weights of the wave's 32 rows are requested row by row (load u: rows
  // 4u + lane/16, 16-byte piece lane%16 of the chunk, so each request covers
  // whole 256-byte row segments) and pass through the wave's LDS tile into
  // the MFMA operand layout (lane = row, 16 contiguous bytes of it).  Rows
  // past N are clamped: computed and dropped.
  // Q8_0: QU loads of 16 int8, rows 8u + lane/8, piece lane%8 of the chunk;
  // the lane's own row (lane%32) fetches that row's 4 block scales per chunk
  constexpr int QU = kSkChunk * 32 / (64 * 16);  // 4
  constexpr int NW = Q8 ? QU : kSkU;
  const void* wr[NW];
#pragma unroll
  for (int u = 0; u < NW; ++u) {
    if (Q8)
      wr[u] = sk_row_q8(a, SWIGLU, min(rt * 128 + w * 32 + 8 * u + (lane >> 3), s.N - 1)) + (lane & 7) * 16;
    else
      wr[u] = sk_row(a, SWIGLU, min(rt * 128 + w * 32 + 4 * u + (lane >> 4), s.N - 1)) + (lane & 15) * 8;
  }
  const uint16_t* wsc = Q8 ? sk_scales_q8(a, SWIGLU, min(rt * 128 + w * 32 + (lane & 31), s.N - 1)) : nullptr;
  uint16_t* wsw = Ws[w];
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  // activation pieces: 32 tokens x 16 pieces of 8 = 512 per array, 2 per
  // thread: token min(e/16, T-1), k offset (e%16)*8, e = tid + 256 i
  constexpr int AP = 32 * (kSkChunk / 8) / 256;
  typedef typename std::conditional<Q8, uint4, bf16x8>::type WRaw;
  WRaw bw[NW];
  bf16x8 ah[AP], al[AP];
  uint2 sc4 = make_uint2(0u, 0u);  // Q8_0: the 4 block scales of the lane's row for the chunk
  const uint16_t* ahp[AP];
  const uint16_t* alp[AP];
#pragma unroll
  for (int i = 0; i < AP; ++i) {
    const int e = tid + i * 256;
    const int64_t off = (int64_t)min(e >> 4, T - 1) * K + (e & 15) * 8;
    ahp[i] = a.act_hi + off;
    alp[i] = a.act_lo + off;
  }
// the weights are read once: non-temporal loads (measured 5-9 % faster for
// the gate/up and down projections at 9..32 tokens)
#define SK_LOAD(kc_)                                                              \
  do {                                                                            \
    if constexpr (Q8) {                                                           \
      typedef unsigned int u32x4_ __attribute__((ext_vector_type(4)));           \
      _Pragma("unroll") for (int u = 0; u < NW; ++u) {                            \
        const u32x4_ v_ = __builtin_nontemporal_load((const u32x4_*)((const int8_t*)wr[u] + (kc_))); \
        bw[u] = make_uint4(v_[0], v_[1], v_[2], v_[3]);                           \
      }                                                                           \
      sc4 = *(const uint2*)(wsc + (kc_) / 32);                                    \
    } else {                                                                      \
      _Pragma("unroll") for (int u = 0; u < NW; ++u)                              \
        bw[u] = __builtin_nontemporal_load((const bf16x8*)((const uint16_t*)wr[u] + (kc_))); \
    }                                                                             \
    _Pragma("unroll") for (int i = 0; i < AP; ++i) {                              \
      ah[i] = *(const bf16x8*)(ahp[i] + (kc_));                                   \
      al[i] = *(const bf16x8*)(alp[i] + (kc_));                                   \
    }                                                                             \
  } while (0)
  SK_LOAD(k0);
  for (int kc = k0; kc < k1; kc += kSkChunk) {
    __syncthreads();  // the previous chunk's readers are done
#pragma unroll
    for (int i = 0; i < AP; ++i) {
      const int e = tid + i * 256;
      const int off = (e >> 4) * kSkPitch + (e & 15) * 8;
      *(bf16x8*)&Ah[off] = ah[i];
      *(bf16x8*)&Al[off] = al[i];
    }
    uint32_t scw[2] = {0u, 0u};  // Q8_0: this chunk's scales, kept across the next chunk's loads
    if constexpr (Q8) {
#pragma unroll
      for (int u = 0; u < NW; ++u) {
        bf16x8 lo8, hi8;
        widen_i8x16(bw[u], lo8, hi8);
        uint16_t* dst = &wsw[(8 * u + (lane >> 3)) * kSkPitch + (lane & 7) * 16];
        *(bf16x8*)dst = lo8;
        *(bf16x8*)(dst + 8) = hi8;
      }
      scw[0] = sc4.x;
      scw[1] = sc4.y;
    } else {
#pragma unroll
      for (int u = 0; u < NW; ++u) *(bf16x8*)&wsw[(4 * u + (lane >> 4)) * kSkPitch + (lane & 15) * 8] = bw[u];
    }
    __syncthreads();
    if (kc + kSkChunk < k1) SK_LOAD(kc + kSkChunk);
    if constexpr (Q8) {
#pragma unroll
      for (int blk = 0; blk < kSkChunk / 32; ++blk) {
        f32x16 tmp;
#pragma unroll
        for (int r = 0; r < 16; ++r) tmp[r] = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int off = (lane & 31) * kSkPitch + (2 * blk + h) * 16 + (lane >> 5) * 8;
          const bf16x8 xh = *(const bf16x8*)&Ah[off];
          const bf16x8 xl = *(const bf16x8*)&Al[off];
          const bf16x8 b = *(const bf16x8*)&wsw[off];
          tmp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, b, tmp, 0, 0, 0);
          tmp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xl, b, tmp, 0, 0, 0);
        }
        const uint32_t pair = scw[blk >> 1];
        const float sc = f16_to_f32((uint16_t)((blk & 1) ? pair >> 16 : pair & 0xFFFFu));
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = fmaf(sc, tmp[r], acc[r]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < kSkU; ++u) {
        const int off = (lane & 31) * kSkPitch + u * 16 + (lane >> 5) * 8;
        const bf16x8 xh = *(const bf16x8*)&Ah[off];
        const bf16x8 xl = *(const bf16x8*)&Al[off];
        const bf16x8 b = *(const bf16x8*)&wsw[off];
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, b, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xl, b, acc, 0, 0, 0);
      }
    }
  }
#undef SK_LOAD
  // acc[r] <-> token (r/4)*8 + (lane/32)*4 + r%4, row rt*128 + w*32 + lane%32
  const int n = rt * 128 + w * 32 + (lane & 31);
  if (n >= s.N) return;
  float* pp = s.part + (int64_t)ks * s.tstride * s.N + n;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
    if (t < T) pp[(int64_t)t * s.N] = acc[r];
  }
}

template <int EPI, typename KvT>
__global__ void __launch_bounds__(256) skinny_epilogue_kernel(SkinnyArgs s) {
  const LinearArgs& a = s.a;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int T = a.T;
  // sum of the K slices, 8 requests in flight at a time (clamped slice
  // indices, the surplus weighted by 0)
  auto total = [&](int t, int n) {
    float y = 0.f;
    for (int k0 = 0; k0 < s.ksplit; k0 += 8) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = s.part[((int64_t)min(k0 + k, s.ksplit - 1) * s.tstride + t) * s.N + n];
#pragma unroll
      for (int k = 0; k < 8; ++k) y = fmaf(v[k], k0 + k < s.ksplit ? 1.f : 0.f, y);
    }
    return y;
  };
  if (EPI == EPI_SWIGLU) {
    const int F = a.n0;
    if (i >= (int64_t)T * F) return;
    const int t = (int)(i / F), f = (int)(i % F);
    const float v = silu(total(t, f)) * total(t, F + f);
    const int64_t o = (int64_t)t * a.ldo + f;
    if (a.out) a.out[o] = v;
    if (a.out_hi) split_bf16(v, a.out_hi[o], a.out_lo[o]);
    return;
  }
  // other epilogues: one thread per adjacent column pair (a RoPE pair)
  const int NP = (s.N + 1) / 2;
  if (i >= (int64_t)T * NP) return;
  const int t = (int)(i / NP), n = 2 * (int)(i % NP);
  const float y0 = total(t, n);
  const float y1 = n + 1 < s.N ? total(t, n + 1) : 0.f;
  if (EPI == EPI_STORE) {
    a.out[(int64_t)t * a.ldo + n] = y0;
    if (n + 1 < s.N) a.out[(int64_t)t * a.ldo + n + 1] = y1;
  } else if (EPI == EPI_RESIDUAL) {
    float* xo = a.out + (int64_t)t * a.ldo;
    xo[n] += y0;
    if (n + 1 < s.N) xo[n + 1] += y1;
  } else if (EPI == EPI_QKV) {
    const int hd = a.head_dim;
    if (n < a.n0 + a.n1) {
      const int lr = n < a.n0 ? n : n - a.n0;
      const int pi = (lr % hd) >> 1;
      const float2 cs = a.rope_cs[(int64_t)t * (hd >> 1) + pi];
      const float z0 = y0 * cs.x - y1 * cs.y, z1 = y0 * cs.y + y1 * cs.x;
      if (n < a.n0) {
        a.q_out[(int64_t)t * a.n0 + lr] = z0;
        a.q_out[(int64_t)t * a.n0 + lr + 1] = z1;
      } else {
        const int64_t ci = ((int64_t)(lr / hd) * a.n_ctx + a.slots[t]) * hd + (lr % hd);
        KvStore<KvT>::store((typename KvStore<KvT>::T*)a.k_cache, ci, z0);
        KvStore<KvT>::store((typename KvStore<KvT>::T*)a.k_cache, ci + 1, z1);
      }
    } else {
      const int lr = n - a.n0 - a.n1;
      const int64_t ci = ((int64_t)(lr / hd) * a.n_ctx + a.slots[t]) * hd + (lr % hd);
      KvStore<KvT>::store((typename KvStore<KvT>::T*)a.v_cache, ci, y0);
      if (n + 1 < s.N) KvStore<KvT>::store((typename KvStore<KvT>::T*)a.v_cache, ci + 1, y1);
    }
  }
}

// Residual pass with the next RMSNorm (EPI_RESIDUAL, norm_out_g set): one
// block of 1024 threads per token holds the token's whole row, so the sum of
// squares of the new residual needs no second pass over memory.  Thread i
// takes columns 4 i + 4096 p (float4), requests every K slice's partial at
// once, adds them to the residual, writes it back, and after the block's
// reduction writes g * x_new * r as a bf16 pair, r = 1 / sqrt(ss / N + eps)
// as rmsnorm_kernel computes it.
constexpr int kSkNormThreads = 1024;
__global__ void __launch_bounds__(kSkNormThreads) skinny_residual_norm_kernel(SkinnyArgs s) {
  const LinearArgs& a = s.a;
  __shared__ float red[kSkNormThreads / 64];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int N = s.N;
  float* xo = a.out + (int64_t)t * a.ldo;
  constexpr int P = 2;  // float4 per thread: rows of up to 8192
  float4 xv[P];
  float ss = 0.f;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int n = tid * 4 + p * 4 * kSkNormThreads;
    xv[p] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (n < N) {
      float4 y = *(const float4*)(xo + n);
      for (int k0 = 0; k0 < s.ksplit; k0 += 8) {
        float4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = *(const float4*)&s.part[((int64_t)min(k0 + k, s.ksplit - 1) * s.tstride + t) * N + n];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float on = k0 + k < s.ksplit ? 1.f : 0.f;
          y.x = fmaf(v[k].x, on, y.x); y.y = fmaf(v[k].y, on, y.y);
          y.z = fmaf(v[k].z, on, y.z); y.w = fmaf(v[k].w, on, y.w);
        }
      }
      *(float4*)(xo + n) = y;
      xv[p] = y;
      ss += y.x * y.x + y.y * y.y + y.z * y.z + y.w * y.w;
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  ss = 0.f;
#pragma unroll
  for (int w = 0; w < kSkNormThreads / 64; ++w) ss += red[w];
  const float r = 1.0f / sqrtf(ss / (float)N + a.norm_out_eps);
  const int64_t ro = (int64_t)t * N;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int n = tid * 4 + p * 4 * kSkNormThreads;
    if (n >= N) break;
    const float4 gv = *(const float4*)(a.norm_out_g + n);
    const float v[4] = {xv[p].x * r * gv.x, xv[p].y * r * gv.y, xv[p].z * r * gv.z, xv[p].w * r * gv.w};
    uint16_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split_bf16(v[e], h[e], l[e]);
    *(uint2*)(a.norm_out_hi + ro + n) = make_uint2(h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16);
    *(uint2*)(a.norm_out_lo + ro + n) = make_uint2(l[0] | (uint32_t)l[1] << 16, l[2] | (uint32_t)l[3] << 16);
  }
}

bool skinny_norm_supported(const LinearArgs& a) {
  return a.epi == EPI_RESIDUAL && a.n0 % 4 == 0 && a.n0 <= 8 * kSkNormThreads && a.ldo % 4 == 0;
}

bool skinny_supported(const LinearArgs& a) {
  const int N = a.epi == EPI_SWIGLU ? 2 * a.n0 : a.n0 + a.n1 + a.n2;
  return (a.weight_dtype == TDF_BF16 || a.weight_dtype == TDF_Q8_0) && a.act_hi && a.act_lo && a.T > 0 &&
         a.T <= 32 && a.K % kSkChunk == 0 &&
         (int64_t)N * 32 <= kSkinnyPartFloats && (a.epi != EPI_QKV || (a.n0 % 2 == 0 && a.n1 % 2 == 0));
}

// Pass 2 with four adjacent columns of a token per thread (16-byte loads of
// every K slice's partials in batches of KB, clamped and weighted 0 past the
// last slice; the same sum order as skinny_epilogue_kernel), then the
// layer's epilogue: SwiGLU on columns f..f+3 of gate and up, or two RoPE
// pairs inside one head, or store / residual add.
template <int EPI, typename KvT, int KB>
__global__ void __launch_bounds__(256) slices4_epilogue_kernel(SkinnyArgs s) {
  const LinearArgs& a = s.a;
  const int NC = EPI == EPI_SWIGLU ? a.n0 : s.N;  // output columns
  const int NQ = NC / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.T * NQ) return;
  const int t = (int)(i / NQ), n = 4 * (int)(i % NQ);
  auto total4 = [&](int c, float* y) {
#pragma unroll
    for (int q = 0; q < 4; ++q) y[q] = 0.f;
    for (int k0 = 0; k0 < s.ksplit; k0 += KB) {
      float4 v[KB];
#pragma unroll
      for (int k = 0; k < KB; ++k)
        v[k] = *(const float4*)&s.part[((int64_t)min(k0 + k, s.ksplit - 1) * s.tstride + t) * s.N + c];
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const float w = k0 + k < s.ksplit ? 1.f : 0.f;
        y[0] = fmaf(v[k].x, w, y[0]); y[1] = fmaf(v[k].y, w, y[1]);
        y[2] = fmaf(v[k].z, w, y[2]); y[3] = fmaf(v[k].w, w, y[3]);
      }
    }
  };
  float y[4];
  total4(n, y);
  if (EPI == EPI_SWIGLU) {
    float u[4], v[4];
    total4(a.n0 + n, u);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = silu(y[q]) * u[q];
    const int64_t o = (int64_t)t * a.ldo + n;
    if (a.out) *(float4*)&a.out[o] = make_float4(v[0], v[1], v[2], v[3]);
    if (a.out_hi) {
      uint16_t hi[4], lo[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) split_bf16(v[q], hi[q], lo[q]);
      *(uint2*)&a.out_hi[o] = make_uint2(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16));
      *(uint2*)&a.out_lo[o] = make_uint2(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16));
    }
  } else if (EPI == EPI_STORE) {
    *(float4*)&a.out[(int64_t)t * a.ldo + n] = make_float4(y[0], y[1], y[2], y[3]);
  } else if (EPI == EPI_RESIDUAL) {
    float4* xo = (float4*)&a.out[(int64_t)t * a.ldo + n];
    const float4 x = *xo;
    *xo = make_float4(x.x + y[0], x.y + y[1], x.z + y[2], x.w + y[3]);
  } else if (EPI == EPI_QKV) {
    const int hd = a.head_dim;
    if (n < a.n0 + a.n1) {
      const int lr = n < a.n0 ? n : n - a.n0;
      float z[4];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float2 cs = a.rope_cs[(int64_t)t * (hd >> 1) + (((lr + 2 * q) % hd) >> 1)];
        z[2 * q] = y[2 * q] * cs.x - y[2 * q + 1] * cs.y;
        z[2 * q + 1] = y[2 * q] * cs.y + y[2 * q + 1] * cs.x;
      }
      if (n < a.n0) {
        *(float4*)&a.q_out[(int64_t)t * a.n0 + lr] = make_float4(z[0], z[1], z[2], z[3]);
      } else {
        const int64_t ci = ((int64_t)(lr / hd) * a.n_ctx + a.slots[t]) * hd + (lr % hd);
#pragma unroll
        for (int q = 0; q < 4; ++q) KvStore<KvT>::store((typename KvStore<KvT>::T*)a.k_cache, ci + q, z[q]);
      }
    } else {
      const int lr = n - a.n0 - a.n1;
      const int64_t ci = ((int64_t)(lr / hd) * a.n_ctx + a.slots[t]) * hd + (lr % hd);
#pragma unroll
      for (int q = 0; q < 4; ++q) KvStore<KvT>::store((typename KvStore<KvT>::T*)a.v_cache, ci + q, y[q]);
    }
  }
}

// four columns per thread fit: every column count, the row pitch and (QKV)
// the head size are multiples of 4
static bool slices4_fit(const SkinnyArgs& s) {
  const LinearArgs& a = s.a;
  if (a.epi == EPI_QKV) return a.n0 % 4 == 0 && a.n1 % 4 == 0 && a.n2 % 4 == 0 && a.head_dim % 4 == 0;
  if (a.epi == EPI_SWIGLU) return a.n0 % 4 == 0 && a.ldo % 4 == 0;
  return s.N % 4 == 0 && a.ldo % 4 == 0;
}

template <int KB>
static hipError_t slices4_epilogue(const SkinnyArgs& s, hipStream_t st) {
  const LinearArgs& a = s.a;
  const int NC = a.epi == EPI_SWIGLU ? a.n0 : s.N;
  const unsigned blocks = (unsigned)(((int64_t)a.T * (NC / 4) + 255) / 256);
  switch (a.epi) {
    case EPI_STORE: slices4_epilogue_kernel<EPI_STORE, float, KB><<<blocks, 256, 0, st>>>(s); break;
    case EPI_RESIDUAL: slices4_epilogue_kernel<EPI_RESIDUAL, float, KB><<<blocks, 256, 0, st>>>(s); break;
    case EPI_SWIGLU: slices4_epilogue_kernel<EPI_SWIGLU, float, KB><<<blocks, 256, 0, st>>>(s); break;
    case EPI_QKV:
      if (a.kv_dtype == TDF_BF16) slices4_epilogue_kernel<EPI_QKV, kv_bf16, KB><<<blocks, 256, 0, st>>>(s);
      else if (a.kv_dtype == TDF_F16) slices4_epilogue_kernel<EPI_QKV, kv_f16, KB><<<blocks, 256, 0, st>>>(s);
      else slices4_epilogue_kernel<EPI_QKV, float, KB><<<blocks, 256, 0, st>>>(s);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Pass 2: sum the K slices of s.part and apply the layer's epilogue (one
// thread per output, or per RoPE pair)
static hipError_t slices_epilogue(const SkinnyArgs& s, hipStream_t st) {
  const LinearArgs& a = s.a;
  const int64_t n_thr = a.epi == EPI_SWIGLU ? (int64_t)a.T * a.n0 : (int64_t)a.T * ((s.N + 1) / 2);
  const unsigned blocks = (unsigned)((n_thr + 255) / 256);
  switch (a.epi) {
    case EPI_STORE: skinny_epilogue_kernel<EPI_STORE, float><<<blocks, 256, 0, st>>>(s); break;
    case EPI_RESIDUAL: skinny_epilogue_kernel<EPI_RESIDUAL, float><<<blocks, 256, 0, st>>>(s); break;
    case EPI_SWIGLU: skinny_epilogue_kernel<EPI_SWIGLU, float><<<blocks, 256, 0, st>>>(s); break;
    case EPI_QKV:
      if (a.kv_dtype == TDF_BF16) skinny_epilogue_kernel<EPI_QKV, kv_bf16><<<blocks, 256, 0, st>>>(s);
      else if (a.kv_dtype == TDF_F16) skinny_epilogue_kernel<EPI_QKV, kv_f16><<<blocks, 256, 0, st>>>(s);
      else skinny_epilogue_kernel<EPI_QKV, float><<<blocks, 256, 0, st>>>(s);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_linear_skinny(const LinearArgs& a, float* part, hipStream_t st) {
  if (!skinny_supported(a)) return hipErrorInvalidValue;
  SkinnyArgs s;
  s.a = a;
  s.N = a.epi == EPI_SWIGLU ? 2 * a.n0 : a.n0 + a.n1 + a.n2;
  s.part = part;
  // K slices: enough blocks to fill the chip (>= 512), each slice a whole
  // number of 128-wide chunks and at least 4 of them, within the workspace
  // (8B widths at 32 tokens, output projection: 8 slices of 4 chunks 15.3 us
  // with the epilogue, 16 slices of 2 chunks 16.7 us)
  const int nrt = (s.N + 127) / 128;
  const int chunks = a.K / kSkChunk;
  int ks = 1;
  while (nrt * ks < 512 && chunks / (ks * 2) >= 4 && (int64_t)s.N * 32 * ks * 2 <= kSkinnyPartFloats) ks *= 2;
  s.kslice = ((chunks + ks - 1) / ks) * kSkChunk;
  s.ksplit = (a.K + s.kslice - 1) / s.kslice;
  const bool q8 = a.weight_dtype == TDF_Q8_0;
  if (a.epi == EPI_SWIGLU) {
    if (q8) skinny_kernel<true, true><<<nrt * s.ksplit, 256, 0, st>>>(s);
    else skinny_kernel<true, false><<<nrt * s.ksplit, 256, 0, st>>>(s);
  } else {
    if (q8) skinny_kernel<false, true><<<nrt * s.ksplit, 256, 0, st>>>(s);
    else skinny_kernel<false, false><<<nrt * s.ksplit, 256, 0, st>>>(s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.norm_out_g) {
    if (!skinny_norm_supported(a)) return hipErrorInvalidValue;
    skinny_residual_norm_kernel<<<a.T, kSkNormThreads, 0, st>>>(s);
    return hipGetLastError();
  }
  if (slices4_fit(s)) return slices4_epilogue<8>(s, st);
  return slices_epilogue(s, st);
}

hipError_t launch_split_epilogue(const LinearArgs& a, float* part, int ksplit, hipStream_t st) {
  if (a.T <= 0 || ksplit < 1 || a.norm_out_g || (a.epi == EPI_QKV && (a.n0 % 2 || a.n1 % 2)))
    return hipErrorInvalidValue;
  SkinnyArgs s;
  s.a = a;
  s.N = a.epi == EPI_SWIGLU ? 2 * a.n0 : a.n0 + a.n1 + a.n2;
  s.part = part;
  s.ksplit = ksplit;
  s.tstride = a.T;
  if (slices4_fit(s)) return ksplit <= 2 ? slices4_epilogue<2>(s, st) : slices4_epilogue<8>(s, st);
  return slices_epilogue(s, st);
}

}  // namespace tdf
