// Prefill linear layers on the gfx950 matrix cores.
//
// C[m][n] = sum_k act[m][k] W[n][k] with bf16 operands and float32
// accumulation (v_mfma_f32_32x32x16_bf16).  Both operands are K-contiguous,
// as stored (W row-major [out][in]).  Prefill is compute-bound (llama.cpp
// walkthrough, "KV-cache and the Prefill / Decode stages"), so the epilogues
// of the Llama layer (Ollama engine page, "Deep dive: the Llama forward pass
// in Go") are fused here: RoPE + K/V cache write for the stacked Q/K/V
// projection, SILU(gate) * up for the gate/up pair, and the residual add
// for the output and down projections.
//
// Tiling: 256 threads = 4 waves in a 2x2 grid; block tile 128 x 128 x 64,
// each wave 64 x 64 = 2 x 2 MFMA tiles of 32 x 32.  Tiles go through LDS
// (row pitch 72 bf16 to spread banks), double-buffered with the next tile
// prefetched into registers during the MFMAs.  Blocks are ordered so that
// the m tiles and K splits of one n tile run back to back on one XCD
// (dispatch is round-robin over the 8 XCDs), which keeps each weight tile's
// re-reads inside that XCD's L2.
#include "k_common.hpp"
#include "kernels.hpp"
#include "tdf.h"

namespace tdf {

constexpr int GBM = 128, GBN = 128, GBK = 64, GPITCH = GBK + 8;

template <typename KvT>
__device__ __forceinline__ void kv_store(void* cache, int64_t idx, float v) {
  KvStore<KvT>::store((typename KvStore<KvT>::T*)cache, idx, v);
}

template <int EPI, typename KvT>
__global__ void __launch_bounds__(256) gemm_kernel(LinearArgs a, int M, int tiles_m, int tiles_n,
                                                   int ksplit) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][GBM * GPITCH];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][GBN * GPITCH];

  const int total = tiles_m * tiles_n * ksplit;
  int b = blockIdx.x;
  if ((total & 7) == 0) b = (b & 7) * (total >> 3) + (b >> 3);
  const int tm = b % tiles_m;
  const int ks = (b / tiles_m) % ksplit;
  const int tn = b / (tiles_m * ksplit);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int K = a.K;
  const int kchunk = K / ksplit;
  const int k_begin = ks * kchunk;
  const int nk = kchunk / GBK;
  const int m0 = tm * GBM;
  const int Ntot = a.n0 + a.n1 + a.n2;
  // column base of this block (SwiGLU: 64 output columns, gate and up rows)
  const int n0 = EPI == EPI_SWIGLU ? tn * 64 : tn * GBN;

  // rows this thread stages: chunk c = tid + 256 i -> row c / 8, k offset (c % 8) * 8
  const int kc = (tid & 7) * 8;
  const uint16_t* arow[4];
  const uint16_t* brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    const int gm = m0 + r;
    arow[i] = gm < M ? a.act_bf16 + (int64_t)gm * K : nullptr;
    const uint16_t* p = nullptr;
    if (EPI == EPI_SWIGLU) {
      const int q = r >> 5;
      const int f = n0 + (q >> 1) * 32 + (r & 31);
      if (f < a.n0) p = (const uint16_t*)((q & 1) ? a.w1 : a.w0) + (int64_t)f * K;
    } else {
      const int gr = n0 + r;
      if (gr < a.n0) p = (const uint16_t*)a.w0 + (int64_t)gr * K;
      else if (gr < a.n0 + a.n1) p = (const uint16_t*)a.w1 + (int64_t)(gr - a.n0) * K;
      else if (gr < Ntot) p = (const uint16_t*)a.w2 + (int64_t)(gr - a.n0 - a.n1) * K;
    }
    brow[i] = p;
  }

  uint4 ra[4], rb[4];
  const uint4 zero = make_uint4(0, 0, 0, 0);
  auto gload = [&](int k) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = arow[i] ? *(const uint4*)(arow[i] + k + kc) : zero;
      rb[i] = brow[i] ? *(const uint4*)(brow[i] + k + kc) : zero;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      *(uint4*)&As[buf][r * GPITCH + kc] = ra[i];
      *(uint4*)&Bs[buf][r * GPITCH + kc] = rb[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  gload(k_begin);
  lstore(0);
  __syncthreads();

  const int frow = lane & 31;
  const int fk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(k_begin + (kt + 1) * GBK);
#pragma unroll
    for (int kk = 0; kk < GBK; kk += 16) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        af[mt] = *(const bf16x8*)&As[cur][(wm * 64 + mt * 32 + frow) * GPITCH + kk + fk];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        bfr[nt] = *(const bf16x8*)&Bs[cur][(wn * 64 + nt * 32 + frow) * GPITCH + kk + fk];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mt], bfr[nt], acc[mt][nt], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds column (lane % 32) and rows i*8 + (lane/32)*4 + j
  const int ccol = lane & 31;
  const int rsub = (lane >> 5) * 4;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * 64 + mt * 32 + (r >> 2) * 8 + rsub + (r & 3);
      const bool row_ok = row < M;
      if (EPI == EPI_SWIGLU) {
        const int f = n0 + wn * 32 + ccol;
        if (row_ok && f < a.n0) {
          const float v = silu(acc[mt][0][r]) * acc[mt][1][r];
          a.out_bf16[(int64_t)row * a.ldo + f] = f32_to_bf16(v);
        }
        continue;
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int col = n0 + wn * 64 + nt * 32 + ccol;
        const float y = acc[mt][nt][r];
        if (EPI == EPI_QKV) {
          const float partner = __shfl_xor(y, 1, kWave);
          if (!row_ok || col >= Ntot) continue;
          const int hd = a.head_dim;
          if (col < a.n0 + a.n1) {
            const int lc = col < a.n0 ? col : col - a.n0;
            const int i = (lc % hd) >> 1;
            double sn, cs;
            sincos((double)a.pos[row] * a.inv_freq[i], &sn, &cs);
            const float c = (float)cs, s = (float)sn;
            const float z = (col & 1) ? partner * s + y * c : y * c - partner * s;
            if (col < a.n0) {
              if (a.q_out) a.q_out[(int64_t)row * a.n0 + lc] = z;
              if (a.q_out_bf16) a.q_out_bf16[(int64_t)row * a.n0 + lc] = f32_to_bf16(z);
            } else {
              kv_store<KvT>(a.k_cache, ((int64_t)(lc / hd) * a.n_ctx + a.slots[row]) * hd + (lc % hd), z);
            }
          } else {
            const int lc = col - a.n0 - a.n1;
            kv_store<KvT>(a.v_cache, ((int64_t)(lc / hd) * a.n_ctx + a.slots[row]) * hd + (lc % hd), y);
          }
        } else if (row_ok && col < Ntot) {
          float* o = a.out + (int64_t)row * a.ldo + col;
          if (EPI == EPI_STORE) *o = y;
          else if (ksplit == 1) *o += y;
          else atomicAdd(o, y);
        }
      }
    }
  }
}

bool gemm_supported(const LinearArgs& a) {
  return a.weight_bf16 && a.act_bf16 && a.K % GBK == 0 && a.K >= GBK;
}

template <int EPI, typename KvT>
static hipError_t gemm_launch_t(const LinearArgs& a, hipStream_t s) {
  const int M = a.T;
  const int tiles_m = (M + GBM - 1) / GBM;
  const int Ntot = a.n0 + a.n1 + a.n2;
  const int tiles_n = EPI == EPI_SWIGLU ? (a.n0 + 63) / 64 : (Ntot + GBN - 1) / GBN;
  int ksplit = 1;
  if (EPI == EPI_RESIDUAL) {
    // fill the 256 CUs: split K (partial sums are added atomically)
    const int nkt = a.K / GBK;
    while (tiles_m * tiles_n * ksplit < 512 && ksplit < 8 && nkt % (ksplit * 2) == 0 &&
           nkt / (ksplit * 2) >= 4)
      ksplit *= 2;
  }
  const int blocks = tiles_m * tiles_n * ksplit;
  gemm_kernel<EPI, KvT><<<blocks, 256, 0, s>>>(a, M, tiles_m, tiles_n, ksplit);
  return hipGetLastError();
}

hipError_t launch_linear_gemm(const LinearArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (!gemm_supported(a)) return hipErrorInvalidValue;
  switch (a.epi) {
    case EPI_STORE: return gemm_launch_t<EPI_STORE, float>(a, s);
    case EPI_RESIDUAL: return gemm_launch_t<EPI_RESIDUAL, float>(a, s);
    case EPI_SWIGLU: return gemm_launch_t<EPI_SWIGLU, float>(a, s);
    case EPI_QKV:
      if (a.kv_dtype == TDF_BF16) return gemm_launch_t<EPI_QKV, kv_bf16>(a, s);
      if (a.kv_dtype == TDF_F16) return gemm_launch_t<EPI_QKV, kv_f16>(a, s);
      return gemm_launch_t<EPI_QKV, float>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tdf
