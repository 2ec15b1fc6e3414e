// Prefill linear layers on the gfx950 matrix cores.
//
// C[m][n] = sum_k act[m][k] W[n][k], float32 accumulation on
// v_mfma_f32_32x32x16_bf16.  W is bf16 as stored (row-major [out][in], both
// operands K-contiguous).  The activations carry about 16 significant bits as
// a pair of bf16 arrays, act = hi + lo (hi = bf16(x), lo = bf16(x - hi)), so
// every weight fragment feeds two MFMAs: act_hi.W + act_lo.W.  A single bf16
// rounding of the activations before each projection would put the logits of
// the 32-layer models far outside the float64 oracle's tolerance (the error
// grows through the layers); the pair keeps the prefill within it.
//
// Prefill is compute-bound (llama.cpp walkthrough, "KV-cache and the Prefill
// / Decode stages"), so the epilogues of the Llama layer (Ollama engine page,
// "Deep dive: the Llama forward pass in Go") are fused: RoPE + K/V cache
// write for the stacked Q/K/V projection, SILU(gate) * up for the gate/up
// pair (written again as a hi/lo pair), and the residual add for the output
// and down projections (split over K with atomic adds when the tiles alone
// would leave CUs idle).
//
// Q8_0 weights (blocks of 32 int8 of a row with one fp16 scale): the int8
// values are exact in bf16, so they are widened to bf16 while being staged
// into LDS and enter the same MFMAs unscaled; each 32-deep block's products
// are collected in a temporary accumulator and added to the tile scaled by
// the block scale of their column (exact weights, one FMA per output per
// block).
//
// Tiling: 256 threads = 4 waves in a 2 x 2 grid; wave tile (32 MT) x (32 NT)
// = MT x NT MFMA tiles of 32 x 32, block tile (64 MT) x (64 NT) x 64.  Tiles
// go through LDS (row pitch 72 bf16 to spread banks) with the next K tile
// prefetched into registers during the MFMAs.  Blocks are ordered so that the
// m tiles and K splits of one n tile run back to back on one XCD (dispatch is
// round-robin over the 8 XCDs), keeping a weight tile's re-reads in that
// XCD's L2.
#include <type_traits>

#include "k_common.hpp"
#include "kernels.hpp"
#include "tdf.h"

namespace tdf {

constexpr int GBK = 64, GPITCH = GBK + 8;

template <typename KvT>
__device__ __forceinline__ void kv_store(void* cache, int64_t idx, float v) {
  KvStore<KvT>::store((typename KvStore<KvT>::T*)cache, idx, v);
}

__device__ __forceinline__ void split_store(uint16_t* hi, uint16_t* lo, int64_t i, float v) {
  split_bf16(v, hi[i], lo[i]);
}

// 8 int8 -> 8 bf16 (exact: at most 8 significant bits)
__device__ __forceinline__ bf16x8 widen_i8x8(uint2 q) {
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = j < 2 ? q.x : q.y;
    const int b = (j & 1) * 2;
    const uint32_t f0 = __builtin_bit_cast(uint32_t, (float)((int32_t)(w << (24 - 8 * b)) >> 24));
    const uint32_t f1 = __builtin_bit_cast(uint32_t, (float)((int32_t)(w << (16 - 8 * b)) >> 24));
    o[j] = (f0 >> 16) | (f1 & 0xFFFF0000u);
  }
  return __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
}

template <int EPI, typename KvT, int MT, int NT, bool Q8>
__global__ void __launch_bounds__(256, 2) gemm_kernel(LinearArgs a, int M, int tiles_m, int tiles_n,
                                                   int ksplit) {
  constexpr int BM = 64 * MT, BN = 64 * NT;
  constexpr int A_PER = BM * 8 / 256;   // 16-byte A pieces per thread (each of hi, lo)
  constexpr int B_PER = BN * 8 / 256;   // B pieces of 8 weights per thread
  static_assert(BN <= 256, "one scale pair per thread");
  __shared__ __attribute__((aligned(16))) uint16_t Ah[BM * GPITCH];
  __shared__ __attribute__((aligned(16))) uint16_t Al[BM * GPITCH];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * GPITCH];
  // Q8_0: the two block scales (fp16) of each B row for the current K tile
  __shared__ uint32_t Ss[Q8 ? BN : 1];

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
  const int m0 = tm * BM;
  const int Ntot = a.n0 + a.n1 + a.n2;
  // SwiGLU: a block covers BN/2 output columns; wave wn holds gate tiles
  // [0, NT/2) and up tiles [NT/2, NT) for the same BN/4 columns
  const int n0 = EPI == EPI_SWIGLU ? tn * (BN / 2) : tn * BN;

  // Each thread stages 16-byte pieces: row (tid / 8) + 32 i, k offset
  // (tid % 8) * 8.  Rows past the end are clamped to a valid row; their
  // products are discarded by the epilogue's bounds checks.
  const int kc = (tid & 7) * 8;
  const uint16_t* ap_hi[A_PER];
  const uint16_t* ap_lo[A_PER];
#pragma unroll
  for (int i = 0; i < A_PER; ++i) {
    const int gm = min(m0 + (tid >> 3) + 32 * i, M - 1);
    ap_hi[i] = a.act_hi + (int64_t)gm * K + kc;
    ap_lo[i] = a.act_lo + (int64_t)gm * K + kc;
  }
  // B row r of the block tile: its matrix, row in that matrix and the
  // matrix's row count (rows past the end clamped to a valid row)
  auto b_row = [&](int r, const void*& w, int64_t& row, int& rows) {
    if (EPI == EPI_SWIGLU) {
      constexpr int WN = BN / 2, HALF = WN / 2;
      const int part = r / WN, rr = r % WN;
      row = min(n0 + part * HALF + (rr % HALF), a.n0 - 1);
      w = rr >= HALF ? a.w1 : a.w0;
      rows = a.n0;
    } else {
      const int gr = min(n0 + r, Ntot - 1);
      if (gr < a.n0) { w = a.w0; row = gr; rows = a.n0; }
      else if (gr < a.n0 + a.n1) { w = a.w1; row = gr - a.n0; rows = a.n1; }
      else { w = a.w2; row = gr - a.n0 - a.n1; rows = a.n2; }
    }
  };
  // B pieces: bf16 element pointers, or Q8_0 pointers to the int8 values
  typedef typename std::conditional<Q8, const int8_t*, const uint16_t*>::type BPtr;
  BPtr bp[B_PER];
#pragma unroll
  for (int i = 0; i < B_PER; ++i) {
    const void* w;
    int64_t row;
    int rows;
    b_row((tid >> 3) + 32 * i, w, row, rows);
    bp[i] = (BPtr)w + row * K + kc;
  }
  // Q8_0: thread r < BN fetches the scale pair of B row r for each K tile
  const uint32_t* sp = nullptr;
  if (Q8 && tid < BN) {
    const void* w;
    int64_t row;
    int rows;
    b_row(tid, w, row, rows);
    sp = (const uint32_t*)((const int8_t*)w + (int64_t)rows * K) + row * (K / 64);
  }
  // B prefetch registers: 8 bf16, or 8 int8 widened when stored to LDS
  typedef typename std::conditional<Q8, uint2, bf16x8>::type BRaw;
  auto load_b = [&](int i, int k) -> BRaw {
    if constexpr (Q8) return *(const uint2*)(bp[i] + k);
    else return *(const bf16x8*)(bp[i] + k);
  };
  auto b_lds = [&](BRaw v) -> bf16x8 {
    if constexpr (Q8) return widen_i8x8(v);
    else return v;
  };

  bf16x8 rah[A_PER], ral[A_PER];
  BRaw rb[B_PER];
  uint32_t rs = 0;

  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // first K tile
#pragma unroll
  for (int i = 0; i < A_PER; ++i) {
    rah[i] = *(const bf16x8*)(ap_hi[i] + k_begin);
    ral[i] = *(const bf16x8*)(ap_lo[i] + k_begin);
  }
#pragma unroll
  for (int i = 0; i < B_PER; ++i) rb[i] = load_b(i, k_begin);
  if (Q8 && sp) rs = sp[k_begin / GBK];
#pragma unroll
  for (int i = 0; i < A_PER; ++i) {
    const int r = (tid >> 3) + 32 * i;
    *(bf16x8*)&Ah[r * GPITCH + kc] = rah[i];
    *(bf16x8*)&Al[r * GPITCH + kc] = ral[i];
  }
#pragma unroll
  for (int i = 0; i < B_PER; ++i) *(bf16x8*)&Bs[((tid >> 3) + 32 * i) * GPITCH + kc] = b_lds(rb[i]);
  if (Q8 && tid < BN) Ss[tid] = rs;
  __syncthreads();

  const int frow = lane & 31;
  const int fk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) {
      // prefetch the next K tile into registers while the MFMAs run
      const int kn = k_begin + (kt + 1) * GBK;
#pragma unroll
      for (int i = 0; i < A_PER; ++i) {
        rah[i] = *(const bf16x8*)(ap_hi[i] + kn);
        ral[i] = *(const bf16x8*)(ap_lo[i] + kn);
      }
#pragma unroll
      for (int i = 0; i < B_PER; ++i) rb[i] = load_b(i, kn);
      if (Q8 && sp) rs = sp[kn / GBK];
    }
    if (Q8) {
      // per 32-deep block and column tile: unscaled products into tmp, then
      // acc += scale(column, block) * tmp (the block's A fragments stay in
      // registers across the column tiles)
#pragma unroll
      for (int blk = 0; blk < GBK / 32; ++blk) {
        bf16x8 ah[2][MT], al[2][MT];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const int r = (wm * 32 * MT + mt * 32 + frow) * GPITCH + blk * 32 + h * 16 + fk;
            ah[h][mt] = *(const bf16x8*)&Ah[r];
            al[h][mt] = *(const bf16x8*)&Al[r];
          }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          bf16x8 bfr[2];
#pragma unroll
          for (int h = 0; h < 2; ++h)
            bfr[h] = *(const bf16x8*)&Bs[(wn * 32 * NT + nt * 32 + frow) * GPITCH + blk * 32 + h * 16 + fk];
          f32x16 tmp[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) tmp[mt][r] = 0.f;
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              tmp[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[h][mt], bfr[h], tmp[mt], 0, 0, 0);
              tmp[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[h][mt], bfr[h], tmp[mt], 0, 0, 0);
            }
          const uint32_t sc2 = Ss[wn * 32 * NT + nt * 32 + frow];
          const float sc = f16_to_f32((uint16_t)(blk ? sc2 >> 16 : sc2 & 0xFFFFu));
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][nt][r] = fmaf(sc, tmp[mt][r], acc[mt][nt][r]);
        }
      }
    } else
#pragma unroll
    for (int kk = 0; kk < GBK; kk += 16) {
      bf16x8 ah[MT], al[MT], bfr[NT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = (wm * 32 * MT + mt * 32 + frow) * GPITCH + kk + fk;
        ah[mt] = *(const bf16x8*)&Ah[r];
        al[mt] = *(const bf16x8*)&Al[r];
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        bfr[nt] = *(const bf16x8*)&Bs[(wn * 32 * NT + nt * 32 + frow) * GPITCH + kk + fk];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mt], bfr[nt], acc[mt][nt], 0, 0, 0);
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[mt], bfr[nt], acc[mt][nt], 0, 0, 0);
        }
    }
    if (more) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < A_PER; ++i) {
        const int r = (tid >> 3) + 32 * i;
        *(bf16x8*)&Ah[r * GPITCH + kc] = rah[i];
        *(bf16x8*)&Al[r * GPITCH + kc] = ral[i];
      }
#pragma unroll
      for (int i = 0; i < B_PER; ++i) *(bf16x8*)&Bs[((tid >> 3) + 32 * i) * GPITCH + kc] = b_lds(rb[i]);
      if (Q8 && tid < BN) Ss[tid] = rs;
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds column (lane % 32) and rows i*8 + (lane/32)*4 + j
  const int ccol = lane & 31;
  const int rsub = (lane >> 5) * 4;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * 32 * MT + mt * 32 + (r >> 2) * 8 + rsub + (r & 3);
      const bool row_ok = row < M;
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int nt = 0; nt < NT / 2; ++nt) {
          const int f = n0 + wn * (BN / 4) + nt * 32 + ccol;
          if (row_ok && f < a.n0) {
            const float v = silu(acc[mt][nt][r]) * acc[mt][nt + NT / 2][r];
            split_store(a.out_hi, a.out_lo, (int64_t)row * a.ldo + f, v);
          }
        }
        continue;
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int col = n0 + wn * 32 * NT + nt * 32 + ccol;
        const float y = acc[mt][nt][r];
        if (EPI == EPI_QKV) {
          const float partner = __shfl_xor(y, 1, kWave);
          if (!row_ok || col >= Ntot) continue;
          const int hd = a.head_dim;
          if (col < a.n0 + a.n1) {
            const int lc = col < a.n0 ? col : col - a.n0;
            const int i = (lc % hd) >> 1;
            const float2 cs = a.rope_cs[(int64_t)row * (hd >> 1) + i];
            const float c = cs.x, s = cs.y;
            const float z = (col & 1) ? partner * s + y * c : y * c - partner * s;
            if (col < a.n0) {
              a.q_out[(int64_t)row * a.n0 + lc] = z;
            } else {
              kv_store<KvT>(a.k_cache, ((int64_t)(lc / hd) * a.n_ctx + a.slots[row]) * hd + (lc % hd), z);
            }
          } else {
            const int lc = col - a.n0 - a.n1;
            kv_store<KvT>(a.v_cache, ((int64_t)(lc / hd) * a.n_ctx + a.slots[row]) * hd + (lc % hd), y);
          }
        } else if (row_ok && col < Ntot) {
          float* o = a.out + (int64_t)row * a.ldo + col;
          if (EPI == EPI_STORE) o[(int64_t)ks * M * a.ldo] = y;  // split ks: its own slab of M rows
          else if (ksplit == 1) *o += y;
          else atomicAdd(o, y);
        }
      }
    }
  }
}

bool gemm_supported(const LinearArgs& a) {
  return (a.weight_dtype == TDF_BF16 || a.weight_dtype == TDF_Q8_0) && a.act_hi && a.act_lo &&
         a.K % GBK == 0 && a.K >= GBK;
}

template <int EPI, typename KvT, int MT, int NT>
static hipError_t gemm_launch_tile(const LinearArgs& a, int ksplit, hipStream_t s) {
  const int M = a.T;
  const int tiles_m = (M + 64 * MT - 1) / (64 * MT);
  const int Ntot = a.n0 + a.n1 + a.n2;
  const int tiles_n = EPI == EPI_SWIGLU ? (a.n0 + 32 * NT - 1) / (32 * NT) : (Ntot + 64 * NT - 1) / (64 * NT);
  if (a.weight_dtype == TDF_Q8_0) {
    if constexpr (MT == 1 && NT == 2)
      gemm_kernel<EPI, KvT, MT, NT, true><<<tiles_m * tiles_n * ksplit, 256, 0, s>>>(a, M, tiles_m, tiles_n, ksplit);
    else
      return hipErrorInvalidValue;
  } else {
    gemm_kernel<EPI, KvT, MT, NT, false><<<tiles_m * tiles_n * ksplit, 256, 0, s>>>(a, M, tiles_m, tiles_n, ksplit);
  }
  return hipGetLastError();
}

// Tile choice.  Plain epilogues: 64x128 for at most 64 rows, else the
// largest of 128x256, 128x128, 64x128 that gives at least 384 blocks (1.5
// per CU).  Residual epilogue: the
// largest tile that reaches 512 blocks with a K split (2, 4) that still
// leaves each split at least 48 K tiles; failing that, the smallest K split
// (1, 2, 4, 8) for which some tile reaches 512 blocks, with the largest such
// tile.  The atomic adds of a split cost less than small tiles' extra
// operand traffic only when the split is deep in K: measured at M = 512,
// K = 14336 (8B down) 128x128 tiles split in 4 take 137.5 us against 146 us
// for 64x128 split in 2; K = 28672 (70B down) 128x256 split in 4 take 441 us
// against 567 us for 64x128 unsplit; K = 8192 (70B output projection)
// 128x128 split in 2 take 156 us against 175 us; at K = 4096 (8B output
// projection) 64x128 tiles split in 2 stay best (51 us; 128x256 split in 8:
// 93 us).
template <int EPI, typename KvT>
static hipError_t gemm_launch_t(const LinearArgs& a, hipStream_t s) {
  const int M = a.T;
  const int Ntot = EPI == EPI_SWIGLU ? 2 * a.n0 : a.n0 + a.n1 + a.n2;
  const int nkt = a.K / GBK;
  // Q8_0 weights take the 64x128 tile only (the block-scale accumulators of
  // the larger tiles do not fit in the registers)
  const bool q8 = a.weight_dtype == TDF_Q8_0;
  const int b24 = q8 ? 0 : ((M + 127) / 128) * ((Ntot + 255) / 256);
  const int b22 = q8 ? 0 : ((M + 127) / 128) * ((Ntot + 127) / 128);
  const int b12 = ((M + 63) / 64) * ((Ntot + 127) / 128);
  if (EPI == EPI_RESIDUAL) {
    for (int ks = 2; ks <= 4; ks *= 2) {
      if (nkt % ks != 0 || nkt / ks < 48) break;
      if (b24 * ks >= 512) return gemm_launch_tile<EPI, KvT, 2, 4>(a, ks, s);
    }
    for (int ks = 2; ks <= 4; ks *= 2) {
      if (nkt % ks != 0 || nkt / ks < 48) break;
      if (b22 * ks >= 512) return gemm_launch_tile<EPI, KvT, 2, 2>(a, ks, s);
    }
    for (int ks = 1; ks <= 8; ks *= 2) {
      // each split keeps at least 4 K tiles
      if (ks > 1 && (nkt % ks != 0 || nkt / ks < 4)) break;
      if (b24 * ks >= 512) return gemm_launch_tile<EPI, KvT, 2, 4>(a, ks, s);
      if (b22 * ks >= 512) return gemm_launch_tile<EPI, KvT, 2, 2>(a, ks, s);
      if (b12 * ks >= 512) return gemm_launch_tile<EPI, KvT, 1, 2>(a, ks, s);
    }
    // small problems: the deepest allowed split of the smallest tile
    int ks = 1;
    while (ks < 8 && nkt % (ks * 2) == 0 && nkt / (ks * 2) >= 4 && b12 * ks < 512) ks *= 2;
    return gemm_launch_tile<EPI, KvT, 1, 2>(a, ks, s);
  }
  // QKV (RoPE and the cache write need whole sums, so no atomic adds): when
  // 128x128 tiles are too few for the chip, K is split in two into float32
  // slabs of the workspace and a second pass sums them and finishes
  if (EPI == EPI_QKV && !q8 && a.split_ws && b22 < 384 && b22 * 2 >= 384 && nkt % 2 == 0 &&
      (int64_t)2 * M * Ntot <= a.split_ws_floats) {
    LinearArgs p = a;
    p.epi = EPI_STORE; p.out = a.split_ws; p.ldo = Ntot;
    const hipError_t e = gemm_launch_tile<EPI_STORE, float, 2, 2>(p, 2, s);
    if (e != hipSuccess) return e;
    return launch_split_epilogue(a, a.split_ws, 2, s);
  }
  // at most 64 rows (the 32-row LM head of a multi-sequence step, small
  // ubatches): 64-row tiles, so that 128-row tiles do not spend three
  // quarters of their matrix-core work on padding rows (LM head of 32 rows
  // at 8B widths: 32 sequences 3745-3752 -> 3756-3763 tok/s on one box)
  if (M <= 64 && b12 >= 384) return gemm_launch_tile<EPI, KvT, 1, 2>(a, 1, s);
  if (b24 >= 384) return gemm_launch_tile<EPI, KvT, 2, 4>(a, 1, s);
  if (b22 >= 384) return gemm_launch_tile<EPI, KvT, 2, 2>(a, 1, s);
  return gemm_launch_tile<EPI, KvT, 1, 2>(a, 1, s);
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
