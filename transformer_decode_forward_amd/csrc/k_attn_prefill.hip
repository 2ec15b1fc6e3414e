// Prefill attention on the gfx950 matrix cores (flash-style, online softmax).
//
// Scaled dot-product attention of the ubatch's queries over the cached keys
// and values of their sequence, causal by position (Ollama engine page,
// "Deep dive: the Llama forward pass in Go" and "KV Cache: memory for causal
// attention"; llama.cpp walkthrough, "KV-cache and the Prefill / Decode
// stages").  Query head j reads KV head j / (n_head / n_head_kv).
//
// Block = one query tile (up to 32 tokens of one sequence) x one KV head;
// wave w of the block handles query head g*G + w, so each K/V tile staged in
// LDS serves the G heads of the group.  Per 64-cell K/V tile a wave computes
//   S^T = K Q^T      (32x32x16 MFMA: lane = query, registers = cells)
// so a query's 64 scores sit in two lanes (lane and lane^32); the running
// max and sum need one cross-lane exchange.  The probabilities are then
// already in the B-operand layout of
//   O^T += V^T P^T   (lane = query, registers = head dims)
// with V staged transposed in LDS, read in the same cell order.  The rescale
// by exp(m_old - m_new) is per lane.  Cells come from the sequence's
// position-ordered cell list; token t sees the first n_vis[t] entries, or in
// a windowed layer the entries [n_lo[t], n_vis[t]) (the block's cell range
// then starts at the tile's smallest n_lo).
//
// K and V are exact in their cache type; Q and the probabilities P are split
// into a pair hi + lo of the MFMA type (hi = round(x), lo = round(x - hi)),
// each product taking two MFMAs, so that the scores and the weighted sums keep
// about 16 significant bits, as the projections do.
//
// Q8_0 caches (blocks of 32 along the head dimension: fp16 scale d, int8
// codes q): the block's staging threads form d * q (exact in float32) and
// store it in LDS as a bf16 pair hi + lo, shared by the G waves; each product
// adds a third MFMA for the low part (Klo Qhi, Vlo Phi), so K and V enter
// with about 16 significant bits.
//
// With n_splits > 1 each block covers one range of `chunk` list entries and
// writes (max, sum, unnormalised accumulator) partials, merged afterwards by
// the decode merge kernel.
#include "k_common.hpp"
#include "kernels.hpp"
#include "tdf.h"

namespace tdf {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <typename KvT> struct MfmaOf;
template <> struct MfmaOf<kv_bf16> {
  typedef bf16x8 vec;
  typedef __bf16 elem;
  __device__ __forceinline__ static f32x16 mma(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct MfmaOf<kv_q8> : MfmaOf<kv_bf16> {};
template <> struct MfmaOf<kv_f16> {
  typedef f16x8 vec;
  typedef _Float16 elem;
  __device__ __forceinline__ static f32x16 mma(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

constexpr int kQT = 32;   // queries per tile
constexpr int kCT = 64;   // cells per K/V tile
constexpr int kPrefStage = 2048;  // cell list entries a block stages in LDS

template <typename KvT, int HD, int G>
__global__ void __launch_bounds__(64 * G) __attribute__((amdgpu_waves_per_eu(2))) attn_prefill_kernel(PrefillAttnArgs a) {
  typedef MfmaOf<KvT> M;
  typedef typename M::vec vec;
  constexpr int KP = HD + 8;     // K row pitch (elements)
  constexpr int VP = kCT + 8;    // V^T row pitch (elements)
  constexpr bool Q8 = std::is_same<KvT, kv_q8>::value;
  constexpr int NB = HD / 32;    // Q8_0 blocks per row
  typedef typename std::conditional<Q8, int8_t, uint16_t>::type ST;
  typedef typename std::conditional<Q8, uint2, uint4>::type Raw;  // 8 stored elements
  __shared__ __attribute__((aligned(16))) uint16_t k_s[kCT * KP];
  __shared__ __attribute__((aligned(16))) uint16_t vt_s[HD * VP];
  // Q8_0: low parts of the dequantized tiles
  __shared__ __attribute__((aligned(16))) uint16_t kl_s[Q8 ? kCT * KP : 8];
  __shared__ __attribute__((aligned(16))) uint16_t vtl_s[Q8 ? HD * VP : 8];

  const int tile = blockIdx.x, g = blockIdx.y, split = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = g * G + w;
  const int ql = lane & 31, qg = lane >> 5;
  const int t = a.tile_tokens[tile * kQT + ql];      // -1 for padding
  const int nvis = t >= 0 ? a.n_vis[t] : 0;
  const int vis_lo = t >= 0 && a.n_lo ? a.n_lo[t] : 0;  // first visible entry (window)
  const int tile_nvis = a.tile_nvis_max[tile];
  const int c_lo = (a.tile_lo ? a.tile_lo[tile] : 0) + split * a.chunk;
  if (c_lo >= tile_nvis) return;
  const int c_hi = min(tile_nvis, c_lo + a.chunk);
  const int32_t* cells = a.cell_list + a.tile_list_off[tile];
  const ST* kc = (const ST*)a.k_cache + (int64_t)g * a.n_ctx * HD;
  const ST* vc = (const ST*)a.v_cache + (int64_t)g * a.n_ctx * HD;
  // Q8_0 scales: [Hkv][n_ctx][NB] fp16 after the codes
  const uint16_t* ksc = nullptr;
  const uint16_t* vsc = nullptr;
  if constexpr (Q8) {
    ksc = (const uint16_t*)((const int8_t*)a.k_cache + (int64_t)a.Hkv * a.n_ctx * HD) + (int64_t)g * a.n_ctx * NB;
    vsc = (const uint16_t*)((const int8_t*)a.v_cache + (int64_t)a.Hkv * a.n_ctx * HD) + (int64_t)g * a.n_ctx * NB;
  }
  const float scale = rsqrtf((float)HD);

  typedef typename M::elem E;
  // Q^T fragments (B operand), hi and lo: lane holds Q[query][ks*16 + qg*8 + 0..7]
  vec qh[HD / 16], qlo[HD / 16];
#pragma unroll
  for (int ks = 0; ks < HD / 16; ++ks) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = t >= 0 ? a.q[((int64_t)t * a.H + h) * HD + ks * 16 + qg * 8 + e] * scale : 0.f;
      const E hi = (E)v;
      qh[ks][e] = hi;
      qlo[ks][e] = (E)(v - (float)hi);
    }
  }

  f32x16 o[HD / 32];
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  constexpr int CHUNKS = kCT * HD / 8;  // 16-byte pieces of one K (or V) tile
  constexpr int PPT = CHUNKS / (64 * G);  // pieces of each per thread
  // The block's cell list entries go to LDS once (ranges up to kPrefStage
  // entries); tile loads then need no index round trip.  Entries past the
  // block's range repeat its last cell: their scores are masked and their
  // probabilities zero.
  __shared__ int32_t cell_s[kPrefStage];
  const int span = c_hi - c_lo;
  const bool staged = span <= kPrefStage;  // block-uniform
  if (staged)
    for (int e = tid; e < span; e += 64 * G) cell_s[e] = cells[c_lo + e];
  __syncthreads();
  // Requests go out SUB pieces at a time (requesting the next tile during
  // the current one would need 32 more registers than the kernel has left:
  // measured slower with the spills).
  constexpr int SUB = PPT < 4 ? PPT : 4;
  Raw kreg[SUB], vreg[SUB];
  uint16_t ksreg[SUB], vsreg[SUB];  // Q8_0: scales of the pieces' blocks
#define TILE_LOAD(c0_, i0_)                                                            \
  do {                                                                                 \
    _Pragma("unroll") for (int i = 0; i < SUB; ++i) {                                  \
      const int ii = tid + ((i0_) + i) * 64 * G;                                       \
      const int cc = min((c0_) + ii % kCT, c_hi - 1);                                  \
      const int64_t cell = staged ? cell_s[cc - c_lo] : cells[cc];                     \
      const int64_t row = cell * HD + (ii / kCT) * 8;                                  \
      kreg[i] = *(const Raw*)(kc + row);                                               \
      vreg[i] = *(const Raw*)(vc + row);                                               \
      if constexpr (Q8) {                                                              \
        ksreg[i] = ksc[cell * NB + (ii / kCT) / 4];                                    \
        vsreg[i] = vsc[cell * NB + (ii / kCT) / 4];                                    \
      }                                                                                \
    }                                                                                  \
  } while (0)
  for (int c0 = c_lo; c0 < c_hi; c0 += kCT) {
    __syncthreads();  // the previous tile's readers are done
#pragma unroll
    for (int i0 = 0; i0 < PPT; i0 += SUB) {
      TILE_LOAD(c0, i0);
#pragma unroll
      for (int i = 0; i < SUB; ++i) {
        const int ii = tid + (i0 + i) * 64 * G;
        const int c = ii % kCT, dchunk = (ii / kCT) * 8;
        if constexpr (Q8) {
          const float dk = f16_to_f32(ksreg[i]), dv = f16_to_f32(vsreg[i]);
          const int8_t* kq = (const int8_t*)&kreg[i];
          const int8_t* vq = (const int8_t*)&vreg[i];
          uint16_t kh[8], kl[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            split_bf16(dk * (float)kq[e], kh[e], kl[e]);
            uint16_t vh, vl;
            split_bf16(dv * (float)vq[e], vh, vl);
            vt_s[(dchunk + e) * VP + c] = vh;
            vtl_s[(dchunk + e) * VP + c] = vl;
          }
          auto pack = [](const uint16_t* x) {
            return make_uint4(x[0] | ((uint32_t)x[1] << 16), x[2] | ((uint32_t)x[3] << 16),
                              x[4] | ((uint32_t)x[5] << 16), x[6] | ((uint32_t)x[7] << 16));
          };
          *(uint4*)&k_s[c * KP + dchunk] = pack(kh);
          *(uint4*)&kl_s[c * KP + dchunk] = pack(kl);
        } else {
          *(uint4*)&k_s[c * KP + dchunk] = kreg[i];
          const uint16_t* vh = (const uint16_t*)&vreg[i];
#pragma unroll
          for (int e = 0; e < 8; ++e) vt_s[(dchunk + e) * VP + c] = vh[e];
        }
      }
    }
    __syncthreads();

    // S^T for two 32-cell halves: s[sub][r] <-> cell sub*32 + (r/4)*8 + qg*4 + r%4
    f32x16 s[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[sub][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < HD / 16; ++ks) {
        const vec kf = *(const vec*)&k_s[(sub * 32 + ql) * KP + ks * 16 + qg * 8];
        s[sub] = M::mma(kf, qh[ks], s[sub]);
        s[sub] = M::mma(kf, qlo[ks], s[sub]);
        if constexpr (Q8) {
          const vec kfl = *(const vec*)&kl_s[(sub * 32 + ql) * KP + ks * 16 + qg * 8];
          s[sub] = M::mma(kfl, qh[ks], s[sub]);
        }
      }
    }
    // causal / range mask and online softmax for this lane's query
    float tmax = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ci = c0 + sub * 32 + (r >> 2) * 8 + qg * 4 + (r & 3);
        if (ci >= nvis || ci >= c_hi || ci < vis_lo) s[sub][r] = -INFINITY;
        tmax = fmaxf(tmax, s[sub][r]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const float m_new = fmaxf(m_run, tmax);
    const bool live = m_new != -INFINITY;
    const float alpha = live ? __expf(m_run - m_new) : 1.f;
    float psum = 0.f;
    vec ph[2][2], plo[2][2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = live ? __expf(s[sub][r] - m_new) : 0.f;
        psum += p;
        const E hi = (E)p;
        ph[sub][r >> 3][r & 7] = hi;
        plo[sub][r >> 3][r & 7] = (E)(p - (float)hi);
      }
    psum += __shfl_xor(psum, 32, kWave);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    // O^T += V^T P^T; A operand lane: d = dt*32 + ql, cells in P's order
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt) {
      const uint16_t* vrow = &vt_s[(dt * 32 + ql) * VP];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int cb = sub * 32 + s2 * 16 + qg * 4;
          const uint2 lo = *(const uint2*)(vrow + cb);
          const uint2 hi = *(const uint2*)(vrow + cb + 8);
          const vec vf = __builtin_bit_cast(vec, make_uint4(lo.x, lo.y, hi.x, hi.y));
          o[dt] = M::mma(vf, ph[sub][s2], o[dt]);
          o[dt] = M::mma(vf, plo[sub][s2], o[dt]);
          if constexpr (Q8) {
            const uint16_t* vrl = &vtl_s[(dt * 32 + ql) * VP];
            const uint2 l2 = *(const uint2*)(vrl + cb);
            const uint2 h2 = *(const uint2*)(vrl + cb + 8);
            o[dt] = M::mma(__builtin_bit_cast(vec, make_uint4(l2.x, l2.y, h2.x, h2.y)), ph[sub][s2], o[dt]);
          }
        }
    }
  }

#undef TILE_LOAD
  // o[dt][r] <-> head dim dt*32 + (r/4)*8 + qg*4 + r%4 of this lane's query
  if (t < 0 || nvis <= c_lo) return;
  if (a.n_splits == 1) {
    const float inv = 1.f / l_run;
    const int64_t base = ((int64_t)t * a.H + h) * HD;
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = dt * 32 + i * 8 + qg * 4;
        const float4 v = make_float4(o[dt][4 * i] * inv, o[dt][4 * i + 1] * inv, o[dt][4 * i + 2] * inv,
                                     o[dt][4 * i + 3] * inv);
        if (a.out) *(float4*)&a.out[base + d] = v;
        if (a.out_hi) {
          uint16_t h[4], l[4];
          split_bf16(v.x, h[0], l[0]);
          split_bf16(v.y, h[1], l[1]);
          split_bf16(v.z, h[2], l[2]);
          split_bf16(v.w, h[3], l[3]);
          *(uint2*)&a.out_hi[base + d] = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
          *(uint2*)&a.out_lo[base + d] = make_uint2(l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16));
        }
      }
  } else {
    const int64_t pb = ((int64_t)t * a.H + h) * a.n_splits + split;
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = dt * 32 + i * 8 + qg * 4;
        *(float4*)&a.part_acc[pb * HD + d] =
            make_float4(o[dt][4 * i], o[dt][4 * i + 1], o[dt][4 * i + 2], o[dt][4 * i + 3]);
      }
    if (qg == 0) {
      a.part_ml[pb * 2] = m_run;
      a.part_ml[pb * 2 + 1] = l_run;
    }
  }
}

template <typename KvT, int HD>
static hipError_t prefill_attn_hd(const PrefillAttnArgs& a, hipStream_t s) {
  const int G = a.H / a.Hkv;
  dim3 grid(a.n_tiles, a.Hkv, a.n_splits);
  switch (G) {
    case 1: attn_prefill_kernel<KvT, HD, 1><<<grid, 64, 0, s>>>(a); break;
    case 2: attn_prefill_kernel<KvT, HD, 2><<<grid, 128, 0, s>>>(a); break;
    case 4: attn_prefill_kernel<KvT, HD, 4><<<grid, 256, 0, s>>>(a); break;
    case 8: attn_prefill_kernel<KvT, HD, 8><<<grid, 512, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool prefill_attention_supported(int kv_dtype, int head_dim) {
  return (kv_dtype == TDF_BF16 || kv_dtype == TDF_F16 || kv_dtype == TDF_Q8_0) && (head_dim == 64 || head_dim == 128);
}

hipError_t launch_attention_prefill(const PrefillAttnArgs& a, hipStream_t s) {
  if (a.n_tiles <= 0) return hipSuccess;
  hipError_t e;
  if (a.kv_dtype == TDF_BF16)
    e = a.hd == 128 ? prefill_attn_hd<kv_bf16, 128>(a, s) : prefill_attn_hd<kv_bf16, 64>(a, s);
  else if (a.kv_dtype == TDF_F16)
    e = a.hd == 128 ? prefill_attn_hd<kv_f16, 128>(a, s) : prefill_attn_hd<kv_f16, 64>(a, s);
  else if (a.kv_dtype == TDF_Q8_0)
    e = a.hd == 128 ? prefill_attn_hd<kv_q8, 128>(a, s) : prefill_attn_hd<kv_q8, 64>(a, s);
  else
    return hipErrorInvalidValue;
  if (e != hipSuccess || a.n_splits == 1) return e;
  return launch_attention_merge(a.merge, s);
}

}  // namespace tdf
