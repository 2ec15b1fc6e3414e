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
// whose V^T operand comes from the V tile as stored (row = cell) through
// gfx950's transposing LDS read (ds_read_b64_tr_b16: four 16-lane groups,
// each turning 4 cells x 16 dimensions into 16 lanes x 4 cells), read in the
// same cell order.  K and V rows are requested as whole rows (16 consecutive
// lanes per 256-byte row).  The rescale by exp(m_old - m_new) is per lane
// and skipped when no lane's max moved; the causal mask is skipped on tiles
// that every query of the wave sees whole.  Cells come from the sequence's
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
// store it in LDS as a bf16 pair hi + lo (V transposed), shared by the G
// waves; each product
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
  constexpr int KP = HD + 8;     // K (and 16-bit V) row pitch (elements)
  constexpr int VP = kCT + 8;    // Q8_0: V^T row pitch (elements)
  constexpr bool Q8 = std::is_same<KvT, kv_q8>::value;
  constexpr int NB = HD / 32;    // Q8_0 blocks per row
  typedef typename std::conditional<Q8, int8_t, uint16_t>::type ST;
  typedef typename std::conditional<Q8, uint2, uint4>::type Raw;  // 8 stored elements
  constexpr int NCH = HD / 8;    // 16-byte chunks per row
  // K tile (row = cell, pitch KP); 16-bit caches: V tile likewise; Q8_0: the
  // dequantized tiles as bf16 pairs, V transposed (pitch VP)
  __shared__ __attribute__((aligned(16))) uint16_t k_s[kCT * KP];
  __shared__ __attribute__((aligned(16))) uint16_t v_s[Q8 ? 8 : kCT * KP];
  __shared__ __attribute__((aligned(16))) uint16_t vt_s[Q8 ? HD * VP : 8];
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
  // Q^T fragments (B operand), hi and lo: lane holds Q[query][ks*16 + qg*8 + 0..7],
  // requested as two 16-byte pieces per ks (one 4-byte request per element
  // put 64 scattered addresses in each of 64 requests: 8-15 us per block)
  vec qh[HD / 16], qlo[HD / 16];
  {
    const float* qrow = a.q + ((int64_t)max(t, 0) * a.H + h) * HD + qg * 8;
#pragma unroll
    for (int ks = 0; ks < HD / 16; ++ks) {
      const float4 x0 = *(const float4*)(qrow + ks * 16), x1 = *(const float4*)(qrow + ks * 16 + 4);
      const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = t >= 0 ? x[e] * scale : 0.f;
        const E hi = (E)v;
        qh[ks][e] = hi;
        qlo[ks][e] = (E)(v - (float)hi);
      }
    }
  }

  f32x16 o[HD / 32];
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

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
  auto cell_at = [&](int cc) -> int64_t { return staged ? cell_s[cc - c_lo] : cells[cc]; };

  // One tile: scores, online softmax and the value product.  kfrag(sub, ks)
  // is the K fragment of cell sub*32 + (lane % 32), dimensions ks*16 +
  // (lane / 32)*8 .. + 8; vfrag(dt, sub, s2) the V^T fragment of dimension
  // dt*32 + (lane % 32), cells base + (lane / 32)*4 + 0..3 and base + 8 +
  // (lane / 32)*4 + 0..3 with base = sub*32 + s2*16.  Q8_0 adds the low parts.
  auto tile_compute = [&](int c0, auto kfrag, auto vfrag, auto klfrag, auto vlfrag) {
    // S^T for two 32-cell halves: s[sub][r] <-> cell sub*32 + (r/4)*8 + qg*4 + r%4
    f32x16 s[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[sub][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < HD / 16; ++ks) {
        const vec kf = kfrag(sub, ks);
        s[sub] = M::mma(kf, qh[ks], s[sub]);
        s[sub] = M::mma(kf, qlo[ks], s[sub]);
        if constexpr (Q8) s[sub] = M::mma(klfrag(sub, ks), qh[ks], s[sub]);
      }
    }
    // causal / range mask and online softmax for this lane's query.  The mask
    // is skipped (wave-uniform) when every real query of the wave sees the
    // whole tile; padding queries (t < 0) are never written.
    const bool part = t >= 0 && (c0 + kCT > min(nvis, c_hi) || c0 < vis_lo);
    float tmax = -INFINITY;
    if (__ballot(part)) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ci = c0 + sub * 32 + (r >> 2) * 8 + qg * 4 + (r & 3);
          if (ci >= nvis || ci >= c_hi || ci < vis_lo) s[sub][r] = -INFINITY;
          tmax = fmaxf(tmax, s[sub][r]);
        }
    } else {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[sub][r]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const float m_new = fmaxf(m_run, tmax);
    const bool live = m_new != -INFINITY;
    // exp(m_run - m_new) is exactly 1 where the max did not move: the
    // accumulators are rescaled only when some lane's max moved
    const bool moved = live && m_new != m_run;
    const float alpha = moved ? __expf(m_run - m_new) : 1.f;
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
    if (__ballot(moved)) {
#pragma unroll
      for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }
    // O^T += V^T P^T; A operand lane: d = dt*32 + ql, cells in P's order
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const vec vf = vfrag(dt, sub, s2);
          o[dt] = M::mma(vf, ph[sub][s2], o[dt]);
          o[dt] = M::mma(vf, plo[sub][s2], o[dt]);
          if constexpr (Q8) o[dt] = M::mma(vlfrag(dt, sub, s2), ph[sub][s2], o[dt]);
        }
  };

  if constexpr (!Q8) {
    // K and V tiles as stored (row = cell, pitch KP), each row requested by
    // NCH consecutive lanes (whole 16-byte chunks of one row), so a wave's
    // request covers 64 / NCH whole rows.  The V^T fragments are read with
    // the LDS transpose load.
    constexpr int PPT = kCT * NCH / (64 * G);  // chunks of each of K and V per thread
    uint4 kreg[PPT], vreg[PPT];
    auto kf = [&](int sub, int ks) -> vec { return *(const vec*)&k_s[(sub * 32 + ql) * KP + ks * 16 + qg * 8]; };
    auto vf = [&](int dt, int sub, int s2) -> vec {
      // two transposed reads of 4 cells x 16 dimensions per 16-lane group:
      // lane j of the group points at cell j / 4 of the four, dimensions
      // 4 (j % 4) .. + 4, and receives its own dimension of the four cells
      const int gi = lane >> 4, j = lane & 15;
      const int d0 = dt * 32 + 16 * (gi & 1) + 4 * (j & 3);
      const int row = sub * 32 + s2 * 16 + (gi >> 1) * 4 + (j >> 2);
      typedef short v4s __attribute__((ext_vector_type(4)));
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)&v_s[row * KP + d0]);
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)&v_s[(row + 8) * KP + d0]);
      const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
      return __builtin_bit_cast(vec, make_uint4(l2.x, l2.y, h2.x, h2.y));
    };
    auto none = [](int, int) -> vec { return vec{}; };
    auto none3 = [](int, int, int) -> vec { return vec{}; };
    for (int c0 = c_lo; c0 < c_hi; c0 += kCT) {
      __syncthreads();  // the previous tile's readers are done
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int ii = tid + i * 64 * G;
        const int64_t off = cell_at(min(c0 + ii / NCH, c_hi - 1)) * HD + (ii % NCH) * 8;
        kreg[i] = *(const uint4*)(kc + off);
        vreg[i] = *(const uint4*)(vc + off);
      }
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int ii = tid + i * 64 * G;
        *(uint4*)&k_s[(ii / NCH) * KP + (ii % NCH) * 8] = kreg[i];
        *(uint4*)&v_s[(ii / NCH) * KP + (ii % NCH) * 8] = vreg[i];
      }
      __syncthreads();
      tile_compute(c0, kf, vf, none, none3);
    }
  } else {
    constexpr int CHUNKS = kCT * HD / 8;  // 16-byte pieces of one K (or V) tile
    constexpr int PPT = CHUNKS / (64 * G);  // pieces of each per thread
    // Requests go out SUB pieces at a time (requesting the next tile during
    // the current one would need 32 more registers than the kernel has left:
    // measured slower with the spills).
    constexpr int SUB = PPT < 4 ? PPT : 4;
    Raw kreg[SUB], vreg[SUB];
    uint16_t ksreg[SUB], vsreg[SUB];  // scales of the pieces' blocks
    for (int c0 = c_lo; c0 < c_hi; c0 += kCT) {
      __syncthreads();  // the previous tile's readers are done
#pragma unroll
      for (int i0 = 0; i0 < PPT; i0 += SUB) {
#pragma unroll
        for (int i = 0; i < SUB; ++i) {
          const int ii = tid + (i0 + i) * 64 * G;
          const int64_t cell = cell_at(min(c0 + ii % kCT, c_hi - 1));
          const int64_t row = cell * HD + (ii / kCT) * 8;
          kreg[i] = *(const Raw*)(kc + row);
          vreg[i] = *(const Raw*)(vc + row);
          ksreg[i] = ksc[cell * NB + (ii / kCT) / 4];
          vsreg[i] = vsc[cell * NB + (ii / kCT) / 4];
        }
#pragma unroll
        for (int i = 0; i < SUB; ++i) {
          const int ii = tid + (i0 + i) * 64 * G;
          const int c = ii % kCT, dchunk = (ii / kCT) * 8;
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
        }
      }
      __syncthreads();
      auto kf = [&](const uint16_t* kb) {
        return [=](int sub, int ks) -> vec { return *(const vec*)&kb[(sub * 32 + ql) * KP + ks * 16 + qg * 8]; };
      };
      auto vf = [&](const uint16_t* vtb) {
        return [=](int dt, int sub, int s2) -> vec {
          const uint16_t* vrow = &vtb[(dt * 32 + ql) * VP];
          const int cb = sub * 32 + s2 * 16 + qg * 4;
          const uint2 lo = *(const uint2*)(vrow + cb);
          const uint2 hi = *(const uint2*)(vrow + cb + 8);
          return __builtin_bit_cast(vec, make_uint4(lo.x, lo.y, hi.x, hi.y));
        };
      };
      tile_compute(c0, kf(k_s), vf(vt_s), kf(kl_s), vf(vtl_s));
    }
  }

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
