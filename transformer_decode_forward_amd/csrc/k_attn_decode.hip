// Decode attention for gfx950 (ubatches of up to 32 tokens): split-K over
// each token's cached cells, then a merge of the splits' partial softmax
// sums.  Scaled dot-product attention over cached K/V with fewer KV heads
// than query heads (Ollama engine page, "Deep dive: the Llama forward pass in
// Go"; "KV Cache: memory for causal attention"): query head j reads KV head
// j / (n_head / n_head_kv); a token sees the cells of its sequence whose
// position is at most its own (in a windowed layer only the last n_swa).
#include <algorithm>
#include <type_traits>

#include "k_common.hpp"
#include "kernels.hpp"
#include "tdf.h"

namespace tdf {

// ---------------------------------------------------------------------------
// Decode attention.  Block (chunk j, kv head g, token t) runs the G = H/Hkv
// query heads of the group over the chunk's cells, one tile of rows at a
// time.  The cache is read in 16-byte pieces, PR = HD/E pieces per row, so a
// row is PR adjacent lanes: each lane dots its E elements with the G queries
// (held in registers), the PR lanes add their parts across the row (DPP), and
// the same lanes apply the row's probabilities to their E elements of V.
// Every row group (the PR lanes of a row) keeps its own online softmax
// (running max m, sum l and rescaled accumulator per head), so the tile loop
// needs no exchange between lanes beyond the row sums; the groups and the
// four waves are combined once at the end.
// Partials of several chunks are merged by attn_merge_kernel.

constexpr int kTile = 64;
constexpr int kCellStage = kDecodeCellStage;  // cell indices a block stages in LDS

// 16 bytes of cache elements -> floats
template <typename KvT> __device__ __forceinline__ void unpack16(uint4 u, float* out);
template <> __device__ __forceinline__ void unpack16<float>(uint4 u, float* out) {
  out[0] = __builtin_bit_cast(float, u.x); out[1] = __builtin_bit_cast(float, u.y);
  out[2] = __builtin_bit_cast(float, u.z); out[3] = __builtin_bit_cast(float, u.w);
}
template <> __device__ __forceinline__ void unpack16<kv_bf16>(uint4 u, float* out) {
  const uint32_t p[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[2 * j] = __builtin_bit_cast(float, p[j] << 16);
    out[2 * j + 1] = __builtin_bit_cast(float, p[j] & 0xFFFF0000u);
  }
}
// Q8_0: 16 int8 codes (the block scale is applied by the caller)
template <> __device__ __forceinline__ void unpack16<kv_q8>(uint4 u, float* out) {
  const uint32_t p[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int b = 0; b < 4; ++b) out[4 * j + b] = (float)((int32_t)(p[j] << (24 - 8 * b)) >> 24);
}
template <> __device__ __forceinline__ void unpack16<kv_f16>(uint4 u, float* out) {
  const uint32_t p[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[2 * j] = f16_to_f32((uint16_t)(p[j] & 0xFFFFu));
    out[2 * j + 1] = f16_to_f32((uint16_t)(p[j] >> 16));
  }
}

// sum over aligned groups of W adjacent lanes (W = 1..32), every lane of a
// group receiving the group's sum: xor 1 and xor 2 inside quads, then the
// half-row and row mirrors (lane i <-> 7-i, i <-> 15-i), then xor 16
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  if (W >= 2) v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  if (W >= 4) v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  if (W >= 8) v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  if (W >= 16) v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  if (W >= 32) v += __shfl_xor(v, 16, kWave);
  return v;
}

template <typename KvT, int HD, int G>
__global__ void __launch_bounds__(256) attn_decode_kernel(AttnArgs a) {
  typedef typename KvStore<KvT>::T ST;
  // Q8_0 rows: 16 codes per 16-byte piece, inside one 32-element block whose
  // fp16 scale (from the scale array after the codes) multiplies the piece's
  // score part and its probability for V
  constexpr bool Q8 = std::is_same<KvT, kv_q8>::value;
  constexpr int E = Q8 ? 16 : sizeof(ST) == 2 ? 8 : 4;  // elements per 16-byte piece
  constexpr int PR = HD / E;                           // pieces per row: 2..32
  constexpr int ROWS = 256 / PR;                       // rows per pass of the block
  constexpr int TILE = ROWS > kTile ? ROWS : kTile;    // rows per tile
  constexpr int PPER = TILE / ROWS;                    // passes per tile
  __shared__ float acc_s[4][G][HD];
  __shared__ float m_s[4][G], l_s[4][G];

  const int g = blockIdx.x, j = blockIdx.y, t = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nvis = a.n_vis[t];
  const int c_lo = j * a.chunk;
  if (c_lo >= nvis) return;
  const int c_hi = min(nvis, c_lo + a.chunk);
  const int32_t* cells = a.cell_list + a.list_off[t];
  const ST* kc = (const ST*)a.k_cache + (int64_t)g * a.n_ctx * HD;
  const ST* vc = (const ST*)a.v_cache + (int64_t)g * a.n_ctx * HD;
  const int r0 = tid / PR;        // row of this lane in each pass
  const int dq = (tid % PR) * E;  // first element of this lane's piece
  constexpr int NB = HD / 32;     // Q8_0 blocks per row
  const uint16_t* ksc = nullptr;
  const uint16_t* vsc = nullptr;
  if (Q8) {
    ksc = (const uint16_t*)((const int8_t*)a.k_cache + (int64_t)a.Hkv * a.n_ctx * HD) + (int64_t)g * a.n_ctx * NB + dq / 32;
    vsc = (const uint16_t*)((const int8_t*)a.v_cache + (int64_t)a.Hkv * a.n_ctx * HD) + (int64_t)g * a.n_ctx * NB + dq / 32;
  }

  // Loads come from clamped addresses, unconditionally: a load under a
  // divergent branch makes the compiler wait for every load in flight.  The
  // first tile's cell indices are requested together with q.
  // A chunk of several tiles stages its cell indices in LDS first (one
  // round trip), so that each next tile's K/V requests need no index load.
  __shared__ int32_t cell_s[kCellStage];
  const int span = c_hi - c_lo;
  const bool staged = span > TILE && span <= kCellStage;  // block-uniform
  if (staged) {
#pragma unroll
    for (int i = 0; i < kCellStage / 256; ++i) {
      const int e = tid + i * 256;
      const int32_t v = cells[c_lo + min(e, span - 1)];
      if (e < span) cell_s[e] = v;
    }
  }
  int row[PPER];
  uint4 kr[PPER], vr[PPER];
  uint16_t ksr[PPER], vsr[PPER];  // Q8_0 scales of the pieces
  if (!staged) {
#pragma unroll
    for (int pi = 0; pi < PPER; ++pi) row[pi] = cells[min(c_lo + r0 + pi * ROWS, c_hi - 1)];
  }
  float qr[G][E];
  {
    const float scale = rsqrtf((float)HD);
    const float* qp = a.q + ((int64_t)t * a.H + g * G) * HD + dq;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < E; e += 4) {
        const float4 v = *(const float4*)(qp + h * HD + e);
        qr[h][e] = v.x * scale; qr[h][e + 1] = v.y * scale;
        qr[h][e + 2] = v.z * scale; qr[h][e + 3] = v.w * scale;
      }
  }
  if (staged) {
    __syncthreads();
#pragma unroll
    for (int pi = 0; pi < PPER; ++pi) row[pi] = cell_s[min(r0 + pi * ROWS, span - 1)];
  }
#pragma unroll
  for (int pi = 0; pi < PPER; ++pi) {
    const int64_t off = (int64_t)row[pi] * HD + dq;
    kr[pi] = *(const uint4*)(kc + off);
    vr[pi] = *(const uint4*)(vc + off);
    if (Q8) {
      ksr[pi] = ksc[(int64_t)row[pi] * NB];
      vsr[pi] = vsc[(int64_t)row[pi] * NB];
    }
  }

  float m_w[G], l_w[G], acc[G][E];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_w[h] = -INFINITY;
    l_w[h] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
  }

  for (int c0 = c_lo; c0 < c_hi; c0 += TILE) {
    const int nc = min(TILE, c_hi - c0);
    uint4 kt[PPER], vt[PPER];
    float kst[PPER], vst[PPER];
#pragma unroll
    for (int pi = 0; pi < PPER; ++pi) {
      kt[pi] = kr[pi];
      vt[pi] = vr[pi];
      kst[pi] = Q8 ? f16_to_f32(ksr[pi]) : 1.f;
      vst[pi] = Q8 ? f16_to_f32(vsr[pi]) : 1.f;
    }
    if (c0 + TILE < c_hi) {  // block-uniform: request the next tile
#pragma unroll
      for (int pi = 0; pi < PPER; ++pi) {
        const int e = min(c0 + TILE + r0 + pi * ROWS, c_hi - 1);
        row[pi] = staged ? cell_s[e - c_lo] : cells[e];
      }
#pragma unroll
      for (int pi = 0; pi < PPER; ++pi) {
        const int64_t off = (int64_t)row[pi] * HD + dq;
        kr[pi] = *(const uint4*)(kc + off);
        vr[pi] = *(const uint4*)(vc + off);
        if (Q8) {
          ksr[pi] = ksc[(int64_t)row[pi] * NB];
          vsr[pi] = vsc[(int64_t)row[pi] * NB];
        }
      }
    }
    // scores of this lane's rows, summed over the PR lanes of each row
    float sc[PPER][G];
#pragma unroll
    for (int pi = 0; pi < PPER; ++pi) {
      float kf[E];
      unpack16<KvT>(kt[pi], kf);
      const bool live = r0 + pi * ROWS < nc;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float x0 = 0.f, x1 = 0.f;
#pragma unroll
        for (int e = 0; e < E; e += 2) {
          x0 = fmaf(qr[h][e], kf[e], x0);
          x1 = fmaf(qr[h][e + 1], kf[e + 1], x1);
        }
        const float x = group_sum<PR>(Q8 ? (x0 + x1) * kst[pi] : x0 + x1);
        sc[pi][h] = live ? x : -INFINITY;
      }
    }
    // online softmax per head over this lane's rows: the PR lanes of a row
    // group hold identical scores, so each group keeps its own running max,
    // sum and accumulator with no exchange between lanes
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = sc[0][h];
#pragma unroll
      for (int pi = 1; pi < PPER; ++pi) mx = fmaxf(mx, sc[pi][h]);
      const float m_new = fmaxf(m_w[h], mx);
      // a group with no live row yet keeps m = -inf, l = 0, acc = 0
      const float alpha = m_new == -INFINITY ? 1.f : __expf(m_w[h] - m_new);
      float ps = 0.f;
#pragma unroll
      for (int pi = 0; pi < PPER; ++pi) {
        const float p = sc[pi][h] == -INFINITY ? 0.f : __expf(sc[pi][h] - m_new);
        sc[pi][h] = p;
        ps += p;
      }
      l_w[h] = fmaf(l_w[h], alpha, ps);
      m_w[h] = m_new;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] *= alpha;
    }
    // probabilities times V (rows past the visible cells have p = 0)
#pragma unroll
    for (int pi = 0; pi < PPER; ++pi) {
      float vf[E];
      unpack16<KvT>(vt[pi], vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pv = Q8 ? sc[pi][h] * vst[pi] : sc[pi][h];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = fmaf(pv, vf[e], acc[h][e]);
      }
    }
  }

  // combine the row groups of the wave (lanes with equal tid % PR): common
  // max, rescale, then sum; afterwards the four waves through LDS
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = m_w[h];
#pragma unroll
    for (int o = PR; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o, kWave));
    const float w = m_w[h] == -INFINITY ? 0.f : __expf(m_w[h] - M);
    float l = l_w[h] * w;
#pragma unroll
    for (int o = PR; o < 64; o <<= 1) l += __shfl_xor(l, o, kWave);
    m_w[h] = M;
    l_w[h] = l;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float v = acc[h][e] * w;
#pragma unroll
      for (int o = PR; o < 64; o <<= 1) v += __shfl_xor(v, o, kWave);
      acc[h][e] = v;
    }
  }
  if (lane < PR) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < E; ++e) acc_s[wv][h][dq + e] = acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m_s[wv][h] = m_w[h];
      l_s[wv][h] = l_w[h];
    }
  }
  __syncthreads();
  // the first row of the chunk is live and belongs to wave 0, so M is finite
  const int nch = (nvis + a.chunk - 1) / a.chunk;
  constexpr int OUT_PER = (G * HD + 255) / 256;
#pragma unroll
  for (int o = 0; o < OUT_PER; ++o) {
    const int id = tid + o * 256;
    if (id < G * HD) {
      const int h = id / HD, d = id % HD;
      const float M = fmaxf(fmaxf(m_s[0][h], m_s[1][h]), fmaxf(m_s[2][h], m_s[3][h]));
      float L = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float wt = __expf(m_s[w][h] - M);
        L = fmaf(l_s[w][h], wt, L);
        A = fmaf(acc_s[w][h][d], wt, A);
      }
      if (nch == 1) {
        // the whole visible range is in this block: normalise and write
        const float r = A / L;
        const int64_t oi = ((int64_t)t * a.H + g * G + h) * HD + d;
        if (a.out) a.out[oi] = r;
        if (a.out_hi) split_bf16(r, a.out_hi[oi], a.out_lo[oi]);
      } else {
        const int64_t base = ((int64_t)t * a.H + g * G + h) * a.n_chunks + j;
        a.part_acc[base * HD + d] = A;
        if (d == 0) {
          a.part_ml[base * 2] = M;
          a.part_ml[base * 2 + 1] = L;
        }
      }
    }
  }
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
// ---------------------------------------------------------------------------
// Decode attention with the scores on the matrix cores (16-bit and Q8_0 caches, head
// dimension 64 or 128).  Block (chunk j, kv head g, token t) as above; each
// wave takes every fourth 16-cell tile of the chunk.  Scores: the G query
// heads (rows of a 16-row operand, the rest zero) times the tile's keys as
// the 32-deep columns of v_mfma_f32_16x16x32, with the query split into a
// 16-bit high part and a 16-bit remainder (two products per 32 dimensions),
// so the scores keep about 16 significant bits of the query; the keys enter
// exactly as stored.  The products leave head h of cell c in lane c + 16 (h / 4),
// component h % 4: row reductions over 16 lanes give each head's tile
// maximum and sum.  Probabilities go through 1 KB of LDS per wave to the
// lanes that own V: each lane keeps 8 dimensions of the output for every
// head and adds p * V over the cells of its row group (vector units, float32).
// Per-wave running maxima and sums are wave-uniform, so the row groups of a
// wave combine without rescaling; the four waves combine through LDS.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
template <typename KvT> struct Mfma16;
template <> struct Mfma16<kv_bf16> {
  typedef bf16x8 vec;
  typedef __bf16 elem;
  typedef s16x4 vec4;  // 4 bf16 bit patterns
  __device__ __forceinline__ static f32x4 mma(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static f32x4 mma4(vec4 a, vec4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  // x ~= hi + lo, both as stored 16-bit patterns
  __device__ __forceinline__ static void split(float x, short& hi, short& lo) {
    const __bf16 h = (__bf16)x;
    hi = __builtin_bit_cast(short, h);
    lo = __builtin_bit_cast(short, (__bf16)(x - (float)h));
  }
};
template <> struct Mfma16<kv_f16> {
  typedef f16x8 vec;
  typedef _Float16 elem;
  typedef f16x4 vec4;
  __device__ __forceinline__ static f32x4 mma(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static f32x4 mma4(vec4 a, vec4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static void split(float x, short& hi, short& lo) {
    const _Float16 h = (_Float16)x;
    hi = __builtin_bit_cast(short, h);
    lo = __builtin_bit_cast(short, (_Float16)(x - (float)h));
  }
};

template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
  return fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, -INFINITY),
                                                                      __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false)));
}
// Q8_0 rows use the bf16 products: the int8 codes are exact in bf16
template <> struct Mfma16<kv_q8> : Mfma16<kv_bf16> {};

// 8 int8 codes -> 8 bf16 (exact: at most 8 significant bits)
__device__ __forceinline__ bf16x8 q8_widen8(uint2 q) {
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
// fp16 scale b of a row's scale word(s)
__device__ __forceinline__ float q8_scale(uint2 r, int b) {
  const uint32_t w = b < 2 ? r.x : r.y;
  return f16_to_f32((uint16_t)(w >> (16 * (b & 1))));
}
__device__ __forceinline__ float q8_scale(uint32_t r, int b) { return f16_to_f32((uint16_t)(r >> (16 * b))); }

// max / sum over each row of 16 lanes, every lane of the row receiving it
__device__ __forceinline__ float row16_max(float v) {
  v = dpp_max<0xB1>(v);
  v = dpp_max<0x4E>(v);
  v = dpp_max<0x141>(v);
  return dpp_max<0x140>(v);
}
__device__ __forceinline__ float row16_sum(float v) { return group_sum<16>(v); }

// Work items of the matrix-core decode attention, one (token, chunk) pair
// each: items 0 .. F-1 are the whole chunks (a.chunk cells) of every token in
// token order, items F .. F+P-1 the last, partial chunks of the tokens whose
// visible count is not a multiple of a.chunk, again in token order.  Blocks
// are placed on the shader engines of an XCD round-robin and in order, and a
// block that must wait for a slot on a full engine holds back the ones after
// it; items of (nearly) equal size in dispatch order keep the engines evenly
// loaded, and the shorter partial chunks fill the end of the launch.  Every
// wave of a block computes the same result; false past the last item.
__device__ __forceinline__ bool decode_item(const int32_t* n_vis, const int32_t* list_off, int T, int chunk,
                                            int item, int lane, int& t_out, int& j_out, int& off_out) {
  int base = 0;  // whole chunks of the tokens before this group of 64
#pragma unroll 1
  for (int t0 = 0; t0 < T; t0 += 64) {
    // the tokens' list offsets ride with their counts (one round trip)
    const int nv = t0 + lane < T ? n_vis[t0 + lane] : 0;
    const int lo = list_off[min(t0 + lane, T - 1)];
    const int full = nv / chunk;
    int incl = full;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    const int tot = __shfl(incl, 63);
    if (item < base + tot) {
      const int tl = __builtin_ctzll(__ballot(base + incl > item));
      t_out = t0 + tl;
      j_out = item - base - __shfl(incl - full, tl);
      off_out = __shfl(lo, tl);
      return true;
    }
    base += tot;
  }
  int rel = item - base;  // among the partial chunks
#pragma unroll 1
  for (int t0 = 0; t0 < T; t0 += 64) {
    const int nv = t0 + lane < T ? n_vis[t0 + lane] : 0;
    const int lo = list_off[min(t0 + lane, T - 1)];
    const int part = nv % chunk != 0 ? 1 : 0;
    int incl = part;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    const int tot = __shfl(incl, 63);
    if (rel < tot) {
      const int tl = __builtin_ctzll(__ballot(incl > rel));
      t_out = t0 + tl;
      j_out = __shfl(nv / chunk, tl);
      off_out = __shfl(lo, tl);
      return true;
    }
    rel -= tot;
  }
  return false;
}

template <typename KvT, int HD, int G>
__global__ void __launch_bounds__(256) attn_decode_mfma_kernel(AttnArgs a) {
  typedef Mfma16<KvT> M;
  typedef typename M::vec vec;
  typedef typename M::elem elem;
  typedef typename M::vec4 vec4;
  typedef typename KvStore<KvT>::T ST;
  static_assert(HD == 64 || HD == 128, "head_dim 64 or 128");
  static_assert(G >= 1 && G <= 8, "at most 8 query heads per kv head");
  // Q8_0 rows: the codes (8 per lane and load) are widened to bf16 for the
  // products; each 32-deep score product is scaled by its cell's key block
  // scale, and the probabilities are multiplied by the value block scales
  // before the value product (one left operand per 32 output dimensions)
  constexpr bool Q8 = std::is_same<KvT, kv_q8>::value;
  constexpr int NB = HD / 32;  // Q8_0 blocks per row
  typedef typename std::conditional<Q8, uint2, vec>::type KRaw;
  typedef typename std::conditional<Q8, uint2, uint4>::type VRaw;
  typedef typename std::conditional<(HD == 128), uint2, uint32_t>::type SRaw;
  constexpr int NKC = HD / 32;   // 32-deep slices of the head dimension (scores)
  constexpr int NN = HD / 16;    // 16-wide output column blocks (P V)
  constexpr int PR = HD / 8;     // V loads: lanes per row (8 dimensions each)
  constexpr int RG = 64 / PR;    // V loads: row groups per wave
  constexpr int CPL = 16 / RG;   // V loads: cells of a tile per lane
  constexpr int VP = HD + 4;     // V tile row pitch in LDS (elements; breaks bank conflicts)
  __shared__ int32_t cell_s[kCellStage];
  __shared__ __attribute__((aligned(16))) short v_s[4][16 * VP];
  __shared__ float pt_s[4][G][16];
  __shared__ float acc_s[4][G][HD];
  __shared__ float m_s[4][G], l_s[4][G];
  __shared__ float vs_s[4][16][Q8 ? NB : 1];  // Q8_0: value block scales of the wave's tile

  // one-dimensional grid: kv head fastest (consecutive blocks go to
  // consecutive XCDs, so with 8 kv heads each XCD takes one head), then the
  // work item
  const int g = blockIdx.x % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int t, j, loff;
  if (a.T == 1) {
    // one token: the dense list is the chunk order itself, so the token's
    // count and list offset are requested together below (one round trip
    // fewer before the cell indices)
    t = 0;
    j = blockIdx.x / a.Hkv;
    loff = a.list_off[0];
  } else {
    if (!decode_item(a.n_vis, a.list_off, a.T, a.chunk, blockIdx.x / a.Hkv, lane, t, j, loff)) return;
    t = __builtin_amdgcn_readfirstlane(t);
    j = __builtin_amdgcn_readfirstlane(j);
    loff = __builtin_amdgcn_readfirstlane(loff);
  }
  if (j >= a.n_chunks) return;  // cells past the launch's split count are not covered
  const int nvis = a.n_vis[t];
  const int c_lo = j * a.chunk;
  if (c_lo >= nvis) return;  // a chunk past the token's cells (one token)
  const int c_hi = min(nvis, c_lo + a.chunk);
  const int span = c_hi - c_lo;  // 1 .. kCellStage (checked at launch)
  const int ntiles = (span + 15) >> 4;
  const int32_t* cells = a.cell_list + loff;
  const ST* kc = (const ST*)a.k_cache + (int64_t)g * a.n_ctx * HD;
  const ST* vc = (const ST*)a.v_cache + (int64_t)g * a.n_ctx * HD;
  // Q8_0 scale rows of this kv head (NB fp16 per cell)
  const SRaw* ksc = nullptr;
  const SRaw* vsc = nullptr;
  if constexpr (Q8) {
    ksc = (const SRaw*)((const int8_t*)a.k_cache + (int64_t)a.Hkv * a.n_ctx * HD) + (int64_t)g * a.n_ctx;
    vsc = (const SRaw*)((const int8_t*)a.v_cache + (int64_t)a.Hkv * a.n_ctx * HD) + (int64_t)g * a.n_ctx;
  }
  // Q8_0, tokens handing over their own K/V rows in float32: thread i takes
  // element i of [K row | V row] of this head and token (requested with q),
  // and the staging loop looks for the token's cell in this chunk
  const bool own = Q8 && a.new_k != nullptr;  // block-uniform
  int32_t slot = -1;
  float xown = 0.f;
  if (own) {
    slot = a.new_slot[t];
    const int i = min(tid, 2 * HD - 1);
    const float* src = i < HD ? a.new_k + i : a.new_v + (i - HD);
    xown = src[g * a.new_hs + (int64_t)t * HD];
  }
  int pos = -1;  // the cell's place in the chunk (at most one: a token sees a cell once)
  for (int e = tid; e < kCellStage; e += 256) {
    const int32_t v = cells[c_lo + min(e, span - 1)];
    cell_s[e] = v;  // entries past the span repeat its last cell
    if (own && e < span && v == slot) pos = e;
  }
  __shared__ int pos_s[4];
  if (own) {
    const uint64_t hit = __ballot(pos >= 0);
    const int p = __builtin_amdgcn_readlane(pos, hit ? (int)__builtin_ctzll(hit) : 0);
    if (lane == 0) pos_s[wv] = hit ? p : -1;
  }
  // query operand: lane l holds head l % 16 (zero past G), dimensions
  // 32 kk + 8 (l / 16) .. + 8, scaled by 1/sqrt(HD), as a high part and the
  // remainder
  vec qh[NKC], ql[NKC];
  {
    const int hq = lane & 15;
    const float scale = rsqrtf((float)HD);
    const float* qp = a.q + ((int64_t)t * a.H + g * G + min(hq, G - 1)) * HD + (lane >> 4) * 8;
#pragma unroll
    for (int kk = 0; kk < NKC; ++kk) {
      const float4 x0 = *(const float4*)(qp + kk * 32), x1 = *(const float4*)(qp + kk * 32 + 4);
      const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = hq < G ? x[e] * scale : 0.f;
        const elem h = (elem)v;
        qh[kk][e] = h;
        ql[kk][e] = (elem)(v - (float)h);
      }
    }
  }
  __syncthreads();

  // The chunk that holds the token's cell quantizes its rows by the Q8_0
  // block rule (32 adjacent threads = one block), stores codes and scales in
  // the cell, and keeps them in LDS for the tile that reads the cell: that
  // tile takes them from there instead of from its loads.
  __shared__ __attribute__((aligned(16))) int8_t oq_s[2][HD];      // K, V codes
  __shared__ __attribute__((aligned(16))) uint16_t osc_s[2][NB];   // K, V scale bits
  int otile = -1, orow = 0;  // tile and row of the cell in this chunk
  if (own) {
    const int p = max(max(pos_s[0], pos_s[1]), max(pos_s[2], pos_s[3]));
    if (p >= 0) {  // block-uniform
      otile = p >> 4;
      orow = p & 15;
      float amax = fabsf(xown);
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
      const uint16_t dbits = q8_scale_bits(amax);
      const int8_t code = q8_code(xown, f16_to_f32(dbits));
      if (tid < 2 * HD) {
        const int which = tid / HD, i = tid % HD;
        oq_s[which][i] = code;
        if ((i & 31) == 0) osc_s[which][i / 32] = dbits;
        int8_t* codes = (int8_t*)(which ? a.v_cache : a.k_cache);
        const int64_t crow = (int64_t)g * a.n_ctx + slot;
        codes[crow * HD + i] = code;
        if ((i & 31) == 0) ((uint16_t*)(codes + (int64_t)a.Hkv * a.n_ctx * HD))[crow * NB + i / 32] = dbits;
      }
      __syncthreads();
    }
  }

  const int rg = lane / PR, pc = lane % PR;  // V loads: row group, 8-dimension piece
  const int hrow = (lane >> 4) * 4;          // heads hrow .. hrow + 3 in the score layout
  // Reference maxima per head (wave-uniform): probabilities are exp(s - m),
  // and m moves only when a score exceeds it by more than kSlack, so the
  // accumulators are rarely rescaled; p stays below e^kSlack.
  constexpr float kSlack = 8.f;
  float m_w[G];
  f32x4 acc[NN], acc_l;
#pragma unroll
  for (int h = 0; h < G; ++h) m_w[h] = -INFINITY;
#pragma unroll
  for (int n = 0; n < NN; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  acc_l = f32x4{0.f, 0.f, 0.f, 0.f};
  vec4 ones;
  {
    short one_hi, one_lo;
    M::split(1.f, one_hi, one_lo);
#pragma unroll
    for (int q = 0; q < 4; ++q) ones[q] = __builtin_bit_cast(typename std::remove_reference<decltype(ones[0])>::type, one_hi);
  }
  short* vw = v_s[wv];
  auto cell_of = [&](int tl, int r) { return cell_s[min(tl * 16 + r, span - 1)]; };
  KRaw kn[NKC];
  VRaw vn[CPL];
  SRaw ksr, vsr;  // Q8_0: key scales of the lane's cell, value scales of cell lane % 16
  int tl = wv;
  {
    const int ck = cell_of(tl, lane & 15);
#pragma unroll
    for (int kk = 0; kk < NKC; ++kk) kn[kk] = *(const KRaw*)(kc + (int64_t)ck * HD + kk * 32 + (lane >> 4) * 8);
#pragma unroll
    for (int pi = 0; pi < CPL; ++pi) vn[pi] = *(const VRaw*)(vc + (int64_t)cell_of(tl, rg * CPL + pi) * HD + pc * 8);
    if constexpr (Q8) {
      ksr = ksc[ck];
      vsr = vsc[ck];
    }
  }
  for (; tl < ntiles; tl += 4) {
    const int nt = min(tl + 4, ntiles - 1);  // next tile of this wave (clamped)
    if constexpr (Q8) {
      if (tl == otile) {  // wave-uniform: the token's own cell is row orow of this tile
        const bool kr = (lane & 15) == orow;
#pragma unroll
        for (int kk = 0; kk < NKC; ++kk) {
          const KRaw o = *(const KRaw*)&oq_s[0][kk * 32 + (lane >> 4) * 8];
          kn[kk] = kr ? o : kn[kk];
        }
        const SRaw ko = *(const SRaw*)&osc_s[0][0], vo = *(const SRaw*)&osc_s[1][0];
        ksr = kr ? ko : ksr;
        vsr = kr ? vo : vsr;
        const VRaw o = *(const VRaw*)&oq_s[1][pc * 8];
#pragma unroll
        for (int pi = 0; pi < CPL; ++pi) vn[pi] = rg * CPL + pi == orow ? o : vn[pi];
      }
    }
    // this tile's V rows into the wave's LDS tile (rows of VP elements), then
    // the next tile's V requested into the same registers
#pragma unroll
    for (int pi = 0; pi < CPL; ++pi) {
      uint4 v4;
      if constexpr (Q8) v4 = __builtin_bit_cast(uint4, q8_widen8(vn[pi]));
      else v4 = vn[pi];
      uint2* dst = (uint2*)(vw + (rg * CPL + pi) * VP + pc * 8);
      dst[0] = make_uint2(v4.x, v4.y);
      dst[1] = make_uint2(v4.z, v4.w);
    }
    if constexpr (Q8) {
      if (lane < 16) {
#pragma unroll
        for (int b = 0; b < NB; ++b) vs_s[wv][lane][b] = q8_scale(vsr, b);
      }
    }
#pragma unroll
    for (int pi = 0; pi < CPL; ++pi) vn[pi] = *(const VRaw*)(vc + (int64_t)cell_of(nt, rg * CPL + pi) * HD + pc * 8);
    if constexpr (Q8) vsr = vsc[cell_of(nt, lane & 15)];
    // scores: component i of lane l is head 4 (l / 16) + i of cell l % 16;
    // then the next tile's K requested into the same registers
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKC; ++kk) {
      if constexpr (Q8) {
        const vec kv = q8_widen8(kn[kk]);
        f32x4 tk = {0.f, 0.f, 0.f, 0.f};
        tk = M::mma(qh[kk], kv, tk);
        tk = M::mma(ql[kk], kv, tk);
        const float dk = q8_scale(ksr, kk);
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = fmaf(dk, tk[i], s[i]);
      } else {
        s = M::mma(qh[kk], kn[kk], s);
        s = M::mma(ql[kk], kn[kk], s);
      }
    }
    {
      const int ck = cell_of(nt, lane & 15);
#pragma unroll
      for (int kk = 0; kk < NKC; ++kk) kn[kk] = *(const KRaw*)(kc + (int64_t)ck * HD + kk * 32 + (lane >> 4) * 8);
      if constexpr (Q8) ksr = ksc[ck];
    }
    const bool live = tl * 16 + (lane & 15) < span;
    float mr[4];  // reference max of this lane's heads
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = (live && hrow + i < G) ? s[i] : -INFINITY;
      float mh = m_w[i < G ? i : 0];
      if (G > 4 && hrow >= 4) mh = m_w[(4 + i) < G ? 4 + i : 0];
      mr[i] = mh;
    }
    bool over = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) over |= s[i] > mr[i] + kSlack;
    if (__ballot(over)) {
      // some score passed its reference by more than the slack: move the
      // references of every head to the exact running max, rescale
      float al[4];
      float mnew[G], alpha[G];
#pragma unroll
      for (int i = 0; i < 4; ++i) mr[i] = row16_max(s[i]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float th = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mr[h & 3]), (h >> 2) * 16));
        mnew[h] = fmaxf(m_w[h], th);  // finite: the tile has a live cell
        alpha[h] = __expf(m_w[h] - mnew[h]);
        m_w[h] = mnew[h];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mh = mnew[i < G ? i : 0], ah = alpha[i < G ? i : 0];
        if (G > 4 && hrow >= 4) {
          mh = mnew[(4 + i) < G ? 4 + i : 0];
          ah = alpha[(4 + i) < G ? 4 + i : 0];
        }
        mr[i] = mh;
        al[i] = ah;
      }
#pragma unroll
      for (int n = 0; n < NN; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[n][i] *= al[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc_l[i] *= al[i];
    }
    float ps[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ps[i] = s[i] == -INFINITY ? 0.f : __expf(s[i] - mr[i]);
    // probabilities to [head][cell] in LDS, read back as the 16 x 16 left
    // operand of the value product: lane l takes head l % 16, cells
    // 4 (l / 16) .. + 4, split into a high part and the remainder
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (hrow + i < G) pt_s[wv][hrow + i][lane & 15] = ps[i];
    __builtin_amdgcn_wave_barrier();
    vec4 ph, pl;
    vec4 phb[Q8 ? NB : 1], plb[Q8 ? NB : 1];  // Q8_0: probabilities times the value block scales
    {
      const int hp = lane & 15;
      const float4 p4 = *(const float4*)&pt_s[wv][min(hp, G - 1)][hrow];
      const float pv[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        short hi, lo;
        M::split(hp < G ? pv[q] : 0.f, hi, lo);
        ph[q] = __builtin_bit_cast(typename std::remove_reference<decltype(ph[0])>::type, hi);
        pl[q] = __builtin_bit_cast(typename std::remove_reference<decltype(pl[0])>::type, lo);
        if constexpr (Q8) {
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            M::split(hp < G ? pv[q] * vs_s[wv][hrow + q][b] : 0.f, hi, lo);
            phb[b][q] = __builtin_bit_cast(typename std::remove_reference<decltype(ph[0])>::type, hi);
            plb[b][q] = __builtin_bit_cast(typename std::remove_reference<decltype(pl[0])>::type, lo);
          }
        }
      }
    }
    // value product: right operand lane l = cells 4 (l / 16) .. + 4 of
    // dimension 16 n + l % 16, read down the LDS tile's column with one
    // transposing LDS load; a column of ones gives the probability sums
#pragma unroll
    for (int n = 0; n < NN; ++n) {
      // transposing LDS read: in each 16-lane group, lane 4e + q points at
      // cell hrow + e, dimensions 16n + 4q .. + 4; lane i of the group
      // receives dimension 16n + i of cells hrow .. hrow + 3
      const s16x4 bt = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)&vw[(hrow + ((lane & 15) >> 2)) * VP + n * 16 + 4 * (lane & 3)]);
      const vec4 b = __builtin_bit_cast(vec4, bt);
      if constexpr (Q8) {
        acc[n] = M::mma4(phb[n / 2], b, acc[n]);
        acc[n] = M::mma4(plb[n / 2], b, acc[n]);
      } else {
        acc[n] = M::mma4(ph, b, acc[n]);
        acc[n] = M::mma4(pl, b, acc[n]);
      }
    }
    acc_l = M::mma4(ph, ones, acc_l);
    acc_l = M::mma4(pl, ones, acc_l);
    __builtin_amdgcn_wave_barrier();
  }

  // accumulator rows are heads: head hrow + i of this lane's row, dimension
  // 16 n + l % 16; the waves combine through LDS
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (hrow + i < G) {
#pragma unroll
      for (int n = 0; n < NN; ++n) acc_s[wv][hrow + i][n * 16 + (lane & 15)] = acc[n][i];
    }
  if ((lane & 15) == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (hrow + i < G) l_s[wv][hrow + i] = acc_l[i];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) m_s[wv][h] = m_w[h];  // -inf for a wave without tiles
  }
  __syncthreads();
  const int nch = (nvis + a.chunk - 1) / a.chunk;
  constexpr int OUT_PER = (G * HD + 255) / 256;
#pragma unroll
  for (int o = 0; o < OUT_PER; ++o) {
    const int id = tid + o * 256;
    if (id < G * HD) {
      const int h = id / HD, d = id % HD;
      const float Mx = fmaxf(fmaxf(m_s[0][h], m_s[1][h]), fmaxf(m_s[2][h], m_s[3][h]));
      float L = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float wt = m_s[w][h] == -INFINITY ? 0.f : __expf(m_s[w][h] - Mx);
        L = fmaf(l_s[w][h], wt, L);
        A = fmaf(acc_s[w][h][d], wt, A);
      }
      if (nch == 1) {
        const float r = A / L;
        const int64_t oi = ((int64_t)t * a.H + g * G + h) * HD + d;
        if (a.out) a.out[oi] = r;
        if (a.out_hi) split_bf16(r, a.out_hi[oi], a.out_lo[oi]);
      } else {
        const int64_t base = ((int64_t)t * a.H + g * G + h) * a.n_chunks + j;
        a.part_acc[base * HD + d] = A;
        if (d == 0) {
          a.part_ml[base * 2] = Mx;
          a.part_ml[base * 2 + 1] = L;
        }
      }
    }
  }
}

// One block of NTH threads (NTH >= 64, a multiple of HD) per (query head,
// token).  Every load goes out before the token's split count is known: the
// NTH/HD thread groups request their splits' accumulators (every
// (NTH/HD)-th of the launch's n_chunks, up to kMergeBatch of them at once)
// while wave 0 requests the per-split maxima and sums; with the count in
// hand, wave 0 turns them into weights exp(m_j - M) and the total L, the
// groups sum their weighted splits (splits past the count are selected away,
// never multiplied: their memory holds stale values) and add up through
// LDS.  Decode ubatches (many splits, few tokens) use 256 threads; larger
// ubatches (few splits, many tokens) the smallest block.
// BATCH (the accumulators a thread requests at once) and R (the maxima and
// sums per lane of wave 0, 64 splits each) are sized at launch from the
// split count, so that a launch with few splits requests no clamped copies.
template <int HD, int NTH, int BATCH, int R>
__global__ void __launch_bounds__(NTH) attn_merge_kernel(AttnArgs a) {
  constexpr int kMergeBatch = BATCH;
  constexpr int NP = NTH / HD;
  __shared__ float w_s[kMergeMaxSplits];
  __shared__ float part_s[NP][HD];
  __shared__ float inv_l;
  const int h = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
  const int nc = a.n_chunks;  // splits launched (>= the token's count)
  const int64_t base = ((int64_t)t * a.H + h) * nc;
  const int d = tid % HD, part = tid / HD;
  const float* pa = a.part_acc + base * HD + d;
  // first batch of accumulators and the maxima / sums, requested together
  float v[kMergeBatch];
#pragma unroll
  for (int b = 0; b < kMergeBatch; ++b) v[b] = pa[(int64_t)min(part + b * NP, nc - 1) * HD];
  float2 ml[R];
  if (tid < 64) {
#pragma unroll
    for (int r = 0; r < R; ++r) ml[r] = *(const float2*)&a.part_ml[(base + min(tid + r * 64, nc - 1)) * 2];
  }
  const int nch = (a.n_vis[t] + a.chunk - 1) / a.chunk;
  if (nch == 1 && !a.merge_single) return;  // the split kernel wrote this token already
  if (tid < 64) {
    float M = -INFINITY;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (tid + r * 64 < nch) M = fmaxf(M, ml[r].x);
    M = wave_max(M);
    float L = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int jj = tid + r * 64;
      const float w = jj < nch ? __expf(ml[r].x - M) : 0.f;
      if (jj < nch) {
        w_s[jj] = w;
        L = fmaf(ml[r].y, w, L);
      }
    }
    L = wave_sum(L);
    if (tid == 0) inv_l = 1.f / L;
  }
  __syncthreads();
  float o = 0.f;
  for (int j0 = part; j0 < nch; j0 += NP * kMergeBatch) {
    if (j0 != part) {
#pragma unroll
      for (int b = 0; b < kMergeBatch; ++b) v[b] = pa[(int64_t)min(j0 + b * NP, nc - 1) * HD];
    }
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b) {
      const int jj = j0 + b * NP;
      if (jj < nch) o = fmaf(v[b], w_s[jj], o);
    }
  }
  part_s[part][d] = o;
  __syncthreads();
  if (tid >= HD) return;
  float r = 0.f;
#pragma unroll
  for (int q = 0; q < NP; ++q) r += part_s[q][tid];
  r *= inv_l;
  const int64_t oi = ((int64_t)t * a.H + h) * HD + tid;
  if (a.out) a.out[oi] = r;
  if (a.out_hi) split_bf16(r, a.out_hi[oi], a.out_lo[oi]);
}

template <typename KvT, int HD>
static hipError_t attn_launch_hd(const AttnArgs& a, hipStream_t s) {
  const int G = a.H / a.Hkv;
  // kv head fastest: consecutive blocks go to consecutive XCDs (block b to
  // XCD b % 8), so with 8 kv heads each XCD takes one head of every
  // (token, chunk) and all XCDs get the same work.  With the chunk index
  // fastest, XCD k would take chunk k of every token: sequences of unequal
  // length leave the XCDs of the high chunks idle.  The matrix-core kernel
  // also packs the (token, chunk) pairs that have cells into a dense list
  // (decode_item), so that no surplus block sits between two working ones.
  dim3 grid(a.Hkv, a.n_chunks, a.T);
  const unsigned items = (unsigned)a.Hkv * a.n_chunks * a.T;
  // 16-bit and Q8_0 caches with head_dim 64 or 128: scores and value
  // products on the matrix cores (chunks of at most kCellStage cells)
  bool done = false;
  // tokens' own rows handed over in float32: Q8_0 cache, the matrix-core
  // kernel (the only one that quantizes them)
  if (a.new_k && (!std::is_same<KvT, kv_q8>::value || !(HD == 64 || HD == 128) || a.chunk > kCellStage ||
                  !a.new_v || !a.new_slot))
    return hipErrorInvalidValue;
  if constexpr (!std::is_same<KvT, float>::value && (HD == 64 || HD == 128)) {
    if (a.chunk <= kCellStage) {
      switch (G) {
        case 1: attn_decode_mfma_kernel<KvT, HD, 1><<<items, 256, 0, s>>>(a); break;
        case 2: attn_decode_mfma_kernel<KvT, HD, 2><<<items, 256, 0, s>>>(a); break;
        case 4: attn_decode_mfma_kernel<KvT, HD, 4><<<items, 256, 0, s>>>(a); break;
        case 8: attn_decode_mfma_kernel<KvT, HD, 8><<<items, 256, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
      }
      done = true;
    }
  }
  if (!done) switch (G) {
    case 1: attn_decode_kernel<KvT, HD, 1><<<grid, 256, 0, s>>>(a); break;
    case 2: attn_decode_kernel<KvT, HD, 2><<<grid, 256, 0, s>>>(a); break;
    case 4: attn_decode_kernel<KvT, HD, 4><<<grid, 256, 0, s>>>(a); break;
    case 8: attn_decode_kernel<KvT, HD, 8><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // a single chunk per token writes its output directly
  if (a.n_chunks == 1) return hipSuccess;
  return launch_attention_merge(a, s);
}

// Merge of at most 8 splits with one wave per (token, head) pair, four
// pairs per block (the prefill's many pairs: half the waves of the block
// form, no LDS or barrier).  Lane i takes dimensions DPL i .. + DPL; the
// splits' maxima and sums sit in lanes 0 .. nch-1.  The same operations in
// the same order as attn_merge_kernel (wave reductions of the maxima and of
// the l w products, then the weighted sum split by split).
template <int HD>
__global__ void __launch_bounds__(256) attn_merge_wave_kernel(AttnArgs a) {
  constexpr int DPL = HD / 64;  // 1 or 2
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= a.T * a.H) return;  // wave-uniform
  const int t = pair / a.H, h = pair % a.H;
  const int nc = a.n_chunks;  // splits launched (>= the token's count), at most 8
  const int64_t base = ((int64_t)t * a.H + h) * nc;
  // every split's accumulators and the maxima / sums, requested together
  float v[8][DPL];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float* p = a.part_acc + (base + min(j, nc - 1)) * HD + lane * DPL;
    if constexpr (DPL == 2) {
      const float2 x = *(const float2*)p;
      v[j][0] = x.x; v[j][1] = x.y;
    } else {
      v[j][0] = *p;
    }
  }
  const float2 ml = *(const float2*)&a.part_ml[(base + min(lane, nc - 1)) * 2];
  const int nch = (a.n_vis[t] + a.chunk - 1) / a.chunk;
  const bool in = lane < nch;
  const float M = wave_max(in ? ml.x : -INFINITY);
  const float w = in ? __expf(ml.x - M) : 0.f;
  const float L = wave_sum(in ? fmaf(ml.y, w, 0.f) : 0.f);
  const float inv_l = 1.f / L;
  float o[DPL];
#pragma unroll
  for (int q = 0; q < DPL; ++q) o[q] = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= nch) break;  // wave-uniform
    const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
#pragma unroll
    for (int q = 0; q < DPL; ++q) o[q] = fmaf(v[j][q], wj, o[q]);
  }
  const int64_t oi = ((int64_t)t * a.H + h) * HD + lane * DPL;
#pragma unroll
  for (int q = 0; q < DPL; ++q) {
    const float r = (0.f + o[q]) * inv_l;
    if (a.out) a.out[oi + q] = r;
    if (a.out_hi) split_bf16(r, a.out_hi[oi + q], a.out_lo[oi + q]);
  }
}

template <int HD, int NTH>
static void merge_launch(const AttnArgs& a, dim3 grid, hipStream_t s) {
  const int per = (a.n_chunks + NTH / HD - 1) / (NTH / HD);  // splits per thread group
  if (per <= 4 && a.n_chunks <= 64) attn_merge_kernel<HD, NTH, 4, 1><<<grid, NTH, 0, s>>>(a);
  else if (per <= 8 && a.n_chunks <= 64) attn_merge_kernel<HD, NTH, 8, 1><<<grid, NTH, 0, s>>>(a);
  else if (a.n_chunks <= 64) attn_merge_kernel<HD, NTH, 16, 1><<<grid, NTH, 0, s>>>(a);
  else attn_merge_kernel<HD, NTH, 16, kMergeMaxSplits / 64><<<grid, NTH, 0, s>>>(a);
}

hipError_t launch_attention_merge(const AttnArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.n_chunks > kMergeMaxSplits) return hipErrorInvalidValue;
  const dim3 grid(a.H, a.T);
  const bool wide = a.n_chunks > 8;
  // many pairs, few splits, every token merged (the prefill): one wave per pair
  if (a.merge_single && a.n_chunks <= 8 && (a.hd == 64 || a.hd == 128) && (int64_t)a.T * a.H >= 1024) {
    const unsigned blocks = (unsigned)(((int64_t)a.T * a.H + 3) / 4);
    if (a.hd == 128) attn_merge_wave_kernel<128><<<blocks, 256, 0, s>>>(a);
    else attn_merge_wave_kernel<64><<<blocks, 256, 0, s>>>(a);
    return hipGetLastError();
  }
  switch (a.hd) {
    case 16:
      if (wide) merge_launch<16, 256>(a, grid, s);
      else merge_launch<16, 64>(a, grid, s);
      break;
    case 32:
      if (wide) merge_launch<32, 256>(a, grid, s);
      else merge_launch<32, 64>(a, grid, s);
      break;
    case 64:
      if (wide) merge_launch<64, 256>(a, grid, s);
      else merge_launch<64, 64>(a, grid, s);
      break;
    case 128:
      if (wide) merge_launch<128, 256>(a, grid, s);
      else merge_launch<128, 128>(a, grid, s);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename KvT>
static hipError_t attn_launch_kv(const AttnArgs& a, hipStream_t s) {
  switch (a.hd) {
    case 16:
      if constexpr (std::is_same<KvT, kv_q8>::value) return hipErrorInvalidValue;  // blocks of 32
      else return attn_launch_hd<KvT, 16>(a, s);
    case 32: return attn_launch_hd<KvT, 32>(a, s);
    case 64: return attn_launch_hd<KvT, 64>(a, s);
    case 128: return attn_launch_hd<KvT, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attention_decode(const AttnArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.kv_dtype == TDF_BF16) return attn_launch_kv<kv_bf16>(a, s);
  if (a.kv_dtype == TDF_F16) return attn_launch_kv<kv_f16>(a, s);
  if (a.kv_dtype == TDF_Q8_0) {
    if (a.hd % 32 != 0) return hipErrorInvalidValue;
    return attn_launch_kv<kv_q8>(a, s);
  }
  return attn_launch_kv<float>(a, s);
}

}  // namespace tdf
