// Launch interface of the gfx950 kernels (host side).  Every launcher
// enqueues on `stream` and returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tdf.h"

namespace tdf {

enum Epilogue : int {
  EPI_STORE = 0,     // out[t][n] = y                         (float32)
  EPI_RESIDUAL = 1,  // out[t][n] += y                        (residual stream)
  EPI_SWIGLU = 2,    // out[t][n] = silu(y_gate) * y_up       (w0 = gate, w1 = up)
  EPI_QKV = 3,       // RoPE on q and k, q -> q_out, k/v -> cache cells
};

// y[t][n] = sum_k W[n][k] act[t][k] for the rows of up to three matrices
// stacked along n (QKV: w0 = W_q, w1 = W_k, w2 = W_v).
struct LinearArgs {
  const void* w0 = nullptr;
  const void* w1 = nullptr;
  const void* w2 = nullptr;
  int n0 = 0, n1 = 0, n2 = 0;  // rows of each matrix
  int K = 0;                   // inner size (row length)
  int T = 0;                   // tokens (rows of act)
  // TDF_BF16, TDF_F32 or TDF_Q8_0 (each matrix one buffer: rows*K int8, then
  // its fp16 block scales [rows][K/32])
  int weight_dtype = TDF_BF16;
  // activations: float32 [T][K] (GEMV), or a bf16 pair hi + lo [T][K] (GEMM)
  const float* act_f32 = nullptr;
  // GEMV RMSNorm consumer: when norm_ssp is set, act_f32 holds u = g * x (the
  // gain times the raw residual) and y = (sum_k W[n][k] u[k]) / sqrt(ss/K + eps)
  // with ss = sum of norm_ssp[t][0 .. norm_nparts) (partial sums of x^2)
  const float* norm_ssp = nullptr;
  int norm_nparts = 0, norm_stride = 0;
  float norm_eps = 0.f;
  // GEMV residual producer: when next_g is set, the EPI_RESIDUAL epilogue also
  // writes next_u[t][n] = next_g[n] * x_new[t][n] and, per block, the partial
  // sum of x_new^2 over its rows to next_ssp[t][blockIdx]
  const float* next_g = nullptr;
  float* next_u = nullptr;
  float* next_ssp = nullptr;
  int next_stride = 0;
  // 9..32-token residual producer (launch_linear_skinny, EPI_RESIDUAL): when
  // norm_out_g is set, the residual pass also writes the next RMSNorm's
  // output g * x_new / sqrt(mean(x_new^2) + norm_out_eps) as a bf16 pair
  const float* norm_out_g = nullptr;
  uint16_t* norm_out_hi = nullptr;
  uint16_t* norm_out_lo = nullptr;
  float norm_out_eps = 0.f;
  const uint16_t* act_hi = nullptr;
  const uint16_t* act_lo = nullptr;
  // epilogue
  int epi = EPI_STORE;
  float* out = nullptr;        // [T][ldo] float32 (STORE / RESIDUAL / SWIGLU)
  uint16_t* out_hi = nullptr;  // [T][ldo] bf16 pair (GEMM SWIGLU)
  uint16_t* out_lo = nullptr;
  int ldo = 0;
  // EPI_QKV
  float* q_out = nullptr;      // [T][n0] float32
  void* k_cache = nullptr;     // layer base [n_head_kv][n_ctx][head_dim]
  void* v_cache = nullptr;
  int kv_dtype = 0;            // tdf_dtype
  int n_ctx = 0;
  int head_dim = 0;
  const int32_t* slots = nullptr;  // [T] cell of each token
  const int32_t* pos = nullptr;    // [T] position of each token
  const float2* rope_cs = nullptr; // [T][head_dim/2] (cos, sin) of pos * theta^(-2i/head_dim)
  // optional float32 workspace of the matrix-core GEMM (K-split partials of
  // an epilogue that needs whole sums)
  float* split_ws = nullptr;
  int64_t split_ws_floats = 0;
};

hipError_t launch_linear_gemv(const LinearArgs& a, hipStream_t s);
hipError_t launch_linear_gemm(const LinearArgs& a, hipStream_t s);
bool gemm_supported(const LinearArgs& a);
// 9..32 tokens on the matrix cores with the weights streamed once (split
// over K into the float32 workspace `part` of kSkinnyPartFloats floats,
// then an epilogue pass); bf16 weights, hi/lo activations, K % 128 == 0
constexpr int64_t kSkinnyPartFloats = 32ll * 65536;
bool skinny_supported(const LinearArgs& a);
// the residual pass can also write the next RMSNorm (norm_out_g)
bool skinny_norm_supported(const LinearArgs& a);
hipError_t launch_linear_skinny(const LinearArgs& a, float* part, hipStream_t s);
// the epilogue of `a` over K-split partials part[ksplit][a.T][N] (their sum)
hipError_t launch_split_epilogue(const LinearArgs& a, float* part, int ksplit, hipStream_t s);

// x[t][:] = E[token[t]][:] (to float32); with g set also u = g * x and
// ssp[t * stride] = sum x^2 (one partial per row).  n_rows: rows of the
// table (a Q8_0 table's scales start at byte n_rows * d)
hipError_t launch_embed(const void* table, int weight_dtype, int n_rows, const int32_t* tokens, int T, int d,
                        float* x, const float* g, float* u, float* ssp, int stride, hipStream_t s);
// number of blocks (= partial sums) a residual GEMV writes for N rows
int gemv_residual_parts(int N);
// out = x / sqrt(mean(x^2) + eps) * g, as float32 and/or a bf16 pair
// (hi = bf16(out), lo = bf16(out - hi))
hipError_t launch_rmsnorm(const float* x, const float* g, int T, int d, float eps, float* out_f32,
                          uint16_t* out_hi, uint16_t* out_lo, hipStream_t s);
// cs[t][i] = (cos, sin)(pos[t] * inv_freq[i]) for i < half, angles in double
hipError_t launch_rope_table(const int32_t* pos, const double* inv_freq, int T, int half, float2* cs,
                             hipStream_t s);
// dst[pairs[2i]] = pairs[2i+1]
hipError_t launch_scatter(int32_t* dst, const int64_t* pairs, int n, hipStream_t s);
// dst[r][:] = src[rows[r]][:] (rows == NULL: identity, dst == NULL: no copy);
// with g set also u[r] = g * src[rows[r]] and ssp[r * stride] = its sum of squares
hipError_t launch_gather_rows(const float* src, const int32_t* rows, int R, int d, float* dst,
                              const float* g, float* u, float* ssp, int stride, hipStream_t s);
// Rotate the cached keys of n_cells cells (every layer and KV head) by the
// per-pair angles whose (cos, sin) are cs[hd/2]: (k[2i], k[2i+1]) ->
// (k[2i] c - k[2i+1] s, k[2i] s + k[2i+1] c), in double, stored back in the
// cache type.  kv: cache base, layer_stride_bytes: distance between the K
// arrays of consecutive layers; each K array is [Hkv][n_ctx][hd].
hipError_t launch_kv_rotate(void* kv, int kv_dtype, size_t layer_stride_bytes, int L, int Hkv, int n_ctx, int hd,
                            const int32_t* cells, int n_cells, const double2* cs, hipStream_t s);

// Q8_0 KV cache (layout per layer array: int8 codes [Hkv][n_ctx][hd], then
// fp16 scales [Hkv][n_ctx][hd/32]).  kv_quantize stores float32 rows (row
// (t, h) at src + t * t_stride + h * h_stride) in cells[t]; kv_rotate_q8
// rotates the stored keys of n_cells cells (every layer) and re-quantizes.
inline size_t kv_q8_array_bytes(int Hkv, int n_ctx, int hd) {
  const size_t b = (size_t)Hkv * n_ctx * hd + (size_t)Hkv * n_ctx * (hd / 32) * 2;
  return (b + 255) / 256 * 256;
}
hipError_t launch_kv_quantize(const float* src_k, const float* src_v, int64_t t_stride, int64_t h_stride, int T,
                              int Hkv, int hd, const int32_t* cells, void* k_dst, void* v_dst, int n_ctx,
                              hipStream_t s);
hipError_t launch_kv_rotate_q8(void* kv, size_t layer_stride_bytes, int L, int Hkv, int n_ctx, int hd,
                               const int32_t* cells, int n_cells, const double2* cs, hipStream_t s);

// Sampling chain of one token per logits row (temperature > 0): Top-K
// (1 <= top_k <= kMaxTopK), temperature, softmax, Top-P, Min-P, draw with
// u[r] in [0, 1) (device array); tok[r] receives the token.
constexpr int kMaxTopK = 1024;
struct SampleParams {
  float temperature = 1.f;
  int top_k = 40;
  float top_p = 1.f;
  float min_p = 0.f;
};
hipError_t launch_sample(const float* logits, int R, int V, const SampleParams& sp, const float* u,
                         int32_t* tok, hipStream_t s);

// tok[r] = argmax_n logits[r][n] (lowest index on ties), in two passes over
// argmax_splits(V) column splits; part_v / part_i hold R * argmax_splits(V)
// partial results
constexpr int kArgmaxMaxSplits = 256;
int argmax_splits(int V);
hipError_t launch_argmax(const float* logits, int R, int V, int32_t* tok, float* part_v, int32_t* part_i,
                         hipStream_t s);

// Attention of T tokens over their visible cells (split over cell chunks,
// then merged).  q [T][H][hd] float32; caches [Hkv][n_ctx][hd]; cell lists
// [n_seq_max][n_ctx]; list_off[t] = seq * n_ctx; n_vis[t] = visible cells.
// most splits of one token's cell range that the attention merge combines
constexpr int kMergeMaxSplits = 256;

struct AttnArgs {
  const float* q = nullptr;
  const void* k_cache = nullptr;
  const void* v_cache = nullptr;
  int kv_dtype = 0;
  const int32_t* cell_list = nullptr;
  const int32_t* list_off = nullptr;
  const int32_t* n_vis = nullptr;
  int T = 0, H = 0, Hkv = 0, hd = 0, n_ctx = 0;
  int chunk = 256;       // cells per split
  int n_chunks = 1;      // splits of the longest token
  float* part_acc = nullptr;  // [T][H][n_chunks][hd]
  float* part_ml = nullptr;   // [T][H][n_chunks][2]
  // merge kernel: also merge tokens with a single chunk (the prefill split
  // kernel always writes partials; the decode split kernel writes such tokens
  // directly)
  int merge_single = 0;
  float* out = nullptr;       // [T][H][hd] float32
  uint16_t* out_hi = nullptr; // optional bf16 pair
  uint16_t* out_lo = nullptr;
  // Q8_0 cache on the matrix cores (optional): token t's own K and V rows
  // arrive as float32 (head g at new_k / new_v + g * new_hs + t * hd) instead
  // of in its cell new_slot[t]; the block whose chunk holds that cell
  // quantizes them, stores them in the cell and uses them itself.  The caller
  // guarantees that no token sees the cell of another token of the launch.
  const float* new_k = nullptr;
  const float* new_v = nullptr;
  int64_t new_hs = 0;
  const int32_t* new_slot = nullptr;
};
hipError_t launch_attention_decode(const AttnArgs& a, hipStream_t s);
// Decode attention stages a block's cell indices in LDS; with 16-bit or Q8_0
// caches and head_dim 64 or 128 it runs on the matrix cores when a.chunk is at most
// this many cells.  (32 sequences at 1.2 k-7.9 k cells: 2048-cell chunks
// give about 720 blocks, one round of the 768 resident slots, 3765 -> 3790
// tok/s bf16 and 4200 -> 4300 Q8_0 against 1024-cell chunks' 1.7 rounds;
// 4096-cell chunks leave slots idle: 3590 / 3610.)
constexpr int kDecodeCellStage = 2048;
inline bool attn_decode_on_mfma(int kv_dtype, int hd) {
  return (kv_dtype == TDF_F16 || kv_dtype == TDF_BF16 || kv_dtype == TDF_Q8_0) && (hd == 64 || hd == 128);
}
// merge of split partials only (part_* -> out / out_bf16)
hipError_t launch_attention_merge(const AttnArgs& a, hipStream_t s);

// Prefill attention on the matrix cores.  Query tiles of up to 32 tokens of
// one sequence: tile_tokens [n_tiles][32] (ubatch token index, -1 padding),
// tile_list_off[i] = seq * n_ctx, tile_nvis_max[i] = largest n_vis in the
// tile.  q is float32 [T][H][hd]; bf16 or f16 caches, head_dim 64 or 128.
struct PrefillAttnArgs {
  const float* q = nullptr;
  const void* k_cache = nullptr;
  const void* v_cache = nullptr;
  int kv_dtype = 0;
  const int32_t* cell_list = nullptr;
  const int32_t* n_vis = nullptr;
  const int32_t* tile_tokens = nullptr;
  const int32_t* tile_list_off = nullptr;
  const int32_t* tile_nvis_max = nullptr;
  // windowed layers: token t sees list entries [n_lo[t], n_vis[t]); a tile's
  // cell range starts at tile_lo (its smallest n_lo); NULL = from entry 0
  const int32_t* n_lo = nullptr;
  const int32_t* tile_lo = nullptr;
  int n_tiles = 0, H = 0, Hkv = 0, hd = 0, n_ctx = 0;
  int chunk = 0, n_splits = 1;
  float* part_acc = nullptr;
  float* part_ml = nullptr;
  float* out = nullptr;
  uint16_t* out_hi = nullptr;
  uint16_t* out_lo = nullptr;
  AttnArgs merge;  // used when n_splits > 1 (T, H, hd, chunk, n_chunks = n_splits, parts, outs; its
                   // n_vis counts entries from the tile's first entry)
};
bool prefill_attention_supported(int kv_dtype, int head_dim);
hipError_t launch_attention_prefill(const PrefillAttnArgs& a, hipStream_t s);

}  // namespace tdf
