// C ABI and host runtime of the decoder forward pass (declared in tdf.h).
//
// One decode call (llama.cpp walkthrough, "Steps 11-12" and "Step 13"):
// intake and defaults (host_plan), an all-or-nothing check that the batch
// fits in the free cells, then per ubatch: place the tokens in cells and
// commit them, upload the ubatch's small integer arrays in one copy, and
// enqueue the layer loop of the Ollama engine page ("Deep dive: the Llama
// forward pass in Go").  Linear layers over at most 8 rows stream the
// weights as GEMVs (float32 activations), larger ones run on the MFMA GEMM;
// ubatches of at most 32 tokens use the split-K decode attention, larger ones
// the MFMA attention.  The logits
// of flagged rows land in one device buffer in batch order ("Steps 14-15"),
// followed by a device argmax per row; the call synchronises its stream
// before returning.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <map>
#include <mutex>
#include <tuple>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "host_plan.hpp"
#include "kernels.hpp"
#include "tdf.h"

using namespace tdf;

namespace {

thread_local std::string g_err;

void set_err(const std::string& s) { g_err = s; }

// test hooks: TDF_FAULT_ALLOC=n in the environment makes the n-th device
// allocation of the process fail; tdf_fault_alloc(n) makes the n-th next one
// fail (host-side failure injection: the allocation is simply not made)
int g_alloc_count = 0;
int g_fail_in = 0;
hipError_t dev_alloc(void** p, size_t bytes) {
  static const int fault_at = [] {
    const char* e = getenv("TDF_FAULT_ALLOC");
    return e ? atoi(e) : 0;
  }();
  ++g_alloc_count;
  const bool planted = g_fail_in > 0 && --g_fail_in == 0;
  if (planted || (fault_at > 0 && g_alloc_count == fault_at)) {
    *p = nullptr;
    return hipErrorOutOfMemory;
  }
  if (bytes == 0) bytes = 256;
  return hipMalloc(p, bytes);
}

// stream-ordered scratch of one call, released on every return path
struct CallScratch {
  hipStream_t s;
  std::vector<void*> p;
  explicit CallScratch(hipStream_t st) : s(st) {}
  hipError_t alloc(void** out, size_t bytes) {
    *out = nullptr;
    hipError_t e = hipMallocAsync(out, bytes ? bytes : 256, s);
    if (e == hipSuccess) p.push_back(*out);
    return e;
  }
  ~CallScratch() {
    for (void* x : p) (void)hipFreeAsync(x, s);
  }
};

size_t dtype_size(int dt) { return dt == TDF_F32 ? 4 : 2; }

constexpr int kGemvMaxT = 8;        // linear layers of up to this many rows stream weights as GEMVs
constexpr int kDecodeMaxT = 32;     // ubatches up to this size use the split-K decode attention
constexpr int kChunkCapDecode = 256; // attention splits per token (decode)
constexpr int kChunkCapPrefill = 32; // attention splits per token (larger ubatches)
static_assert(kChunkCapDecode <= kMergeMaxSplits && kChunkCapPrefill <= kMergeMaxSplits, "merge width");

constexpr int kQTile = 32;           // tokens per prefill attention query tile

// int32 entries of the per-call staging area.  A ubatch of U tokens stores 5
// per token, its selected rows (<= U), its query tiles (at most
// U/32 + 1 + min(U, n_seq_max) tiles of 34 entries) and, for windowed
// attention, 4 more per token and 1 more per tile; rounded up to 4.
size_t staging_i32(int n_batch, int n_ubatch, int n_seq_max) {
  const size_t U = (size_t)n_ubatch;
  const size_t n_ub = ((size_t)n_batch + U - 1) / U;
  const size_t tiles = U / kQTile + 1 + std::min<size_t>(U, (size_t)n_seq_max);
  return n_ub * (10 * U + (kQTile + 3) * tiles + 4) + 16;
}
size_t staging_i64_base(int n_batch, int n_ubatch, int n_seq_max) {
  return (staging_i32(n_batch, n_ubatch, n_seq_max) * 4 + 15) & ~(size_t)15;
}

}  // namespace

struct tdf_model {
  tdf_hparams hp;               // swa_layers cleared; the flags live in `windowed`
  std::vector<uint8_t> windowed;  // per layer: attention limited to the n_swa window
  bool any_window = false;
  const void* token_embd;
  const float* output_norm;
  const void* output;
  std::vector<tdf_layer_weights> layers;
};

struct tdf_context {
  const tdf_model* m = nullptr;
  int n_ctx = 0, n_batch = 0, n_ubatch = 0, n_seq_max = 0, kv_dtype = 0;
  bool output_all = false, dry_run = false;
  int n_cu = 0;                     // compute units of the context's device
  hipStream_t stream = nullptr;
  bool own_stream = false;
  KvBook book;

  // device memory
  void* kv = nullptr;               // [L][2][Hkv][n_ctx][hd]
  size_t kv_layer_bytes = 0;        // one of K or V of one layer
  int32_t* cell_list = nullptr;     // [n_seq_max][n_ctx]
  double* inv_freq = nullptr;       // [hd/2]
  float2* rope_cs = nullptr;        // [U][hd/2] (cos, sin) of the ubatch's positions
  float *x = nullptr, *xs = nullptr, *q = nullptr, *o = nullptr, *mb = nullptr;
  // decode-path RMSNorm hand-off: u = g * x rows and partial sums of x^2
  float *u = nullptr, *ssp = nullptr;
  int ssp_stride = 0;
  // bf16 hi/lo pairs of the matrix-core inputs: normed rows, attention output, MLP product
  uint16_t *h_hi = nullptr, *h_lo = nullptr, *o_hi = nullptr, *o_lo = nullptr, *m_hi = nullptr, *m_lo = nullptr;
  float *part_acc = nullptr, *part_ml = nullptr;
  float* kv_stage = nullptr;        // Q8_0 cache: float32 K/V rows of the ubatch [2][Hkv][n_ubatch][hd]
  int32_t* iota = nullptr;          // Q8_0 cache: 0 .. n_ubatch-1 (staging rows)
  size_t part_rows = 0;             // capacity in (token, head, chunk) triples
  void* ints = nullptr;             // per-call packed integers
  size_t ints_bytes = 0;
  char* ints_host = nullptr;        // pinned staging
  float* logits = nullptr;          // [cap][V]
  int32_t* d_tok = nullptr;         // [cap]
  float* skinny_part = nullptr;     // K-split partials of the 9..32-token linear layers
  float* qkv_split = nullptr;       // K-split partials of the ubatch QKV GEMM [2][n_ubatch][(H + 2 Hkv) hd]
  int64_t qkv_split_floats = 0;
  float* amax_v = nullptr;          // [cap][argmax_splits(V)] partial maxima
  int32_t* amax_i = nullptr;        // [cap][argmax_splits(V)] their indices
  int32_t* h_tok = nullptr;         // pinned [cap]
  int logits_cap = 0;
  // tdf_sample_logits buffers (caller's rows), grown on demand
  float* ext_u = nullptr;           // [ext_rows]
  int32_t* ext_tok = nullptr;       // [ext_rows]
  int32_t* ext_htok = nullptr;      // pinned [ext_rows]
  float* ext_pv = nullptr;          // [ext_parts] argmax partials
  int32_t* ext_pi = nullptr;
  size_t ext_rows = 0, ext_parts = 0;
  std::vector<void*> owned;

  // TDF_CTX_PROFILE: event pairs of the current call, totals per (op, path)
  bool profile = false;
  std::vector<hipEvent_t> ev_pool;
  size_t ev_used = 0;
  std::vector<int> ev_slot;          // slot of each recorded pair
  int64_t prof_n[2 * TDF_OP_COUNT] = {};
  double prof_ms[2 * TDF_OP_COUNT] = {};

  // launch replay: one instantiated graph per decode ubatch shape
  bool use_graphs = true;
  std::map<std::tuple<int, int, int, int, int, const void*, const void*, const void*, int, int, int, int, int>,
           hipGraphExec_t> graphs;
  int64_t n_graph_captures = 0, n_graph_replays = 0;

  // results of the last decode
  int n_outputs = 0;
  std::vector<int32_t> out_ids;     // batch index of each output row
  std::vector<int32_t> row_of;      // batch index -> output row or -1
  std::vector<int32_t> last_slots;
  std::vector<float> logits_host;
  std::vector<char> host_row_ok;
};

// ---------------------------------------------------------------------------
// helpers

#define TDF_HIP(expr)                                                        \
  do {                                                                       \
    hipError_t _e = (expr);                                                  \
    if (_e != hipSuccess) {                                                  \
      set_err(std::string(#expr) + ": " + hipGetErrorString(_e));            \
      return TDF_E_DEVICE;                                                   \
    }                                                                        \
  } while (0)

static int ctx_alloc(tdf_context* c, void** p, size_t bytes) {
  hipError_t e = dev_alloc(p, bytes);
  if (e != hipSuccess) {
    set_err(std::string("device allocation failed: ") + hipGetErrorString(e));
    return TDF_E_ALLOC;
  }
  c->owned.push_back(*p);
  return TDF_OK;
}

static void ctx_free(tdf_context* c, void* p) {
  if (!p) return;
  auto it = std::find(c->owned.begin(), c->owned.end(), p);
  if (it != c->owned.end()) c->owned.erase(it);
  (void)hipFree(p);
}

// ---- profiling (TDF_CTX_PROFILE) ----

static hipEvent_t prof_event(tdf_context* c) {
  if (c->ev_used == c->ev_pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    c->ev_pool.push_back(e);
  }
  return c->ev_pool[c->ev_used++];
}

// records a start event; returns the slot to pass to prof_end (or -1)
static int prof_begin(tdf_context* c, int op, bool mfma) {
  if (!c->profile) return -1;
  hipEvent_t e = prof_event(c);
  if (!e || hipEventRecord(e, c->stream) != hipSuccess) return -1;
  return 2 * op + (mfma ? 1 : 0);
}

static void prof_end(tdf_context* c, int slot) {
  if (slot < 0) return;
  hipEvent_t e = prof_event(c);
  if (!e || hipEventRecord(e, c->stream) != hipSuccess) return;
  c->ev_slot.push_back(slot);
}

// after the stream has been synchronised: fold the recorded pairs in
static void prof_collect(tdf_context* c) {
  if (!c->profile) return;
  for (size_t i = 0; i < c->ev_slot.size(); ++i) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, c->ev_pool[2 * i], c->ev_pool[2 * i + 1]) == hipSuccess) {
      c->prof_ms[c->ev_slot[i]] += ms;
      c->prof_n[c->ev_slot[i]] += 1;
    }
  }
  c->ev_slot.clear();
  c->ev_used = 0;
}

static void ctx_release(tdf_context* c) {
  for (auto& kv : c->graphs) (void)hipGraphExecDestroy(kv.second);
  c->graphs.clear();
  for (hipEvent_t e : c->ev_pool) (void)hipEventDestroy(e);
  c->ev_pool.clear();
  for (void* p : c->owned) (void)hipFree(p);
  c->owned.clear();
  if (c->ints_host) (void)hipHostFree(c->ints_host);
  if (c->h_tok) (void)hipHostFree(c->h_tok);
  if (c->ext_htok) (void)hipHostFree(c->ext_htok);
  c->ints_host = nullptr;
  c->h_tok = nullptr;
  c->ext_htok = nullptr;
  if (c->own_stream && c->stream) (void)hipStreamDestroy(c->stream);
  c->stream = nullptr;
}

static int ensure_logits(tdf_context* c, int rows) {
  if (rows <= c->logits_cap) return TDF_OK;
  const int V = c->m->hp.n_vocab;
  void *lg = nullptr, *tk = nullptr, *av = nullptr, *ai = nullptr;
  const size_t n_part = (size_t)rows * argmax_splits(V);
  hipError_t e = dev_alloc(&lg, (size_t)rows * V * sizeof(float));
  if (e == hipSuccess) e = dev_alloc(&tk, (size_t)rows * sizeof(int32_t));
  if (e == hipSuccess) e = dev_alloc(&av, n_part * sizeof(float));
  if (e == hipSuccess) e = dev_alloc(&ai, n_part * sizeof(int32_t));
  void* htk = nullptr;
  if (e == hipSuccess) e = hipHostMalloc(&htk, (size_t)rows * sizeof(int32_t), hipHostMallocDefault);
  if (e != hipSuccess) {
    if (lg) (void)hipFree(lg);
    if (tk) (void)hipFree(tk);
    if (av) (void)hipFree(av);
    if (ai) (void)hipFree(ai);
    set_err(std::string("logits allocation failed: ") + hipGetErrorString(e));
    return TDF_E_ALLOC;
  }
  auto drop = [&](void* p) {
    if (!p) return;
    auto it = std::find(c->owned.begin(), c->owned.end(), p);
    if (it != c->owned.end()) c->owned.erase(it);
    (void)hipFree(p);
  };
  (void)hipStreamSynchronize(c->stream);
  for (auto& kv : c->graphs) (void)hipGraphExecDestroy(kv.second);
  c->graphs.clear();
  drop(c->logits);
  drop(c->d_tok);
  drop(c->amax_v);
  drop(c->amax_i);
  if (c->h_tok) (void)hipHostFree(c->h_tok);
  c->logits = (float*)lg;
  c->d_tok = (int32_t*)tk;
  c->amax_v = (float*)av;
  c->amax_i = (int32_t*)ai;
  c->h_tok = (int32_t*)htk;
  c->owned.push_back(lg);
  c->owned.push_back(tk);
  c->owned.push_back(av);
  c->owned.push_back(ai);
  c->logits_cap = rows;
  return TDF_OK;
}

static void* kv_k(const tdf_context* c, int l) { return (char*)c->kv + (size_t)(2 * l) * c->kv_layer_bytes; }
static void* kv_v(const tdf_context* c, int l) { return (char*)c->kv + (size_t)(2 * l + 1) * c->kv_layer_bytes; }

// ---------------------------------------------------------------------------
// model

extern "C" tdf_model* tdf_model_create(const tdf_hparams* hp, const tdf_weights* w) {
  if (!hp || !w) { set_err("hparams or weights is NULL"); return nullptr; }
  const tdf_hparams& h = *hp;
  if (h.n_vocab <= 0 || h.n_embd <= 0 || h.n_layer < 0 || h.n_head <= 0 || h.n_head_kv <= 0 ||
      h.head_dim <= 0 || (h.head_dim & 1) || h.n_ff <= 0 || h.n_head % h.n_head_kv != 0 ||
      !(h.rms_eps >= 0.f) || !(h.rope_theta > 0.f)) {
    set_err("invalid hparams");
    return nullptr;
  }
  if (h.weight_dtype != TDF_F32 && h.weight_dtype != TDF_BF16 && h.weight_dtype != TDF_Q8_0) {
    set_err("weight_dtype must be F32, BF16 or Q8_0");
    return nullptr;
  }
  if (h.weight_dtype == TDF_Q8_0 && (h.n_embd % 32 || (h.n_head * h.head_dim) % 32 || h.n_ff % 32)) {
    set_err("Q8_0 weights need n_embd, n_head*head_dim and n_ff to be multiples of 32");
    return nullptr;
  }
  const int G = h.n_head / h.n_head_kv;
  if (!(G == 1 || G == 2 || G == 4 || G == 8)) { set_err("n_head / n_head_kv must be 1, 2, 4 or 8"); return nullptr; }
  if (!(h.head_dim == 16 || h.head_dim == 32 || h.head_dim == 64 || h.head_dim == 128)) {
    set_err("head_dim must be 16, 32, 64 or 128");
    return nullptr;
  }
  if (h.n_swa < 0) { set_err("n_swa must be >= 0"); return nullptr; }
  if (!w->token_embd || !w->output_norm || (h.n_layer > 0 && !w->layers)) { set_err("missing weight pointer"); return nullptr; }
  for (int l = 0; l < h.n_layer; ++l) {
    const tdf_layer_weights& L = w->layers[l];
    if (!L.attn_norm || !L.wq || !L.wk || !L.wv || !L.wo || !L.ffn_norm || !L.w_gate || !L.w_up || !L.w_down) {
      set_err("missing layer weight pointer");
      return nullptr;
    }
  }
  tdf_model* m = new tdf_model();
  m->hp = h;
  m->hp.swa_layers = nullptr;
  m->windowed.assign(h.n_layer, 0);
  for (int l = 0; l < h.n_layer; ++l) {
    m->windowed[l] = h.n_swa > 0 && (!h.swa_layers || h.swa_layers[l] != 0);
    m->any_window = m->any_window || m->windowed[l];
  }
  m->token_embd = w->token_embd;
  m->output_norm = (const float*)w->output_norm;
  m->output = w->output ? w->output : w->token_embd;
  m->layers.assign(w->layers, w->layers + h.n_layer);
  return m;
}

extern "C" void tdf_model_free(tdf_model* m) { delete m; }

// ---------------------------------------------------------------------------
// context

extern "C" tdf_context* tdf_context_create(const tdf_model* m, const tdf_context_params* p) {
  if (!m || !p) { set_err("model or params is NULL"); return nullptr; }
  if (p->n_ctx <= 0 || p->n_seq_max < 1 || p->n_seq_max > kMaxSeq || p->n_ubatch <= 0 || p->n_batch <= 0) {
    set_err("invalid context parameters");
    return nullptr;
  }
  if (p->kv_dtype != TDF_F32 && p->kv_dtype != TDF_F16 && p->kv_dtype != TDF_BF16 && p->kv_dtype != TDF_Q8_0) {
    set_err("invalid kv_dtype");
    return nullptr;
  }
  if (p->kv_dtype == TDF_Q8_0 && m->hp.head_dim % 32 != 0) {
    set_err("a Q8_0 cache needs head_dim to be a multiple of 32");
    return nullptr;
  }
  tdf_context* c = new tdf_context();
  c->m = m;
  c->n_ctx = p->n_ctx;
  c->n_batch = std::min(p->n_ctx, p->n_batch);
  c->n_ubatch = std::min(c->n_batch, p->n_ubatch);
  c->n_seq_max = p->n_seq_max;
  c->kv_dtype = p->kv_dtype;
  c->output_all = p->output_all != 0;
  c->dry_run = (p->flags & TDF_CTX_DRY_RUN) != 0;
  c->profile = !c->dry_run && (p->flags & TDF_CTX_PROFILE) != 0;
  {
    const char* e = getenv("TDF_NO_GRAPH");
    c->use_graphs = !c->profile && !(e && atoi(e) != 0);
  }
  c->book.init(c->n_ctx, c->n_seq_max);
  if (c->dry_run) return c;

  const tdf_hparams& h = m->hp;
  const int d = h.n_embd, H = h.n_head, Hkv = h.n_head_kv, hd = h.head_dim, F = h.n_ff;
  const int U = c->n_ubatch;
  int rc = TDF_OK;
  auto A = [&](void** ptr, size_t bytes) {
    if (rc == TDF_OK) rc = ctx_alloc(c, ptr, bytes);
  };
  if (p->stream) {
    c->stream = (hipStream_t)p->stream;
  } else {
    if (hipStreamCreateWithFlags(&c->stream, hipStreamNonBlocking) != hipSuccess) {
      set_err("stream creation failed");
      delete c;
      return nullptr;
    }
    c->own_stream = true;
  }
  {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&c->n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      set_err("device query failed");
      if (c->own_stream) (void)hipStreamDestroy(c->stream);
      delete c;
      return nullptr;
    }
  }
  c->kv_layer_bytes = c->kv_dtype == TDF_Q8_0 ? kv_q8_array_bytes(Hkv, c->n_ctx, hd)
                                              : (size_t)Hkv * c->n_ctx * hd * dtype_size(c->kv_dtype);
  A(&c->kv, c->kv_layer_bytes * 2 * std::max(1, h.n_layer));
  A((void**)&c->cell_list, (size_t)c->n_seq_max * c->n_ctx * sizeof(int32_t));
  // every entry a kernel reads is written first; zeros keep any entry in bounds regardless
  if (rc == TDF_OK && hipMemset(c->cell_list, 0, (size_t)c->n_seq_max * c->n_ctx * sizeof(int32_t)) != hipSuccess) {
    set_err("cell list initialisation failed");
    rc = TDF_E_DEVICE;
  }
  A((void**)&c->inv_freq, (size_t)(hd / 2) * sizeof(double));
  A((void**)&c->rope_cs, (size_t)U * (hd / 2) * sizeof(float2));
  A((void**)&c->x, (size_t)U * d * 4);
  A((void**)&c->xs, (size_t)U * d * 4);
  A((void**)&c->u, (size_t)U * d * 4);
  c->ssp_stride = std::max(1, gemv_residual_parts(d));
  A((void**)&c->ssp, (size_t)U * c->ssp_stride * 4);
  A((void**)&c->q, (size_t)U * H * hd * 4);
  A((void**)&c->o, (size_t)U * H * hd * 4);
  A((void**)&c->mb, (size_t)U * F * 4);
  A((void**)&c->h_hi, (size_t)U * d * 2);
  A((void**)&c->h_lo, (size_t)U * d * 2);
  A((void**)&c->o_hi, (size_t)U * H * hd * 2);
  A((void**)&c->o_lo, (size_t)U * H * hd * 2);
  A((void**)&c->m_hi, (size_t)U * F * 2);
  A((void**)&c->m_lo, (size_t)U * F * 2);
  c->part_rows = std::max((size_t)std::min(U, kDecodeMaxT) * H * kChunkCapDecode,
                          (size_t)U * H * kChunkCapPrefill);
  A((void**)&c->part_acc, c->part_rows * hd * 4);
  A((void**)&c->part_ml, c->part_rows * 2 * 4);
  if (U > kGemvMaxT) A((void**)&c->skinny_part, (size_t)kSkinnyPartFloats * 4);
  if (U > kDecodeMaxT && m->hp.weight_dtype == TDF_BF16) {
    c->qkv_split_floats = (int64_t)2 * U * (H + 2 * Hkv) * hd;
    A((void**)&c->qkv_split, (size_t)c->qkv_split_floats * 4);
  }
  if (c->kv_dtype == TDF_Q8_0) {
    A((void**)&c->kv_stage, (size_t)2 * Hkv * U * hd * 4);
    A((void**)&c->iota, (size_t)U * 4);
    if (rc == TDF_OK) {
      std::vector<int32_t> io(U);
      for (int i = 0; i < U; ++i) io[i] = i;
      if (hipMemcpy(c->iota, io.data(), (size_t)U * 4, hipMemcpyHostToDevice) != hipSuccess) {
        set_err("upload of the staging rows failed");
        rc = TDF_E_DEVICE;
      }
    }
  }
  // per-call integers: 5 int32 per token + selected rows, then int64 list writes
  c->ints_bytes = staging_i64_base(c->n_batch, c->n_ubatch, c->n_seq_max) +
                  (size_t)2 * c->n_batch * c->n_seq_max * 8;
  A(&c->ints, c->ints_bytes);
  if (rc == TDF_OK && hipHostMalloc((void**)&c->ints_host, c->ints_bytes, hipHostMallocDefault) != hipSuccess) {
    set_err("pinned staging allocation failed");
    rc = TDF_E_ALLOC;
  }
  if (rc == TDF_OK) rc = ensure_logits(c, 1);
  if (rc == TDF_OK) {
    std::vector<double> inv(hd / 2);
    for (int i = 0; i < hd / 2; ++i) inv[i] = std::pow((double)h.rope_theta, -2.0 * i / hd);
    if (hipMemcpy(c->inv_freq, inv.data(), inv.size() * sizeof(double), hipMemcpyHostToDevice) != hipSuccess) {
      set_err("upload of rope frequencies failed");
      rc = TDF_E_DEVICE;
    }
  }
  if (rc != TDF_OK) {
    ctx_release(c);
    delete c;
    return nullptr;
  }
  return c;
}

extern "C" void tdf_context_free(tdf_context* c) {
  if (!c) return;
  if (c->stream) (void)hipStreamSynchronize(c->stream);
  ctx_release(c);
  delete c;
}

// ---------------------------------------------------------------------------
// forward pass of one ubatch

struct UbatchDev {
  int T = 0, R = 0;
  const int32_t *tokens, *pos, *slots, *list_off, *n_vis, *sel;
  const int64_t* list_writes;
  int n_list_writes = 0;
  const int32_t *tile_tokens = nullptr, *tile_off = nullptr, *tile_nvis = nullptr;
  int n_tiles = 0;
  bool sel_identity = false;  // selected rows are exactly 0..T-1
  // the tokens' sequence sets are pairwise disjoint, so no token sees the
  // cell of another token of the ubatch
  bool own_rows = false;
  int attn_chunk = 64, attn_grid = 1;  // split-K decode attention: cells per split, splits launched
  int nvis_max = 0;
  // windowed layers: first visible list entry per token (n_lo), the shifted
  // list start and count (decode attention), per-tile first entry and the
  // per-token count from it (matrix-core attention and its merge)
  const int32_t *n_lo = nullptr, *list_off_w = nullptr, *n_vis_w = nullptr;
  const int32_t *n_vis_rel = nullptr, *tile_lo = nullptr;
  int attn_chunk_w = 64, attn_grid_w = 1, nvis_max_w = 0, span_max_w = 0;
  int out_row0 = 0;  // first logits row of this ubatch
};

static int run_linear(tdf_context* c, LinearArgs& a, bool mfma, int op) {
  const int slot = prof_begin(c, op, mfma);
  hipError_t e;
  if (!mfma)
    e = launch_linear_gemv(a, c->stream);
  else if (a.T <= kDecodeMaxT && c->skinny_part && skinny_supported(a))
    e = launch_linear_skinny(a, c->skinny_part, c->stream);
  else
    e = launch_linear_gemm(a, c->stream);
  prof_end(c, slot);
  if (e != hipSuccess) {
    set_err(std::string("linear launch failed: ") + hipGetErrorString(e));
    return TDF_E_DEVICE;
  }
  return TDF_OK;
}

static int forward_ubatch(tdf_context* c, const UbatchDev& u) {
  const tdf_model* m = c->m;
  const tdf_hparams& h = m->hp;
  const int d = h.n_embd, H = h.n_head, Hkv = h.n_head_kv, hd = h.head_dim, F = h.n_ff, V = h.n_vocab;
  const int L = h.n_layer;
  // bf16 and Q8_0 weights have matrix-core paths
  const bool wmfma = h.weight_dtype == TDF_BF16 || h.weight_dtype == TDF_Q8_0;
  hipStream_t s = c->stream;
  int T = u.T;
  auto use_mfma = [&](int rows, int K) { return wmfma && rows > kGemvMaxT && K % 64 == 0; };
  auto attn_gain = [&](int l) { return (const float*)(l < L ? m->layers[l].attn_norm : m->output_norm); };

  // RMSNorm hand-off to the decode GEMV: c->u holds g * x of the rows in
  // `cur`, c->ssp their partial sums of x^2 (u_parts per row), produced by the
  // kernel that last wrote `cur` (embedding, residual GEMV, row gather) or by
  // an explicit pass when that kernel could not (matrix-core producer).
  int u_parts = 0;  // 0: not ready
  // c->h_hi / h_lo already hold the next RMSNorm of `cur` (written by a
  // 9..32-token residual projection's last pass)
  bool h_ready = false;
  auto on_skinny = [&](const LinearArgs& a, bool mfma) {
    return mfma && a.T <= kDecodeMaxT && c->skinny_part && skinny_supported(a);
  };
  // a residual projection on the 9..32-token path also writes the next norm
  // for a matrix-core consumer of the same rows
  auto fuse_next_norm = [&](LinearArgs& a, bool mfma, const float* g) {
    if (!on_skinny(a, mfma)) return;
    LinearArgs t = a;
    t.norm_out_g = g;
    if (!skinny_norm_supported(t)) return;
    a.norm_out_g = g; a.norm_out_hi = c->h_hi; a.norm_out_lo = c->h_lo; a.norm_out_eps = h.rms_eps;
  };
  float* cur = c->x;  // residual rows being carried
  auto prep_norm = [&](const float* g, int rows) -> int {
    const int ps = prof_begin(c, TDF_OP_NORM, false);
    TDF_HIP(launch_gather_rows(cur, nullptr, rows, d, nullptr, g, c->u, c->ssp, c->ssp_stride, s));
    prof_end(c, ps);
    u_parts = 1;
    return TDF_OK;
  };

  const bool first_gemv = !use_mfma(T, d);
  int ps = prof_begin(c, TDF_OP_EMBED, !first_gemv);
  TDF_HIP(launch_embed(m->token_embd, h.weight_dtype, V, u.tokens, T, d, c->x, first_gemv ? attn_gain(0) : nullptr,
                       c->u, c->ssp, c->ssp_stride, s));
  TDF_HIP(launch_scatter(c->cell_list, u.list_writes, u.n_list_writes, s));
  TDF_HIP(launch_rope_table(u.pos, c->inv_freq, T, hd / 2, c->rope_cs, s));
  prof_end(c, ps);
  if (first_gemv) u_parts = 1;

  for (int l = 0; l < L; ++l) {
    const tdf_layer_weights& W = m->layers[l];
    // attention block
    const bool big = use_mfma(T, d);
    if (big && !h_ready) {
      ps = prof_begin(c, TDF_OP_NORM, big);
      TDF_HIP(launch_rmsnorm(cur, (const float*)W.attn_norm, T, d, h.rms_eps, nullptr, c->h_hi, c->h_lo, s));
      prof_end(c, ps);
    } else if (!big && !u_parts) {
      if (int rc = prep_norm((const float*)W.attn_norm, T)) return rc;
    }
    LinearArgs qa;
    qa.w0 = W.wq; qa.w1 = W.wk; qa.w2 = W.wv;
    qa.n0 = H * hd; qa.n1 = Hkv * hd; qa.n2 = Hkv * hd;
    qa.K = d; qa.T = T; qa.weight_dtype = h.weight_dtype;
    qa.act_f32 = c->u; qa.act_hi = c->h_hi; qa.act_lo = c->h_lo;
    qa.norm_ssp = c->ssp; qa.norm_nparts = u_parts; qa.norm_stride = c->ssp_stride; qa.norm_eps = h.rms_eps;
    qa.epi = EPI_QKV;
    qa.q_out = c->q;
    qa.k_cache = kv_k(c, l); qa.v_cache = kv_v(c, l);
    qa.kv_dtype = c->kv_dtype; qa.n_ctx = c->n_ctx; qa.head_dim = hd;
    qa.slots = u.slots; qa.pos = u.pos; qa.rope_cs = c->rope_cs;
    qa.split_ws = c->qkv_split; qa.split_ws_floats = c->qkv_split_floats;
    // Q8_0 cache: the projection writes float32 K/V rows to the staging area
    // (row t of head h at [h][t]), and they are quantized into their cells
    //  - with matrix-core decode attention, when no token sees another
    //    token's cell (one token, or one token per sequence), by the
    //    attention block whose chunk holds the cell (a single token's GEMV
    //    keeps its 8-row blocks: 32-row quantizing blocks are 192 for 256 CUs
    //    at 8B widths, 14.6 against 12.6 us; 32 lock-step sequences drop the
    //    separate pass);
    //  - for a single token otherwise, by the GEMV itself when its 32-row
    //    blocks fit on the compute units at once (no staging);
    //  - else by a separate pass.
    const bool win = m->windowed[l] != 0;
    const int dchunk = win ? u.attn_chunk_w : u.attn_chunk;
    const bool q8_attn = c->kv_dtype == TDF_Q8_0 && T <= kDecodeMaxT && u.own_rows &&
                         attn_decode_on_mfma(TDF_Q8_0, hd) && dchunk <= kDecodeCellStage;
    const bool q8_fold = !q8_attn && T == 1 && !big && (H + 2 * Hkv) * hd / 32 <= c->n_cu;
    const bool kvq8 = c->kv_dtype == TDF_Q8_0 && !q8_fold;
    if (kvq8) {
      qa.k_cache = c->kv_stage; qa.v_cache = c->kv_stage + (size_t)Hkv * c->n_ubatch * hd;
      qa.kv_dtype = TDF_F32; qa.n_ctx = c->n_ubatch; qa.slots = c->iota;
    }
    if (int rc = run_linear(c, qa, big, TDF_OP_QKV)) return rc;
    if (kvq8 && !q8_attn) {
      ps = prof_begin(c, TDF_OP_QKV, big);
      TDF_HIP(launch_kv_quantize(c->kv_stage, c->kv_stage + (size_t)Hkv * c->n_ubatch * hd, hd,
                                 (int64_t)c->n_ubatch * hd, T, Hkv, hd, u.slots, kv_k(c, l), kv_v(c, l), c->n_ctx, s));
      prof_end(c, ps);
    }
    u_parts = 0;

    if (T > kDecodeMaxT && prefill_attention_supported(c->kv_dtype, hd)) {
      PrefillAttnArgs pa;
      pa.q = c->q;
      pa.k_cache = kv_k(c, l); pa.v_cache = kv_v(c, l);
      pa.kv_dtype = c->kv_dtype;
      pa.cell_list = c->cell_list; pa.n_vis = u.n_vis;
      pa.tile_tokens = u.tile_tokens; pa.tile_list_off = u.tile_off; pa.tile_nvis_max = u.tile_nvis;
      pa.n_tiles = u.n_tiles; pa.H = H; pa.Hkv = Hkv; pa.hd = hd; pa.n_ctx = c->n_ctx;
      if (win) { pa.n_lo = u.n_lo; pa.tile_lo = u.tile_lo; }
      // split the cell range only when the tiles alone leave CUs idle; at
      // least 256 cells per split, at most kChunkCapPrefill splits
      const int span = win ? u.span_max_w : u.nvis_max;
      const int blocks = u.n_tiles * Hkv;
      int want = std::max(1, (512 + blocks - 1) / blocks);
      int chunk = std::max(256, (span + want - 1) / want);
      chunk = std::max(chunk, (span + kChunkCapPrefill - 1) / kChunkCapPrefill);
      chunk = (chunk + 63) / 64 * 64;
      pa.chunk = chunk;
      pa.n_splits = (span + chunk - 1) / chunk;
      pa.part_acc = c->part_acc; pa.part_ml = c->part_ml;
      pa.out = c->o; pa.out_hi = c->o_hi; pa.out_lo = c->o_lo;
      pa.merge.T = T; pa.merge.H = H; pa.merge.Hkv = Hkv; pa.merge.hd = hd;
      pa.merge.n_vis = win ? u.n_vis_rel : u.n_vis; pa.merge.chunk = chunk; pa.merge.n_chunks = pa.n_splits;
      pa.merge.merge_single = 1;
      pa.merge.part_acc = c->part_acc; pa.merge.part_ml = c->part_ml;
      pa.merge.out = c->o; pa.merge.out_hi = c->o_hi; pa.merge.out_lo = c->o_lo;
      ps = prof_begin(c, TDF_OP_ATTN, big);
      TDF_HIP(launch_attention_prefill(pa, s));
      prof_end(c, ps);
    } else {
      AttnArgs at;
      at.q = c->q;
      at.k_cache = kv_k(c, l); at.v_cache = kv_v(c, l);
      at.kv_dtype = c->kv_dtype;
      at.cell_list = c->cell_list;
      at.list_off = win ? u.list_off_w : u.list_off;
      at.n_vis = win ? u.n_vis_w : u.n_vis;
      at.T = T; at.H = H; at.Hkv = Hkv; at.hd = hd; at.n_ctx = c->n_ctx;
      at.chunk = dchunk;
      at.n_chunks = win ? u.attn_grid_w : u.attn_grid;
      if (q8_attn) {
        at.new_k = c->kv_stage; at.new_v = c->kv_stage + (size_t)Hkv * c->n_ubatch * hd;
        at.new_hs = (int64_t)c->n_ubatch * hd; at.new_slot = u.slots;
      }
      at.part_acc = c->part_acc; at.part_ml = c->part_ml;
      at.out = c->o;
      at.out_hi = big ? c->o_hi : nullptr;
      at.out_lo = big ? c->o_lo : nullptr;
      ps = prof_begin(c, TDF_OP_ATTN, big);
      TDF_HIP(launch_attention_decode(at, s));
      prof_end(c, ps);
    }

    const bool last = l == L - 1;
    // the last layer keeps only the rows whose logits are wanted before its MLP
    const bool narrow = last && !(u.R == T && u.sel_identity);
    const int T_mlp = last ? u.R : T;
    const bool bigm = use_mfma(T_mlp, d) && use_mfma(T_mlp, F);
    LinearArgs oa;
    oa.w0 = W.wo; oa.n0 = d; oa.K = H * hd; oa.T = T; oa.weight_dtype = h.weight_dtype;
    oa.act_f32 = c->o; oa.act_hi = c->o_hi; oa.act_lo = c->o_lo;
    oa.epi = EPI_RESIDUAL; oa.out = cur; oa.ldo = d;
    const bool wo_mfma = big && use_mfma(T, H * hd);
    if (!wo_mfma && !bigm && !narrow) {
      oa.next_g = (const float*)W.ffn_norm; oa.next_u = c->u; oa.next_ssp = c->ssp; oa.next_stride = c->ssp_stride;
    }
    if (bigm && !narrow) fuse_next_norm(oa, wo_mfma, (const float*)W.ffn_norm);
    if (int rc = run_linear(c, oa, wo_mfma, TDF_OP_WO)) return rc;
    u_parts = oa.next_g ? gemv_residual_parts(d) : 0;
    h_ready = oa.norm_out_g != nullptr;

    if (last) {
      if (u.R == 0) return TDF_OK;
      if (narrow) {
        ps = prof_begin(c, TDF_OP_NORM, big);
        TDF_HIP(launch_gather_rows(cur, u.sel, u.R, d, c->xs, bigm ? nullptr : (const float*)W.ffn_norm,
                                   c->u, c->ssp, c->ssp_stride, s));
        prof_end(c, ps);
        cur = c->xs;
        u_parts = bigm ? 0 : 1;
      }
      T = u.R;
    }
    // MLP block
    if (bigm && !h_ready) {
      ps = prof_begin(c, TDF_OP_NORM, bigm);
      TDF_HIP(launch_rmsnorm(cur, (const float*)W.ffn_norm, T, d, h.rms_eps, nullptr, c->h_hi, c->h_lo, s));
      prof_end(c, ps);
    } else if (!bigm && !u_parts) {
      if (int rc = prep_norm((const float*)W.ffn_norm, T)) return rc;
    }
    LinearArgs ga;
    ga.w0 = W.w_gate; ga.w1 = W.w_up; ga.n0 = F; ga.K = d; ga.T = T; ga.weight_dtype = h.weight_dtype;
    ga.act_f32 = c->u; ga.act_hi = c->h_hi; ga.act_lo = c->h_lo;
    ga.norm_ssp = c->ssp; ga.norm_nparts = u_parts; ga.norm_stride = c->ssp_stride; ga.norm_eps = h.rms_eps;
    ga.epi = EPI_SWIGLU; ga.out = c->mb; ga.out_hi = c->m_hi; ga.out_lo = c->m_lo; ga.ldo = F;
    if (int rc = run_linear(c, ga, bigm, TDF_OP_GATE_UP)) return rc;
    u_parts = 0;
    LinearArgs da;
    da.w0 = W.w_down; da.n0 = d; da.K = F; da.T = T; da.weight_dtype = h.weight_dtype;
    da.act_f32 = c->mb; da.act_hi = c->m_hi; da.act_lo = c->m_lo;
    da.epi = EPI_RESIDUAL; da.out = cur; da.ldo = d;
    const bool next_gemv = last ? !use_mfma(T, d) : !use_mfma(T, d);
    if (!bigm && next_gemv) {
      da.next_g = attn_gain(l + 1); da.next_u = c->u; da.next_ssp = c->ssp; da.next_stride = c->ssp_stride;
    }
    // the next consumer (next layer's QKV, or the LM head) reads the same rows
    if (!next_gemv) fuse_next_norm(da, bigm, attn_gain(l + 1));
    if (int rc = run_linear(c, da, bigm, TDF_OP_DOWN)) return rc;
    u_parts = da.next_g ? gemv_residual_parts(d) : 0;
    h_ready = da.norm_out_g != nullptr;
  }
  if (L == 0) {
    if (u.R == 0) return TDF_OK;
    if (!(u.R == T && u.sel_identity)) {
      TDF_HIP(launch_gather_rows(cur, u.sel, u.R, d, c->xs, nullptr, nullptr, nullptr, 0, s));
      cur = c->xs;
      u_parts = 0;
    }
    T = u.R;
  }
  // output norm + LM head into this ubatch's logits rows
  const bool bigo = use_mfma(T, d);
  if (bigo && !h_ready) {
    ps = prof_begin(c, TDF_OP_NORM, bigo);
    TDF_HIP(launch_rmsnorm(cur, m->output_norm, T, d, h.rms_eps, nullptr, c->h_hi, c->h_lo, s));
    prof_end(c, ps);
  } else if (!bigo && !u_parts) {
    if (int rc = prep_norm(m->output_norm, T)) return rc;
  }
  LinearArgs la;
  la.w0 = m->output; la.n0 = V; la.K = d; la.T = T; la.weight_dtype = h.weight_dtype;
  la.act_f32 = c->u; la.act_hi = c->h_hi; la.act_lo = c->h_lo;
  la.norm_ssp = c->ssp; la.norm_nparts = u_parts; la.norm_stride = c->ssp_stride; la.norm_eps = h.rms_eps;
  la.epi = EPI_STORE; la.out = c->logits + (size_t)u.out_row0 * V; la.ldo = V;
  return run_linear(c, la, bigo, TDF_OP_LM_HEAD);
}

// Replay of the decode launch sequence (the graph reuse of llama.cpp
// walkthrough "Step 13": same-shape ubatches skip rebuilding).  Every
// per-call value the kernels read lives in device memory at fixed addresses
// (the ubatch's integers, cell lists, caches); the key holds everything that
// enters a kernel argument.
static int run_graphed(tdf_context* c, const UbatchDev& u) {
  // the list writes sit after those of the call's earlier ubatches, whose
  // count depends on how many sequences their tokens carry: the address is
  // part of the key as the integers' address is
  const auto key = std::make_tuple(u.T, u.R, u.n_list_writes, u.attn_chunk, u.attn_grid,
                                   (const void*)c->logits, (const void*)u.tokens, (const void*)u.list_writes,
                                   u.out_row0, (int)u.sel_identity, u.attn_chunk_w, u.attn_grid_w, (int)u.own_rows);
  auto it = c->graphs.find(key);
  if (it == c->graphs.end()) {
    if (c->graphs.size() >= 64) {
      for (auto& kv : c->graphs) (void)hipGraphExecDestroy(kv.second);
      c->graphs.clear();
    }
    TDF_HIP(hipStreamBeginCapture(c->stream, hipStreamCaptureModeThreadLocal));
    const int rc = forward_ubatch(c, u);
    hipGraph_t graph = nullptr;
    const hipError_t e = hipStreamEndCapture(c->stream, &graph);
    if (rc != TDF_OK) {
      if (graph) (void)hipGraphDestroy(graph);
      return rc;
    }
    if (e != hipSuccess) {
      set_err(std::string("graph capture failed: ") + hipGetErrorString(e));
      return TDF_E_DEVICE;
    }
    hipGraphExec_t exec = nullptr;
    const hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (ei != hipSuccess) {
      set_err(std::string("graph instantiation failed: ") + hipGetErrorString(ei));
      return TDF_E_DEVICE;
    }
    it = c->graphs.emplace(key, exec).first;
    ++c->n_graph_captures;
  } else {
    ++c->n_graph_replays;
  }
  TDF_HIP(hipGraphLaunch(it->second, c->stream));
  return TDF_OK;
}

// ---------------------------------------------------------------------------
// decode

extern "C" int32_t tdf_decode(tdf_context* c, const tdf_batch* b) {
  if (!c) { set_err("context is NULL"); return TDF_E_INVALID; }
  g_err.clear();
  Intake in;
  std::string err;
  int rc = intake_batch(c->book, b, c->m->hp.n_vocab, c->n_batch, c->output_all, in, err);
  if (rc != TDF_OK) { set_err(err); return rc; }
  const int n = in.n_tokens;
  if (c->book.n_free() < n) {
    set_err("not enough free KV cells");
    return TDF_NO_SLOT;
  }
  int n_out = 0;
  for (int i = 0; i < n; ++i) n_out += in.output[i] ? 1 : 0;
  if (!c->dry_run) {
    rc = ensure_logits(c, std::max(1, n_out));
    if (rc != TDF_OK) return rc;
  }
  c->n_outputs = n_out;
  c->out_ids.clear();
  c->row_of.assign(n, -1);
  c->last_slots.assign(n, -1);
  c->logits_host.clear();
  c->host_row_ok.assign(n_out, 0);
  for (int i = 0; i < n; ++i)
    if (in.output[i]) {
      c->row_of[i] = (int32_t)c->out_ids.size();
      c->out_ids.push_back(i);
    }

  // integers of every ubatch of this call go into one pinned staging area;
  // region of a ubatch: tokens, pos, slots, list_off, n_vis, sel | list writes
  size_t i32_off = 0, i64_off = 0;
  const size_t i64_base = staging_i64_base(c->n_batch, c->n_ubatch, c->n_seq_max);
  std::vector<int32_t> slots;
  std::vector<int64_t> writes;
  int out_row = 0;
  for (int u0 = 0; u0 < n; u0 += c->n_ubatch) {
    const int T = std::min(c->n_ubatch, n - u0);
    if (!c->book.find_slots(T, slots)) {
      set_err("internal: cells vanished during decode");
      return TDF_E_DEVICE;
    }
    writes.clear();
    std::vector<int32_t> list_off(T), n_vis(T), sel, n_lo;
    int nvis_max = 0;
    const bool win = c->m->any_window;
    if (win) n_lo.resize(T);
    for (int i = 0; i < T; ++i) {
      const int t = u0 + i;
      const int32_t idx = c->book.place(slots[i], in.pos[t], in.seq_mask[t], in.seq0[t], &writes);
      list_off[i] = in.seq0[t] * c->n_ctx;
      n_vis[i] = idx + 1;
      nvis_max = std::max(nvis_max, n_vis[i]);
      // first list entry inside the window: position > pos - n_swa
      if (win) n_lo[i] = c->book.first_at_or_after(in.seq0[t], n_vis[i], in.pos[t] - c->m->hp.n_swa + 1);
      c->last_slots[t] = slots[i];
      if (in.output[t]) sel.push_back(i);
    }
    if (c->dry_run) continue;

    int32_t* h32 = (int32_t*)(c->ints_host + i32_off * 4);
    int32_t* d32 = (int32_t*)((char*)c->ints + i32_off * 4);
    memcpy(h32, &in.token[u0], T * 4);
    memcpy(h32 + T, &in.pos[u0], T * 4);
    memcpy(h32 + 2 * T, slots.data(), T * 4);
    memcpy(h32 + 3 * T, list_off.data(), T * 4);
    memcpy(h32 + 4 * T, n_vis.data(), T * 4);
    if (!sel.empty()) memcpy(h32 + 5 * T, sel.data(), sel.size() * 4);
    // query tiles for the matrix-core attention: tokens of one sequence in
    // batch order, 32 at a time
    std::vector<int32_t> tile_tok, tile_off, tile_nvis, tile_lo;
    if (T > kDecodeMaxT) {
      std::vector<int> order(T);
      for (int i = 0; i < T; ++i) order[i] = i;
      std::stable_sort(order.begin(), order.end(),
                       [&](int x, int y) { return in.seq0[u0 + x] < in.seq0[u0 + y]; });
      for (int k = 0; k < T;) {
        const int s0 = in.seq0[u0 + order[k]];
        int nmax = 0, cnt = 0;
        const size_t base = tile_tok.size();
        tile_tok.resize(base + kQTile, -1);
        int lmin = INT32_MAX;
        while (k < T && cnt < kQTile && in.seq0[u0 + order[k]] == s0) {
          tile_tok[base + cnt++] = order[k];
          nmax = std::max(nmax, n_vis[order[k]]);
          if (win) lmin = std::min(lmin, n_lo[order[k]]);
          ++k;
        }
        tile_off.push_back(s0 * c->n_ctx);
        tile_nvis.push_back(nmax);
        if (win) tile_lo.push_back(lmin);
      }
    }
    const int n_tiles = (int)tile_off.size();
    if (n_tiles) {
      int32_t* tp = h32 + 5 * T + sel.size();
      memcpy(tp, tile_tok.data(), tile_tok.size() * 4);
      memcpy(tp + tile_tok.size(), tile_off.data(), n_tiles * 4);
      memcpy(tp + tile_tok.size() + n_tiles, tile_nvis.data(), n_tiles * 4);
    }
    size_t n32 = 5 * (size_t)T + sel.size() + (size_t)(kQTile + 2) * n_tiles;
    // windowed attention: n_lo, list_off_w, n_vis_w, n_vis_rel per token, tile_lo per tile
    int nvis_max_w = 0, span_max_w = 0;
    const size_t w_base = n32;
    if (win) {
      std::vector<int32_t> rel(T, 0), tile_of(T, -1);
      for (int k = 0; k < n_tiles; ++k)
        for (int q = 0; q < kQTile; ++q) {
          const int tt = tile_tok[(size_t)k * kQTile + q];
          if (tt >= 0) tile_of[tt] = k;
        }
      int32_t* wp = h32 + w_base;
      for (int i = 0; i < T; ++i) {
        wp[i] = n_lo[i];
        wp[T + i] = list_off[i] + n_lo[i];
        wp[2 * T + i] = n_vis[i] - n_lo[i];
        nvis_max_w = std::max(nvis_max_w, n_vis[i] - n_lo[i]);
        rel[i] = tile_of[i] >= 0 ? n_vis[i] - tile_lo[tile_of[i]] : n_vis[i] - n_lo[i];
        wp[3 * T + i] = rel[i];
      }
      for (int k = 0; k < n_tiles; ++k) {
        wp[4 * T + k] = tile_lo[k];
        span_max_w = std::max(span_max_w, tile_nvis[k] - tile_lo[k]);
      }
      n32 += 4 * (size_t)T + n_tiles;
    }
    int64_t* h64 = (int64_t*)(c->ints_host + i64_base + i64_off * 8);
    int64_t* d64 = (int64_t*)((char*)c->ints + i64_base + i64_off * 8);
    if (!writes.empty()) memcpy(h64, writes.data(), writes.size() * 8);
    TDF_HIP(hipMemcpyAsync(d32, h32, n32 * 4, hipMemcpyHostToDevice, c->stream));
    if (!writes.empty())
      TDF_HIP(hipMemcpyAsync(d64, h64, writes.size() * 8, hipMemcpyHostToDevice, c->stream));

    UbatchDev ud;
    ud.T = T;
    ud.R = (int)sel.size();
    ud.sel_identity = ud.R == T;
    {
      uint64_t seen = 0;
      ud.own_rows = true;
      for (int i = 0; i < T; ++i) {
        if (in.seq_mask[u0 + i] & seen) ud.own_rows = false;
        seen |= in.seq_mask[u0 + i];
      }
    }
    ud.tokens = d32; ud.pos = d32 + T; ud.slots = d32 + 2 * T;
    ud.list_off = d32 + 3 * T; ud.n_vis = d32 + 4 * T; ud.sel = d32 + 5 * T;
    ud.list_writes = d64;
    ud.n_list_writes = (int)writes.size() / 2;
    ud.nvis_max = nvis_max;
    ud.n_tiles = n_tiles;
    ud.tile_tokens = d32 + 5 * T + sel.size();
    ud.tile_off = ud.tile_tokens + (size_t)kQTile * n_tiles;
    ud.tile_nvis = ud.tile_off + n_tiles;
    ud.out_row0 = out_row;
    if (win) {
      ud.n_lo = d32 + w_base;
      ud.list_off_w = ud.n_lo + T;
      ud.n_vis_w = ud.n_lo + 2 * T;
      ud.n_vis_rel = ud.n_lo + 3 * T;
      ud.tile_lo = ud.n_lo + 4 * T;
      ud.nvis_max_w = nvis_max_w;
      ud.span_max_w = span_max_w;
    }
    auto split_cells = [&](int nmax, int& chunk_out, int& grid_out) {
      if (T <= kDecodeMaxT) {
        // cells per split grow past 256 splits; the launched grid is the
        // split count rounded up to a power of two (surplus blocks exit), so
        // a captured launch sequence stays valid while the context grows
        int chunk = (nmax + kChunkCapDecode - 1) / kChunkCapDecode;
        chunk = std::max(64, (chunk + 63) / 64 * 64);
        const int64_t heads = (int64_t)T * c->m->hp.n_head_kv;
        if (attn_decode_on_mfma(c->kv_dtype, c->m->hp.head_dim)) {
          // matrix-core kernel: about 256 blocks in all, 128..2048 cells each
          // (measured best from one sequence at 2k to 32 sequences at 8k)
          const int64_t want = (nmax * heads + 255) / 256;
          int ch = 128;
          while (ch < kDecodeCellStage && ch < want) ch *= 2;
          chunk = std::max(chunk, std::min(ch, std::max(64, (nmax + 63) / 64 * 64)));
        } else {
          // several tiles per block once there are blocks to spare (long
          // contexts, many tokens): fewer partials, per-block costs amortised
          while (chunk < 512 && heads * ((nmax + 2 * chunk - 1) / (2 * chunk)) >= 4096) chunk *= 2;
        }
        const int need = (nmax + chunk - 1) / chunk;
        int grid = 1;
        while (grid < need) grid *= 2;
        chunk_out = chunk;
        grid_out = std::min(grid, kChunkCapDecode);
      } else {
        int chunk = (nmax + kChunkCapPrefill - 1) / kChunkCapPrefill;
        chunk = std::max(64, (chunk + 63) / 64 * 64);
        chunk_out = chunk;
        grid_out = (nmax + chunk - 1) / chunk;
      }
    };
    split_cells(nvis_max, ud.attn_chunk, ud.attn_grid);
    if (win) split_cells(nvis_max_w, ud.attn_chunk_w, ud.attn_grid_w);
    if (c->use_graphs && T <= kDecodeMaxT) {
      rc = run_graphed(c, ud);
    } else {
      rc = forward_ubatch(c, ud);
    }
    if (rc != TDF_OK) return rc;
    out_row += ud.R;
    i32_off += (n32 + 3) & ~(size_t)3;
    i64_off += writes.size();
  }
  if (c->dry_run) return TDF_OK;
  if (n_out > 0) {
    const int ps = prof_begin(c, TDF_OP_ARGMAX, false);
    TDF_HIP(launch_argmax(c->logits, n_out, c->m->hp.n_vocab, c->d_tok, c->amax_v, c->amax_i, c->stream));
    prof_end(c, ps);
    TDF_HIP(hipMemcpyAsync(c->h_tok, c->d_tok, (size_t)n_out * 4, hipMemcpyDeviceToHost, c->stream));
  }
  TDF_HIP(hipStreamSynchronize(c->stream));
  prof_collect(c);
  return TDF_OK;
}

extern "C" int32_t tdf_n_outputs(const tdf_context* c) { return c ? c->n_outputs : TDF_E_INVALID; }

extern "C" int32_t tdf_output_ids(const tdf_context* c, int32_t* out) {
  if (!c) return TDF_E_INVALID;
  if (out) std::copy(c->out_ids.begin(), c->out_ids.end(), out);
  return c->n_outputs;
}

extern "C" const float* tdf_get_logits_ith(tdf_context* c, int32_t i) {
  if (!c || c->dry_run || i < 0 || i >= (int32_t)c->row_of.size() || c->row_of[i] < 0) {
    set_err("no logits for this batch index");
    return nullptr;
  }
  const int V = c->m->hp.n_vocab;
  const int r = c->row_of[i];
  if (c->logits_host.size() < (size_t)c->n_outputs * V) c->logits_host.resize((size_t)c->n_outputs * V);
  if (!c->host_row_ok[r]) {
    if (hipMemcpy(&c->logits_host[(size_t)r * V], c->logits + (size_t)r * V, (size_t)V * 4,
                  hipMemcpyDeviceToHost) != hipSuccess) {
      set_err("logits copy failed");
      return nullptr;
    }
    c->host_row_ok[r] = 1;
  }
  return &c->logits_host[(size_t)r * V];
}

extern "C" const float* tdf_get_logits_device(tdf_context* c) {
  if (!c || c->dry_run) return nullptr;
  return c->logits;
}

extern "C" int32_t tdf_argmax_ith(const tdf_context* c, int32_t i) {
  if (!c || c->dry_run || i < 0 || i >= (int32_t)c->row_of.size() || c->row_of[i] < 0) return TDF_E_INVALID;
  return c->h_tok[c->row_of[i]];
}

extern "C" int32_t tdf_seq_pos_max(const tdf_context* c, int32_t s) {
  if (!c || s < 0 || s >= c->n_seq_max) return TDF_E_INVALID;
  return c->book.seq_pos_max(s);
}

extern "C" int32_t tdf_kv_clear(tdf_context* c) {
  if (!c) return TDF_E_INVALID;
  if (c->stream) (void)hipStreamSynchronize(c->stream);
  c->book.clear();
  c->n_outputs = 0;
  c->out_ids.clear();
  c->row_of.clear();
  c->logits_host.clear();
  c->host_row_ok.clear();
  return TDF_OK;
}

extern "C" int32_t tdf_kv_cell(const tdf_context* c, int32_t cell, int32_t* pos, uint64_t* seq_mask) {
  if (!c || cell < 0 || cell >= c->n_ctx) return TDF_E_INVALID;
  if (pos) *pos = c->book.cell_pos(cell);
  if (seq_mask) *seq_mask = c->book.cell_seq(cell);
  return TDF_OK;
}

extern "C" int32_t tdf_last_slots(const tdf_context* c, int32_t* slots) {
  if (!c) return TDF_E_INVALID;
  if (slots) std::copy(c->last_slots.begin(), c->last_slots.end(), slots);
  return (int32_t)c->last_slots.size();
}

// ---------------------------------------------------------------------------
// cache import

template <typename E>
__global__ void kv_import_kernel(E* __restrict__ dst, const E* __restrict__ src,
                                 const int32_t* __restrict__ cells, int n, int Hkv, int hd, int n_ctx) {
  const int64_t total = (int64_t)n * Hkv * hd;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int d = (int)(i % hd);
    const int g = (int)((i / hd) % Hkv);
    const int p = (int)(i / ((int64_t)hd * Hkv));
    dst[((int64_t)g * n_ctx + cells[p]) * hd + d] = src[i];
  }
}

extern "C" int32_t tdf_kv_import(tdf_context* c, int32_t s, int32_t pos0, int32_t n,
                                 const void* const* k_layers, const void* const* v_layers) {
  if (!c || s < 0 || s >= c->n_seq_max || n <= 0 || pos0 < 0 || pos0 <= c->book.seq_pos_max(s)) {
    set_err("invalid kv_import arguments");
    return TDF_E_INVALID;
  }
  const int L = c->m->hp.n_layer;
  if (!c->dry_run && L > 0 && (!k_layers || !v_layers)) { set_err("missing layer arrays"); return TDF_E_INVALID; }
  if (!c->dry_run)
    for (int l = 0; l < L; ++l)
      if (!k_layers[l] || !v_layers[l]) { set_err("missing layer array"); return TDF_E_INVALID; }
  std::vector<int32_t> slots;
  if (!c->book.find_slots(n, slots)) { set_err("not enough free KV cells"); return TDF_NO_SLOT; }
  // the placement is worked out on a copy and committed only once the
  // device holds the rows and the cell lists
  KvBook next = c->book;
  std::vector<int64_t> writes;
  for (int i = 0; i < n; ++i) next.place(slots[i], pos0 + i, 1ull << s, s, &writes);
  if (c->dry_run) {
    c->book = std::move(next);
    c->last_slots = slots;
    return TDF_OK;
  }
  const int Hkv = c->m->hp.n_head_kv, hd = c->m->hp.head_dim;
  CallScratch scratch(c->stream);
  void *dcells = nullptr, *dwrites = nullptr;
  TDF_HIP(scratch.alloc(&dcells, (size_t)n * 4));
  TDF_HIP(scratch.alloc(&dwrites, writes.size() * 8));
  TDF_HIP(hipMemcpyAsync(dcells, slots.data(), (size_t)n * 4, hipMemcpyHostToDevice, c->stream));
  TDF_HIP(hipMemcpyAsync(dwrites, writes.data(), writes.size() * 8, hipMemcpyHostToDevice, c->stream));
  TDF_HIP(launch_scatter(c->cell_list, (const int64_t*)dwrites, (int)writes.size() / 2, c->stream));
  const int64_t total = (int64_t)n * Hkv * hd;
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 65536);
  for (int l = 0; l < L; ++l) {
    if (c->kv_dtype == TDF_Q8_0) {
      // float32 rows [n][Hkv][hd], quantized into their cells
      TDF_HIP(launch_kv_quantize((const float*)k_layers[l], (const float*)v_layers[l], (int64_t)Hkv * hd, hd, n, Hkv,
                                 hd, (const int32_t*)dcells, kv_k(c, l), kv_v(c, l), c->n_ctx, c->stream));
    } else if (c->kv_dtype == TDF_F32) {
      kv_import_kernel<float><<<blocks, 256, 0, c->stream>>>((float*)kv_k(c, l), (const float*)k_layers[l],
                                                            (const int32_t*)dcells, n, Hkv, hd, c->n_ctx);
      kv_import_kernel<float><<<blocks, 256, 0, c->stream>>>((float*)kv_v(c, l), (const float*)v_layers[l],
                                                            (const int32_t*)dcells, n, Hkv, hd, c->n_ctx);
    } else {
      kv_import_kernel<uint16_t><<<blocks, 256, 0, c->stream>>>((uint16_t*)kv_k(c, l), (const uint16_t*)k_layers[l],
                                                               (const int32_t*)dcells, n, Hkv, hd, c->n_ctx);
      kv_import_kernel<uint16_t><<<blocks, 256, 0, c->stream>>>((uint16_t*)kv_v(c, l), (const uint16_t*)v_layers[l],
                                                               (const int32_t*)dcells, n, Hkv, hd, c->n_ctx);
    }
    TDF_HIP(hipGetLastError());
  }
  TDF_HIP(hipStreamSynchronize(c->stream));
  c->book = std::move(next);
  c->last_slots = slots;
  return TDF_OK;
}

static int check_sampling(const tdf_sampling* p, const float* u, int R, const char* who) {
  if (!(p->temperature > 0.f)) return TDF_OK;  // greedy: the other fields are ignored
  if (!u || p->top_k < 1 || p->top_k > kMaxTopK || !(p->min_p >= 0.f && p->min_p <= 1.f) ||
      !(p->top_p == p->top_p) || !std::isfinite(p->temperature)) {
    set_err(std::string(who) + ": invalid sampling parameters");
    return TDF_E_INVALID;
  }
  for (int i = 0; i < R; ++i)
    if (!(u[i] >= 0.f && u[i] < 1.f)) {
      set_err(std::string(who) + ": u must lie in [0, 1)");
      return TDF_E_INVALID;
    }
  return TDF_OK;
}

// greedy (argmax) or the sampling chain over R rows of V logits at the
// device pointer lg; d_u, d_tok, pv, pi, h_tok are the context's buffers for
// that many rows
static int sample_rows(tdf_context* c, const float* lg, int R, int V, const tdf_sampling* p, const float* u,
                       int32_t* tokens, float* d_u, int32_t* d_tok, float* pv, int32_t* pi, int32_t* h_tok) {
  if (!(p->temperature > 0.f)) {
    TDF_HIP(launch_argmax(lg, R, V, d_tok, pv, pi, c->stream));
  } else {
    TDF_HIP(hipMemcpyAsync(d_u, u, (size_t)R * 4, hipMemcpyHostToDevice, c->stream));
    SampleParams sp;
    sp.temperature = p->temperature;
    sp.top_k = p->top_k;
    sp.top_p = p->top_p;
    sp.min_p = p->min_p;
    TDF_HIP(launch_sample(lg, R, V, sp, d_u, d_tok, c->stream));
  }
  TDF_HIP(hipMemcpyAsync(h_tok, d_tok, (size_t)R * 4, hipMemcpyDeviceToHost, c->stream));
  TDF_HIP(hipStreamSynchronize(c->stream));
  memcpy(tokens, h_tok, (size_t)R * 4);
  return TDF_OK;
}

extern "C" int32_t tdf_sample(tdf_context* c, const tdf_sampling* p, const float* u, int32_t* tokens) {
  if (!c || !p || !tokens || c->dry_run) {
    set_err("tdf_sample: invalid arguments");
    return TDF_E_INVALID;
  }
  const int R = c->n_outputs, V = c->m->hp.n_vocab;
  if (R == 0) return TDF_OK;
  if (int rc = check_sampling(p, u, R, "tdf_sample")) return rc;
  // u goes through the argmax partials buffer (>= R floats)
  return sample_rows(c, c->logits, R, V, p, u, tokens, c->amax_v, c->d_tok, c->amax_v, c->amax_i, c->h_tok);
}

extern "C" int32_t tdf_sample_logits(tdf_context* c, const float* logits, int32_t n_rows, int32_t n_vocab,
                                     const tdf_sampling* p, const float* u, int32_t* tokens) {
  if (!c || !p || !tokens || c->dry_run || !logits || n_rows < 0 || n_vocab < 1) {
    set_err("tdf_sample_logits: invalid arguments");
    return TDF_E_INVALID;
  }
  if (n_rows == 0) return TDF_OK;
  if (int rc = check_sampling(p, u, n_rows, "tdf_sample_logits")) return rc;
  const size_t parts = (size_t)n_rows * argmax_splits(n_vocab);
  if ((size_t)n_rows > c->ext_rows) {
    void *du = nullptr, *dt = nullptr, *ht = nullptr;
    if (int rc = ctx_alloc(c, &du, (size_t)n_rows * 4)) return rc;
    if (int rc = ctx_alloc(c, &dt, (size_t)n_rows * 4)) return rc;
    if (hipHostMalloc(&ht, (size_t)n_rows * 4, hipHostMallocDefault) != hipSuccess) {
      set_err("tdf_sample_logits: pinned allocation failed");
      return TDF_E_ALLOC;
    }
    if (c->ext_htok) (void)hipHostFree(c->ext_htok);
    ctx_free(c, c->ext_u);  // the previous call synchronised the stream
    ctx_free(c, c->ext_tok);
    c->ext_u = (float*)du;
    c->ext_tok = (int32_t*)dt;
    c->ext_htok = (int32_t*)ht;
    c->ext_rows = (size_t)n_rows;
  }
  if (parts > c->ext_parts) {
    void *pv = nullptr, *pi = nullptr;
    if (int rc = ctx_alloc(c, &pv, parts * 4)) return rc;
    if (int rc = ctx_alloc(c, &pi, parts * 4)) return rc;
    ctx_free(c, c->ext_pv);
    ctx_free(c, c->ext_pi);
    c->ext_pv = (float*)pv;
    c->ext_pi = (int32_t*)pi;
    c->ext_parts = parts;
  }
  return sample_rows(c, logits, n_rows, n_vocab, p, u, tokens, c->ext_u, c->ext_tok, c->ext_pv, c->ext_pi,
                     c->ext_htok);
}

// ---------------------------------------------------------------------------
// allocation-free sampling: the argmax partials live in a static device array
// (one copy per GPU, kept until the process ends) instead of memory the
// library allocates

namespace {
constexpr size_t kStaticScratchBytes = 1u << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// Device address of this GPU's `scratch` (looked up once per device with
// that device current; the array's name is only a host-side stand-in).
static int static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_err(std::string("tdf_sample_logits_static: no usable current device: ") + hipGetErrorString(e));
    return TDF_E_DEVICE;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      set_err(std::string("tdf_sample_logits_static: scratch lookup failed: ") + hipGetErrorString(e));
      return TDF_E_DEVICE;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TDF_OK;
}

extern "C" int32_t tdf_sample_logits_static(const float* logits, int32_t n_rows, int32_t n_vocab,
                                            const tdf_sampling* p, const float* u, int32_t* tokens,
                                            void* stream) {
  g_err.clear();
  if (!logits || !p || !tokens || n_rows < 0 || n_vocab < 1) {
    set_err("tdf_sample_logits_static: invalid arguments");
    return TDF_E_INVALID;
  }
  if (n_rows == 0) return TDF_OK;
  hipStream_t s = (hipStream_t)stream;
  if (p->temperature > 0.f) {
    // the chain needs no scratch: one block per row, its candidates in LDS
    if (!u || p->top_k < 1 || p->top_k > kMaxTopK || !(p->min_p >= 0.f && p->min_p <= 1.f) ||
        !(p->top_p == p->top_p) || !std::isfinite(p->temperature)) {
      set_err("tdf_sample_logits_static: invalid sampling parameters");
      return TDF_E_INVALID;
    }
    SampleParams sp;
    sp.temperature = p->temperature;
    sp.top_k = p->top_k;
    sp.top_p = p->top_p;
    sp.min_p = p->min_p;
    TDF_HIP(launch_sample(logits, n_rows, n_vocab, sp, u, tokens, s));
    return TDF_OK;
  }
  // greedy: per row argmax_splits(n_vocab) partial (value, index) pairs
  const size_t n_part = (size_t)n_rows * argmax_splits(n_vocab);
  const size_t v_bytes = (n_part * sizeof(float) + 255) & ~(size_t)255;
  if (v_bytes + n_part * sizeof(int32_t) > kStaticScratchBytes) {
    set_err("tdf_sample_logits_static: " + std::to_string(n_rows) + " rows of " + std::to_string(n_vocab) +
            " logits need more than the " + std::to_string(kStaticScratchBytes) + "-byte static scratch");
    return TDF_E_INVALID;
  }
  void* ptr = nullptr;
  if (int rc = static_scratch(&ptr)) return rc;
  float* pv = (float*)ptr;
  int32_t* pi = (int32_t*)((char*)ptr + v_bytes);
  TDF_HIP(launch_argmax(logits, n_rows, n_vocab, tokens, pv, pi, s));
  return TDF_OK;
}

extern "C" int32_t tdf_kv_seq_rm(tdf_context* c, int32_t seq, int32_t p0, int32_t p1) {
  if (!c || seq < 0 || seq >= c->n_seq_max || p0 < 0 || (p1 >= 0 && p1 < p0)) {
    set_err("invalid kv_seq_rm arguments");
    return TDF_E_INVALID;
  }
  KvBook next = c->book;
  next.seq_rm(seq, p0, p1);
  // rewrite the device copy of seq's (compacted) cell list, then commit
  const std::vector<int32_t>& lst = next.seq_cells(seq);
  if (!c->dry_run && !lst.empty()) {
    std::vector<int64_t> writes(2 * lst.size());
    for (size_t i = 0; i < lst.size(); ++i) {
      writes[2 * i] = (int64_t)seq * c->n_ctx + (int64_t)i;
      writes[2 * i + 1] = lst[i];
    }
    CallScratch scratch(c->stream);
    void* dw = nullptr;
    TDF_HIP(scratch.alloc(&dw, writes.size() * 8));
    TDF_HIP(hipMemcpyAsync(dw, writes.data(), writes.size() * 8, hipMemcpyHostToDevice, c->stream));
    TDF_HIP(launch_scatter(c->cell_list, (const int64_t*)dw, (int)lst.size(), c->stream));
    TDF_HIP(hipStreamSynchronize(c->stream));
  }
  c->book = std::move(next);
  return TDF_OK;
}

extern "C" int32_t tdf_kv_seq_shift(tdf_context* c, int32_t seq, int32_t p0, int32_t p1, int32_t delta) {
  if (!c || seq < 0 || seq >= c->n_seq_max || p0 < 0 || (p1 >= 0 && p1 < p0)) {
    set_err("invalid kv_seq_shift arguments");
    return TDF_E_INVALID;
  }
  if (delta == 0) return TDF_OK;
  std::vector<int32_t> cells;
  if (!c->book.shift_cells(seq, p0, p1, delta, cells)) {
    set_err("kv_seq_shift: a shifted cell is shared, a position would be negative, or the order would change");
    return TDF_E_INVALID;
  }
  if (cells.empty()) return TDF_OK;
  if (c->dry_run) {
    c->book.seq_shift(seq, delta, cells);
    return TDF_OK;
  }
  const tdf_hparams& h = c->m->hp;
  const int hd = h.head_dim, half = hd / 2;
  // angles delta * theta^(-2i/hd), as the RoPE table of a ubatch
  std::vector<double> cs(2 * half);
  for (int i = 0; i < half; ++i) {
    const double phi = (double)delta * std::pow((double)h.rope_theta, -2.0 * i / hd);
    cs[2 * i] = std::cos(phi);
    cs[2 * i + 1] = std::sin(phi);
  }
  CallScratch scratch(c->stream);
  void *dcells = nullptr, *dcs = nullptr;
  TDF_HIP(scratch.alloc(&dcells, cells.size() * 4));
  TDF_HIP(scratch.alloc(&dcs, cs.size() * 8));
  TDF_HIP(hipMemcpyAsync(dcells, cells.data(), cells.size() * 4, hipMemcpyHostToDevice, c->stream));
  TDF_HIP(hipMemcpyAsync(dcs, cs.data(), cs.size() * 8, hipMemcpyHostToDevice, c->stream));
  if (c->kv_dtype == TDF_Q8_0)
    TDF_HIP(launch_kv_rotate_q8(c->kv, 2 * c->kv_layer_bytes, h.n_layer, h.n_head_kv, c->n_ctx, hd,
                                (const int32_t*)dcells, (int)cells.size(), (const double2*)dcs, c->stream));
  else
    TDF_HIP(launch_kv_rotate(c->kv, c->kv_dtype, 2 * c->kv_layer_bytes, h.n_layer, h.n_head_kv, c->n_ctx, hd,
                             (const int32_t*)dcells, (int)cells.size(), (const double2*)dcs, c->stream));
  TDF_HIP(hipStreamSynchronize(c->stream));
  // positions move only once the keys are rotated
  c->book.seq_shift(seq, delta, cells);
  return TDF_OK;
}

extern "C" int32_t tdf_profile_read(const tdf_context* c, int32_t op, int32_t mfma, int64_t* launches, double* ms) {
  if (!c || !c->profile || op < 0 || op >= TDF_OP_COUNT) return TDF_E_INVALID;
  const int slot = 2 * op + (mfma ? 1 : 0);
  if (launches) *launches = c->prof_n[slot];
  if (ms) *ms = c->prof_ms[slot];
  return TDF_OK;
}

extern "C" int32_t tdf_profile_reset(tdf_context* c) {
  if (!c || !c->profile) return TDF_E_INVALID;
  for (int i = 0; i < 2 * TDF_OP_COUNT; ++i) {
    c->prof_n[i] = 0;
    c->prof_ms[i] = 0.0;
  }
  return TDF_OK;
}

extern "C" int32_t tdf_graph_counts(const tdf_context* c, int64_t* captures, int64_t* replays) {
  if (!c) return TDF_E_INVALID;
  if (captures) *captures = c->n_graph_captures;
  if (replays) *replays = c->n_graph_replays;
  return TDF_OK;
}

extern "C" int32_t tdf_time_op(tdf_context* c, int32_t op, int32_t n_tokens, int32_t reps, double* avg_us) {
  if (!c || !avg_us || c->dry_run || reps < 1 || n_tokens < 1 || n_tokens > c->n_ubatch) {
    set_err("tdf_time_op: invalid arguments");
    return TDF_E_INVALID;
  }
  if (op != TDF_OP_GATE_UP && op != TDF_OP_DOWN && op != TDF_OP_LM_HEAD) {
    set_err("tdf_time_op: op must be TDF_OP_GATE_UP, TDF_OP_DOWN or TDF_OP_LM_HEAD");
    return TDF_E_INVALID;
  }
  const tdf_model* m = c->m;
  const tdf_hparams& h = m->hp;
  const int d = h.n_embd, F = h.n_ff, V = h.n_vocab, L = h.n_layer, T = n_tokens;
  const bool wmfma = h.weight_dtype == TDF_BF16 || h.weight_dtype == TDF_Q8_0;
  if (op == TDF_OP_LM_HEAD && c->logits_cap < T) {
    if (int rc = ensure_logits(c, T)) return rc;
  }
  if ((op != TDF_OP_LM_HEAD && L == 0)) {
    set_err("tdf_time_op: model has no layers");
    return TDF_E_INVALID;
  }
  const int K = op == TDF_OP_DOWN ? F : d;
  const bool mfma = wmfma && T > kGemvMaxT && K % 64 == 0;
  auto args = [&](int l) {
    LinearArgs a;
    a.T = T; a.weight_dtype = h.weight_dtype;
    if (op == TDF_OP_GATE_UP) {
      const tdf_layer_weights& W = m->layers[l];
      a.w0 = W.w_gate; a.w1 = W.w_up; a.n0 = F; a.K = d;
      a.act_f32 = c->u; a.act_hi = c->h_hi; a.act_lo = c->h_lo;
      if (!mfma) {
        a.norm_ssp = c->ssp; a.norm_nparts = gemv_residual_parts(d); a.norm_stride = c->ssp_stride;
        a.norm_eps = h.rms_eps;
      }
      a.epi = EPI_SWIGLU; a.out = c->mb; a.out_hi = c->m_hi; a.out_lo = c->m_lo; a.ldo = F;
    } else if (op == TDF_OP_DOWN) {
      const tdf_layer_weights& W = m->layers[l];
      a.w0 = W.w_down; a.n0 = d; a.K = F;
      a.act_f32 = c->mb; a.act_hi = c->m_hi; a.act_lo = c->m_lo;
      a.epi = EPI_RESIDUAL; a.out = c->x; a.ldo = d;
    } else {
      a.w0 = m->output; a.n0 = V; a.K = d;
      a.act_f32 = c->u; a.act_hi = c->h_hi; a.act_lo = c->h_lo;
      if (!mfma) {
        a.norm_ssp = c->ssp; a.norm_nparts = gemv_residual_parts(d); a.norm_stride = c->ssp_stride;
        a.norm_eps = h.rms_eps;
      }
      a.epi = EPI_STORE; a.out = c->logits; a.ldo = V;
    }
    return a;
  };
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) e = hipEventRecord(e0, c->stream);
  for (int i = 0; i < reps && e == hipSuccess; ++i) {
    LinearArgs a = args(op == TDF_OP_LM_HEAD ? 0 : i % L);
    // the dispatch of the forward pass (GEMV, 9..32-token streaming kernel, GEMM)
    if (!mfma)
      e = launch_linear_gemv(a, c->stream);
    else if (a.T <= kDecodeMaxT && c->skinny_part && skinny_supported(a))
      e = launch_linear_skinny(a, c->skinny_part, c->stream);
    else
      e = launch_linear_gemm(a, c->stream);
  }
  if (e == hipSuccess) e = hipEventRecord(e1, c->stream);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess) {
    set_err(std::string("tdf_time_op: ") + hipGetErrorString(e));
    return TDF_E_DEVICE;
  }
  *avg_us = 1000.0 * ms / reps;
  return TDF_OK;
}

extern "C" int32_t tdf_fault_alloc(int32_t n) {
  g_fail_in = n > 0 ? n : 0;
  return TDF_OK;
}

extern "C" const char* tdf_last_error(void) { return g_err.c_str(); }
