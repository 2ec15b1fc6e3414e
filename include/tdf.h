/*
 * tdf.h -- C ABI of the MI355X (gfx950) Llama-style decoder forward pass.
 *
 * The calls follow the problem statement of the pages:
 *  - a model made from hyper-parameters plus named weight tensors
 *    (Ollama engine page "Inside the inference engine: model architectures
 *    and the forward pass", sections on the model registry and reflection
 *    based initialisation; llama.cpp walkthrough "Step 4: loading
 *    hyper-parameters");
 *  - a context owning the KV cache (llama.cpp walkthrough "Step 7: creating
 *    the inference context"; Ollama page "KV Cache: memory for causal
 *    attention");
 *  - decode(batch of tokens, positions, sequence ids, output flags)
 *    (llama.cpp walkthrough "Step 10: forming the batch for one call" and
 *    "Steps 11-12: running the batch through the model"), logits per
 *    flagged row ("Steps 14-15") and the greedy token (Ollama page "Token
 *    sampling pipeline": temperature 0 is argmax).
 *
 * Conventions
 *  - All functions are callable from any host thread, one call per context
 *    at a time.  Errors are reported by the return value; a human-readable
 *    message for the calling thread is available from tdf_last_error().
 *  - "device" pointers are HIP device addresses on the current device;
 *    "host" pointers are ordinary process memory.
 *  - Matrices are row-major [out][in] in the model's weight dtype; norm
 *    gains are float32.
 */
#ifndef TDF_H
#define TDF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* TDF_Q8_0 (llama.cpp walkthrough and the Ollama backends chapter name the
 * "Q8_0" type without defining it; the common reading is taken): every block
 * of 32 consecutive elements of a row is one fp16 scale d times 32 int8
 * values q, w = d * q.  A Q8_0 matrix [rows][K] (K a multiple of 32) is one
 * buffer: rows*K int8 values q, row-major, then rows*K/32 fp16 scales,
 * row-major [rows][K/32], starting at byte rows*K.  As a cache type each
 * cached K or V row of head_dim values is quantized the same way when it is
 * stored: d = fp16(max|x| / 127), q = round-half-even(x / d) clamped to
 * [-127, 127] (0 when d is 0), decided in float32. */
typedef enum { TDF_F32 = 0, TDF_F16 = 1, TDF_BF16 = 2, TDF_Q8_0 = 3 } tdf_dtype;

/* Return codes of tdf_decode / tdf_kv_import (llama.cpp walkthrough,
 * "Steps 11-12": 0 success, 1 non-fatal, negative error). */
enum {
  TDF_OK = 0,
  TDF_NO_SLOT = 1,        /* not enough free KV cells: nothing was changed */
  TDF_E_INVALID = -1,     /* invalid argument or batch: nothing was changed */
  TDF_E_ALLOC = -2,       /* device allocation failed */
  TDF_E_DEVICE = -3       /* launch or device failure: clear the context */
};

/* Context flags. */
enum {
  TDF_CTX_DRY_RUN = 1,    /* bookkeeping only: validate, place cells, commit;
                             no device memory, no kernels, no logits; the
                             model's weight pointers are never read */
  TDF_CTX_PROFILE = 2     /* time every kernel launch with HIP events on the
                             context's stream (see tdf_profile_read) */
};

/* Operation classes timed by TDF_CTX_PROFILE. */
enum {
  TDF_OP_EMBED = 0,   /* embedding gather and cell-list update */
  TDF_OP_NORM = 1,    /* RMSNorm and output-row gather */
  TDF_OP_QKV = 2,     /* Q/K/V projection + RoPE + KV write */
  TDF_OP_ATTN = 3,    /* attention (split + merge) */
  TDF_OP_WO = 4,      /* output projection + residual */
  TDF_OP_GATE_UP = 5, /* gate/up projection + SwiGLU */
  TDF_OP_DOWN = 6,    /* down projection + residual */
  TDF_OP_LM_HEAD = 7, /* LM head */
  TDF_OP_ARGMAX = 8,  /* greedy argmax */
  TDF_OP_COUNT = 9
};

/* Hyper-parameters (llama.cpp walkthrough, "Step 4": n_vocab, n_embd,
 * n_layer, n_head, n_head_kv, n_ff, rope base).  head_dim is given
 * explicitly; rope frequency scale is 1 and RMSNorm eps sits inside the
 * square root. weight_dtype is TDF_F32, TDF_BF16 or TDF_Q8_0 (then n_embd,
 * n_head*head_dim and n_ff must be multiples of 32); it applies to the
 * matrices and the embedding table, never to the norm gains. */
typedef struct {
  int32_t n_vocab, n_embd, n_layer, n_head, n_head_kv, head_dim, n_ff;
  float rms_eps, rope_theta;
  int32_t weight_dtype;
  /* Sliding-window attention (Ollama engine page, "KV Cache: memory for
   * causal attention": a windowed layer's mask keeps only the most recent
   * tokens).  n_swa = W > 0: in a windowed layer a token at position p sees
   * only its sequence's cells with position > p - W (the W most recent
   * positions, its own included); 0 = no window.  swa_layers: HOST array of
   * n_layer flags (nonzero = windowed), copied by tdf_model_create; NULL =
   * every layer windowed.  Cells outside the window stay in the cache. */
  int32_t n_swa;
  const int8_t *swa_layers;
} tdf_hparams;

/* Device pointers of one layer (GGUF names blk.<i>.*): attn_norm, attn_q
 * [n_head*head_dim][n_embd], attn_k / attn_v [n_head_kv*head_dim][n_embd],
 * attn_output [n_embd][n_head*head_dim], ffn_norm, ffn_gate / ffn_up
 * [n_ff][n_embd], ffn_down [n_embd][n_ff]. */
typedef struct {
  const void *attn_norm, *wq, *wk, *wv, *wo, *ffn_norm, *w_gate, *w_up, *w_down;
} tdf_layer_weights;

/* token_embd [n_vocab][n_embd]; output_norm [n_embd] f32; output
 * [n_vocab][n_embd] or NULL to reuse token_embd (tied embeddings, the
 * "alt:token_embd" fallback of the Ollama model struct).  `layers` is a
 * HOST array of n_layer entries; it is copied by tdf_model_create. */
typedef struct {
  const void *token_embd, *output_norm, *output;
  const tdf_layer_weights *layers;
} tdf_weights;

/* n_ctx = KV cells; n_batch = largest batch per decode (clamped to n_ctx);
 * n_ubatch = tokens per forward chunk (clamped to n_batch); n_seq_max <= 64;
 * kv_dtype = TDF_F32, TDF_F16, TDF_BF16 or TDF_Q8_0 (head_dim a multiple of
 * 32; blocks of 32 along head_dim); output_all = default output flag
 * of every token instead of the last; stream = hipStream_t to run on (NULL:
 * the context creates its own). */
typedef struct {
  int32_t n_ctx, n_batch, n_ubatch, n_seq_max;
  int32_t kv_dtype;
  int32_t output_all;
  int32_t flags;
  void *stream;
} tdf_context_params;

/* One decode call (llama.cpp walkthrough, "Step 10": struct llama_batch
 * without the embedding input).  HOST arrays of n_tokens entries, read only
 * during tdf_decode.  pos == NULL: each sequence continues at
 * seq_pos_max(s)+1 in batch order.  n_seq_id/seq_id == NULL: sequence 0.
 * logits == NULL: only the last token (or all, with output_all). */
typedef struct {
  int32_t n_tokens;
  const int32_t *token;
  const int32_t *pos;
  const int32_t *n_seq_id;
  const int32_t *const *seq_id;
  const int8_t *logits;
} tdf_batch;

typedef struct tdf_model tdf_model;
typedef struct tdf_context tdf_context;

/* Model from hparams and DEVICE weight pointers.  The weights are NOT
 * copied or owned: they must stay valid until tdf_model_free.  NULL on
 * error (invalid hparams, missing pointer). */
tdf_model *tdf_model_create(const tdf_hparams *hp, const tdf_weights *w);
void tdf_model_free(tdf_model *m);

/* Context (KV cache, scratch, logits) for a model; the model must outlive
 * it.  NULL on error (invalid parameters, allocation failure). */
tdf_context *tdf_context_create(const tdf_model *m, const tdf_context_params *p);
void tdf_context_free(tdf_context *c);

/* Run the batch: validate and fill defaults, split into ubatches of at most
 * n_ubatch tokens in order, place each ubatch's tokens in KV cells, run the
 * forward pass, keep the logits of flagged rows and their greedy tokens.
 * Returns TDF_OK, TDF_NO_SLOT (nothing changed), TDF_E_INVALID (nothing
 * changed), TDF_E_ALLOC or TDF_E_DEVICE.  Synchronises the context's stream
 * before returning. */
int32_t tdf_decode(tdf_context *c, const tdf_batch *b);

/* Rows with logits after the last successful tdf_decode: the tokens whose
 * logits flag was set (llama.cpp walkthrough, "Steps 14-15": the context keeps
 * logits only for positions flagged in the batch).  TDF_E_INVALID for a NULL
 * context. */
int32_t tdf_n_outputs(const tdf_context *c);

/* Batch indices (batch order) of those rows ("Steps 14-15": one row per
 * flagged position, over every ubatch of the call) into the HOST array
 * out[n_outputs] (may be NULL to query the count); returns n_outputs, or
 * TDF_E_INVALID for a NULL context. */
int32_t tdf_output_ids(const tdf_context *c, int32_t *out);

/* HOST pointer to the n_vocab float32 logits of batch index i of the last
 * decode (llama.cpp walkthrough, "Steps 14-15": llama_get_logits_ith gives
 * n_vocab floats for a position of the batch), or NULL if i was not flagged,
 * is out of range, the context is a dry run, or the copy failed (message in
 * tdf_last_error).  The memory belongs to the context: valid until the next
 * tdf_decode, tdf_kv_clear or tdf_context_free (copied from the device on
 * first use). */
const float *tdf_get_logits_ith(tdf_context *c, int32_t i);

/* DEVICE pointer to the [n_outputs][n_vocab] float32 logits of the last
 * decode (the same rows as tdf_get_logits_ith, "Steps 14-15"), row r for
 * batch index tdf_output_ids[r]; owned by the context, valid as above, NULL
 * for a NULL or dry-run context.  Read it on the context's stream or after
 * tdf_decode returned (it synchronises). */
const float *tdf_get_logits_device(tdf_context *c);

/* Greedy token (argmax, lowest index on ties) of batch index i, or
 * TDF_E_INVALID if i was not flagged. */
int32_t tdf_argmax_ith(const tdf_context *c, int32_t i);

/* Largest position held by sequence s, -1 if none (llama.cpp walkthrough,
 * "KV-cache and the Prefill / Decode stages"); TDF_E_INVALID for a bad s. */
int32_t tdf_seq_pos_max(const tdf_context *c, int32_t s);

/* Free every cell: every sequence becomes empty (seq_pos_max -1) and the
 * next decode places its tokens from cell 0 again (llama.cpp walkthrough,
 * "KV-cache and the Prefill / Decode stages": the cache is sized for n_ctx
 * at creation and filled position by position; clearing makes the stored
 * K/V unreachable without touching the device memory).  Also drops the
 * logits of the last decode.  TDF_OK, or TDF_E_INVALID for a NULL context. */
int32_t tdf_kv_clear(tdf_context *c);

/* Inspection of one cell's bookkeeping (Ollama engine page, "KV Cache: memory
 * for causal attention": each cached slot records its position and the
 * sequences it belongs to, from which the mask is built): *pos = position
 * (-1 if free), *seq_mask = bit s set if sequence s holds the cell.  Either
 * output pointer (HOST) may be NULL.  TDF_OK, or TDF_E_INVALID for a NULL
 * context or a cell outside [0, n_ctx). */
int32_t tdf_kv_cell(const tdf_context *c, int32_t cell, int32_t *pos, uint64_t *seq_mask);

/* Cells given to the tokens of the last successful decode or import (batch
 * order; Ollama engine page, "KV Cache": the slots found for the batch's K/V)
 * into the HOST array slots[n_tokens] (may be NULL to query the count);
 * returns n_tokens, or TDF_E_INVALID for a NULL context. */
int32_t tdf_last_slots(const tdf_context *c, int32_t *slots);

/* Restore cached K/V (llama.cpp walkthrough, "KV-cache and the Prefill /
 * Decode stages": the cache holds, per layer and position, the keys and
 * values already computed, so later steps only read them).  Places positions
 * [pos0, pos0+n) of sequence s in cells (one chunk, the ubatch placement
 * rule) and fills them with the given post-RoPE keys and values:
 * k_layers[l] / v_layers[l] are DEVICE pointers to [n][n_head_kv][head_dim]
 * arrays in the context's kv dtype, float32 for a TDF_Q8_0 cache (quantized
 * on import); k_layers / v_layers are HOST arrays of n_layer pointers, read
 * only during the call.  The cells are committed only after the device
 * holds the rows; on any error nothing changes in the bookkeeping.  Returns
 * TDF_OK, TDF_NO_SLOT, TDF_E_INVALID (pos0 must exceed seq_pos_max(s)) or
 * TDF_E_DEVICE. */
int32_t tdf_kv_import(tdf_context *c, int32_t s, int32_t pos0, int32_t n,
                      const void *const *k_layers, const void *const *v_layers);

/* Token sampling (Ollama engine page, "Token sampling pipeline"): for each
 * output row i of the last tdf_decode (i in [0, tdf_n_outputs)), one token
 * from its logits.  temperature <= 0: greedy (argmax, lowest index on ties;
 * the other fields are ignored).  Otherwise the chain Top-K (the top_k
 * highest logits, ties to the lower token id; 1 <= top_k <= 1024) ->
 * temperature (logits divided by it) -> softmax -> Top-P (tokens in ranking
 * order while the cumulative probability is <= top_p; the first always;
 * top_p >= 1 keeps all) ->
 * Min-P (probability >= min_p times the largest; 0 <= min_p <= 1) -> draw:
 * the first survivor whose cumulative probability exceeds u[i] times the
 * survivors' total.  u: HOST array of n_outputs uniform numbers in [0, 1)
 * (the caller's seeded generator makes the draw reproducible); tokens: HOST
 * array of n_outputs entries, written on success.  Returns TDF_OK,
 * TDF_E_INVALID (bad parameters or u outside [0, 1); nothing written) or
 * TDF_E_DEVICE. */
typedef struct {
  float temperature;
  int32_t top_k;
  float top_p, min_p;
} tdf_sampling;
int32_t tdf_sample(tdf_context *c, const tdf_sampling *p, const float *u, int32_t *tokens);

/* The same chain (or greedy argmax) on the caller's logits: n_rows rows of
 * n_vocab float32 values at the DEVICE pointer logits (row-major, rows
 * n_vocab apart, read only), e.g. rows the caller edited after tdf_decode.
 * Runs on the context's stream and synchronises it; u and tokens are HOST
 * arrays of n_rows entries as for tdf_sample.  The context keeps small
 * buffers for the rows' draws and tokens, grown on demand.  Returns TDF_OK,
 * TDF_E_INVALID (bad arguments or parameters; nothing written), TDF_E_ALLOC
 * or TDF_E_DEVICE. */
int32_t tdf_sample_logits(tdf_context *c, const float *logits, int32_t n_rows, int32_t n_vocab,
                          const tdf_sampling *p, const float *u, int32_t *tokens);

/* Allocation-free variant of tdf_sample_logits, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid hipMalloc.  It makes no allocation of any kind.
 * logits: DEVICE [n_rows][n_vocab] float32 (read only); u: DEVICE array of
 * n_rows uniform numbers (read only; needed when temperature > 0; values
 * are not checked on the host: u >= 1 picks the last survivor); tokens:
 * DEVICE array of n_rows entries, written by the kernels.  The work is
 * enqueued on stream (a hipStream_t; NULL: the null stream) and the call
 * returns without waiting for it.  Greedy (temperature <= 0) keeps its
 * per-row partial maxima in a static device array of 1 MiB per GPU (shared
 * by every call on that GPU, held until the process ends, fully overwritten
 * by each call; calls that overlap on one GPU race on it); rows x partials
 * beyond that size (more than 2080 rows of 128256 logits) are rejected with
 * TDF_E_INVALID before anything is enqueued.  The sampling chain needs no
 * scratch.  Returns TDF_OK, TDF_E_INVALID or TDF_E_DEVICE (launch failure,
 * message in tdf_last_error). */
int32_t tdf_sample_logits_static(const float *logits, int32_t n_rows, int32_t n_vocab,
                                 const tdf_sampling *p, const float *u, int32_t *tokens, void *stream);

/* Sliding the context window (Ollama engine page, "KV Cache: memory for
 * causal attention": when the cache is full, the model's shift function
 * re-encodes the RoPE positions of the cached keys and the window moves
 * forward instead of the context being dropped).
 *
 * tdf_kv_seq_rm: remove sequence seq from its cells with position in
 * [p0, p1) (p1 < 0: no upper end); cells left with no sequence become free
 * for later calls.  tdf_kv_seq_shift: add delta to the positions of seq's
 * cells with position in [p0, p1) and rotate their cached keys (every layer
 * and KV head) by delta, so that they equal keys computed at the new
 * positions (RoPE rotations compose); the result is stored in the cache type
 * again.  The shifted cells must belong to seq alone, and seq's positions
 * must stay >= 0, distinct and in their order.  Both return TDF_OK or
 * TDF_E_INVALID (bad arguments or a shift that breaks these rules: nothing
 * changed) or TDF_E_DEVICE. */
int32_t tdf_kv_seq_rm(tdf_context *c, int32_t seq, int32_t p0, int32_t p1);
int32_t tdf_kv_seq_shift(tdf_context *c, int32_t seq, int32_t p0, int32_t p1, int32_t delta);

/* Accumulated launches and GPU time (ms, HIP events) of operation class op
 * since the last reset, for the matrix-core path (mfma = 1: ubatches above
 * 32 tokens) or the decode path (mfma = 0).  Only for TDF_CTX_PROFILE
 * contexts; TDF_E_INVALID otherwise. */
int32_t tdf_profile_read(const tdf_context *c, int32_t op, int32_t mfma, int64_t *launches, double *ms);
int32_t tdf_profile_reset(tdf_context *c);

/* Measurement hook: launch the linear layer of operation op (TDF_OP_GATE_UP,
 * TDF_OP_DOWN or TDF_OP_LM_HEAD) for an ubatch of n_tokens rows (the decode
 * GEMV up to 8 rows, the streaming matrix-core kernel with its epilogue pass
 * for 9..32 rows, the matrix-core GEMM above, as tdf_decode chooses)
 * reps times back to back on the context's stream, cycling over the layers
 * so that no launch finds its weights cached, and store the mean duration
 * per launch in microseconds (HIP events on that stream) in *avg_us.  The
 * inputs are whatever the context's scratch holds (run tdf_decode first);
 * the outputs overwrite scratch, the residual rows and the logits, so the
 * logits of the last tdf_decode are no longer valid afterwards.  The KV cache
 * and the cell bookkeeping are untouched.  Returns TDF_OK, TDF_E_INVALID
 * (bad op, n_tokens outside [1, n_ubatch], reps < 1, dry-run context) or
 * TDF_E_DEVICE. */
int32_t tdf_time_op(tdf_context *c, int32_t op, int32_t n_tokens, int32_t reps, double *avg_us);

/* Launch replay (llama.cpp walkthrough, "Step 13": graph reuse for same-shape
 * ubatches): ubatches of up to 32 tokens run as a captured HIP graph, one per
 * shape, replayed on later calls.  Counts of captures and replays so far.
 * Disabled in TDF_CTX_PROFILE contexts and when TDF_NO_GRAPH=1 is set. */
int32_t tdf_graph_counts(const tdf_context *c, int64_t *captures, int64_t *replays);

/* Failure injection for tests of the error paths (not part of the forward
 * pass): the n-th device allocation the library makes from now on fails as
 * if the device were out of memory (n <= 0 disarms).  The creators then
 * return NULL and tdf_decode TDF_E_ALLOC with nothing changed.  Process-wide;
 * the environment variable TDF_FAULT_ALLOC=n does the same for the n-th
 * allocation of the process.  Returns TDF_OK. */
int32_t tdf_fault_alloc(int32_t n);

/* Message of the last failure on the calling thread ("" if none). */
const char *tdf_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TDF_H */
