"""GPU parity of Q8_0 weights (blocks of 32 elements of a row: one fp16
scale times 32 int8 values) against the float64 oracle, which dequantizes
the same buffers exactly.

Every product d * q is exact in float32.  Where every step runs on the
vector units (the GEMV for ubatches of up to 8 tokens, or inner sizes that
are not multiples of 64) with a float32 cache, the only differences are
float32 rounding of the sums: the float32 tolerance (max-abs 1e-4, rel-L2
1e-5) applies.  Larger ubatches run the matrix cores (int8 values widened
exactly to bf16, activations as a bf16 hi/lo pair, one block scale per 32
products), and a bf16 cache feeds the matrix-core attention: there the bf16
tolerance applies.

Sizes: the GEMV reads a row in chunks of 1024 int8 (16 per lane), so the
inner sizes 1056 and 2080 take full chunks plus a ragged 32-element tail;
128, 256 and 512 are tail-only rows.  A vocabulary of 8200 rows gives the
LM head more than 4096 row pairs (the deeper-batched launch).  Prompts of
more than 8 tokens pass through the GEMV eight tokens at a time; steps of
three sequences take the four-token GEMV.
"""
import numpy as np
import pytest

import tdf_synth

from gpu_common import TOL_BF16, TOL_F32, log, make_weights
from test_gpu_parity import SMALL, run_pair, teacher_forced

pytestmark = pytest.mark.gpu

Q8_SMALL = dict(SMALL, weight_dtype="q8_0", seed=21)
# inner sizes 512 and 1024: four and eight 128-wide chunks for the 9..32-token path
Q8_SK = dict(n_vocab=1000, n_embd=512, n_layer=2, n_head=8, n_head_kv=2, head_dim=64, n_ff=1024,
             rms_eps=1e-5, rope_theta=10000.0, tied=False, weight_dtype="q8_0", seed=25,
             weight_std=0.04, gain_std=0.1)
Q8_MID = dict(n_vocab=8200, n_embd=1056, n_layer=2, n_head=8, n_head_kv=2, head_dim=64, n_ff=2080,
              rms_eps=1e-5, rope_theta=10000.0, tied=False, weight_dtype="q8_0", seed=23,
              weight_std=0.03, gain_std=0.1)


@pytest.mark.parametrize("kv_dtype,tied", [("f32", False), ("bf16", False), ("f32", True)])
def test_q8_small_prefill_and_steps(kv_dtype, tied):
    """150 tokens in ubatches of 64, 64, 22 (matrix cores: a 22-row tile
    included), logits for every row, then three single-token steps (GEMV);
    tied: the LM head reads the Q8_0 embedding table."""
    cfg, w = make_weights(dict(Q8_SMALL, tied=tied))
    prompt = tdf_synth.prompt(cfg, 0, 150)
    nxt = tdf_synth.prompt(cfg, 1, 3)
    calls = [dict(tokens=prompt)] + [dict(tokens=[int(t)]) for t in nxt]
    log(f"q8 small kv={kv_dtype} tied={tied}")
    run_pair(cfg, w, dict(n_ctx=256, n_ubatch=64, output_all=True), calls, TOL_BF16, kv_dtype, "q8-small")


def test_q8_small_vector_units_f32_tolerance():
    """Ubatches of at most 8 tokens stay on the vector units: with a float32
    cache the float32 tolerance holds."""
    cfg, w = make_weights(Q8_SMALL)
    prompt = tdf_synth.prompt(cfg, 0, 24)
    calls = [dict(tokens=prompt[i:i + 8], logits=np.ones(8, dtype=np.int8)) for i in range(0, 24, 8)]
    calls += [dict(tokens=[int(t)]) for t in tdf_synth.prompt(cfg, 1, 2)]
    run_pair(cfg, w, dict(n_ctx=64, n_ubatch=8), calls, TOL_F32, "f32", "q8-small-gemv")


def test_q8_llama1b_width_two_layers():
    """1B-class widths with Q8_0 weights, two layers: 300-token prompt in
    ubatches of 128, 128, 44 on the matrix cores (several 64x128 tiles, the
    residual projections split over K, a ragged last tile), then 4 steps."""
    cfg = dict(tdf_synth.CONFIGS["llama1b"], weight_dtype="q8_0")
    cfg, w = make_weights(cfg, layers=2)
    prompt = tdf_synth.prompt(cfg, 0, 300)
    teacher_forced(cfg, w, 512, prompt, 4, TOL_BF16, "f16", n_ubatch=128, label="q8-1b-2L")


def test_q8_nine_to_32_token_ubatches():
    """Ubatches of 9..32 tokens (the K-sliced matrix-core path: int8 chunks
    widened into LDS, block scales per row): 48 tokens of 16 interleaved
    sequences in ubatches of 24, then two lock-step steps of one token per
    sequence (16 tokens), every row's logits."""
    cfg, w = make_weights(Q8_SK)
    rng = np.random.default_rng(7)
    S = 16
    seqs = [int(x) for x in rng.integers(0, S, size=48)]
    calls = [dict(tokens=tdf_synth.prompt(cfg, 0, 48), seq_ids=[[q] for q in seqs], logits=np.ones(48, dtype=np.int8))]
    for step in range(2):
        calls.append(dict(tokens=tdf_synth.prompt(cfg, 20 + step, S), seq_ids=[[q] for q in range(S)],
                          logits=np.ones(S, dtype=np.int8)))
    log("q8 9..32-token ubatches")
    run_pair(cfg, w, dict(n_ctx=128, n_ubatch=24, n_seq_max=S), calls, TOL_BF16, "bf16", "q8-skinny")


def test_q8_four_row_waves_ragged():
    """Single-token GEMVs with four rows per wave: a vocabulary of 16390 rows
    (the LM head's last wave holds two rows) and a stacked Q/K/V of 20480 rows
    (128 query heads of 128, 16 KV heads), then decode steps; f32 cache, so
    the float32 tolerance applies to the steps after a vector-unit prompt."""
    cfg = dict(n_vocab=16390, n_embd=256, n_layer=1, n_head=128, n_head_kv=16, head_dim=128, n_ff=512,
               rms_eps=1e-5, rope_theta=10000.0, tied=False, weight_dtype="q8_0", seed=27,
               weight_std=0.05, gain_std=0.1)
    cfg, w = make_weights(cfg)
    prompt = tdf_synth.prompt(cfg, 0, 8)
    calls = [dict(tokens=prompt[:4]), dict(tokens=prompt[4:])] + \
        [dict(tokens=[int(t)]) for t in tdf_synth.prompt(cfg, 1, 4)]
    log("q8 four-row waves")
    run_pair(cfg, w, dict(n_ctx=32, n_ubatch=8), calls, TOL_F32, "f32", "q8-r4")


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16"])
def test_q8_ragged_chunks_teacher_forced(kv_dtype):
    """40-token prompt in ubatches of 16, 16, 8, then 6 teacher-forced steps."""
    cfg, w = make_weights(Q8_MID)
    prompt = tdf_synth.prompt(cfg, 0, 40)
    tol = TOL_F32 if kv_dtype == "f32" else TOL_BF16
    log(f"q8 mid kv={kv_dtype}")
    teacher_forced(cfg, w, 128, prompt, 6, tol, kv_dtype, n_ubatch=16, label=f"q8-mid-{kv_dtype}")


def test_q8_three_sequences_lock_step():
    """Three interleaved sequences, then steps of one token per sequence."""
    cfg, w = make_weights(Q8_MID)
    rng = np.random.default_rng(5)
    seqs = [int(s) for s in rng.integers(0, 3, size=30)]
    toks = tdf_synth.prompt(cfg, 0, 30)
    calls = [dict(tokens=toks, seq_ids=[[s] for s in seqs], logits=np.ones(30, dtype=np.int8))]
    for step in range(2):
        calls.append(dict(tokens=tdf_synth.prompt(cfg, 10 + step, 3), seq_ids=[[0], [1], [2]],
                          logits=np.ones(3, dtype=np.int8)))
    log("q8 mid three sequences")
    run_pair(cfg, w, dict(n_ctx=64, n_ubatch=32, n_seq_max=3), calls, TOL_F32, "f32", "q8-multiseq")
