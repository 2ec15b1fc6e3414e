"""GPU parity of Q8_0 weights (blocks of 32 elements of a row: one fp16
scale times 32 int8 values) against the float64 oracle, which dequantizes
the same buffers exactly.

Every product d * q is exact in float32, so with a float32 cache the only
differences are float32 rounding of the sums: the float32 tolerance
(max-abs 1e-4, rel-L2 1e-5) applies.  With a bf16 cache the cache
rounding is shared with the oracle but the attention runs on the matrix
cores with bf16 hi/lo operands: the bf16 tolerance applies.

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
Q8_MID = dict(n_vocab=8200, n_embd=1056, n_layer=2, n_head=8, n_head_kv=2, head_dim=64, n_ff=2080,
              rms_eps=1e-5, rope_theta=10000.0, tied=False, weight_dtype="q8_0", seed=23,
              weight_std=0.03, gain_std=0.1)


@pytest.mark.parametrize("kv_dtype,tied", [("f32", False), ("bf16", False), ("f32", True)])
def test_q8_small_prefill_and_steps(kv_dtype, tied):
    """150 tokens in ubatches of 64, 64, 22, logits for every row, then three
    single-token steps; tied: the LM head reads the Q8_0 embedding table."""
    cfg, w = make_weights(dict(Q8_SMALL, tied=tied))
    prompt = tdf_synth.prompt(cfg, 0, 150)
    nxt = tdf_synth.prompt(cfg, 1, 3)
    calls = [dict(tokens=prompt)] + [dict(tokens=[int(t)]) for t in nxt]
    tol = TOL_F32 if kv_dtype == "f32" else TOL_BF16
    log(f"q8 small kv={kv_dtype} tied={tied}")
    run_pair(cfg, w, dict(n_ctx=256, n_ubatch=64, output_all=True), calls, tol, kv_dtype, "q8-small")


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
