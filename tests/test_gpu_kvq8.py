"""GPU parity of the Q8_0 KV cache (each cached K/V row stored as blocks of
32: fp16 scale, int8 codes decided in float32) against the float64 oracle,
whose cache stores the same rule's values.

Both sides quantize their own float32 K/V rows.  The GPU's rows come from
float32 (vector units) or hi/lo bf16 (matrix cores) projections and differ
from the oracle's in the last bits, so a code can differ by one where x / d
falls next to a rounding boundary; the bf16 tolerance (max-abs 3e-2, rel-L2
1e-2) covers that.  Imported rows are the same float32 values on both sides,
so their codes agree exactly.  Cells, positions and output rows: bit-exact.
"""
import numpy as np
import pytest

import tdf_synth
from oracle import OracleContext

from gpu_common import TOL_BF16, check_logits, check_token, device_model, log, make_weights, oracle_model
from test_gpu_parity import SMALL, run_pair, teacher_forced
from test_gpu_swa import SMALL64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg0", [SMALL, SMALL64], ids=["hd32", "hd64"])
def test_prefill_and_steps(cfg0):
    """150 tokens in ubatches of 64, 64, 22, logits for every row, then three
    steps (head_dim 32: vector-unit attention; 64: matrix cores)."""
    cfg, w = make_weights(cfg0)
    prompt = tdf_synth.prompt(cfg, 0, 150)
    calls = [dict(tokens=prompt)] + [dict(tokens=[int(t)]) for t in tdf_synth.prompt(cfg, 1, 3)]
    log(f"q8 cache hd={cfg['head_dim']}")
    run_pair(cfg, w, dict(n_ctx=256, n_ubatch=64, output_all=True), calls, TOL_BF16, "q8_0", "kvq8")


def test_multi_sequence_steps():
    cfg, w = make_weights(SMALL64)
    rng = np.random.default_rng(4)
    seqs = [int(s) for s in rng.integers(0, 3, size=90)]
    calls = [dict(tokens=tdf_synth.prompt(cfg, 0, 90), seq_ids=[[s] for s in seqs],
                  logits=np.ones(90, dtype=np.int8))]
    for step in range(3):
        calls.append(dict(tokens=tdf_synth.prompt(cfg, 10 + step, 3), seq_ids=[[0], [1], [2]],
                          logits=np.ones(3, dtype=np.int8)))
    run_pair(cfg, w, dict(n_ctx=200, n_ubatch=40, n_seq_max=4), calls, TOL_BF16, "q8_0", "kvq8-multiseq")


def test_lock_step_sequences_own_rows():
    """12 sequences (prompts of 20..119 tokens, ubatches of 64), then three
    lock-step steps of 12 tokens, one per sequence: no token sees another's
    new cell, so the decode attention quantizes each token's own K/V rows
    (9..32-token projections write them as float32).  Then a step whose two
    tokens share a sequence (the separate quantization pass), and one more
    lock-step step.  Every row's logits, cells and output rows checked."""
    cfg, w = make_weights(SMALL64)
    calls = [dict(tokens=tdf_synth.prompt(cfg, 50 + q, 20 + 9 * q), seq_ids=[[q]] * (20 + 9 * q)) for q in range(12)]
    lock = lambda seed: dict(tokens=[int(x) for x in tdf_synth.prompt(cfg, seed, 12)], seq_ids=[[q] for q in range(12)],
                             logits=np.ones(12, dtype=np.int8))
    calls += [lock(70 + k) for k in range(3)]
    calls.append(dict(tokens=[int(x) for x in tdf_synth.prompt(cfg, 80, 3)], seq_ids=[[4], [4], [9]],
                      logits=np.ones(3, dtype=np.int8)))
    calls.append(lock(81))
    log("q8 cache lock-step own rows")
    run_pair(cfg, w, dict(n_ctx=2048, n_ubatch=64, n_seq_max=16), calls, TOL_BF16, "q8_0", "kvq8-lockstep")


def test_graph_key_tracks_own_rows():
    """Steps of the same shape (3 tokens, every row's logits, three list
    writes) that alternate between one token per sequence (the decode
    attention quantizes the tokens' own rows) and two tokens of one sequence
    (the separate quantization pass): replayed launch sequences must follow
    the difference."""
    cfg, w = make_weights(SMALL64)
    calls = [dict(tokens=tdf_synth.prompt(cfg, 60 + q, 30 + 10 * q), seq_ids=[[q]] * (30 + 10 * q)) for q in range(3)]
    for k in range(6):
        seqs = [[0], [1], [2]] if k % 2 == 0 else [[0], [0], [1]]
        calls.append(dict(tokens=[int(x) for x in tdf_synth.prompt(cfg, 90 + k, 3)], seq_ids=seqs,
                          logits=np.ones(3, dtype=np.int8)))
    log("q8 cache: alternating own-row and shared-sequence steps")
    gc, _ = run_pair(cfg, w, dict(n_ctx=512, n_ubatch=64, n_seq_max=4), calls, TOL_BF16, "q8_0", "kvq8-graph-own-rows")
    # captured: the 30-token prompt, the first step of each kind; replayed:
    # the other four steps (one key per kind: without the own-row flag in
    # the key a shared-sequence step would replay the own-row graph, and
    # there would be 2 captures)
    assert gc.graph_counts() == (3, 4), gc.graph_counts()


def test_import_then_decode():
    """300 positions of float32 N(0,1) rows imported (quantized on both sides
    by the same rule from the same values), then decode steps."""
    import transformer_decode_forward_amd as tdf
    from transformer_decode_forward_amd.device import to_device
    cfg, w = make_weights(SMALL64)
    L, P = cfg["n_layer"], 300
    ks = [tdf_synth.kv_fill(cfg, l, "k", 0, P, "f32") for l in range(L)]
    vs = [tdf_synth.kv_fill(cfg, l, "v", 0, P, "f32") for l in range(L)]
    gc = tdf.Context(device_model(cfg, w), n_ctx=512, kv_dtype="q8_0")
    kd = [to_device(k) for k in ks]
    vd = [to_device(v) for v in vs]
    assert gc.kv_import(0, 0, P, [t.data_ptr() for t in kd], [t.data_ptr() for t in vd]) == 0
    oc = OracleContext(oracle_model(cfg, w), n_ctx=512, kv_dtype="q8_0")
    assert oc.kv_import(0, 0, P, ks, vs) == 0
    for t in tdf_synth.prompt(cfg, 2, 3):
        assert gc.decode([int(t)]) == 0
        ro = oc.decode([int(t)])
        assert gc.last_slots() == ro.slots
        check_logits(gc.logits_ith(0), ro.logits[0], TOL_BF16, "kvq8 import")
        check_token(gc.argmax_ith(0), ro.logits[0], "kvq8 import")


def test_import_long_context_own_rows():
    """20000 imported positions (8 KV heads of 128, 2 query heads each),
    then three single-token steps: 1024-cell chunks, the token's own K/V
    rows quantized by the block whose partial last chunk holds its cell, 20
    chunks merged."""
    import transformer_decode_forward_amd as tdf
    from transformer_decode_forward_amd.device import to_device
    cfg0 = dict(SMALL, n_embd=256, n_head=16, n_head_kv=8, head_dim=128, n_ff=256, seed=77)
    cfg, w = make_weights(cfg0)
    L, P, n_ctx = cfg["n_layer"], 20000, 20480
    ks = [tdf_synth.kv_fill(cfg, l, "k", 0, P, "f32") for l in range(L)]
    vs = [tdf_synth.kv_fill(cfg, l, "v", 0, P, "f32") for l in range(L)]
    gc = tdf.Context(device_model(cfg, w), n_ctx=n_ctx, kv_dtype="q8_0")
    kd = [to_device(k) for k in ks]
    vd = [to_device(v) for v in vs]
    assert gc.kv_import(0, 0, P, [t.data_ptr() for t in kd], [t.data_ptr() for t in vd]) == 0
    oc = OracleContext(oracle_model(cfg, w), n_ctx=n_ctx, kv_dtype="q8_0")
    assert oc.kv_import(0, 0, P, ks, vs) == 0
    log("q8 cache 20k imported cells, single-token steps")
    for k, t in enumerate(tdf_synth.prompt(cfg, 5, 3)):
        assert gc.decode([int(t)]) == 0, tdf.tdf_last_error()
        ro = oc.decode([int(t)])
        assert gc.last_slots() == ro.slots
        check_logits(gc.logits_ith(0), ro.logits[0], TOL_BF16, f"kvq8 long own rows step {k}")
        check_token(gc.argmax_ith(0), ro.logits[0], f"kvq8 long own rows step {k}")


def test_drop_and_shift_then_decode():
    """Drop positions [0, 30) of a 100-token prompt, shift the rest down by 30
    (the stored keys rotated and re-quantized), then 5 steps."""
    import transformer_decode_forward_amd as tdf
    cfg, w = make_weights(SMALL64)
    gc = tdf.Context(device_model(cfg, w), n_ctx=256, n_ubatch=64, kv_dtype="q8_0")
    oc = OracleContext(oracle_model(cfg, w), n_ctx=256, n_ubatch=64, kv_dtype="q8_0")
    prompt = tdf_synth.prompt(cfg, 0, 100)
    assert gc.decode(prompt) == 0 and oc.decode(prompt).status == 0
    assert gc.kv_seq_rm(0, 0, 30) == oc.kv_seq_rm(0, 0, 30) == 0
    assert gc.kv_seq_shift(0, 30, -1, -30) == oc.kv_seq_shift(0, 30, -1, -30) == 0
    for k, t in enumerate(tdf_synth.prompt(cfg, 1, 5)):
        assert gc.decode([int(t)]) == 0
        ro = oc.decode([int(t)])
        assert gc.last_slots() == ro.slots
        check_logits(gc.logits_ith(0), ro.logits[0], TOL_BF16, f"kvq8 shift step {k}")


@pytest.mark.parametrize("hd,n_head,n_head_kv", [(128, 8, 2), (128, 2, 2), (64, 8, 1)], ids=["hd128g4", "hd128g1", "hd64g8"])
def test_matrix_core_long_context(hd, n_head, n_head_kv):
    """Matrix-core attention over Q8_0 rows: a 1100-token prompt in ubatches
    of 512, 512, 76 (prefill attention: blocks dequantized into LDS as bf16
    hi/lo pairs), then four steps (decode attention: codes widened to bf16,
    key block scales on the 32-deep score products, value block scales folded
    into the probabilities) whose 1100+ cells split into chunks of 128 that
    are merged, a ragged last tile in each."""
    cfg0 = dict(SMALL, n_embd=256, n_head=n_head, n_head_kv=n_head_kv, head_dim=hd, n_ff=256, seed=31 + hd + n_head)
    cfg, w = make_weights(cfg0)
    prompt = tdf_synth.prompt(cfg, 0, 1100)
    log(f"q8 cache matrix cores hd={hd} G={n_head // n_head_kv}")
    teacher_forced(cfg, w, 1200, prompt, 4, TOL_BF16, "q8_0", n_ubatch=512, label=f"kvq8-mfma-hd{hd}")


def test_llama8b_width_single_token_quantize():
    """8B-class widths (32 query heads, 8 KV heads of 128), two layers, Q8_0
    cache: a 600-token prompt in ubatches of 512 and 88 (the matrix-core
    projections write float32 rows that a separate pass quantizes), then four
    single-token steps, whose QKV GEMV writes the token's K/V rows as
    float32 and whose decode attention quantizes them into the cell (the
    block whose chunk holds the cell)."""
    cfg = dict(tdf_synth.CONFIGS["llama8b"])
    cfg, w = make_weights(cfg, layers=2)
    prompt = tdf_synth.prompt(cfg, 0, 600)
    log("q8 cache at 8B widths")
    teacher_forced(cfg, w, 1024, prompt, 4, TOL_BF16, "q8_0", n_ubatch=512, label="kvq8-8b-2L")
