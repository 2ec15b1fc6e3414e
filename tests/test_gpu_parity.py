"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
the same seeded inputs, the oracle's cache holding K/V in the same element
type as the GPU context's cache.

Logits: max-abs <= 3e-2 and rel-L2 <= 1e-2 for bf16 weights; 1e-4 / 1e-5 for
the float32 model.  Greedy tokens: equal wherever the oracle's top-2 gap
exceeds 5e-2.  Cells, positions and output rows: bit-exact.  Decode steps
are teacher-forced with the oracle's token so that one near-tie cannot make
the two sides diverge.
"""
import numpy as np
import pytest

import tdf_synth
from oracle import OracleContext

from gpu_common import (TOL_BF16, TOL_F32, check_logits, check_token, device_model, log, make_weights,
                        oracle_model)

pytestmark = pytest.mark.gpu

# small bf16 model whose sizes exercise the MFMA path (multiples of 64), two
# KV heads per query-head group of 4, and a vocabulary that is not a power of 2
SMALL = dict(n_vocab=1000, n_embd=128, n_layer=2, n_head=8, n_head_kv=2, head_dim=32, n_ff=256,
             rms_eps=1e-5, rope_theta=10000.0, tied=False, weight_dtype="bf16", seed=11,
             weight_std=0.08, gain_std=0.1)


def run_pair(cfg, tensors, ctx_kw, calls, tol, kv_dtype, label):
    """Run the same decode calls on both sides; compare everything."""
    import transformer_decode_forward_amd as tdf
    gm = device_model(cfg, tensors)
    gc = tdf.Context(gm, kv_dtype=kv_dtype, **ctx_kw)
    oc = OracleContext(oracle_model(cfg, tensors), kv_dtype=kv_dtype, **ctx_kw)
    for k, call in enumerate(calls):
        call = dict(call)
        rg = gc.decode(**call)
        ro = oc.decode(**call)
        assert rg == ro.status == 0, (label, k, rg, tdf.tdf_last_error())
        assert gc.last_slots() == ro.slots, (label, k)
        assert gc.output_ids() == ro.out_index, (label, k)
        for r, i in enumerate(ro.out_index):
            got = gc.logits_ith(i)
            check_logits(got, ro.logits[r], tol, f"{label} call {k} row {i}")
            check_token(gc.argmax_ith(i), ro.logits[r], f"{label} call {k} row {i}")
    return gc, oc


def teacher_forced(cfg, tensors, n_ctx, prompt, steps, tol, kv_dtype, n_ubatch=512, label=""):
    import transformer_decode_forward_amd as tdf
    gm = device_model(cfg, tensors)
    gc = tdf.Context(gm, n_ctx=n_ctx, n_ubatch=n_ubatch, kv_dtype=kv_dtype)
    oc = OracleContext(oracle_model(cfg, tensors), n_ctx=n_ctx, n_ubatch=n_ubatch, kv_dtype=kv_dtype)
    assert gc.decode(prompt) == 0, tdf.tdf_last_error()
    ro = oc.decode(prompt)
    assert gc.last_slots() == ro.slots
    errs = [check_logits(gc.logits_ith(len(prompt) - 1), ro.logits[0], tol, f"{label} prefill")]
    check_token(gc.argmax_ith(len(prompt) - 1), ro.logits[0], f"{label} prefill")
    nxt = int(ro.tokens[0])
    for step in range(steps):
        assert gc.decode([nxt]) == 0, tdf.tdf_last_error()
        ro = oc.decode([nxt])
        assert gc.last_slots() == ro.slots
        assert gc.seq_pos_max(0) == oc.seq_pos_max(0)
        errs.append(check_logits(gc.logits_ith(0), ro.logits[0], tol, f"{label} step {step}"))
        check_token(gc.argmax_ith(0), ro.logits[0], f"{label} step {step}")
        nxt = int(ro.tokens[0])
    log(f"{label}: worst max-abs {max(e[0] for e in errs):.2e}, worst rel-L2 {max(e[1] for e in errs):.2e}")
    return errs


def test_tiny_fp32_workload():
    """16-token prompt in one ubatch, then 16 greedy steps; fp32 weights and cache."""
    cfg = tdf_synth.CONFIGS["tiny"]
    cfg, w = make_weights(cfg)
    prompt = tdf_synth.prompt(cfg, 0, cfg["prompt_len"])
    teacher_forced(cfg, w, cfg["n_ctx"], prompt, cfg["decode_steps"], TOL_F32, "f32", label="tiny")


@pytest.mark.parametrize("kv_dtype", ["bf16", "f16", "f32"])
def test_small_prefill_ragged_ubatches_all_rows(kv_dtype):
    """150 tokens in ubatches of 64, 64, 22 (two MFMA ubatches, one GEMV
    ubatch), logits for every row, then three single-token steps."""
    cfg, w = make_weights(SMALL)
    prompt = tdf_synth.prompt(cfg, 0, 150)
    nxt = tdf_synth.prompt(cfg, 1, 3)
    calls = [dict(tokens=prompt)] + [dict(tokens=[int(t)]) for t in nxt]
    run_pair(cfg, w, dict(n_ctx=256, n_ubatch=64, output_all=True), calls, TOL_BF16, kv_dtype, "small")


def test_small_selected_rows_and_no_rows():
    cfg, w = make_weights(SMALL)
    prompt = tdf_synth.prompt(cfg, 0, 100)
    flags = np.zeros(100, dtype=np.int8)
    flags[[0, 37, 64, 99]] = 1
    calls = [dict(tokens=prompt[:40], logits=np.zeros(40, dtype=np.int8)),
             dict(tokens=prompt[40:], logits=flags[40:]),
             dict(tokens=[5])]
    run_pair(cfg, w, dict(n_ctx=128, n_ubatch=48), calls, TOL_BF16, "bf16", "rows")


def test_small_multi_sequence_batches():
    """Three interleaved sequences in one batch, then lock-step steps of one
    token per sequence (each with its own position and sequence id)."""
    cfg, w = make_weights(SMALL)
    rng = np.random.default_rng(3)
    seqs = [int(s) for s in rng.integers(0, 3, size=120)]
    toks = tdf_synth.prompt(cfg, 0, 120)
    calls = [dict(tokens=toks, seq_ids=[[s] for s in seqs], logits=np.ones(120, dtype=np.int8))]
    for step in range(3):
        calls.append(dict(tokens=tdf_synth.prompt(cfg, 10 + step, 3), seq_ids=[[0], [1], [2]],
                          logits=np.ones(3, dtype=np.int8)))
    run_pair(cfg, w, dict(n_ctx=200, n_ubatch=50, n_seq_max=4), calls, TOL_BF16, "bf16", "multiseq")


def test_small_kv_import_then_decode():
    """Restore 300 positions of post-RoPE K/V (N(0,1) bf16), then decode."""
    import transformer_decode_forward_amd as tdf
    from transformer_decode_forward_amd.device import to_device
    cfg, w = make_weights(SMALL)
    L, P = cfg["n_layer"], 300
    ks = [tdf_synth.kv_fill(cfg, l, "k", 0, P, "bf16") for l in range(L)]
    vs = [tdf_synth.kv_fill(cfg, l, "v", 0, P, "bf16") for l in range(L)]
    gm = device_model(cfg, w)
    gc = tdf.Context(gm, n_ctx=512, kv_dtype="bf16")
    kd = [to_device(k) for k in ks]
    vd = [to_device(v) for v in vs]
    assert gc.kv_import(0, 0, P, [t.data_ptr() for t in kd], [t.data_ptr() for t in vd]) == 0
    oc = OracleContext(oracle_model(cfg, w), n_ctx=512, kv_dtype="bf16")
    assert oc.kv_import(0, 0, P, ks, vs) == 0
    for t in tdf_synth.prompt(cfg, 2, 3):
        assert gc.decode([int(t)]) == 0
        ro = oc.decode([int(t)])
        assert gc.last_slots() == ro.slots
        check_logits(gc.logits_ith(0), ro.logits[0], TOL_BF16, "import")


def test_llama1b_width_two_layers():
    """1B-class widths (d 2048, 32/8 heads of 64, ffn 8192, vocab 128256),
    two layers: 512-token prompt in one ubatch, then 4 steps."""
    cfg = dict(tdf_synth.CONFIGS["llama1b"])
    cfg, w = make_weights(cfg, layers=2)
    prompt = tdf_synth.prompt(cfg, 0, 512)
    teacher_forced(cfg, w, 1024, prompt, 4, TOL_BF16, "f16", label="1b-2L")


def test_llama8b_width_two_layers():
    """8B-class widths, two layers: 2048-token prompt in ubatches of 512,
    logits for the last position only, then 3 steps."""
    cfg = dict(tdf_synth.CONFIGS["llama8b"])
    cfg, w = make_weights(cfg, layers=2)
    prompt = tdf_synth.prompt(cfg, 0, 2048)
    teacher_forced(cfg, w, 4096, prompt, 3, TOL_BF16, "bf16", label="8b-2L")


def test_graph_replay_matches_eager_launches(monkeypatch):
    """Decode steps replayed from captured HIP graphs give the same logits as
    plain launches, over a context that grows across several attention grid
    sizes (replays interleaved with eager host work and synchronisations)."""
    import transformer_decode_forward_amd as tdf
    cfg, w = make_weights(SMALL)
    gm = device_model(cfg, w)
    monkeypatch.setenv("TDF_NO_GRAPH", "1")
    eager = tdf.Context(gm, n_ctx=1024, n_ubatch=64, kv_dtype="bf16")
    monkeypatch.delenv("TDF_NO_GRAPH")
    graphed = tdf.Context(gm, n_ctx=1024, n_ubatch=64, kv_dtype="bf16")
    prompt = tdf_synth.prompt(cfg, 0, 200)
    assert eager.decode(prompt) == 0 and graphed.decode(prompt) == 0
    toks = tdf_synth.prompt(cfg, 1, 80)
    for i, t in enumerate(toks):
        assert eager.decode([int(t)]) == 0 and graphed.decode([int(t)]) == 0
        a, b = eager.logits_ith(0), graphed.logits_ith(0)
        assert np.array_equal(a, b), (i, float(np.max(np.abs(a - b))))
        assert eager.argmax_ith(0) == graphed.argmax_ith(0)
    cap, rep = graphed.graph_counts()
    assert rep >= 70 and cap >= 1, (cap, rep)
    assert eager.graph_counts() == (0, 0)


def test_graph_key_tracks_list_writes_of_earlier_ubatches(monkeypatch):
    """A replayed tail ubatch must scatter its own cell-list writes.  The
    writes of a call's ubatches are packed one after the other, so the tail's
    writes start later when the first ubatch's tokens belong to two
    sequences.  Call A: 64 + 20 tokens of sequence 0.  Call B: 64 tokens of
    sequences {1, 2}, then 20 tokens of sequence 1: the tail has the same
    size, rows and attention split as call A's, but its writes sit at another
    offset.  Both calls' logits must match the oracle and plain launches."""
    import transformer_decode_forward_amd as tdf
    cfg, w = make_weights(SMALL)
    gm = device_model(cfg, w)
    kw = dict(n_ctx=512, n_ubatch=64, n_seq_max=3)
    monkeypatch.setenv("TDF_NO_GRAPH", "1")
    eager = tdf.Context(gm, kv_dtype="bf16", **kw)
    monkeypatch.delenv("TDF_NO_GRAPH")
    graphed = tdf.Context(gm, kv_dtype="bf16", **kw)
    oc = OracleContext(oracle_model(cfg, w), kv_dtype="bf16", **kw)
    calls = [dict(tokens=tdf_synth.prompt(cfg, 60, 84)),
             dict(tokens=tdf_synth.prompt(cfg, 61, 84), seq_ids=[[1, 2]] * 64 + [[1]] * 20)]
    for k, call in enumerate(calls):
        assert eager.decode(**call) == 0 and graphed.decode(**call) == 0, tdf.tdf_last_error()
        ro = oc.decode(**call)
        assert graphed.last_slots() == eager.last_slots() == ro.slots
        a, b = eager.logits_ith(83), graphed.logits_ith(83)
        assert np.array_equal(a, b), (k, float(np.max(np.abs(a - b))))
        check_logits(b, ro.logits[0], TOL_BF16, f"call {k}")
        check_token(graphed.argmax_ith(83), ro.logits[0], f"call {k}")
    # the two tails were captured separately
    assert graphed.graph_counts()[0] == 2
    # sequence 2 holds only the shared first ubatch: a step on it sees those cells
    step = dict(tokens=[5], seq_ids=[[2]])
    assert graphed.decode(**step) == 0
    ro = oc.decode(**step)
    assert ro.positions == [64]
    check_logits(graphed.logits_ith(0), ro.logits[0], TOL_BF16, "seq 2 step")


@pytest.mark.parametrize("kv_dtype", ["bf16", "f16"])
def test_mid_size_ubatches_matrix_cores_streaming(kv_dtype):
    """Ubatches of 9..32 tokens (several sequences' decode steps) run the
    matrix-core path that streams the weights once (K split into partial
    sums, then the epilogue): 1B-class widths, two layers, three sequences
    prefilled, then steps of 12, 24 and 32 tokens with every row's logits."""
    cfg = dict(tdf_synth.CONFIGS["llama1b"])
    cfg, w = make_weights(cfg, layers=2)
    calls = []
    for s in range(3):
        toks = tdf_synth.prompt(cfg, 40 + s, 70 + 30 * s)
        calls.append(dict(tokens=toks, seq_ids=[[s]] * len(toks)))
    for k, n in enumerate((12, 24, 32)):
        calls.append(dict(tokens=tdf_synth.prompt(cfg, 50 + k, n), seq_ids=[[j % 3] for j in range(n)],
                          logits=np.ones(n, dtype=np.int8)))
    run_pair(cfg, w, dict(n_ctx=512, n_ubatch=64, n_seq_max=3), calls, TOL_BF16, kv_dtype, "mid ubatch")


def _lock_step_calls(cfg, n_seq, seed, base_len, step_len):
    """n_seq sequences prefilled in their own calls, then two lock-step steps
    of one token per sequence, a step whose three tokens share sequences, and
    one more lock-step step; every row's logits in the steps."""
    calls = [dict(tokens=tdf_synth.prompt(cfg, seed + q, base_len + step_len * q), seq_ids=[[q]] * (base_len + step_len * q))
             for q in range(n_seq)]
    lock = lambda k: dict(tokens=[int(x) for x in tdf_synth.prompt(cfg, seed + 100 + k, n_seq)],
                          seq_ids=[[q] for q in range(n_seq)], logits=np.ones(n_seq, dtype=np.int8))
    calls += [lock(0), lock(1)]
    calls.append(dict(tokens=[int(x) for x in tdf_synth.prompt(cfg, seed + 150, 3)], seq_ids=[[1], [1], [n_seq - 1]],
                      logits=np.ones(3, dtype=np.int8)))
    calls.append(lock(2))
    return calls


@pytest.mark.parametrize("kv_dtype,hd", [("bf16", 64), ("f16", 64), ("bf16", 128)], ids=["bf16-hd64", "f16-hd64", "bf16-hd128"])
def test_lock_step_one_token_per_sequence(kv_dtype, hd):
    """12 sequences (prompts of 20..119 tokens, ubatches of 64), then
    lock-step steps of 12 tokens, one per sequence (the 9..32-token
    matrix-core projections with their K-split epilogue passes, the decode
    attention over 12 separate cell lists), with a step whose tokens share a
    sequence between them; every row's logits."""
    from test_gpu_swa import SMALL64
    cfg0 = SMALL64 if hd == 64 else dict(SMALL, n_embd=256, n_head=8, n_head_kv=2, head_dim=128, n_ff=256, seed=41)
    cfg, w = make_weights(cfg0)
    log(f"lock-step, one token per sequence: {kv_dtype} cache, head_dim {hd}")
    run_pair(cfg, w, dict(n_ctx=2048, n_ubatch=64, n_seq_max=16), _lock_step_calls(cfg, 12, 300, 20, 9), TOL_BF16,
             kv_dtype, f"lockstep-{kv_dtype}-hd{hd}")


def test_llama8b_width_lock_step_one_token_per_sequence():
    """8B widths (32 query heads, 8 KV heads of 128), two layers: 16
    sequences of 40..115 tokens, then lock-step steps of 16 tokens, one per
    sequence (the 9..32-token projections at full width), with a
    shared-sequence step between them; every row's logits."""
    cfg = dict(tdf_synth.CONFIGS["llama8b"])
    cfg, w = make_weights(cfg, layers=2)
    log("8B widths, 16 lock-step sequences")
    run_pair(cfg, w, dict(n_ctx=2560, n_ubatch=512, n_seq_max=16), _lock_step_calls(cfg, 16, 400, 40, 5), TOL_BF16,
             "bf16", "lockstep-8b-2L")
