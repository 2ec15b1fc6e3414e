"""GPU parity of cache removal and shift (Ollama engine page, "KV Cache:
memory for causal attention": the window slides forward by re-encoding the
cached keys' RoPE positions) against the float64 oracle; same tolerances as
test_gpu_parity, bookkeeping bit-exact."""
import numpy as np
import pytest

import tdf_synth
from oracle import OracleContext

from gpu_common import TOL_BF16, TOL_F32, check_logits, check_token, device_model, make_weights, oracle_model
from test_gpu_swa import SMALL64

pytestmark = pytest.mark.gpu


def _same_cells(gc, oc):
    for c in range(oc.n_ctx):
        p, m = gc.kv_cell(c)
        assert p == int(oc.cell_pos[c]) and m == int(oc.cell_seq[c]), c
    for s in range(oc.n_seq_max):
        assert gc.seq_pos_max(s) == oc.seq_pos_max(s)


def _pair(cfg, w, kv_dtype, **kw):
    import transformer_decode_forward_amd as tdf
    gc = tdf.Context(device_model(cfg, w), kv_dtype=kv_dtype, **kw)
    oc = OracleContext(oracle_model(cfg, w), kv_dtype=kv_dtype, **kw)
    return gc, oc


def _steps(gc, oc, toks, tol, label, seq_ids=None):
    for k, t in enumerate(toks):
        kw = {} if seq_ids is None else dict(seq_ids=seq_ids)
        t = [int(x) for x in np.atleast_1d(t)]
        assert gc.decode(t, **kw) == 0
        ro = oc.decode(t, **kw)
        assert gc.last_slots() == ro.slots, (label, k)
        for r, i in enumerate(ro.out_index):
            check_logits(gc.logits_ith(i), ro.logits[r], tol, f"{label} step {k} row {i}")
            check_token(gc.argmax_ith(i), ro.logits[r], f"{label} step {k} row {i}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "f16"])
def test_drop_and_shift_down_then_decode(kv_dtype):
    """100-token prompt, drop positions [0, 30), shift the rest down by 30,
    then 5 steps (the re-rotated keys are read by every later token)."""
    cfg, w = make_weights(SMALL64)
    gc, oc = _pair(cfg, w, kv_dtype, n_ctx=256, n_ubatch=64)
    prompt = tdf_synth.prompt(cfg, 0, 100)
    assert gc.decode(prompt) == 0 and oc.decode(prompt).status == 0
    assert gc.kv_seq_rm(0, 0, 30) == oc.kv_seq_rm(0, 0, 30) == 0
    assert gc.kv_seq_shift(0, 30, -1, -30) == oc.kv_seq_shift(0, 30, -1, -30) == 0
    _same_cells(gc, oc)
    _steps(gc, oc, tdf_synth.prompt(cfg, 1, 5), TOL_BF16, f"shift {kv_dtype}")
    _same_cells(gc, oc)


def test_shift_up_middle_range_and_multi_sequence():
    """Two sequences: sequence 1 loses a middle range, its tail moves up by
    40; sequence 0 is untouched; lock-step decode of both."""
    cfg, w = make_weights(SMALL64)
    gc, oc = _pair(cfg, w, "bf16", n_ctx=256, n_ubatch=64, n_seq_max=2)
    for s, n in ((0, 50), (1, 70)):
        toks = tdf_synth.prompt(cfg, 2 + s, n)
        assert gc.decode(toks, seq_ids=[[s]] * n) == 0 and oc.decode(toks, seq_ids=[[s]] * n).status == 0
    assert gc.kv_seq_rm(1, 20, 35) == oc.kv_seq_rm(1, 20, 35) == 0
    assert gc.kv_seq_shift(1, 35, -1, 40) == oc.kv_seq_shift(1, 35, -1, 40) == 0
    assert gc.kv_seq_shift(1, 0, 20, 60) == oc.kv_seq_shift(1, 0, 20, 60) == -1  # would pass later cells
    _same_cells(gc, oc)
    toks = tdf_synth.prompt(cfg, 9, 8).reshape(4, 2)
    for k in range(4):
        calls = dict(tokens=[int(x) for x in toks[k]], seq_ids=[[0], [1]], logits=np.ones(2, np.int8))
        assert gc.decode(**calls) == 0
        ro = oc.decode(**calls)
        assert gc.last_slots() == ro.slots
        for r, i in enumerate(ro.out_index):
            check_logits(gc.logits_ith(i), ro.logits[r], TOL_BF16, f"multiseq step {k} row {i}")
    _same_cells(gc, oc)


def test_fp32_shift():
    cfg = tdf_synth.CONFIGS["tiny"]
    cfg, w = make_weights(cfg)
    gc, oc = _pair(cfg, w, "f32", n_ctx=64)
    prompt = tdf_synth.prompt(cfg, 0, 20)
    assert gc.decode(prompt) == 0 and oc.decode(prompt).status == 0
    assert gc.kv_seq_rm(0, 0, 7) == oc.kv_seq_rm(0, 0, 7) == 0
    assert gc.kv_seq_shift(0, 7, -1, -7) == oc.kv_seq_shift(0, 7, -1, -7) == 0
    _steps(gc, oc, tdf_synth.prompt(cfg, 1, 6), TOL_F32, "f32 shift")


def test_sliding_context_loop():
    """A 96-cell cache filled by a 90-token prompt; 40 greedy steps, and
    whenever the cache is full both sides drop the oldest 24 positions and
    shift the rest down (graph-replayed steps between slides)."""
    cfg, w = make_weights(SMALL64)
    gc, oc = _pair(cfg, w, "bf16", n_ctx=96, n_ubatch=64)
    prompt = tdf_synth.prompt(cfg, 5, 90)
    assert gc.decode(prompt) == 0
    ro = oc.decode(prompt)
    nxt = int(ro.tokens[0])
    slides = 0
    for k in range(40):
        rg = gc.decode([nxt])
        if rg == 1:
            assert oc.decode([nxt]).status == 1
            top = oc.seq_pos_max(0)
            lo = top - (96 - 24) + 1
            assert gc.kv_seq_rm(0, 0, lo) == oc.kv_seq_rm(0, 0, lo) == 0
            assert gc.kv_seq_shift(0, lo, -1, -lo) == oc.kv_seq_shift(0, lo, -1, -lo) == 0
            slides += 1
            rg = gc.decode([nxt])
        assert rg == 0
        ro = oc.decode([nxt])
        assert gc.last_slots() == ro.slots
        check_logits(gc.logits_ith(0), ro.logits[0], TOL_BF16, f"slide step {k}")
        check_token(gc.argmax_ith(0), ro.logits[0], f"slide step {k}")
        nxt = int(ro.tokens[0])
    assert slides >= 1
    _same_cells(gc, oc)
