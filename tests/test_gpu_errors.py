"""Error paths of the C ABI on the device (llama.cpp walkthrough, "Steps
11-12": decode returns 0 on success, 1 when nothing could be done, and a
negative code on failure; creators return NULL).

Device allocation failures are injected from the host with tdf_fault_alloc
(the allocation is simply not made, as if the device were out of memory):
every kernel that runs still runs on valid memory.  After a failed call the
bookkeeping must be unchanged, and the context must go on to match the
oracle.
"""
import numpy as np
import pytest

import tdf_synth
from oracle import OracleContext

from gpu_common import TOL_BF16, check_logits, check_token, device_model, make_weights, oracle_model

pytestmark = pytest.mark.gpu

SMALL = dict(n_vocab=1000, n_embd=128, n_layer=2, n_head=8, n_head_kv=2, head_dim=32, n_ff=256,
             rms_eps=1e-5, rope_theta=10000.0, tied=False, weight_dtype="bf16", seed=11,
             weight_std=0.08, gain_std=0.1)


@pytest.fixture
def disarm():
    import transformer_decode_forward_amd as tdf
    yield
    tdf.tdf_fault_alloc(0)


@pytest.mark.parametrize("nth", [1, 2, 7, 15, 20])
def test_context_create_returns_null_on_allocation_failure(nth, disarm):
    import transformer_decode_forward_amd as tdf
    cfg, w = make_weights(SMALL)
    gm = device_model(cfg, w)
    tdf.tdf_fault_alloc(nth)
    with pytest.raises(RuntimeError, match="allocation failed"):
        tdf.Context(gm, n_ctx=256, n_ubatch=64, kv_dtype="bf16")
    tdf.tdf_fault_alloc(0)
    # the library is usable afterwards
    ctx = tdf.Context(gm, n_ctx=256, n_ubatch=64, kv_dtype="bf16")
    assert ctx.decode([1, 2, 3]) == 0


def test_decode_returns_alloc_error_and_changes_nothing(disarm):
    """A decode that needs more logits rows than the context holds grows the
    buffer first; when that allocation fails the call returns -2 before any
    cell is placed, and the same call then succeeds and matches the oracle."""
    import transformer_decode_forward_amd as tdf
    cfg, w = make_weights(SMALL)
    gm = device_model(cfg, w)
    ctx = tdf.Context(gm, n_ctx=256, n_ubatch=64, kv_dtype="bf16")
    oc = OracleContext(oracle_model(cfg, w), n_ctx=256, n_ubatch=64, kv_dtype="bf16")
    first = list(tdf_synth.prompt(cfg, 70, 10))
    assert ctx.decode(first) == 0 and oc.decode(first).status == 0
    toks = list(tdf_synth.prompt(cfg, 71, 40))
    flags = np.ones(40, np.int8)
    cells_before = [ctx.kv_cell(c) for c in range(64)]
    tdf.tdf_fault_alloc(1)
    assert ctx.decode(toks, logits=flags) == tdf.TDF_E_ALLOC
    assert "allocation failed" in tdf.tdf_last_error()
    tdf.tdf_fault_alloc(0)
    assert ctx.seq_pos_max(0) == 9
    assert [ctx.kv_cell(c) for c in range(64)] == cells_before
    assert ctx.decode(toks, logits=flags) == 0
    ro = oc.decode(toks, logits=flags)
    assert ctx.last_slots() == ro.slots and ctx.output_ids() == ro.out_index
    for r, i in enumerate(ro.out_index):
        check_logits(ctx.logits_ith(i), ro.logits[r], TOL_BF16, f"row {i}")
        check_token(ctx.argmax_ith(i), ro.logits[r], f"row {i}")


def test_invalid_and_full_calls_change_nothing_on_device():
    """-1 (invalid token) and 1 (no room) leave cells and positions as they
    were, and the next step still matches the oracle."""
    import transformer_decode_forward_amd as tdf
    cfg, w = make_weights(SMALL)
    gm = device_model(cfg, w)
    ctx = tdf.Context(gm, n_ctx=64, n_ubatch=64, kv_dtype="bf16")
    oc = OracleContext(oracle_model(cfg, w), n_ctx=64, n_ubatch=64, kv_dtype="bf16")
    prompt = list(tdf_synth.prompt(cfg, 72, 60))
    assert ctx.decode(prompt) == 0 and oc.decode(prompt).status == 0
    assert ctx.decode([1, 2, cfg["n_vocab"]]) == tdf.TDF_E_INVALID
    assert ctx.decode(list(range(5))) == tdf.TDF_NO_SLOT
    assert ctx.seq_pos_max(0) == 59
    ro = oc.decode([7])
    assert ctx.decode([7]) == 0
    assert ctx.last_slots() == ro.slots == [60]
    check_logits(ctx.logits_ith(0), ro.logits[0], TOL_BF16, "step after errors")
