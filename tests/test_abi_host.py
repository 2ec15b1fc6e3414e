"""The C-ABI library loads, exports what include/tdf.h declares, and its host
bookkeeping (run through bookkeeping-only contexts: no device memory, no
kernels) matches the oracle's independent bookkeeping bit for bit:
positions, cells, per-cell (position, sequences), seq_pos_max, output rows
and return codes."""
import ctypes

import numpy as np
import pytest

import transformer_decode_forward_amd as tdf
from oracle import OracleContext, OracleModel

HP = dict(n_vocab=100, n_embd=64, n_layer=2, n_head=4, n_head_kv=2, head_dim=16, n_ff=128,
          rms_eps=1e-5, rope_theta=10000.0, tied=False, weight_dtype="bf16")


def test_library_exports_every_declared_symbol():
    L = tdf.lib()
    names = tdf.header_symbols()
    assert "tdf_decode" in names and "tdf_model_create" in names
    for n in names:
        assert hasattr(L, n), n
        ctypes.cast(getattr(L, n), ctypes.c_void_p)


def test_model_create_rejects_bad_hparams():
    bad = dict(HP, n_head=3)
    with pytest.raises(RuntimeError):
        tdf.Model(bad, dry_run=True)
    with pytest.raises(RuntimeError):
        tdf.Model(dict(HP, head_dim=12), dry_run=True)


def test_context_create_rejects_bad_params():
    m = tdf.Model(HP, dry_run=True)
    with pytest.raises(RuntimeError):
        tdf.Context(m, n_ctx=16, n_seq_max=65, dry_run=True)
    with pytest.raises(RuntimeError):
        tdf.Context(m, n_ctx=0, dry_run=True)


def pair(n_ctx=64, n_ubatch=5, n_seq_max=4, output_all=False, n_batch=None):
    m = tdf.Model(HP, dry_run=True)
    g = tdf.Context(m, n_ctx=n_ctx, n_batch=n_batch, n_ubatch=n_ubatch, n_seq_max=n_seq_max,
                    output_all=output_all, dry_run=True)
    o = OracleContext(OracleModel(HP, {}), n_ctx=n_ctx, n_batch=n_batch, n_ubatch=n_ubatch,
                      n_seq_max=n_seq_max, output_all=output_all, compute=False)
    return g, o


def assert_same_state(g, o, n_seq_max):
    for c in range(o.n_ctx):
        p, m = g.kv_cell(c)
        assert p == int(o.cell_pos[c]) and m == int(o.cell_seq[c]), c
    for s in range(n_seq_max):
        assert g.seq_pos_max(s) == o.seq_pos_max(s)


def test_defaults_match_oracle():
    g, o = pair()
    for toks in ([1, 2, 3], [4], [5, 6]):
        assert g.decode(toks) == 0
        r = o.decode(toks)
        assert g.last_slots() == r.slots
        assert g.output_ids() == r.out_index
    assert_same_state(g, o, 4)


@pytest.mark.parametrize("seed", range(6))
def test_random_scripts_match_oracle(seed):
    rng = np.random.default_rng(seed)
    n_seq = int(rng.integers(1, 6))
    g, o = pair(n_ctx=int(rng.integers(20, 80)), n_ubatch=int(rng.integers(1, 9)), n_seq_max=n_seq,
                output_all=bool(rng.integers(0, 2)), n_batch=int(rng.integers(8, 30)))
    for step in range(25):
        n = int(rng.integers(1, 12))
        toks = rng.integers(-2 if step % 7 == 6 else 0, 100, size=n)
        kw = {}
        if rng.random() < 0.6:
            kw["seq_ids"] = [list(rng.choice(n_seq, size=int(rng.integers(1, min(3, n_seq) + 1)), replace=False))
                             for _ in range(n)]
        if rng.random() < 0.3:
            kw["logits"] = rng.integers(0, 2, size=n)
        if rng.random() < 0.2:
            # explicit positions: sometimes valid, sometimes not
            base = max([o.seq_pos_max(s) for s in range(n_seq)]) + 1
            kw["pos"] = base + np.cumsum(rng.integers(0 if rng.random() < 0.3 else 1, 3, size=n))
        rg = g.decode(list(toks), **kw)
        ro = o.decode(list(toks), **kw)
        assert rg == ro.status, (step, rg, ro.status, tdf.tdf_last_error())
        if ro.status == 0:
            assert g.last_slots() == ro.slots
            assert g.output_ids() == ro.out_index
            assert g.n_outputs() == len(ro.out_index)
        assert_same_state(g, o, n_seq)


def test_error_codes_and_full_cache():
    g, o = pair(n_ctx=8, n_ubatch=8, n_seq_max=2)
    assert g.decode([1, 100]) == tdf.TDF_E_INVALID        # token id == n_vocab
    assert "invalid token" in tdf.tdf_last_error()
    assert g.decode([1], seq_ids=[[2]]) == tdf.TDF_E_INVALID
    assert g.decode([1, 2], pos=[4, 4]) == tdf.TDF_E_INVALID
    assert g.decode(list(range(6))) == 0
    assert g.decode([1, 2, 3]) == tdf.TDF_NO_SLOT           # nothing changed
    assert g.seq_pos_max(0) == 5
    assert g.decode([1, 2]) == 0
    assert g.kv_clear() == 0 and g.seq_pos_max(0) == -1
    assert g.decode([7]) == 0 and g.last_slots() == [0]


def test_kv_import_bookkeeping_matches_oracle():
    g, o = pair(n_ctx=32, n_seq_max=2)
    assert g.decode([1, 2, 3], seq_ids=[[1]] * 3) == 0
    o.decode([1, 2, 3], seq_ids=[[1]] * 3)
    assert g.kv_import(0, 4, 10, [], []) == 0
    assert o.kv_import(0, 4, 14, None, None) == 0
    assert g.last_slots() == list(o.last_import_cells)
    assert g.kv_import(0, 5, 3, [], []) == tdf.TDF_E_INVALID  # must follow position 13
    assert g.kv_import(1, 3, 40, [], []) == tdf.TDF_NO_SLOT
    assert_same_state(g, o, 2)
    assert g.decode([9], seq_ids=[[0]]) == 0
    assert o.decode([9], seq_ids=[[0]]).positions == [14]
    assert_same_state(g, o, 2)


def test_time_op_rejects_bookkeeping_contexts_and_bad_ops():
    """The measurement hook launches nothing on a bookkeeping-only context and
    checks its operation and row count before any launch."""
    m = tdf.Model(HP, dry_run=True)
    c = tdf.Context(m, n_ctx=32, dry_run=True)
    for op, n, reps in (("gate_up", 1, 4), ("qkv", 1, 4), ("down", 0, 4), ("lm_head", 1, 0)):
        with pytest.raises(RuntimeError, match=r"\(-1\)"):
            c.time_op(op, n, reps)


def test_window_hparams_accepted_and_checked():
    tdf.Model(dict(HP, n_swa=8, swa_layers=[1] * HP["n_layer"]), dry_run=True)
    tdf.Model(dict(HP, n_swa=8), dry_run=True)
    with pytest.raises(Exception):
        tdf.Model(dict(HP, n_swa=-1), dry_run=True)


def test_q8_0_weights_accepted_and_sizes_checked():
    """Q8_0 blocks are 32 elements of a row: every inner size must be a
    multiple of 32 (n_embd, n_head*head_dim, n_ff)."""
    tdf.Model(dict(HP, weight_dtype="q8_0"), dry_run=True)
    for bad in (dict(n_embd=48), dict(n_ff=144), dict(n_head=1, n_head_kv=1)):
        with pytest.raises(RuntimeError, match="multiples of 32"):
            tdf.Model(dict(HP, weight_dtype="q8_0", **bad), dry_run=True)


def test_q8_0_cache_needs_head_dim_multiple_of_32():
    m16 = tdf.Model(HP, dry_run=True)  # head_dim 16
    with pytest.raises(RuntimeError):
        tdf.Context(m16, n_ctx=16, kv_dtype="q8_0", dry_run=True)
    m32 = tdf.Model(dict(HP, head_dim=32), dry_run=True)
    tdf.Context(m32, n_ctx=16, kv_dtype="q8_0", dry_run=True)


@pytest.mark.parametrize("seed", range(6))
def test_random_scripts_with_removal_and_shift_match_oracle(seed):
    """Decode calls interleaved with range removals and shifts (valid and
    invalid): return codes, cells and positions bit-exact with the oracle."""
    rng = np.random.default_rng(100 + seed)
    n_seq = int(rng.integers(1, 4))
    g, o = pair(n_ctx=int(rng.integers(16, 48)), n_ubatch=int(rng.integers(1, 9)), n_seq_max=n_seq,
                n_batch=int(rng.integers(8, 20)))
    for step in range(40):
        r = rng.random()
        s = int(rng.integers(0, n_seq + (1 if step % 11 == 10 else 0)))  # sometimes an invalid id
        if r < 0.5:
            n = int(rng.integers(1, 8))
            kw = {}
            if rng.random() < 0.5:
                kw["seq_ids"] = [list(rng.choice(n_seq, size=int(rng.integers(1, min(2, n_seq) + 1)),
                                                 replace=False)) for _ in range(n)]
            toks = list(rng.integers(0, 100, size=n))
            rg, ro = g.decode(toks, **kw), o.decode(toks, **kw).status
            if ro == 0:
                pass
        elif r < 0.75:
            top = max(0, o.seq_pos_max(min(s, n_seq - 1)))
            p0 = int(rng.integers(0, top + 2))
            p1 = -1 if rng.random() < 0.3 else int(rng.integers(p0 - 1, top + 3))
            rg, ro = g.kv_seq_rm(s, p0, p1), o.kv_seq_rm(s, p0, p1)
        else:
            top = max(0, o.seq_pos_max(min(s, n_seq - 1)))
            p0 = int(rng.integers(0, top + 2))
            p1 = -1 if rng.random() < 0.5 else int(rng.integers(p0, top + 3))
            delta = int(rng.integers(-top - 2, top + 3))
            rg, ro = g.kv_seq_shift(s, p0, p1, delta), o.kv_seq_shift(s, p0, p1, delta)
        assert rg == ro, (step, r, rg, ro, tdf.tdf_last_error())
        assert_same_state(g, o, n_seq)
    # the device-side lists were rewritten after removals: placements still agree
    assert g.decode([1]) == o.decode([1]).status
