"""Pins of the oracle's cache shift and removal (Ollama engine page, "KV
Cache: memory for causal attention": when the cache is full the model's
shift function re-encodes the cached keys' RoPE positions so that the window
slides forward).  Pins:

* RoPE rotations compose: rotating a key stored at position p by delta gives
  the key of position p + delta (closed form, any delta);
* shifting a whole sequence by delta changes no later logits compared with a
  context that saw the same tokens at positions offset by delta (attention
  depends on position differences only);
* shifting by delta and back restores the cache and the logits;
* after removing a position range, decoding sees exactly the remaining cells
  (equal to a fresh context holding those cells' K/V);
* bookkeeping: freed cells are reused, shared cells keep their other
  sequences, invalid shifts change nothing.
"""
import numpy as np
import pytest

import tdf_synth
from oracle import OracleContext, OracleModel
from oracle.ops import rope

CFG = dict(tdf_synth.CONFIGS["tiny"])


@pytest.fixture(scope="module")
def w():
    return tdf_synth.make_all(CFG)


def _ctx(w, n_ctx=64, **kw):
    return OracleContext(OracleModel(tdf_synth.hparams(CFG), w), n_ctx=n_ctx, **kw)


def test_rope_rotations_compose():
    rng = np.random.default_rng(0)
    k = rng.normal(size=(5, 3, 16))
    for a, b in [(0, 7), (13, -5), (1000, 2345), (-40, 40)]:
        two = rope(rope(k, np.full(5, a), 1e4), np.full(5, b), 1e4)
        np.testing.assert_allclose(two, rope(k, np.full(5, a + b), 1e4), rtol=0, atol=1e-9)


@pytest.mark.parametrize("delta", [7, -3])
def test_shift_equals_offset_positions(w, delta):
    toks = tdf_synth.prompt(CFG, 0, 10)
    nxt = [int(t) for t in tdf_synth.prompt(CFG, 1, 3)]
    start = 3  # so that a shift by -3 keeps positions >= 0
    a = _ctx(w)
    assert a.decode(toks, pos=list(range(start, start + 10))).status == 0
    assert a.kv_seq_shift(0, 0, -1, delta) == 0
    assert a.seq_pos_max(0) == start + 9 + delta
    b = _ctx(w)
    assert b.decode(toks, pos=list(range(start + delta, start + delta + 10))).status == 0
    for t in nxt:
        ra, rb = a.decode([t]), b.decode([t])
        np.testing.assert_allclose(ra.logits, rb.logits, rtol=0, atol=1e-9)


def test_shift_and_back_restores(w):
    toks = tdf_synth.prompt(CFG, 2, 12)
    a, b = _ctx(w), _ctx(w)
    assert a.decode(toks).status == 0 and b.decode(toks).status == 0
    k0 = a.k_cache[1].copy()
    assert a.kv_seq_shift(0, 4, 9, 20) == -1  # would jump over positions 9..11
    assert a.kv_seq_shift(0, 0, -1, 20) == 0 and a.kv_seq_shift(0, 20, -1, -20) == 0
    np.testing.assert_allclose(a.k_cache[1], k0, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(a.cell_pos, b.cell_pos)
    np.testing.assert_allclose(a.decode([9]).logits, b.decode([9]).logits, rtol=0, atol=1e-10)


def test_removed_cells_are_invisible(w):
    """Remove positions [0, 5) of 12, decode: equals a fresh context that
    holds the 7 remaining cells' K/V at the same positions."""
    toks = tdf_synth.prompt(CFG, 3, 12)
    a = _ctx(w)
    assert a.decode(toks).status == 0
    keep = np.flatnonzero(a.cell_pos >= 5)
    L = CFG["n_layer"]
    ks = [a.k_cache[l][keep].copy() for l in range(L)]
    vs = [a.v_cache[l][keep].copy() for l in range(L)]
    assert a.kv_seq_rm(0, 0, 5) == 0
    assert a.n_free() == 64 - 7 and a.seq_pos_max(0) == 11
    b = _ctx(w)
    assert b.kv_import(0, 5, 12, ks, vs) == 0
    np.testing.assert_allclose(a.decode([42]).logits, b.decode([42]).logits, rtol=0, atol=1e-12)


def test_context_shift_pattern(w):
    """The sliding step: drop the oldest 6 positions, shift the rest down by
    6, continue; the next token lands at position n - 6 and freed cells are
    reused from the lowest index."""
    toks = tdf_synth.prompt(CFG, 4, 16)
    a = _ctx(w, n_ctx=16)
    assert a.decode(toks).status == 0
    assert a.decode([1]).status == 1  # full
    assert a.kv_seq_rm(0, 0, 6) == 0 and a.kv_seq_shift(0, 6, -1, -6) == 0
    assert a.seq_pos_max(0) == 9
    r = a.decode([1, 2])
    assert r.status == 0 and r.positions == [10, 11] and r.slots == [0, 1]


def test_bookkeeping_rules(w):
    c = _ctx(w, n_seq_max=3)
    assert c.decode([1, 2, 3, 4], seq_ids=[[0, 1], [0, 1], [0], [1]]).status == 0
    # shared cells: removal from one sequence keeps them for the other
    assert c.kv_seq_rm(0, 0, 2) == 0
    assert c.n_free() == 64 - 4 and c.seq_pos_max(0) == 2 and c.seq_pos_max(1) == 2
    assert c.kv_seq_rm(1, 0, 1) == 0 and c.n_free() == 64 - 3
    # a shift may not move a cell that another sequence also holds
    c2 = _ctx(w, n_seq_max=2)
    assert c2.decode([1, 2], seq_ids=[[0, 1], [0]]).status == 0
    before = c2.cell_pos.copy()
    assert c2.kv_seq_shift(0, 0, -1, 5) == -1
    np.testing.assert_array_equal(c2.cell_pos, before)
    # negative positions, bad ranges and sequence ids are invalid
    assert c2.kv_seq_shift(0, 1, -1, -5) == -1
    assert c2.kv_seq_rm(5, 0, -1) == -1 and c2.kv_seq_rm(0, 3, 1) == -1
