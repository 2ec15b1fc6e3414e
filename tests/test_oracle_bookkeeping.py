"""Pins of the oracle's batch intake, ubatch split and KV-cell bookkeeping.

Sources: llama.cpp walkthrough, "Step 10: forming the batch for one call"
(token range check, default sequence 0, positions from seq_pos_max + 1,
default output flag on the last token), "Step 7: creating the inference
context" (n_batch / n_ubatch clamps), "Steps 11-12" (ubatches of at most
n_ubatch tokens, return codes 0 / 1 / negative), "KV-cache and the Prefill /
Decode stages" (seq_pos_max); Ollama engine page, "KV Cache: memory for
causal attention" (contiguous slots, per-cell position and sequence).
"""
import numpy as np
import pytest

from oracle import OracleContext, OracleModel

HP = dict(n_vocab=100, n_embd=8, n_layer=1, n_head=2, n_head_kv=1, head_dim=4, n_ff=8,
          rms_eps=1e-5, rope_theta=10000.0, tied=True)


def ctx(**kw):
    args = dict(n_ctx=16, n_ubatch=4, n_seq_max=4, compute=False)
    args.update(kw)
    return OracleContext(OracleModel(HP, {}), **args)


def test_defaults_seq0_positions_and_last_logit():
    c = ctx()
    r = c.decode([5, 6, 7])
    assert r.status == 0
    assert r.positions == [0, 1, 2]
    assert r.seq_ids == [[0], [0], [0]]
    assert r.output_flags == [False, False, True]
    assert r.out_index == [2]
    r = c.decode([8])
    assert r.positions == [3] and c.seq_pos_max(0) == 3
    c2 = ctx(output_all=True)
    assert c2.decode([1, 2]).output_flags == [True, True]


def test_default_positions_run_per_sequence():
    c = ctx()
    c.decode([1, 2], seq_ids=[[1], [1]])
    r = c.decode([3, 4, 5, 6], seq_ids=[[0], [1], [0], [2]])
    assert r.positions == [0, 2, 1, 0]
    assert [c.seq_pos_max(s) for s in range(4)] == [1, 2, 0, -1]


def test_clamps_of_batch_sizes():
    c = ctx(n_ctx=6, n_batch=100, n_ubatch=50)
    assert c.n_batch == 6 and c.n_ubatch == 6
    with pytest.raises(ValueError):
        ctx(n_seq_max=65)


@pytest.mark.parametrize("kw", [
    dict(tokens=[]),
    dict(tokens=[1, 100]),                                  # token id == n_vocab
    dict(tokens=[-1]),
    dict(tokens=[1, 2], seq_ids=[[0], [4]]),                # seq id >= n_seq_max
    dict(tokens=[1], seq_ids=[[]]),
    dict(tokens=[1], seq_ids=[[2, 2]]),                     # duplicate id
    dict(tokens=[1, 2], pos=[3, 3]),                        # not increasing
    dict(tokens=[1], pos=[-1]),
    dict(tokens=list(range(17))),                           # more than n_batch
    dict(tokens=[1, 2], logits=[1]),
])
def test_invalid_batches_return_minus_one_and_change_nothing(kw):
    c = ctx()
    c.decode([9, 9])
    before = (c.cell_pos.copy(), c.cell_seq.copy())
    tokens = kw.pop("tokens")
    r = c.decode(tokens, **kw)
    assert r.status == -1
    assert np.array_equal(c.cell_pos, before[0]) and np.array_equal(c.cell_seq, before[1])


def test_explicit_position_must_follow_cache():
    c = ctx()
    c.decode([1, 2, 3])
    assert c.decode([4], pos=[2]).status == -1
    assert c.decode([4], pos=[10]).status == 0   # gaps are allowed
    assert c.seq_pos_max(0) == 10


def test_multi_sequence_token_positions():
    c = ctx()
    c.decode([1, 2, 3], seq_ids=[[0], [0], [0]])
    # a token shared by sequences 0 and 1 takes the first sequence's next position
    r = c.decode([4], seq_ids=[[0, 1]])
    assert r.positions == [3]
    assert c.seq_pos_max(1) == 3
    # then sequence 1 may not go back to position 0
    assert c.decode([5], seq_ids=[[1]], pos=[0]).status == -1
    # default position of a token whose second sequence is ahead is invalid
    c.decode([6, 7], seq_ids=[[2], [2]], pos=[8, 9])
    assert c.decode([8], seq_ids=[[3, 2]]).status == -1


def test_full_cache_returns_one_and_changes_nothing():
    c = ctx(n_ctx=8, n_ubatch=8)
    assert c.decode(list(range(6))).status == 0
    before = c.cell_pos.copy()
    assert c.decode([1, 2, 3]).status == 1
    assert np.array_equal(c.cell_pos, before)
    assert c.decode([1, 2]).status == 0
    assert c.n_free() == 0


def test_ubatch_split_is_consecutive_in_order():
    c = ctx(n_ctx=16, n_ubatch=4)
    r = c.decode(list(range(10)))
    assert [list(u) for u in r.ubatches] == [[0, 1, 2, 3], [4, 5, 6, 7], [8, 9]]
    assert r.slots == list(range(10))


def test_find_slots_first_fit_then_lowest_free():
    c = ctx(n_ctx=12)
    # occupancy pattern: X X . X . . X . . . X .
    occ = [0, 1, 3, 6, 10]
    c.cell_pos[occ] = 0
    assert list(c.find_slots(1)) == [2]
    assert list(c.find_slots(2)) == [4, 5]
    assert list(c.find_slots(3)) == [7, 8, 9]
    assert list(c.find_slots(4)) == [2, 4, 5, 7]    # no run of 4: lowest free cells
    assert list(c.find_slots(7)) == [2, 4, 5, 7, 8, 9, 11]
    assert c.find_slots(8) is None


def test_interleaved_script_invariants():
    rng = np.random.default_rng(5)
    c = ctx(n_ctx=64, n_ubatch=5, n_seq_max=4)
    used = 0
    for step in range(12):
        n = int(rng.integers(1, 7))
        seqs = [[int(s)] for s in rng.integers(0, 4, size=n)]
        r = c.decode(list(rng.integers(0, 100, size=n)), seq_ids=seqs)
        if r.status == 1:
            break
        assert r.status == 0
        used += n
        # slots are the next cells in order (nothing is ever freed)
        assert r.slots == list(range(used - n, used))
    live = c.cell_pos >= 0
    assert int(live.sum()) == used
    pairs = set()
    for cell in np.flatnonzero(live):
        for s in range(4):
            if (int(c.cell_seq[cell]) >> s) & 1:
                key = (s, int(c.cell_pos[cell]))
                assert key not in pairs
                pairs.add(key)
    for s in range(4):
        ps = [p for (q, p) in pairs if q == s]
        assert c.seq_pos_max(s) == (max(ps) if ps else -1)


def test_clear_resets():
    c = ctx()
    c.decode([1, 2, 3])
    c.clear()
    assert c.n_free() == 16 and c.seq_pos_max(0) == -1
    assert c.decode([4]).positions == [0]
