"""Pins of the oracle's sliding-window attention (Ollama engine page, "KV
Cache: memory for causal attention": a windowed layer's mask keeps only the
most recent positions).  Each pin is a consequence of the definition that a
wrong window (off by one, wrong layers) breaks:

* a window wider than every position gap changes nothing;
* per-layer flags that switch the window off everywhere change nothing, and
  flags on every layer equal the flags being absent;
* a window of 1 makes attention return the token's own value vector, so a
  token's logits depend on its id alone, not on its position or context;
* with L windowed layers of width W, the logits at position p depend exactly
  on the tokens at positions p - L(W-1) .. p (the receptive field).
"""
import numpy as np
import pytest

import oracle.context as octx
import tdf_synth
from oracle import OracleContext, OracleModel

CFG = dict(tdf_synth.CONFIGS["tiny"])  # 2 layers, fp32


def _weights():
    return tdf_synth.make_all(CFG)


def _logits(hp_extra, toks, w, n_ubatch=512):
    hp = dict(tdf_synth.hparams(CFG), **hp_extra)
    ctx = OracleContext(OracleModel(hp, w), n_ctx=64, n_ubatch=n_ubatch, output_all=True)
    return ctx.decode(list(toks)).logits


@pytest.fixture(scope="module")
def w():
    return _weights()


def test_wide_window_equals_full_attention(w):
    toks = tdf_synth.prompt(CFG, 0, 12)
    full = _logits({}, toks, w)
    assert np.array_equal(_logits({"n_swa": 12}, toks, w), full)
    assert np.array_equal(_logits({"n_swa": 1000}, toks, w), full)
    assert not np.allclose(_logits({"n_swa": 11}, toks, w), full, rtol=0, atol=1e-9)


def test_layer_flags(w):
    toks = tdf_synth.prompt(CFG, 1, 10)
    full = _logits({}, toks, w)
    assert np.array_equal(_logits({"n_swa": 3, "swa_layers": [0, 0]}, toks, w), full)
    both = _logits({"n_swa": 3}, toks, w)
    assert np.array_equal(_logits({"n_swa": 3, "swa_layers": [1, 1]}, toks, w), both)
    first = _logits({"n_swa": 3, "swa_layers": [1, 0]}, toks, w)
    second = _logits({"n_swa": 3, "swa_layers": [0, 1]}, toks, w)
    for a, b in ((first, full), (second, full), (first, second), (first, both)):
        assert not np.allclose(a, b, rtol=0, atol=1e-9)


def test_window_one_sees_only_itself(w):
    toks = [5, 17, 300, 5, 42, 5]
    lg = _logits({"n_swa": 1}, toks, w)
    # the same id at positions 0, 3 and 5 gives the same logits exactly
    assert np.array_equal(lg[0], lg[3]) and np.array_equal(lg[0], lg[5])
    assert not np.allclose(lg[0], lg[1], rtol=0, atol=1e-9)


@pytest.mark.parametrize("W", [2, 3])
def test_receptive_field(w, W):
    L = CFG["n_layer"]
    toks = list(tdf_synth.prompt(CFG, 2, 14))
    p = 13
    reach = L * (W - 1)  # positions p - reach .. p influence position p
    base = _logits({"n_swa": W}, toks, w)[p]
    for q in range(p + 1):
        alt = list(toks)
        alt[q] = (alt[q] + 1) % CFG["n_vocab"]
        got = _logits({"n_swa": W}, alt, w)[p]
        if q < p - reach:
            assert np.array_equal(got, base), (W, q)
        else:
            assert np.max(np.abs(got - base)) > 1e-6, (W, q)


def test_window_through_the_cache_and_ubatches(w):
    """The window is a predicate on positions: decoding token by token
    through the cache, or in ubatches of 3, gives the logits of one pass."""
    toks = tdf_synth.prompt(CFG, 3, 11)
    hp = dict(tdf_synth.hparams(CFG), n_swa=4, swa_layers=[1, 0])
    one = _logits({"n_swa": 4, "swa_layers": [1, 0]}, toks, w)
    np.testing.assert_allclose(_logits({"n_swa": 4, "swa_layers": [1, 0]}, toks, w, n_ubatch=3), one,
                               rtol=0, atol=1e-12)
    ctx = OracleContext(OracleModel(hp, w), n_ctx=64)
    inc = [ctx.decode([int(t)]).logits[0] for t in toks]
    np.testing.assert_allclose(np.stack(inc), one, rtol=0, atol=1e-12)


def test_off_by_one_window_is_caught(w, monkeypatch):
    """A window one position too wide (p - W <= c instead of <) breaks the
    receptive-field pin."""
    def wide(cell_pos, pos, window):
        cell_pos = np.asarray(cell_pos)
        return (cell_pos >= pos - window) & (cell_pos <= pos)
    monkeypatch.setattr(octx, "window_visible", wide)
    toks = list(tdf_synth.prompt(CFG, 2, 14))
    base = _logits({"n_swa": 2}, toks, w)[13]
    alt = list(toks)
    alt[13 - 3] = (alt[13 - 3] + 1) % CFG["n_vocab"]
    assert not np.array_equal(_logits({"n_swa": 2}, alt, w)[13], base)
