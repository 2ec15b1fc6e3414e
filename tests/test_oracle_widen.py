"""Pins of the oracle's bf16 widening (``oracle.model.widen`` and the bf16
path of ``OracleModel.embed_rows`` / ``OracleModel.w``).

Every bf16 weight of the 1B, 8B and 70B shapes enters the oracle through
these functions, so they are pinned against values fixed by the format
itself: a bf16 number is the upper half of an IEEE-754 binary32 (sign, 8
exponent bits, 7 fraction bits), so each hand-written bit pattern below has
an exact value written out from that definition, and all 65,536 patterns
are compared with torch's own bfloat16 -> float64 conversion (an independent
implementation).  Plausible mistakes (a shift of 15, reading the bits as
fp16, taking them as the low half of the binary32) are planted on the CPU
and each is caught.
"""
import math

import numpy as np
import pytest
import torch

import oracle.model as omodel
from oracle import OracleModel

# (bits, exact value) from the binary32 layout: value = (-1)^s * 1.f * 2^(e-127),
# subnormal (e = 0): (-1)^s * 0.f * 2^-126, with f the 7 stored fraction bits
# followed by 16 zero bits
HAND = [
    (0x3F80, 1.0),                               # e = 127, f = 0
    (0xC040, -3.0),                              # s = 1, e = 128, f = 0b1000000 -> 1.5 * 2
    (0x4049, 3.140625),                          # e = 128, f = 0b1001001 -> (1 + 73/128) * 2
    (0x3C00, 2.0 ** -7),                         # e = 120
    (0x0001, 2.0 ** -133),                       # subnormal: fraction 1/128, times 2^-126
    (0x0080, 2.0 ** -126),                       # smallest normal
    (0x007F, (127 / 128) * 2.0 ** -126),         # largest subnormal
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),    # largest finite
    (0xFF7F, -(2.0 - 2.0 ** -7) * 2.0 ** 127),
    (0x3DCD, (1 + 77 / 128) * 2.0 ** -4),        # 0.10009765625, a typical N(0, 0.02) tail weight
    (0xBCA4, -(1 + 36 / 128) * 2.0 ** -6),       # -0.02001953125
    (0x0000, 0.0),
]


def _check(widen_fn):
    """Mismatches of ``widen_fn`` on the hand patterns, -0.0, the infinities
    and NaN; empty when it widens bf16 bits exactly."""
    bad = []
    bits = np.array([b for b, _ in HAND], dtype=np.uint16)
    got = widen_fn(bits)
    for (b, v), g in zip(HAND, got):
        if not (g == v and got.dtype == np.float64):
            bad.append((hex(b), v, g))
    z = widen_fn(np.array([0x8000], dtype=np.uint16))[0]
    if not (z == 0.0 and math.copysign(1.0, z) < 0):
        bad.append(("0x8000", -0.0, z))
    inf = widen_fn(np.array([0x7F80, 0xFF80, 0x7FC0], dtype=np.uint16))
    if not (inf[0] == math.inf and inf[1] == -math.inf and math.isnan(inf[2])):
        bad.append(("inf/nan", inf))
    return bad


def test_hand_patterns_exact():
    assert _check(omodel.widen) == []


def test_all_patterns_match_torch_bfloat16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns
        got = omodel.widen(bits)
    np.testing.assert_array_equal(got, ref)  # NaN positions must coincide too
    # signs of the zeros
    assert np.array_equal(np.signbit(got[[0x0000, 0x8000]]), [False, True])


def test_shape_kept_and_float32_untouched():
    bits = np.array([[0x3F80, 0xC040, 0x4049], [0x0001, 0x7F7F, 0x3C00]], dtype=np.uint16)
    got = omodel.widen(bits)
    assert got.shape == (2, 3)
    np.testing.assert_array_equal(got[0], [1.0, -3.0, 3.140625])
    f = np.array([0.1, -2.5e-30, 3.0e38], dtype=np.float32)
    w = omodel.widen(f)
    assert w.dtype == np.float64 and np.array_equal(w, f.astype(np.float64))


def _table():
    """A 4 x 3 bf16 embedding table written by hand, and its exact values."""
    bits = np.array([[0x3F80, 0x0000, 0xC040],
                     [0x4049, 0x3C00, 0x0001],
                     [0x7F7F, 0x3DCD, 0xBCA4],
                     [0x8000, 0x0080, 0x007F]], dtype=np.uint16)
    vals = np.array([[1.0, 0.0, -3.0],
                     [3.140625, 2.0 ** -7, 2.0 ** -133],
                     [(2.0 - 2.0 ** -7) * 2.0 ** 127, (1 + 77 / 128) * 2.0 ** -4, -(1 + 36 / 128) * 2.0 ** -6],
                     [-0.0, 2.0 ** -126, (127 / 128) * 2.0 ** -126]])
    return bits, vals


HP = dict(n_vocab=4, n_embd=3, n_layer=0, n_head=1, n_head_kv=1, head_dim=2, n_ff=2,
          rms_eps=1e-5, rope_theta=1e4, tied=True)


@pytest.mark.parametrize("cache", [True, False])
def test_embed_rows_gathers_exact_rows(cache):
    bits, vals = _table()
    m = OracleModel(HP, {"token_embd.weight": bits, "output_norm.weight": np.ones(3, np.float32)}, cache=cache)
    idx = [2, 0, 2, 3, 1]
    got = m.embed_rows(np.array(idx))
    np.testing.assert_array_equal(got, vals[idx])
    assert np.signbit(got[3, 0])
    # the cached full table (after a w() call) gives the same rows
    np.testing.assert_array_equal(m.w("token_embd.weight"), vals)
    np.testing.assert_array_equal(m.embed_rows(np.array(idx)), vals[idx])


def _widen_shift15(a):
    if a.dtype == np.uint16:
        with np.errstate(invalid="ignore"):
            return (a.astype(np.uint32) << 15).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _widen_as_fp16(a):
    if a.dtype == np.uint16:
        return a.view(np.float16).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _widen_low_half(a):
    if a.dtype == np.uint16:
        return a.astype(np.uint32).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _widen_dropping_last_fraction_bit(a):
    # keeps only 6 of the 7 fraction bits
    if a.dtype == np.uint16:
        return ((a.astype(np.uint32) & 0xFFFE) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


@pytest.mark.parametrize("fn", [_widen_shift15, _widen_as_fp16, _widen_low_half,
                                _widen_dropping_last_fraction_bit])
def test_planted_widen_mistakes_are_caught(fn):
    assert _check(fn) != []


def test_planted_embed_mistake_is_caught(monkeypatch):
    bits, vals = _table()
    monkeypatch.setattr(omodel, "widen", _widen_as_fp16)
    m = OracleModel(HP, {"token_embd.weight": bits, "output_norm.weight": np.ones(3, np.float32)}, cache=False)
    got = m.embed_rows(np.array([1, 2]))
    assert not np.array_equal(got, vals[[1, 2]])
