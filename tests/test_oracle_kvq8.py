"""Pins of the oracle's Q8_0 cache rows (blocks of 32 along head_dim: an fp16
scale d = fp16(max|x| / 127) and codes q = round-half-even(x / d) clamped to
[-127, 127], decided in float32; stored value d * q).

* A hand-made row: the scale, ties to even (0.5 -> 0, 1.5 -> 2) and the sign.
* Zero blocks and blocks whose scale underflows fp16 store zeros.
* On random rows: |d q - x| <= d / 2, the largest |q| of a block is 127, and
  re-quantizing stored values changes nothing.
* A decode over a Q8_0 cache stays close to the same decode over a float32
  cache, and a cache shift re-quantizes the rotated keys (shift and back
  stays within the quantization error of the unshifted keys).
"""
import numpy as np

import tdf_synth
from oracle import OracleContext, OracleModel
from oracle.context import quantize_q8_0_rows


def test_hand_row():
    x = np.zeros(64)
    x[0], x[1], x[2], x[3], x[31] = 63.5, -0.5, 0.25, 0.75, -10.0
    x[32:] = 1.0 / 1024
    got = quantize_q8_0_rows(x)
    want = np.zeros(64)
    want[0], want[1], want[2], want[3], want[31] = 63.5, -0.5, 0.0, 1.0, -10.0
    d2 = np.float64(np.float16(np.float32(1.0 / 1024) / np.float32(127)))
    want[32:] = 127 * d2
    assert np.array_equal(got, want)


def test_zero_and_underflowing_blocks():
    x = np.zeros((2, 32))
    x[1, 5] = 1e-9  # max / 127 underflows fp16 to 0
    assert np.array_equal(quantize_q8_0_rows(x), np.zeros((2, 32)))


def test_random_rows_bound_and_idempotence():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 4, 128)) * rng.uniform(1e-3, 10, size=(50, 4, 1))
    got = quantize_q8_0_rows(x)
    f = x.astype(np.float32).astype(np.float64).reshape(50, 4, 4, 32)
    amax = np.abs(x.astype(np.float32)).reshape(50, 4, 4, 32).max(axis=-1)
    d = (amax / np.float32(127)).astype(np.float16).astype(np.float64)
    g = got.reshape(50, 4, 4, 32)
    assert np.all(np.abs(g - f) <= d[..., None] / 2 * (1 + 1e-12))
    q = g / d[..., None]
    assert np.array_equal(q, np.rint(q))
    assert np.all(np.abs(q).max(axis=-1) == 127)
    assert np.array_equal(quantize_q8_0_rows(got), got)


CFG = dict(n_vocab=200, n_embd=64, n_layer=2, n_head=4, n_head_kv=2, head_dim=32, n_ff=96,
           rms_eps=1e-5, rope_theta=10000.0, tied=False, weight_dtype="f32", seed=3,
           weight_std=0.2, gain_std=0.1)


def _ctx(kv):
    w = tdf_synth.make_all(CFG)
    return OracleContext(OracleModel(CFG, w), n_ctx=64, kv_dtype=kv)


def test_decode_close_to_float32_cache():
    toks = list(tdf_synth.prompt(CFG, 0, 20))
    a = _ctx("q8_0").decode(toks)
    b = _ctx("f32").decode(toks)
    # each cached value moves by at most d/2 = max|x|/254 of its block; two
    # layers of sharp attention (weight std 0.2) amplify that to a few percent
    rel = np.linalg.norm(a.logits - b.logits) / np.linalg.norm(b.logits)
    assert 0 < rel < 1e-1


def test_shift_requantizes_keys():
    toks = list(tdf_synth.prompt(CFG, 0, 12))
    c = _ctx("q8_0")
    c.decode(toks)
    before = c.k_cache[0][:12].copy()
    assert c.kv_seq_shift(0, 0, 12, 5) == 0
    after = c.k_cache[0][:12]
    assert np.array_equal(quantize_q8_0_rows(after), after)  # stored values are Q8_0 rows
    assert not np.array_equal(after, before)
    assert c.kv_seq_shift(0, 0, 17, -5) == 0
    back = c.k_cache[0][:12]
    f = _ctx("q8_0")
    f.decode(toks)
    rel = np.linalg.norm(back - f.k_cache[0][:12]) / np.linalg.norm(f.k_cache[0][:12])
    assert rel < 2e-2
