"""Pins of the Q8_0 weight format in the oracle and the generator.

Q8_0 (named, not defined, by the llama.cpp walkthrough's quantisation types
and the Ollama backends chapter) is read as: every block of 32 consecutive
weights of a row is one fp16 scale d times 32 int8 values q; w = d * q.

* A hand-made buffer with known scales and values at known positions
  dequantizes to those exact products (layout: all q row-major, then the
  [rows][K/32] scales).
* The generator's blocks satisfy the format's construction: |q| <= 127, the
  largest |q| of a non-zero block is 127, d = fp16(max|w| / 127) of the same
  float32 draws as the unquantized weights, and |d q - w| <= d / 2.
* The forward pass over Q8_0 weights equals the forward pass over the same
  values stored as float32 (every d * q is exact in float32), for a model
  with untied and tied output weights.
"""
import numpy as np

import tdf_synth
from oracle import OracleContext, OracleModel
from oracle.model import dequant_q8_0


def test_hand_buffer_layout_and_values():
    rows, K = 2, 64
    q = np.zeros((rows, K), dtype=np.int8)
    q[0, 0], q[0, 31], q[0, 32], q[1, 5], q[1, 63] = 127, -1, 3, -127, 64
    d = np.array([[0.5, 0.25], [2.0, 0.125]], dtype=np.float16)
    buf = np.concatenate([q.reshape(-1).view(np.uint8), d.reshape(-1).view(np.uint8)])
    w = dequant_q8_0(buf, rows, K)
    want = np.zeros((rows, K))
    want[0, 0], want[0, 31], want[0, 32], want[1, 5], want[1, 63] = 63.5, -0.5, 0.75, -254.0, 8.0
    assert np.array_equal(w, want)
    assert np.array_equal(dequant_q8_0(buf, rows, K, row_idx=np.array([1, 1, 0])), want[[1, 1, 0]])


def test_generator_blocks_follow_the_format():
    rows, K, std = 7, 96, 0.02
    buf = tdf_synth.normal_q8_0(5, "blk.0.ffn_up.weight", rows, K, std)
    q = buf[:rows * K].view(np.int8).reshape(rows, K // 32, 32).astype(np.int64)
    d = buf[rows * K:].view(np.float16).reshape(rows, K // 32)
    w = tdf_synth.normal(5, "blk.0.ffn_up.weight", rows * K, std).reshape(rows, K // 32, 32)
    assert buf.size == rows * K + rows * K // 32 * 2
    assert np.abs(q).max() <= 127
    assert np.all(np.abs(q).max(axis=2) == 127)
    amax = np.abs(w).max(axis=2).astype(np.float32)
    assert np.array_equal(d, (amax / np.float32(127)).astype(np.float16))
    err = np.abs(q * d.astype(np.float64)[..., None] - w.astype(np.float64))
    assert np.all(err <= d.astype(np.float64)[..., None] / 2 * (1 + 1e-6))


def _as_f32(cfg, tensors, model):
    out = {}
    for name, a in tensors.items():
        out[name] = model.w(name).astype(np.float32) if a.dtype == np.uint8 else a
    return out


def test_forward_equals_float32_copy():
    for tied in (False, True):
        cfg = dict(n_vocab=70, n_embd=64, n_layer=2, n_head=4, n_head_kv=2, head_dim=16, n_ff=96,
                   rms_eps=1e-5, rope_theta=10000.0, tied=tied, weight_dtype="q8_0", seed=9,
                   weight_std=0.2, gain_std=0.1)
        tensors = tdf_synth.make_all(cfg)
        assert tensors["blk.0.attn_q.weight"].dtype == np.uint8
        mq = OracleModel(cfg, tensors)
        f32 = _as_f32(cfg, tensors, mq)
        mf = OracleModel(dict(cfg, weight_dtype="f32"), f32)
        toks = tdf_synth.prompt(cfg, 0, 9)
        a = OracleContext(mq, n_ctx=32).decode(list(toks))
        b = OracleContext(mf, n_ctx=32).decode(list(toks))
        assert np.array_equal(a.logits, b.logits)
