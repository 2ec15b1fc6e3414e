"""Pins of the oracle's element operations against closed forms, invariants,
brute force and library routines (not against a retyped copy of the oracle).

Sources: Ollama engine page ("Deep dive: the Llama forward pass in Go") for
the operations; llama.cpp walkthrough ("Step 4: loading hyper-parameters")
for the rope base frequency.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import ops

rng = np.random.default_rng(1234)


# ---- RMSNorm ---------------------------------------------------------------

def test_rmsnorm_unit_rms_before_gain():
    x = rng.normal(size=(7, 96)) * 3.0
    eps = 1e-5
    y = ops.rms_norm(x, np.ones(96), eps)
    m = np.mean(x * x, axis=1)
    # closed form: RMS(y) = sqrt(m / (m + eps)), i.e. ~1 for m >> eps
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), np.sqrt(m / (m + eps)), rtol=1e-12)


def test_rmsnorm_constant_vector_and_linear_gain():
    c, eps = 0.37, 1e-5
    y = ops.rms_norm(np.full((1, 16), c), np.ones(16), eps)
    np.testing.assert_allclose(y, c / math.sqrt(c * c + eps), rtol=1e-14)
    x = rng.normal(size=(3, 16))
    g = rng.normal(size=16)
    np.testing.assert_allclose(ops.rms_norm(x, g, eps), ops.rms_norm(x, np.ones(16), eps) * g, rtol=1e-13)
    # eps sits inside the root: a tiny vector is damped, not blown up
    tiny = np.full((1, 8), 1e-4)
    np.testing.assert_allclose(ops.rms_norm(tiny, np.ones(8), 1e-5), 1e-4 / math.sqrt(1e-8 + 1e-5), rtol=1e-12)


def test_rmsnorm_matches_torch_library():
    x = rng.normal(size=(5, 40))
    g = rng.normal(size=40)
    ref = F.rms_norm(torch.from_numpy(x), (40,), torch.from_numpy(g), eps=1e-5).numpy()
    np.testing.assert_allclose(ops.rms_norm(x, g, 1e-5), ref, rtol=1e-12, atol=1e-14)


# ---- RoPE ------------------------------------------------------------------

def test_rope_identity_at_zero_and_norm_preserved():
    y = rng.normal(size=(4, 3, 16))
    np.testing.assert_allclose(ops.rope(y, np.zeros(4), 10000.0), y, rtol=0, atol=0)
    z = ops.rope(y, np.array([1, 17, 300, 32767]), 500000.0)
    # every rotated pair keeps its length
    np.testing.assert_allclose(np.hypot(z[..., 0::2], z[..., 1::2]), np.hypot(y[..., 0::2], y[..., 1::2]), rtol=1e-12)


def test_rope_pair0_rotates_by_position_radians():
    y = np.zeros((1, 1, 8))
    y[0, 0, 0] = 1.0
    p = 3
    z = ops.rope(y, np.array([p]), 10000.0)
    np.testing.assert_allclose(z[0, 0, :2], [math.cos(p), math.sin(p)], rtol=1e-14, atol=1e-15)
    assert np.all(z[0, 0, 2:] == 0)


def test_rope_hand_example_second_pair():
    # head_dim 4, base 100: pair 1 turns at 100^(-2/4) = 0.1 rad per position
    y = np.array([[[0.0, 0.0, 1.0, 0.0]]])
    z = ops.rope(y, np.array([5]), 100.0)
    np.testing.assert_allclose(z[0, 0], [0.0, 0.0, math.cos(0.5), math.sin(0.5)], atol=1e-15)
    # counter-clockwise: the second component of each pair gains +sin
    y2 = np.array([[[0.0, 1.0, 0.0, 0.0]]])
    z2 = ops.rope(y2, np.array([1]), 100.0)
    np.testing.assert_allclose(z2[0, 0, :2], [-math.sin(1.0), math.cos(1.0)], atol=1e-15)


def test_rope_equals_complex_multiplication():
    # the textbook complex form: (y0 + i y1) * exp(i p theta^(-2k/d))
    hd, theta = 32, 500000.0
    y = rng.normal(size=(6, 2, hd))
    pos = np.array([0, 1, 5, 100, 4096, 32767])
    z = ops.rope(y, pos, theta)
    yc = y[..., 0::2] + 1j * y[..., 1::2]
    freq = theta ** (-np.arange(0, hd, 2) / hd)
    zc = yc * np.exp(1j * pos[:, None, None] * freq[None, None, :])
    np.testing.assert_allclose(z[..., 0::2], zc.real, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(z[..., 1::2], zc.imag, rtol=1e-11, atol=1e-12)


def test_rope_dot_depends_only_on_position_difference():
    hd = 64
    q = rng.normal(size=(1, 1, hd))
    k = rng.normal(size=(1, 1, hd))
    dots = []
    for base_pos in (0, 7, 1000, 20000):
        rq = ops.rope(q, np.array([base_pos + 13]), 500000.0)
        rk = ops.rope(k, np.array([base_pos]), 500000.0)
        dots.append(float(np.sum(rq * rk)))
    np.testing.assert_allclose(dots, dots[0], rtol=1e-9)


# ---- SiLU / SwiGLU -----------------------------------------------------------

def test_silu_closed_forms_and_library():
    assert ops.silu(np.array([0.0]))[0] == 0.0
    z = rng.normal(size=200) * 5
    # silu(z) - silu(-z) = z  (z*s(z) + z*s(-z) = z)
    np.testing.assert_allclose(ops.silu(z) - ops.silu(-z), z, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ops.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-13, atol=1e-15)
    assert np.isfinite(ops.silu(np.array([-1000.0, 1000.0]))).all()


def test_swiglu_mlp_against_torch_modules():
    d, f = 24, 40
    h = rng.normal(size=(3, d))
    wg, wu, wd = rng.normal(size=(f, d)), rng.normal(size=(f, d)), rng.normal(size=(d, f))
    th = torch.from_numpy(h)
    ref = F.linear(F.silu(F.linear(th, torch.from_numpy(wg))) * F.linear(th, torch.from_numpy(wu)),
                   torch.from_numpy(wd)).numpy()
    np.testing.assert_allclose(ops.swiglu_mlp(h, wg, wu, wd), ref, rtol=1e-12, atol=1e-12)
    # operand order matters: silu is applied to the gate, not the up projection
    swapped = ops.swiglu_mlp(h, wu, wg, wd)
    assert np.max(np.abs(swapped - ref)) > 1e-3


# ---- attention -------------------------------------------------------------

def _brute_attend(q, k, v):
    """Explicit loops: weights exp(s_c - max) / sum, then weighted sum of V."""
    H, hd = q.shape
    n, Hkv, _ = k.shape
    out = np.zeros((H, hd))
    for j in range(H):
        g = j * Hkv // H
        s = [sum(q[j, i] * k[c, g, i] for i in range(hd)) / math.sqrt(hd) for c in range(n)]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        z = sum(w)
        for c in range(n):
            for i in range(hd):
                out[j, i] += w[c] / z * v[c, g, i]
    return out


def test_attend_matches_brute_force_loops():
    q = rng.normal(size=(4, 8))
    k = rng.normal(size=(5, 2, 8))
    v = rng.normal(size=(5, 2, 8))
    np.testing.assert_allclose(ops.attend(q, k, v), _brute_attend(q, k, v), rtol=1e-12, atol=1e-14)


def test_attend_single_key_gives_value_and_equal_scores_give_mean():
    q = rng.normal(size=(2, 8))
    k = rng.normal(size=(1, 1, 8))
    v = rng.normal(size=(1, 1, 8))
    np.testing.assert_allclose(ops.attend(q, k, v), np.repeat(v[0], 2, axis=0), rtol=1e-14)
    kz = np.zeros((6, 1, 8))
    v6 = rng.normal(size=(6, 1, 8))
    np.testing.assert_allclose(ops.attend(q, kz, v6), np.repeat(v6.mean(axis=0), 2, axis=0), rtol=1e-13)


def test_gqa_equals_mha_with_replicated_heads_and_mha_special_case():
    H, Hkv, hd, n = 8, 2, 16, 11
    q = rng.normal(size=(H, hd))
    k = rng.normal(size=(n, Hkv, hd))
    v = rng.normal(size=(n, Hkv, hd))
    rep_k = np.repeat(k, H // Hkv, axis=1)  # contiguous groups: heads 0-3 -> kv 0
    rep_v = np.repeat(v, H // Hkv, axis=1)
    np.testing.assert_allclose(ops.attend(q, k, v), ops.attend(q, rep_k, rep_v), rtol=1e-13, atol=1e-15)
    # n_head_kv == n_head is plain multi-head attention (torch library, fp64)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[:, None, :], torch.from_numpy(rep_k).transpose(0, 1),
                                         torch.from_numpy(rep_v).transpose(0, 1))[:, 0, :].numpy()
    np.testing.assert_allclose(ops.attend(q, rep_k, rep_v), ref, rtol=1e-12, atol=1e-14)


def test_causal_attention_against_torch_sdpa():
    # a prompt of T tokens attending causally == SDPA(is_causal=True) per query
    T, H, Hkv, hd = 9, 4, 2, 8
    q = rng.normal(size=(T, H, hd))
    k = rng.normal(size=(T, Hkv, hd))
    v = rng.normal(size=(T, Hkv, hd))
    ours = np.stack([ops.attend(q[t], k[: t + 1], v[: t + 1]) for t in range(T)])
    tq = torch.from_numpy(q).transpose(0, 1)                                  # [H, T, hd]
    tk = torch.from_numpy(np.repeat(k, H // Hkv, axis=1)).transpose(0, 1)
    tv = torch.from_numpy(np.repeat(v, H // Hkv, axis=1)).transpose(0, 1)
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True).transpose(0, 1).numpy()
    np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-13)


# ---- cache storage type ------------------------------------------------------

def test_cache_storage_rounding_matches_numpy_and_bit_rule():
    from oracle.context import _round_storage
    x = rng.normal(size=4000) * 3
    np.testing.assert_array_equal(_round_storage(x, "f32"), x.astype(np.float32).astype(np.float64))
    np.testing.assert_array_equal(_round_storage(x, "f16"), x.astype(np.float16).astype(np.float64))
    b = _round_storage(x, "bf16")
    # bf16 keeps 8 significant bits: the result is a bf16 value, the nearest one
    u = b.astype(np.float32).view(np.uint32)
    assert np.all(u & 0xFFFF == 0)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(x))) - 7)
    assert np.all(np.abs(b - x) <= ulp / 2 + 1e-300)
    # ties go to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert _round_storage(np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8]), "bf16").tolist() == [1.0, 1 + 2 ** -6]
    assert _round_storage(x, None) is x
