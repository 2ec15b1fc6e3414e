"""Plant plausible mistakes in the oracle (on the CPU) and check that the
whole-forward library pin notices each one.  This shows the pins are
sensitive enough: a dropped term, a wrong sign or index, or a transposed
operand anywhere in the forward pass moves the logits far outside the
agreement the correct oracle reaches."""
import numpy as np
import pytest

import oracle.context as octx
import oracle.ops as ops
import tdf_synth
from oracle import OracleContext, OracleModel

from test_oracle_forward import PIN, hf_logits, prompt_tokens


def _rope_half_split(y, pos, theta):
    y = np.asarray(y, dtype=np.float64)
    hd = y.shape[-1]
    phi = ops.rope_angles(pos, hd, theta)[:, None, :]
    a, b = y[..., : hd // 2], y[..., hd // 2:]
    return np.concatenate([a * np.cos(phi) - b * np.sin(phi), a * np.sin(phi) + b * np.cos(phi)], axis=-1)


def _rope_clockwise(y, pos, theta):
    return ops.rope(y, -np.asarray(pos), theta)


def _rope_wrong_freq(y, pos, theta):
    return ops.rope(y, pos, theta ** 0.5)


def _rms_eps_outside(x, g, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * g


def _rms_no_mean(x, g, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * g


def _attend_scale_hd(q, k, v):
    return ops.attend(q / np.sqrt(q.shape[1]), k, v)


def _attend_interleaved_groups(q, k, v):
    H, Hkv = q.shape[0], k.shape[1]
    # head j -> kv head j % Hkv instead of j // (H / Hkv)
    idx = np.array([j % Hkv for j in range(H)])
    out = np.empty_like(q)
    for j in range(H):
        out[j] = ops.attend(q[j:j + 1], k[:, idx[j]:idx[j] + 1], v[:, idx[j]:idx[j] + 1])[0]
    return out


def _swiglu_swapped(h, wg, wu, wd):
    return ops.swiglu_mlp(h, wu, wg, wd)


def _swiglu_no_gate(h, wg, wu, wd):
    return ((h @ wg.T) * (h @ wu.T)) @ wd.T


MUTATIONS = {
    "rope_half_split": ("rope", _rope_half_split),
    "rope_clockwise": ("rope", _rope_clockwise),
    "rope_wrong_frequency": ("rope", _rope_wrong_freq),
    "rmsnorm_eps_outside_root": ("rms_norm", _rms_eps_outside),
    "rmsnorm_sum_not_mean": ("rms_norm", _rms_no_mean),
    "attention_scale_1_over_hd": ("attend", _attend_scale_hd),
    "gqa_interleaved_groups": ("attend", _attend_interleaved_groups),
    "swiglu_silu_on_up": ("swiglu_mlp", _swiglu_swapped),
    "swiglu_without_silu": ("swiglu_mlp", _swiglu_no_gate),
}


def _oracle_error(cfg, tensors, toks, model_cls=OracleModel):
    ctx = OracleContext(model_cls(cfg, tensors), n_ctx=64, output_all=True)
    got = ctx.decode(toks).logits
    ref = hf_logits(cfg, tensors, toks)
    return np.max(np.abs(got - ref)) / np.max(np.abs(ref))


@pytest.fixture(scope="module")
def case():
    cfg = PIN
    return cfg, tdf_synth.make_all(cfg), prompt_tokens(cfg, 17)


AGREE = 2e-6          # relative agreement of the correct oracle with the library
CAUGHT = 50 * AGREE    # a planted mistake must move the logits well beyond it


def test_correct_oracle_agrees(case):
    assert _oracle_error(*case) < AGREE


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(case, monkeypatch, name):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(octx, attr, fn)
    assert _oracle_error(*case) > CAUGHT, name


class _TransposedWo(OracleModel):
    def w(self, name):
        a = super().w(name)
        return a.T if name.endswith("attn_output.weight") else a


def test_transposed_output_projection_is_caught(case):
    cfg, tensors, toks = case
    assert cfg["n_head"] * cfg["head_dim"] == cfg["n_embd"]  # square, so the mistake runs
    assert _oracle_error(cfg, tensors, toks, _TransposedWo) > CAUGHT


def test_dropped_mlp_branch_is_caught(case, monkeypatch):
    cfg, tensors, toks = case
    real = octx.swiglu_mlp
    calls = {}

    # drop the MLP branch of the residual stream in every layer
    def mlp_then_drop(h2, wg, wu, wd):
        calls["n"] = calls.get("n", 0) + 1
        return real(h2, wg, wu, wd) * 0.0
    monkeypatch.setattr(octx, "swiglu_mlp", mlp_then_drop)
    assert _oracle_error(cfg, tensors, toks) > CAUGHT
    assert calls["n"] == cfg["n_layer"]


def test_non_causal_mask_is_caught(case, monkeypatch):
    cfg, tensors, toks = case
    real_forward = OracleContext._forward

    def leaky(self, toks_, pos, seq0, cells, sel):
        # report every live cell at position 0 while the ubatch runs, so the
        # visibility test (cell.pos <= pos_t) also admits later tokens; RoPE
        # still uses the true positions, which are passed separately
        saved = self.cell_pos.copy()
        self.cell_pos[self.cell_pos >= 0] = 0
        try:
            return real_forward(self, toks_, pos, seq0, cells, sel)
        finally:
            self.cell_pos[:] = saved

    monkeypatch.setattr(OracleContext, "_forward", leaky)
    assert _oracle_error(cfg, tensors, toks) > CAUGHT
