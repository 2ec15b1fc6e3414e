"""Element operations of the decoder layer, float64, one function per step.

TEST INFRASTRUCTURE: imported only by tests, smoke() and bench.py's
cpu_baseline leg.

Sources (cited by page title and section):
* Ollama engine page, "Inside the inference engine: model architectures and
  the forward pass", section "Deep dive: the Llama forward pass in Go" -- the
  per-layer order (attention RMSNorm, Q/K/V, RoPE, scaled dot-product
  attention with the cache, output projection, residual, MLP RMSNorm, gated
  SiLU MLP, residual), GQA with fewer KV heads broadcast over query heads, and
  the MLP ``Down(SILU(Gate(h)) * Up(h))``.
* llama.cpp walkthrough, "Step 4: loading hyper-parameters" -- rope base
  frequency; "KV-cache and the Prefill / Decode stages" -- cached K/V of all
  earlier positions, masked softmax.

Readings where the pages leave a step open:
* RMSNorm: ``x / sqrt(mean(x^2) + eps) * g`` (eps inside the root).
* RoPE: adjacent pairs (2i, 2i+1) rotated by ``pos * theta^(-2i/hd)``.
* Attention scale 1/sqrt(head_dim); query head j uses KV head
  ``j // (n_head / n_head_kv)`` (contiguous groups).
* SwiGLU: ``silu(gate) * up`` with ``silu(z) = z / (1 + exp(-z))``.
* Sliding window (Ollama engine page, "KV Cache: memory for causal
  attention"): a windowed layer attends only to the ``window`` most recent
  positions, the token's own included.
"""
from __future__ import annotations

import numpy as np


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """Row-wise RMSNorm of ``x`` [..., d] with gain ``g`` [d]."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


def rope_angles(pos: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """phi[t, i] = pos[t] * theta^(-2i/head_dim) for i < head_dim/2."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = np.power(float(theta), -2.0 * i / head_dim)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope(y: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate each head of ``y`` [T, n_heads, head_dim] at its token's position.

    Pair (y[2i], y[2i+1]) -> (y[2i] cos phi - y[2i+1] sin phi,
                              y[2i] sin phi + y[2i+1] cos phi).
    """
    y = np.asarray(y, dtype=np.float64)
    hd = y.shape[-1]
    phi = rope_angles(pos, hd, theta)[:, None, :]  # [T, 1, hd/2]
    c, s = np.cos(phi), np.sin(phi)
    ye, yo = y[..., 0::2], y[..., 1::2]
    out = np.empty_like(y)
    out[..., 0::2] = ye * c - yo * s
    out[..., 1::2] = ye * s + yo * c
    return out


def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_mlp(h: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """``W_down (silu(W_gate h) * (W_up h))`` for rows of ``h``; W are [out][in]."""
    return (silu(h @ w_gate.T) * (h @ w_up.T)) @ w_down.T


def attend(q: np.ndarray, k_vis: np.ndarray, v_vis: np.ndarray) -> np.ndarray:
    """Scaled dot-product attention of one token over its visible cells.

    q      [n_head, hd]          rotated queries of the token
    k_vis  [n, n_head_kv, hd]    rotated keys of the visible cells
    v_vis  [n, n_head_kv, hd]    values of the visible cells
    returns [n_head, hd]

    Query head j uses KV head j // (n_head / n_head_kv): the heads are viewed
    as [n_head_kv, group, hd] and each group is scored against its KV head.
    """
    n_head, hd = q.shape
    n_head_kv = k_vis.shape[1]
    group = n_head // n_head_kv
    qg = q.reshape(n_head_kv, group, hd)
    s = np.matmul(qg, k_vis.transpose(1, 2, 0)) / np.sqrt(hd)      # [Hkv, group, n]
    a = np.exp(s - np.max(s, axis=-1, keepdims=True))
    a /= np.sum(a, axis=-1, keepdims=True)
    return np.matmul(a, v_vis.transpose(1, 0, 2)).reshape(n_head, hd)  # [Hkv, group, hd]


def window_visible(cell_pos: np.ndarray, pos: int, window: int) -> np.ndarray:
    """Cells a token at position ``pos`` sees in a windowed layer, by cell
    position: pos - window < p <= pos (the ``window`` most recent positions)."""
    cell_pos = np.asarray(cell_pos)
    return (cell_pos > pos - window) & (cell_pos <= pos)
