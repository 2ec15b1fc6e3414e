"""Model weights for the oracle: exact float64 views of the stored values.

TEST INFRASTRUCTURE: imported only by tests, smoke() and bench.py's
cpu_baseline leg.

The model is hyper-parameters plus named tensors, as in the Ollama engine
page ("Inside the inference engine: model architectures and the forward
pass", section "Model initialisation with reflection"): ``token_embd``,
``blk.<i>.*``, ``output_norm`` and ``output`` which falls back to
``token_embd`` when absent (tied input/output embeddings).

Stored values are fp32 (float32 arrays), bf16 (uint16 bit patterns) or
Q8_0 (uint8 buffers, see ``dequant_q8_0``); all widen to float64 exactly.  Tensors are fetched through a provider callable so
that very large models can be regenerated layer by layer instead of held.
"""
from __future__ import annotations

from typing import Callable, Dict, Optional

import numpy as np


def widen(a: np.ndarray) -> np.ndarray:
    """Exact float64 value of stored weights (float32, or uint16 bf16 bits).
    A bf16 value is the float32 whose upper 16 bits are the stored bits."""
    if a.dtype == np.uint16:
        src = np.ascontiguousarray(a).reshape(-1)
        out = np.empty(src.size, dtype=np.float64)
        step = 1 << 22
        for i in range(0, src.size, step):
            out[i:i + step] = (src[i:i + step].astype(np.uint32) << 16).view(np.float32)
        return out.reshape(a.shape)
    return np.asarray(a, dtype=np.float64)


def dequant_q8_0(buf: np.ndarray, rows: int, K: int, row_idx=None) -> np.ndarray:
    """Exact float64 values of a Q8_0 matrix [rows][K] (llama.cpp walkthrough
    and Ollama backends chapter name the "Q8_0" type without defining it; the
    reading here is the common one): every block of 32 consecutive elements
    of a row is one scale d (fp16) times 32 int8 values q, w = d * q.  The
    buffer holds rows*K int8 values q (row-major), then rows*K/32 fp16 scales
    (row-major [rows][K/32]).  row_idx selects rows (default all)."""
    nb = K // 32
    q = np.frombuffer(buf, dtype=np.int8, count=rows * K).reshape(rows, nb, 32)
    d = np.frombuffer(buf, dtype=np.float16, count=rows * nb, offset=rows * K).reshape(rows, nb)
    if row_idx is not None:
        q, d = q[row_idx], d[row_idx]
    return (q.astype(np.float64) * d.astype(np.float64)[..., None]).reshape(q.shape[0], K)


class OracleModel:
    """hparams: n_vocab, n_embd, n_layer, n_head, n_head_kv, head_dim, n_ff,
    rms_eps, rope_theta, tied; optionally n_swa (attention window, 0 = none)
    and swa_layers (per-layer flags, absent = every layer windowed).

    ``tensors`` is either a dict name -> stored array, or a callable
    ``provider(name) -> stored array`` (used to stream huge models).
    """

    def __init__(self, hparams: dict, tensors, cache: bool = True):
        self.hp = dict(hparams)
        self._provider: Callable[[str], np.ndarray]
        if isinstance(tensors, dict):
            self._provider = tensors.__getitem__
            self._names = set(tensors)
        else:
            self._provider = tensors
            self._names = None
        self._cache: Optional[Dict[str, np.ndarray]] = {} if cache else None

    def has(self, name: str) -> bool:
        if self._names is not None:
            return name in self._names
        try:
            self._provider(name)
            return True
        except KeyError:
            return False

    def shape(self, name: str):
        """[rows][cols] of a matrix of this model (from the hyper-parameters)."""
        hp = self.hp
        d, F, V = hp["n_embd"], hp["n_ff"], hp["n_vocab"]
        q_rows, kv_rows = hp["n_head"] * hp["head_dim"], hp["n_head_kv"] * hp["head_dim"]
        if name in ("token_embd.weight", "output.weight"):
            return V, d
        suffix = name.split(".", 2)[-1]
        return {"attn_q.weight": (q_rows, d), "attn_k.weight": (kv_rows, d), "attn_v.weight": (kv_rows, d),
                "attn_output.weight": (d, q_rows), "ffn_gate.weight": (F, d), "ffn_up.weight": (F, d),
                "ffn_down.weight": (d, F)}[suffix]

    def _widen(self, name: str, a: np.ndarray) -> np.ndarray:
        if a.dtype == np.uint8:
            return dequant_q8_0(a, *self.shape(name))
        return widen(a)

    def w(self, name: str) -> np.ndarray:
        if self._cache is not None and name in self._cache:
            return self._cache[name]
        a = self._widen(name, self._provider(name))
        if self._cache is not None:
            self._cache[name] = a
        return a

    def output_weight(self) -> np.ndarray:
        """LM head [n_vocab][n_embd]; the embedding table when tied."""
        if self.hp.get("tied", False) or not self.has("output.weight"):
            return self.w("token_embd.weight")
        return self.w("output.weight")

    def embed_rows(self, tokens: np.ndarray) -> np.ndarray:
        """Rows ``token[i]`` of the [n_vocab][n_embd] embedding table."""
        idx = np.asarray(tokens, dtype=np.int64)
        if self._cache is not None and "token_embd.weight" in self._cache:
            return self._cache["token_embd.weight"][idx]
        a = self._provider("token_embd.weight")
        if a.dtype == np.uint8:
            return dequant_q8_0(a, *self.shape("token_embd.weight"), row_idx=idx)
        return widen(a[idx])
