"""Model weights for the oracle: exact float64 views of the stored values.

TEST INFRASTRUCTURE: imported only by tests, smoke() and bench.py's
cpu_baseline leg.

The model is hyper-parameters plus named tensors, as in the Ollama engine
page ("Inside the inference engine: model architectures and the forward
pass", section "Model initialisation with reflection"): ``token_embd``,
``blk.<i>.*``, ``output_norm`` and ``output`` which falls back to
``token_embd`` when absent (tied input/output embeddings).

Stored values are fp32 (float32 arrays) or bf16 (uint16 bit patterns); both
widen to float64 exactly.  Tensors are fetched through a provider callable so
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

    def w(self, name: str) -> np.ndarray:
        if self._cache is not None and name in self._cache:
            return self._cache[name]
        a = widen(self._provider(name))
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
        return widen(self._provider("token_embd.weight")[idx])
