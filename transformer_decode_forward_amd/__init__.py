"""Python binding of libtdf.so, the gfx950 Llama-style decoder forward pass.

Argument marshalling only: every step of the forward pass runs in the HIP
kernels of the library.  The functions mirror ``include/tdf.h`` one to one
(``tdf_model_create``, ``tdf_decode``, ...); ``Model`` and ``Context`` wrap
them for convenience.  PyTorch is used only to hold device memory and to
name streams.  Importing raises if the library has not been built
(``python -m transformer_decode_forward_amd.build``): there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtdf.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "tdf.h")

TDF_F32, TDF_F16, TDF_BF16, TDF_Q8_0 = 0, 1, 2, 3
DTYPES = {"f32": TDF_F32, "f16": TDF_F16, "bf16": TDF_BF16, "q8_0": TDF_Q8_0}
TDF_OK, TDF_NO_SLOT, TDF_E_INVALID, TDF_E_ALLOC, TDF_E_DEVICE = 0, 1, -1, -2, -3
TDF_CTX_DRY_RUN, TDF_CTX_PROFILE = 1, 2
OPS = ["embed", "norm", "qkv", "attn", "wo", "gate_up", "down", "lm_head", "argmax"]

_i32, _u64, _f32 = ctypes.c_int32, ctypes.c_uint64, ctypes.c_float
_vp = ctypes.c_void_p


class tdf_hparams(ctypes.Structure):
    _fields_ = [("n_vocab", _i32), ("n_embd", _i32), ("n_layer", _i32), ("n_head", _i32),
                ("n_head_kv", _i32), ("head_dim", _i32), ("n_ff", _i32),
                ("rms_eps", _f32), ("rope_theta", _f32), ("weight_dtype", _i32),
                ("n_swa", _i32), ("swa_layers", ctypes.POINTER(ctypes.c_int8))]


class tdf_layer_weights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")]


class tdf_weights(ctypes.Structure):
    _fields_ = [("token_embd", _vp), ("output_norm", _vp), ("output", _vp),
                ("layers", ctypes.POINTER(tdf_layer_weights))]


class tdf_sampling(ctypes.Structure):
    _fields_ = [("temperature", _f32), ("top_k", _i32), ("top_p", _f32), ("min_p", _f32)]


class tdf_context_params(ctypes.Structure):
    _fields_ = [("n_ctx", _i32), ("n_batch", _i32), ("n_ubatch", _i32), ("n_seq_max", _i32),
                ("kv_dtype", _i32), ("output_all", _i32), ("flags", _i32), ("stream", _vp)]


class tdf_batch(ctypes.Structure):
    _fields_ = [("n_tokens", _i32), ("token", ctypes.POINTER(_i32)), ("pos", ctypes.POINTER(_i32)),
                ("n_seq_id", ctypes.POINTER(_i32)), ("seq_id", ctypes.POINTER(ctypes.POINTER(_i32))),
                ("logits", ctypes.POINTER(ctypes.c_int8))]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m transformer_decode_forward_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "tdf_model_create": (_vp, [ctypes.POINTER(tdf_hparams), ctypes.POINTER(tdf_weights)]),
            "tdf_model_free": (None, [_vp]),
            "tdf_context_create": (_vp, [_vp, ctypes.POINTER(tdf_context_params)]),
            "tdf_context_free": (None, [_vp]),
            "tdf_decode": (_i32, [_vp, ctypes.POINTER(tdf_batch)]),
            "tdf_n_outputs": (_i32, [_vp]),
            "tdf_output_ids": (_i32, [_vp, ctypes.POINTER(_i32)]),
            "tdf_get_logits_ith": (ctypes.POINTER(_f32), [_vp, _i32]),
            "tdf_get_logits_device": (_vp, [_vp]),
            "tdf_argmax_ith": (_i32, [_vp, _i32]),
            "tdf_seq_pos_max": (_i32, [_vp, _i32]),
            "tdf_kv_clear": (_i32, [_vp]),
            "tdf_kv_cell": (_i32, [_vp, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_u64)]),
            "tdf_last_slots": (_i32, [_vp, ctypes.POINTER(_i32)]),
            "tdf_kv_import": (_i32, [_vp, _i32, _i32, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp)]),
            "tdf_profile_read": (_i32, [_vp, _i32, _i32, ctypes.POINTER(ctypes.c_int64),
                                        ctypes.POINTER(ctypes.c_double)]),
            "tdf_profile_reset": (_i32, [_vp]),
            "tdf_graph_counts": (_i32, [_vp, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]),
            "tdf_time_op": (_i32, [_vp, _i32, _i32, _i32, ctypes.POINTER(ctypes.c_double)]),
            "tdf_kv_seq_rm": (_i32, [_vp, _i32, _i32, _i32]),
            "tdf_sample": (_i32, [_vp, ctypes.POINTER(tdf_sampling), ctypes.POINTER(_f32), ctypes.POINTER(_i32)]),
            "tdf_sample_logits": (_i32, [_vp, ctypes.c_void_p, _i32, _i32, ctypes.POINTER(tdf_sampling),
                                         ctypes.POINTER(_f32), ctypes.POINTER(_i32)]),
            "tdf_kv_seq_shift": (_i32, [_vp, _i32, _i32, _i32, _i32]),
            "tdf_fault_alloc": (_i32, [_i32]),
            "tdf_sample_logits_static": (_i32, [ctypes.c_void_p, _i32, _i32, ctypes.POINTER(tdf_sampling),
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
            "tdf_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def header_symbols() -> list:
    """Function names declared in include/tdf.h."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tdf_[a-z_]+)\s*\(", text)))


# ---- one-to-one wrappers ---------------------------------------------------

def tdf_model_create(hp: tdf_hparams, w: tdf_weights):
    return lib().tdf_model_create(ctypes.byref(hp), ctypes.byref(w))


def tdf_model_free(m) -> None:
    lib().tdf_model_free(m)


def tdf_context_create(m, p: tdf_context_params):
    return lib().tdf_context_create(m, ctypes.byref(p))


def tdf_context_free(c) -> None:
    lib().tdf_context_free(c)


def tdf_decode(c, b: tdf_batch) -> int:
    return lib().tdf_decode(c, ctypes.byref(b))


def tdf_last_error() -> str:
    return lib().tdf_last_error().decode()


def tdf_fault_alloc(n: int) -> int:
    return lib().tdf_fault_alloc(n)


def tdf_sample_logits_static(logits_ptr: int, n_rows: int, n_vocab: int, p: tdf_sampling, u_ptr: int,
                             tokens_ptr: int, stream: int = 0) -> int:
    """Device addresses in, device tokens out, enqueued on ``stream``."""
    return lib().tdf_sample_logits_static(ctypes.c_void_p(logits_ptr), n_rows, n_vocab, ctypes.byref(p),
                                          ctypes.c_void_p(u_ptr or None), ctypes.c_void_p(tokens_ptr),
                                          ctypes.c_void_p(stream or None))


# ---- convenience objects ---------------------------------------------------

def _hparams(hp: dict) -> tdf_hparams:
    flags = hp.get("swa_layers")
    arr = None if flags is None else (ctypes.c_int8 * max(1, len(flags)))(*[1 if f else 0 for f in flags])
    h = tdf_hparams(hp["n_vocab"], hp["n_embd"], hp["n_layer"], hp["n_head"], hp["n_head_kv"],
                    hp["head_dim"], hp["n_ff"], hp["rms_eps"], hp["rope_theta"],
                    DTYPES[hp["weight_dtype"]], int(hp.get("n_swa") or 0),
                    ctypes.cast(arr, ctypes.POINTER(ctypes.c_int8)) if arr is not None else None)
    h._keep = arr  # the flags must outlive the create call
    return h


class Model:
    """A tdf_model over device tensors named as in GGUF (``token_embd.weight``,
    ``blk.<i>.attn_q.weight``, ...).  ``tensors`` values are torch device
    tensors (kept alive here) or raw device addresses.  ``dry_run`` makes a
    model whose weights are never read (for bookkeeping-only contexts)."""

    def __init__(self, hp: dict, tensors: Optional[Dict[str, object]] = None, dry_run: bool = False):
        self.hp = dict(hp)
        self._keep = tensors
        L = hp["n_layer"]

        def addr(name):
            if dry_run:
                return 0x1000
            t = tensors.get(name) if tensors is not None else None
            if t is None:
                return None
            return t if isinstance(t, int) else t.data_ptr()

        self._layers = (tdf_layer_weights * max(1, L))()
        for l in range(L):
            p = f"blk.{l}."
            self._layers[l] = tdf_layer_weights(*[addr(p + n) for n in (
                "attn_norm.weight", "attn_q.weight", "attn_k.weight", "attn_v.weight", "attn_output.weight",
                "ffn_norm.weight", "ffn_gate.weight", "ffn_up.weight", "ffn_down.weight")])
        out = None if (hp.get("tied") and not dry_run) else addr("output.weight")
        w = tdf_weights(addr("token_embd.weight"), addr("output_norm.weight"), out, self._layers)
        self.handle = tdf_model_create(_hparams(hp), w)
        if not self.handle:
            raise RuntimeError("tdf_model_create failed: " + tdf_last_error())

    def close(self):
        if getattr(self, "handle", None):
            tdf_model_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _i32_array(values) -> ctypes.Array:
    a = np.ascontiguousarray(np.asarray(values, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.POINTER(_i32))


class Context:
    def __init__(self, model: Model, n_ctx: int, n_batch: Optional[int] = None, n_ubatch: int = 512,
                 n_seq_max: int = 1, kv_dtype: str = "bf16", output_all: bool = False,
                 stream: Optional[int] = None, dry_run: bool = False, profile: bool = False):
        self.model = model
        flags = (TDF_CTX_DRY_RUN if dry_run else 0) | (TDF_CTX_PROFILE if profile else 0)
        p = tdf_context_params(n_ctx, n_batch if n_batch is not None else n_ctx, n_ubatch, n_seq_max,
                               DTYPES[kv_dtype], int(output_all), flags, stream)
        self.handle = tdf_context_create(model.handle, p)
        if not self.handle:
            raise RuntimeError("tdf_context_create failed: " + tdf_last_error())
        self.n_vocab = model.hp["n_vocab"]
        self.last_n_tokens = 0

    def close(self):
        if getattr(self, "handle", None):
            tdf_context_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def decode(self, tokens: Sequence[int], pos=None, seq_ids=None, logits=None) -> int:
        n = len(tokens)
        keep = []
        tok, tp = _i32_array(tokens)
        keep.append(tok)
        b = tdf_batch()
        b.n_tokens = n
        b.token = tp
        if pos is not None:
            pa, pp = _i32_array(pos)
            keep.append(pa)
            b.pos = pp
        if seq_ids is not None:
            ns, nsp = _i32_array([len(s) for s in seq_ids])
            keep.append(ns)
            rows = (ctypes.POINTER(_i32) * n)()
            for i, s in enumerate(seq_ids):
                a, ap = _i32_array(s if len(s) else [0])
                keep.append(a)
                rows[i] = ap
            keep.append(rows)
            b.n_seq_id = nsp
            b.seq_id = rows
        if logits is not None:
            la = np.ascontiguousarray(np.asarray(logits, dtype=np.int8))
            keep.append(la)
            b.logits = la.ctypes.data_as(ctypes.POINTER(ctypes.c_int8))
        rc = tdf_decode(self.handle, b)
        if rc == TDF_OK:
            self.last_n_tokens = n
        return rc

    def n_outputs(self) -> int:
        return lib().tdf_n_outputs(self.handle)

    def output_ids(self) -> list:
        n = self.n_outputs()
        out = (_i32 * max(1, n))()
        lib().tdf_output_ids(self.handle, out)
        return list(out[:n])

    def logits_ith(self, i: int) -> Optional[np.ndarray]:
        p = lib().tdf_get_logits_ith(self.handle, i)
        if not p:
            return None
        return np.ctypeslib.as_array(p, shape=(self.n_vocab,)).copy()

    def logits_device_ptr(self) -> int:
        return lib().tdf_get_logits_device(self.handle) or 0

    def argmax_ith(self, i: int) -> int:
        return lib().tdf_argmax_ith(self.handle, i)

    def seq_pos_max(self, s: int) -> int:
        return lib().tdf_seq_pos_max(self.handle, s)

    def kv_clear(self) -> int:
        return lib().tdf_kv_clear(self.handle)

    def kv_cell(self, cell: int):
        p, m = _i32(), _u64()
        rc = lib().tdf_kv_cell(self.handle, cell, ctypes.byref(p), ctypes.byref(m))
        if rc != TDF_OK:
            raise IndexError(cell)
        return p.value, m.value

    def last_slots(self) -> list:
        n = self.last_n_tokens
        out = (_i32 * max(1, n))()
        n = lib().tdf_last_slots(self.handle, out)
        return list(out[:n])

    def profile(self) -> dict:
        """{(op name, "mfma"|"decode"): (launches, total ms)} for profiled contexts."""
        out = {}
        for i, name in enumerate(OPS):
            for mfma in (0, 1):
                n, ms = ctypes.c_int64(), ctypes.c_double()
                if lib().tdf_profile_read(self.handle, i, mfma, ctypes.byref(n), ctypes.byref(ms)) == TDF_OK \
                        and n.value:
                    out[(name, "mfma" if mfma else "decode")] = (n.value, ms.value)
        return out

    def graph_counts(self):
        """(captures, replays) of the decode launch graphs."""
        cap, rep = ctypes.c_int64(), ctypes.c_int64()
        lib().tdf_graph_counts(self.handle, ctypes.byref(cap), ctypes.byref(rep))
        return cap.value, rep.value

    def sample(self, temperature: float, top_k: int = 40, top_p: float = 1.0, min_p: float = 0.0,
               u: Optional[Sequence[float]] = None):
        """One token per output row of the last decode (tdf_sample); u: one
        uniform number in [0, 1) per row.  Returns (rc, tokens)."""
        n = self.n_outputs()
        ua = (_f32 * max(1, n))(*([0.0] * n if u is None else [float(x) for x in u]))
        out = (_i32 * max(1, n))()
        p = tdf_sampling(float(temperature), int(top_k), float(top_p), float(min_p))
        rc = lib().tdf_sample(self.handle, ctypes.byref(p), ua, out)
        return rc, list(out)[:n]

    def sample_logits(self, logits_ptr: int, n_rows: int, n_vocab: int, temperature: float, top_k: int = 40,
                      top_p: float = 1.0, min_p: float = 0.0, u: Optional[Sequence[float]] = None):
        """The same chain on n_rows rows of n_vocab float32 logits at the
        device address logits_ptr (tdf_sample_logits).  Returns (rc, tokens)."""
        n = int(n_rows)
        ua = (_f32 * max(1, n))(*([0.0] * n if u is None else [float(x) for x in u]))
        out = (_i32 * max(1, n))()
        p = tdf_sampling(float(temperature), int(top_k), float(top_p), float(min_p))
        rc = lib().tdf_sample_logits(self.handle, ctypes.c_void_p(int(logits_ptr)), n, int(n_vocab),
                                     ctypes.byref(p), ua, out)
        return rc, list(out)[:n]

    def kv_seq_rm(self, seq: int, p0: int, p1: int) -> int:
        return lib().tdf_kv_seq_rm(self.handle, seq, p0, p1)

    def kv_seq_shift(self, seq: int, p0: int, p1: int, delta: int) -> int:
        return lib().tdf_kv_seq_shift(self.handle, seq, p0, p1, delta)

    def time_op(self, op: str, n_tokens: int, reps: int) -> float:
        """Mean duration (us) of `reps` back-to-back launches of one linear layer
        (op "gate_up", "down" or "lm_head") for n_tokens rows; tdf_time_op."""
        us = ctypes.c_double()
        rc = lib().tdf_time_op(self.handle, OPS.index(op), n_tokens, reps, ctypes.byref(us))
        if rc != TDF_OK:
            raise RuntimeError(f"tdf_time_op failed ({rc}): {tdf_last_error()}")
        return us.value

    def profile_reset(self) -> int:
        return lib().tdf_profile_reset(self.handle)

    def kv_import(self, seq: int, pos0: int, n: int, k_ptrs: Sequence[int], v_ptrs: Sequence[int]) -> int:
        L = max(1, len(k_ptrs))
        ka = (_vp * L)(*k_ptrs) if len(k_ptrs) else (_vp * 1)()
        va = (_vp * L)(*v_ptrs) if len(v_ptrs) else (_vp * 1)()
        rc = lib().tdf_kv_import(self.handle, seq, pos0, n, ka, va)
        if rc == TDF_OK:
            self.last_n_tokens = n
        return rc
