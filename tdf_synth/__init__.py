"""Seeded synthetic inputs shared by the CPU oracle and the GPU path's tests.

This module only makes numbers: weights, prompts, lengths, cache fills and
logits rows, each a pure function of (seed, name, element index).  It holds no step
of the decoder forward pass.  The generator itself is C (``synth.c``) so that
an 8B- or 70B-shaped model can be produced in seconds with OpenMP; this file
loads it with ctypes and wraps it in numpy.

Tensor names follow the GGUF naming used by the Ollama engine's reflection
binding (page "Inside the inference engine: model architectures and the
forward pass", section on reflection-based model initialisation):
``token_embd.weight``, ``output_norm.weight``, ``output.weight`` and
``blk.<i>.{attn_norm,attn_q,attn_k,attn_v,attn_output,ffn_norm,ffn_gate,
ffn_up,ffn_down}.weight``.  Matrices are row-major ``[out][in]``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libtdfsynth.so")
_lib = None

WEIGHT_STD = 0.02  # N(0, 0.02): standard deviation 0.02


def build(force: bool = True) -> str:
    """Compile synth.c into libtdfsynth.so next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64, f64 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double
        vp = ctypes.c_void_p
        lib.tdfs_fnv1a64.restype = u64
        lib.tdfs_fnv1a64.argtypes = [ctypes.c_char_p]
        lib.tdfs_stream_key.restype = u64
        lib.tdfs_stream_key.argtypes = [u64, ctypes.c_char_p]
        lib.tdfs_word.restype = u64
        lib.tdfs_word.argtypes = [u64, u64]
        lib.tdfs_normal_f32.argtypes = [u64, u64, i64, f64, vp]
        lib.tdfs_normal_bf16.argtypes = [u64, u64, i64, f64, vp]
        lib.tdfs_uniform_i32.argtypes = [u64, u64, i64, i64, i64, vp]
        lib.tdfs_f32_to_bf16.argtypes = [vp, i64, vp]
        lib.tdfs_normal_q8_0.argtypes = [u64, i64, i64, f64, vp, vp]
        _lib = lib
    return _lib


def stream_key(seed: int, name: str) -> int:
    return _load().tdfs_stream_key(seed, name.encode())


def words(seed: int, name: str, n: int, first: int = 0) -> np.ndarray:
    """Raw 64-bit counter words (for tests of the stream definition)."""
    lib = _load()
    key = lib.tdfs_stream_key(seed, name.encode())
    return np.array([lib.tdfs_word(key, first + i) for i in range(n)], dtype=np.uint64)


def normal(seed: int, name: str, n: int, std: float = 1.0, dtype: str = "f32", first: int = 0) -> np.ndarray:
    """``n`` draws of fp32(std * N(0,1)) from stream (seed, name), starting at ``first``.

    dtype "f32" returns float32; "bf16" returns uint16 bf16 bit patterns.
    """
    lib = _load()
    key = lib.tdfs_stream_key(seed, name.encode())
    if dtype == "f32":
        out = np.empty(n, dtype=np.float32)
        lib.tdfs_normal_f32(key, first, n, std, out.ctypes.data)
    elif dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        lib.tdfs_normal_bf16(key, first, n, std, out.ctypes.data)
    else:
        raise ValueError(f"unsupported dtype {dtype!r}")
    return out


def normal_q8_0(seed: int, name: str, rows: int, K: int, std: float) -> np.ndarray:
    """The [rows][K] matrix of draws fp32(std * N(0,1)) of stream (seed, name)
    (element (r, k) is draw r*K + k, as ``normal``) stored as Q8_0: per block
    of 32 consecutive elements of a row a scale d = fp16(max|w| / 127) and
    q = round-to-nearest-even(w / d) in [-127, 127].  Returned as one uint8
    buffer: rows*K int8 values q (row-major) followed by rows*K/32 fp16 scales
    (row-major [rows][K/32])."""
    if K % 32:
        raise ValueError("Q8_0 rows must be a multiple of 32 long")
    lib = _load()
    key = lib.tdfs_stream_key(seed, name.encode())
    out = np.empty(rows * K + rows * (K // 32) * 2, dtype=np.uint8)
    lib.tdfs_normal_q8_0(key, rows, K, std, out.ctypes.data, out[rows * K:].ctypes.data)
    return out


def uniform_int(seed: int, name: str, n: int, lo: int, hi: int, first: int = 0) -> np.ndarray:
    """``n`` integers uniform on [lo, hi] (inclusive) from stream (seed, name)."""
    if hi < lo:
        raise ValueError("empty range")
    lib = _load()
    key = lib.tdfs_stream_key(seed, name.encode())
    out = np.empty(n, dtype=np.int32)
    lib.tdfs_uniform_i32(key, first, n, lo, hi, out.ctypes.data)
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().tdfs_f32_to_bf16(x.ctypes.data, x.size, out.ctypes.data)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# Model shapes and workloads.  Each is a Llama-class decoder as named on the
# pages (page "romankryvolapov.com/ru/llama-cpp", preface: Llama/Qwen/Gemma
# class models; hyper-parameters as listed in "Step 4: loading
# hyper-parameters").  eps is 1e-5 everywhere; gains are exactly 1.0.
# ---------------------------------------------------------------------------

CONFIGS = {
    "tiny": dict(
        n_vocab=512, n_embd=64, n_layer=2, n_head=4, n_head_kv=2, head_dim=16, n_ff=172,
        rms_eps=1e-5, rope_theta=10000.0, tied=True, weight_dtype="f32", kv_dtype="f32",
        n_ctx=64, n_ubatch=512, seed=1, prompt_len=16, decode_steps=16,
    ),
    "llama1b": dict(
        n_vocab=128256, n_embd=2048, n_layer=16, n_head=32, n_head_kv=8, head_dim=64, n_ff=8192,
        rms_eps=1e-5, rope_theta=500000.0, tied=False, weight_dtype="bf16", kv_dtype="f16",
        n_ctx=4096, n_ubatch=512, seed=2, prompt_len=512, decode_steps=128,
    ),
    "llama8b": dict(
        n_vocab=128256, n_embd=4096, n_layer=32, n_head=32, n_head_kv=8, head_dim=128, n_ff=14336,
        rms_eps=1e-5, rope_theta=500000.0, tied=False, weight_dtype="bf16", kv_dtype="bf16",
        n_ctx=8192, n_ubatch=512, seed=3, prompt_len=2048, decode_steps=256,
    ),
    "llama8b_multiseq": dict(
        n_vocab=128256, n_embd=4096, n_layer=32, n_head=32, n_head_kv=8, head_dim=128, n_ff=14336,
        rms_eps=1e-5, rope_theta=500000.0, tied=False, weight_dtype="bf16", kv_dtype="bf16",
        n_ctx=32 * (8192 + 64), n_ubatch=512, seed=4, n_seqs=32, len_lo=1024, len_hi=8192,
        decode_steps=64,
    ),
    "llama70b": dict(
        n_vocab=128256, n_embd=8192, n_layer=80, n_head=64, n_head_kv=8, head_dim=128, n_ff=28672,
        rms_eps=1e-5, rope_theta=500000.0, tied=False, weight_dtype="bf16", kv_dtype="bf16",
        n_ctx=32768, n_ubatch=512, seed=5, prompt_len=4096, decode_windows=(4096, 16384, 32752),
        window_steps=16,
    ),
}


def hparams(cfg: dict) -> dict:
    keys = ("n_vocab", "n_embd", "n_layer", "n_head", "n_head_kv", "head_dim", "n_ff",
            "rms_eps", "rope_theta", "tied", "weight_dtype")
    out = {k: cfg[k] for k in keys}
    if cfg.get("n_swa"):
        out["n_swa"] = int(cfg["n_swa"])
        out["swa_layers"] = cfg.get("swa_layers")
    return out


def derive(cfg: dict, **overrides) -> dict:
    """A copy of ``cfg`` with some fields replaced (e.g. fewer layers)."""
    out = dict(cfg)
    out.update(overrides)
    return out


def tensor_shapes(cfg: dict, layer: int | None = None) -> dict:
    """Row-major [out][in] shapes of the tensors of one layer, or of the globals."""
    d, hd, F = cfg["n_embd"], cfg["head_dim"], cfg["n_ff"]
    H, Hkv, V = cfg["n_head"], cfg["n_head_kv"], cfg["n_vocab"]
    if layer is None:
        shapes = {"token_embd.weight": (V, d), "output_norm.weight": (d,)}
        if not cfg["tied"]:
            shapes["output.weight"] = (V, d)
        return shapes
    p = f"blk.{layer}."
    return {
        p + "attn_norm.weight": (d,),
        p + "attn_q.weight": (H * hd, d),
        p + "attn_k.weight": (Hkv * hd, d),
        p + "attn_v.weight": (Hkv * hd, d),
        p + "attn_output.weight": (d, H * hd),
        p + "ffn_norm.weight": (d,),
        p + "ffn_gate.weight": (F, d),
        p + "ffn_up.weight": (F, d),
        p + "ffn_down.weight": (d, F),
    }


def make_tensor(cfg: dict, name: str, shape: tuple) -> np.ndarray:
    """One tensor: norm gains are exactly 1.0 (fp32) unless the config sets
    ``gain_std`` (then 1 + N(0, gain_std) in fp32); matrices N(0, weight_std)
    (default 0.02) in the config's weight dtype (float32, uint16 bf16 bits, or
    the uint8 Q8_0 buffer of ``normal_q8_0``)."""
    n = int(np.prod(shape))
    if name.endswith("norm.weight"):
        gs = cfg.get("gain_std", 0.0)
        if not gs:
            return np.ones(shape, dtype=np.float32)
        return (1.0 + normal(cfg["seed"], name, n, gs, "f32").astype(np.float64)).astype(np.float32).reshape(shape)
    std = cfg.get("weight_std", WEIGHT_STD)
    if cfg["weight_dtype"] == "q8_0":
        return normal_q8_0(cfg["seed"], name, shape[0], shape[1], std)
    return normal(cfg["seed"], name, n, std, cfg["weight_dtype"]).reshape(shape)


def make_globals(cfg: dict) -> dict:
    return {n: make_tensor(cfg, n, s) for n, s in tensor_shapes(cfg).items()}


def make_layer(cfg: dict, layer: int) -> dict:
    return {n: make_tensor(cfg, n, s) for n, s in tensor_shapes(cfg, layer).items()}


def make_all(cfg: dict) -> dict:
    """Every tensor of the model (small models only)."""
    out = make_globals(cfg)
    for l in range(cfg["n_layer"]):
        out.update(make_layer(cfg, l))
    return out


def prompt(cfg: dict, seq: int, length: int) -> np.ndarray:
    """Uniform-random token ids in [0, n_vocab) for sequence ``seq``."""
    return uniform_int(cfg["seed"], f"prompt.{seq}", length, 0, cfg["n_vocab"] - 1)


def seq_lengths(cfg: dict) -> np.ndarray:
    """Multi-sequence prompt lengths, uniform on [len_lo, len_hi] inclusive."""
    return uniform_int(cfg["seed"], "lengths", cfg["n_seqs"], cfg["len_lo"], cfg["len_hi"])


def kv_fill(cfg: dict, layer: int, which: str, pos0: int, pos1: int, dtype: str) -> np.ndarray:
    """Synthetic cache contents N(0,1) for positions [pos0, pos1) of one layer,
    shaped [pos][n_head_kv][head_dim]; element (p, h, i) is index
    (p * n_head_kv + h) * head_dim + i of stream "kvfill.<which>.<layer>"."""
    Hkv, hd = cfg["n_head_kv"], cfg["head_dim"]
    n = (pos1 - pos0) * Hkv * hd
    vals = normal(cfg["seed"], f"kvfill.{which}.{layer}", n, 1.0, dtype, first=pos0 * Hkv * hd)
    return vals.reshape(pos1 - pos0, Hkv, hd)


def logit_rows(seed: int, kind: str, n_rows: int, n_vocab: int) -> np.ndarray:
    """float32 rows of synthetic logits [n_rows][n_vocab] with a chosen
    structure: "normal" N(0, 2); "coarse" N(0, 1) rounded to whole numbers
    (large groups of equal values); "comb" N(0, 1) with 10 + N(0, 1) at the
    evenly spaced ids floor(t * n_vocab / 1024), t < 1024; "masked" N(0, 2)
    with every other id set to -inf."""
    n = n_rows * n_vocab
    z = normal(seed, f"logits.{kind}", n, 1.0).astype(np.float64).reshape(n_rows, n_vocab)
    if kind == "normal":
        out = 2.0 * z
    elif kind == "coarse":
        out = np.rint(z)
    elif kind == "comb":
        out = z.copy()
        ids = (np.arange(1024, dtype=np.int64) * n_vocab) // 1024
        out[:, ids] = 10.0 + normal(seed, "logits.comb.peaks", n_rows * ids.size, 1.0).reshape(n_rows, -1)
    elif kind == "masked":
        out = 2.0 * z
        out[:, 1::2] = -np.inf
    else:
        raise ValueError(kind)
    return out.astype(np.float32)
