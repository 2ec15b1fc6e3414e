"""Per-site precision study of the prefill path (a measurement script, not a
test: pytest does not collect it).

The decoder forward pass (Ollama engine page, "Deep dive: the Llama forward
pass in Go") is computed in float64 exactly as the oracle computes it, with
the cache holding K/V rounded to the cache type (bf16), and with ONE
rounding inserted at a chosen site of every layer: the input of a matrix
product, or the query / probabilities of the attention.  The logits of
sampled prompt rows are compared with the unrounded computation, which is
the oracle's result (``--check`` verifies that on a two-layer model against
``oracle.OracleContext``).  The study shows which inputs of the prefill's
matrix-core products need more than one bf16 rounding to stay within the
logits tolerance (max-abs 3e-2, rel-L2 1e-2) at full depth.

Sites (per layer):
  qkv_in    attention RMSNorm output, input of the Q/K/V projection
  q         rotated query entering the scores
  p         softmax probabilities entering the product with V
  wo_in     attention output, input of the output projection
  gu_in     FFN RMSNorm output, input of the gate/up projection
  down_in   SwiGLU product, input of the down projection
Formats: bf16 (round to nearest even via float32), f16 (round to nearest
even), pair (bf16 hi + bf16 lo of the remainder: about 16 significant bits).

    python tests/precision_study.py --layers 32 --prompt 512
    python tests/precision_study.py --check
"""
from __future__ import annotations

import argparse
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import tdf_synth  # noqa: E402
from oracle.ops import rms_norm, rope, silu  # noqa: E402

SITES = ("qkv_in", "q", "p", "wo_in", "gu_in", "down_in")


def to_bf16(a):
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32)
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


def rounder(fmt):
    if fmt is None:
        return lambda a: a
    if fmt == "bf16":
        return to_bf16
    if fmt == "f16":
        return lambda a: np.asarray(a, dtype=np.float64).astype(np.float16).astype(np.float64)
    if fmt == "pair":
        def pair(a):
            hi = to_bf16(a)
            return hi + to_bf16(np.asarray(a, dtype=np.float64) - hi)
        return pair
    raise ValueError(fmt)


def wide(bits):
    return tdf_synth.bf16_bits_to_f32(bits).astype(np.float64)


class Variant:
    """fmts: site -> format; optional keys "layers" (range of layers the
    roundings apply to; all by default), "base" (format of every site outside
    that range; exact by default) and "cache" ("f64": keep K/V unrounded, the
    storage rounding switched off)."""

    def __init__(self, name, fmts, cfg, tokens, emb):
        self.name = name
        fmts = dict(fmts)
        self.layers = fmts.pop("layers", None)
        base = fmts.pop("base", None)
        self.cache_f64 = fmts.pop("cache", None) == "f64"
        self.r_in = {s: rounder(fmts.get(s)) for s in SITES}
        self.r_out = {s: rounder(base) for s in SITES}
        self.x = emb.copy()
        self.cfg = cfg

    def layer(self, W, l, pos):
        self.r = self.r_in if self.layers is None or l in self.layers else self.r_out
        cfg = self.cfg
        H, Hkv, hd = cfg["n_head"], cfg["n_head_kv"], cfg["head_dim"]
        eps, theta = cfg["rms_eps"], cfg["rope_theta"]
        P = self.x.shape[0]
        p = f"blk.{l}."
        h = self.r["qkv_in"](rms_norm(self.x, W[p + "attn_norm.weight"], eps))
        q = rope((h @ W[p + "attn_q.weight"].T).reshape(P, H, hd), pos, theta)
        k = rope((h @ W[p + "attn_k.weight"].T).reshape(P, Hkv, hd), pos, theta)
        v = (h @ W[p + "attn_v.weight"].T).reshape(P, Hkv, hd)
        if not self.cache_f64:
            k, v = to_bf16(k), to_bf16(v)     # the bf16 cache
        q = self.r["q"](q)
        G = H // Hkv
        o = np.empty((P, H, hd))
        mask = np.triu(np.ones((P, P), dtype=bool), 1)
        for g in range(Hkv):
            qg = q[:, g * G:(g + 1) * G, :].transpose(1, 0, 2)          # [G][P][hd]
            s = qg @ k[:, g, :].T / np.sqrt(hd)                           # [G][P][P]
            s[:, mask] = -np.inf
            a = np.exp(s - s.max(axis=-1, keepdims=True))
            a /= a.sum(axis=-1, keepdims=True)
            a = self.r["p"](a)
            o[:, g * G:(g + 1) * G, :] = (a @ v[:, g, :]).transpose(1, 0, 2)
        o = self.r["wo_in"](o.reshape(P, H * hd))
        self.x = self.x + o @ W[p + "attn_output.weight"].T
        h2 = self.r["gu_in"](rms_norm(self.x, W[p + "ffn_norm.weight"], eps))
        m = silu(h2 @ W[p + "ffn_gate.weight"].T) * (h2 @ W[p + "ffn_up.weight"].T)
        self.x = self.x + self.r["down_in"](m) @ W[p + "ffn_down.weight"].T


def run(cfg, P, variants, rows, log=print):
    toks = tdf_synth.prompt(cfg, 0, P)
    g = tdf_synth.make_globals(cfg)
    emb = wide(g["token_embd.weight"][toks])
    pos = np.arange(P)
    vs = [Variant(n, f, cfg, toks, emb) for n, f in variants]
    t0 = time.time()
    for l in range(cfg["n_layer"]):
        W = {n: (wide(a) if a.dtype == np.uint16 else a.astype(np.float64))
             for n, a in tdf_synth.make_layer(cfg, l).items()}
        for v in vs:
            v.layer(W, l, pos)
        log(f"layer {l} done ({time.time() - t0:.0f}s)", flush=True)
    out = g["output.weight"] if not cfg["tied"] else g["token_embd.weight"]
    gain = g["output_norm.weight"].astype(np.float64)
    res = {}
    for v in vs:
        hn = rms_norm(v.x[rows], gain, cfg["rms_eps"])
        logits = np.empty((len(rows), cfg["n_vocab"]))
        for c0 in range(0, cfg["n_vocab"], 16384):
            logits[:, c0:c0 + 16384] = hn @ wide(out[c0:c0 + 16384]).T
        res[v.name] = logits
    return res


def check():
    """The unrounded study forward equals the oracle (two full-width layers)."""
    from oracle import OracleContext, OracleModel
    cfg = dict(tdf_synth.CONFIGS["llama8b"], n_layer=2)
    P = 96
    res = run(cfg, P, [("exact", {})], [P - 1], log=lambda s, **k: None)["exact"][0]
    w = tdf_synth.make_all(cfg)
    oc = OracleContext(OracleModel(tdf_synth.hparams(cfg), w), n_ctx=256, kv_dtype="bf16")
    r = oc.decode(tdf_synth.prompt(cfg, 0, P))
    err = float(np.max(np.abs(res - r.logits[0])))
    print(f"study forward vs oracle, 2 layers, {P} tokens: max-abs {err:.2e}")
    assert err < 1e-9


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--prompt", type=int, default=512)
    ap.add_argument("--check", action="store_true")
    ap.add_argument("--set", default="sites", choices=["sites", "designs", "depth"])
    a = ap.parse_args()
    if a.check:
        check()
        return
    cfg = dict(tdf_synth.CONFIGS["llama8b"], n_layer=a.layers)
    if a.set == "sites":
        variants = [("exact", {})]
        variants += [(f"{s} bf16", {s: "bf16"}) for s in SITES]
        variants += [(f"{s} f16", {s: "f16"}) for s in ("qkv_in", "wo_in", "gu_in", "down_in")]
        variants += [("all bf16", {s: "bf16" for s in SITES}), ("all pair", {s: "pair" for s in SITES})]
    elif a.set == "depth":
        L = a.layers
        allb = {s: "bf16" for s in SITES}
        variants = [("exact", {})]
        variants += [("f64 cache (no storage rounding)", {"cache": "f64"})]
        variants += [("all pair", {s: "pair" for s in SITES})]
        for lo, hi in ((0, L // 4), (L // 4, L // 2), (L // 2, 3 * L // 4), (3 * L // 4, L),
                       (L - L // 8, L)):
            variants += [(f"bf16 layers {lo}-{hi - 1}, pair else", dict(allb, layers=range(lo, hi), base="pair"))]
        mm = ("wo_in", "gu_in", "down_in")
        variants += [("mm f16, qkv/q/p pair", dict({s: "f16" for s in mm}, qkv_in="pair", q="pair", p="pair"))]
    else:
        mm = ("wo_in", "gu_in", "down_in")
        variants = [("exact", {})]
        variants += [("qkv pair, q/p pair, rest f16", dict({s: "f16" for s in mm}, qkv_in="pair", q="pair", p="pair"))]
        variants += [("qkv pair, q/p bf16, rest f16", dict({s: "f16" for s in mm}, qkv_in="pair", q="bf16", p="bf16"))]
        variants += [("all f16, q/p pair", dict({s: "f16" for s in mm}, qkv_in="f16", q="pair", p="pair"))]
        variants += [("qkv pair, q/p pair, rest bf16", dict({s: "bf16" for s in mm}, qkv_in="pair", q="pair", p="pair"))]
    P = a.prompt
    rows = sorted(set([P // 8 * i - 1 for i in range(1, 9)]))
    res = run(cfg, P, variants, rows)
    ref = res["exact"]
    print(f"\n8B width, {a.layers} layers, {P}-token prompt, rows {rows}")
    print(f"{'variant':34s} {'max-abs':>10s} {'rel-L2':>10s}   (worst row; tolerance 3e-2 / 1e-2)")
    for name, _ in variants[1:]:
        d = res[name] - ref
        ma = float(np.max(np.abs(d)))
        rel = float(np.max(np.linalg.norm(d, axis=1) / np.linalg.norm(ref, axis=1)))
        print(f"{name:34s} {ma:10.2e} {rel:10.2e}")


if __name__ == "__main__":
    main()
