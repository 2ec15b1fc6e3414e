"""Benchmark of the decoder forward pass on one MI355X.

Workload (8B-class Llama shape, bf16 weights N(0, 0.02), bf16 KV cache of
8192 cells): a 2048-token uniform-random prompt decoded in ubatches of 512
with logits for the last position only (prefill), then greedy decode steps of
one token each, every step feeding back the GPU's own argmax.

A timed "step" is one decode call: the whole forward pass for one token
(embedding, 32 layers, output norm, LM head, device argmax, 4-byte token
readback), replayed as a HIP graph.  ``value`` is decode tokens/s; the
prefill rate of the same model is reported beside it.  ``roofline`` covers
the dominant decode kernel (the fused gate/up GEMV) and ``roofline_prefill``
the dominant prefill kernel (the gate/up MFMA GEMM): their average launch
durations come from tdf_time_op, back-to-back launches of that kernel on the
library's stream between two HIP events, cycling over the 32 layers' weights.
``traffic`` is read from the committed rocprofv3 counter summary of that
kernel when the kernel source still matches it (else null).
``multiseq`` (32 sequences in lock-step steps, same weights) and ``llama1b``
(the 1B shape, its own weights) are compact sections of other workloads.
``kernels`` is a per-operation breakdown from an eager repeat with a HIP
event pair around every launch (it includes the events' own overhead):
``prefill`` covers the prompt, ``decode`` the timed single-token steps.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-peaks]
    python bench.py --calibrate-copy     # plain 1 GiB device copy, for counter scaling
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16
COPY_BYTES = 1 << 30         # calibration copy: 1 GiB read + 1 GiB written
TRAFFIC_FILES = {"decode": "profiles/gemv_gate_up_decode_llama8b_traffic.json",
                 "prefill": "profiles/gemm_gate_up_prefill512_llama8b_traffic.json",
                 "decode_q8_0": "profiles/gemv_gate_up_decode_llama8b_q8_0_traffic.json",
                 "prefill_q8_0": "profiles/gemm_gate_up_prefill512_llama8b_q8_0_traffic.json"}
KERNEL_SOURCES = {"decode": "transformer_decode_forward_amd/csrc/k_decode.hip",
                  "prefill": "transformer_decode_forward_amd/csrc/k_gemm.hip",
                  "decode_q8_0": "transformer_decode_forward_amd/csrc/k_decode.hip",
                  "prefill_q8_0": "transformer_decode_forward_amd/csrc/k_gemm.hip"}
# rocprofv3 matrix-core counters of the prefill kernels (GEMMs and attention)
MFMA_FILES = {"prefill": "profiles/llama8b_prefill_mfma.json",
              "prefill_q8_0": "profiles/llama8b_q8_0_prefill_mfma.json"}


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def build_model(cfg, keep_host=True):
    import tdf_synth
    import transformer_decode_forward_amd as tdf
    from transformer_decode_forward_amd.device import to_device
    host, dev = {}, {}
    names = list(tdf_synth.tensor_shapes(cfg).items())
    for l in range(cfg["n_layer"]):
        names += list(tdf_synth.tensor_shapes(cfg, l).items())
    t0 = time.time()
    for i, (name, shape) in enumerate(names):
        a = tdf_synth.make_tensor(cfg, name, shape)
        if keep_host:
            host[name] = a
        dev[name] = to_device(a)
        if i % 36 == 0:
            log(f"weights {i}/{len(names)} ({time.time() - t0:.0f}s)")
    return tdf.Model(tdf_synth.hparams(cfg), dev), host


def weight_bytes_per_element(cfg):
    """bf16: 2; float32: 4; Q8_0: 34 bytes per block of 32 (int8 + fp16 scale)."""
    return {"bf16": 2.0, "f32": 4.0, "q8_0": 34.0 / 32.0}[cfg["weight_dtype"]]


def kv_cell_bytes(cfg):
    """Bytes of one cached cell (K and V of every layer) in the cache type."""
    per = {"bf16": 2.0, "f16": 2.0, "f32": 4.0, "q8_0": 34.0 / 32.0}[cfg["kv_dtype"]]
    return cfg["n_layer"] * 2 * cfg["n_head_kv"] * cfg["head_dim"] * per


def decode_bytes(cfg, ctx_len):
    """Algorithmic HBM bytes of one single-token decode step at context ctx_len:
    every weight once, K/V of the visible cells, the new K/V, the logits."""
    d, H, Hkv, hd, F, V, L = (cfg[k] for k in ("n_embd", "n_head", "n_head_kv", "head_dim", "n_ff",
                                             "n_vocab", "n_layer"))
    p_layer = d * H * hd + 2 * d * Hkv * hd + H * hd * d + 3 * d * F
    weights = weight_bytes_per_element(cfg) * (L * p_layer + V * d)
    kv_cell = kv_cell_bytes(cfg)
    return weights + kv_cell * ctx_len + kv_cell + 4 * V


def prefill_flops(cfg, n_tok, n_ubatch, n_out_last=1):
    """Algorithmic FLOPs of the prompt: projections and MLP of every token
    (last layer's MLP only for output rows), causal attention pairs, LM head."""
    d, H, Hkv, hd, F, V, L = (cfg[k] for k in ("n_embd", "n_head", "n_head_kv", "head_dim", "n_ff",
                                             "n_vocab", "n_layer"))
    p_attn = d * H * hd + 2 * d * Hkv * hd + H * hd * d
    p_mlp = 3 * d * F
    fl = 2 * n_tok * L * (p_attn + p_mlp) - 2 * (n_tok - n_out_last) * p_mlp
    fl += 4 * H * hd * L * sum(p + 1 for p in range(n_tok))
    fl += 2 * n_out_last * V * d
    return fl


def source_hash(rel):
    import hashlib
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic(kind):
    """HBM bytes per launch from the committed counter summary, or None when
    the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, TRAFFIC_FILES[kind])
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kind]):
        return None
    return rec.get("traffic_bytes_per_launch")


def mfma_busy(kind):
    """MFMA-busy fraction of each prefill kernel (SQ_VALU_MFMA_BUSY_CYCLES over
    the SIMDs' active cycles) from the committed counter summary, or None when
    a kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, MFMA_FILES[kind])
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if any(h != source_hash(src) for src, h in rec.get("sources", {}).items()):
        return None
    return {k: v["mfma_busy"] for k, v in rec["kernels"].items()}


def calibrate_copy():
    """A plain device-to-device copy of COPY_BYTES (4 launches), so that the
    FETCH_SIZE / WRITE_SIZE counters can be scaled by a transfer of known size."""
    import torch
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(4):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copied {COPY_BYTES} bytes 4 times")


def measured_peaks():
    """Practical peaks on this GPU: a device copy (bytes read + written) and a
    large bf16 GEMM from the vendor library (torch.matmul), for context."""
    import torch
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        b.copy_(a)
    s.record()
    for _ in range(10):
        b.copy_(a)
    e.record()
    e.synchronize()
    copy_gbs = 10 * 2 * COPY_BYTES / (s.elapsed_time(e) * 1e-3) / 1e9
    del a, b
    n = 8192
    x = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    y = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(2):
        torch.matmul(x, y)
    s.record()
    for _ in range(10):
        torch.matmul(x, y)
    e.record()
    e.synchronize()
    gemm_tfs = 10 * 2 * n ** 3 / (s.elapsed_time(e) * 1e-3) / 1e12
    return {"copy_GBs": round(copy_gbs, 1), "bf16_gemm_8192_TFLOPs": round(gemm_tfs, 1),
            "note": "torch device copy (read + write bytes) and torch.matmul bf16 8192^3 (hipBLASLt)"}


def cpu_baseline(cfg, host_weights, ctx_len):
    """The oracle, as it stands, on a bounded sample: one decode step of the
    same model at context ctx_len (the cache restored from synthetic
    post-RoPE K/V, since replaying the prompt on the CPU would take hours)."""
    import tdf_synth
    from oracle import OracleContext, OracleModel
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 0) for i in threadpool_info()) or None
    except Exception:
        pass
    m = OracleModel(tdf_synth.hparams(cfg), host_weights, cache=False)
    oc = OracleContext(m, n_ctx=ctx_len + 8)
    L = cfg["n_layer"]
    rc = oc.kv_import(0, 0, ctx_len, lambda l: tdf_synth.kv_fill(cfg, l, "k", 0, ctx_len, "bf16"),
                      lambda l: tdf_synth.kv_fill(cfg, l, "v", 0, ctx_len, "bf16"))
    assert rc == 0
    tok = int(tdf_synth.prompt(cfg, 7, 1)[0])
    t0 = time.perf_counter()
    r = oc.decode([tok])
    dt = time.perf_counter() - t0
    assert r.status == 0 and r.logits.shape == (1, cfg["n_vocab"])
    # prefill: one ubatch of the prompt through the first layers only (the
    # whole prompt would take minutes), rate scaled to the full depth
    Lp, U = 2, cfg["n_ubatch"]
    pm = OracleModel(dict(tdf_synth.hparams(cfg), n_layer=Lp), host_weights, cache=False)
    pc = OracleContext(pm, n_ctx=U, n_ubatch=U)
    t0 = time.perf_counter()
    r = pc.decode(tdf_synth.prompt(cfg, 0, U))
    dtp = time.perf_counter() - t0
    assert r.status == 0
    pre_tps = U / (dtp * L / Lp)
    return {"value": 1.0 / dt, "unit": "decode tok/s", "cores": threads or os.cpu_count(),
            "kind": "oracle",
            "sample": f"1 decode step of the {L}-layer model at context {ctx_len} (cache restored "
                      f"from synthetic K/V), float64 numpy, {dt:.1f} s",
            "prefill": {"value": pre_tps, "unit": "prefill tok/s",
                        "sample": f"one {U}-token ubatch (positions 0..{U - 1}) through the first {Lp} of the "
                                  f"{L} layers plus the LM head row, {dtp:.1f} s, rate scaled by {L}/{Lp} "
                                  f"(the LM head is counted {L // Lp} times: an upper bound on the time)"}}


def decode_bytes_multi(cfg, ctxs):
    """Algorithmic bytes of one decode step of len(ctxs) tokens (one per
    sequence at the given contexts): weights once, each token's visible K/V,
    the new K/V and the logits rows."""
    d, H, Hkv, hd, F, V, L = (cfg[k] for k in ("n_embd", "n_head", "n_head_kv", "head_dim", "n_ff",
                                             "n_vocab", "n_layer"))
    p_layer = d * H * hd + 2 * d * Hkv * hd + H * hd * d + 3 * d * F
    kv_cell = kv_cell_bytes(cfg)
    return (weight_bytes_per_element(cfg) * (L * p_layer + V * d) + kv_cell * (sum(ctxs) + len(ctxs))
            + 4 * V * len(ctxs))


def run_multiseq(args, cfg, model=None, steps=None, warmup=None):
    """32 sequences sharing one cache: prompts of 1024..8192 tokens prefilled
    one call per sequence, then lock-step decode steps of 32 tokens (one per
    sequence, its own position and id), logits for all 32 rows.  ``model``:
    an uploaded model of the same shape to reuse (else one is made)."""
    import torch
    import tdf_synth
    import transformer_decode_forward_amd as tdf
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    S, lens = cfg["n_seqs"], tdf_synth.seq_lengths(cfg)
    if model is None:
        log(f"generating and uploading weights; {S} sequences, {int(lens.sum())} prompt tokens")
        model, _ = build_model(cfg, keep_host=False)
    ctx = tdf.Context(model, n_ctx=cfg["n_ctx"], n_batch=8192, n_ubatch=cfg["n_ubatch"], n_seq_max=S,
                      kv_dtype=cfg["kv_dtype"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(S):
        toks = tdf_synth.prompt(cfg, s, int(lens[s]))
        assert ctx.decode(toks, seq_ids=[[s]] * len(toks)) == 0, tdf.tdf_last_error()
    t_pre = time.perf_counter() - t0
    seq_ids = [[s] for s in range(S)]
    flags = np.ones(S, dtype=np.int8)
    toks = [ctx.argmax_ith(int(lens[S - 1]) - 1)] * S
    for _ in range(warmup):
        assert ctx.decode(toks, seq_ids=seq_ids, logits=flags) == 0, tdf.tdf_last_error()
        toks = [ctx.argmax_ith(i) for i in range(S)]
    ctx0 = [int(lens[s]) + warmup for s in range(S)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        assert ctx.decode(toks, seq_ids=seq_ids, logits=flags) == 0, tdf.tdf_last_error()
        toks = [ctx.argmax_ith(i) for i in range(S)]
    torch.cuda.synchronize()
    t_dec = time.perf_counter() - t0
    ctx.close()
    mean = [c + (steps - 1) / 2.0 for c in ctx0]
    step_bytes = decode_bytes_multi(cfg, mean)
    ms = 1000.0 * t_dec / steps
    tps = S * steps / t_dec
    log(f"prefill {lens.sum() / t_pre:.0f} tok/s, decode {tps:.1f} tok/s ({ms:.3f} ms per 32-token step)")
    return {
        "metric": ("decode tok/s (% HBM peak), 8B-shape bf16, 32 sequences" if cfg["weight_dtype"] == "bf16" else
                   f"decode tok/s (% HBM peak), 8B-shape {cfg['weight_dtype'].upper()} weights, 32 sequences")
                  + ("" if cfg["kv_dtype"] == "bf16" else f", {cfg['kv_dtype'].upper()} cache"),
        "value": round(tps, 2), "unit": "tok/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg["weight_dtype"] == "bf16" else f"f32 ({cfg['weight_dtype']} weights)",
        "data": "synthetic",
        "config": {"workload": f"llama8b_multiseq: {S} sequences, prompts {int(lens.min())}..{int(lens.max())} "
                               f"tokens prefilled per sequence, then lock-step steps of {S} tokens, all rows' logits; "
                               f"KV {cfg['kv_dtype']} {cfg['n_ctx']} cells"},
        "decode": {"tok_s": round(tps, 2), "sum_ctx_mean": round(sum(mean), 1),
                   "algorithmic_bytes_per_step": int(step_bytes),
                   "achieved_GBs": round(step_bytes / (ms * 1e-3) / 1e9, 1),
                   "frac_hbm_peak": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "prefill": {"tok_s": round(float(lens.sum()) / t_pre, 1), "tokens": int(lens.sum()),
                    "s": round(t_pre, 3)},
        "roofline": None, "cpu_baseline": None,
    }


def run_small(cfg, steps=64, warmup=8):
    """A compact single-sequence run of another shape (its own prompt in
    ubatches, then graph-replayed greedy decode steps): decode tok/s and
    fraction of the HBM peak, prefill tok/s and fraction of the MFMA peak."""
    import torch
    import tdf_synth
    import transformer_decode_forward_amd as tdf
    P, U = cfg["prompt_len"], cfg["n_ubatch"]
    model, _ = build_model(cfg, keep_host=False)
    ctx = tdf.Context(model, n_ctx=cfg["n_ctx"], n_ubatch=U, kv_dtype=cfg["kv_dtype"])
    prompt = tdf_synth.prompt(cfg, 0, P)
    for _ in range(2):  # the second prefill is timed
        ctx.kv_clear()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        assert ctx.decode(prompt) == 0, tdf.tdf_last_error()
        t_pre = time.perf_counter() - t0
    tok = ctx.argmax_ith(P - 1)
    for _ in range(warmup):
        assert ctx.decode([tok]) == 0, tdf.tdf_last_error()
        tok = ctx.argmax_ith(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        assert ctx.decode([tok]) == 0, tdf.tdf_last_error()
        tok = ctx.argmax_ith(0)
    torch.cuda.synchronize()
    t_dec = time.perf_counter() - t0
    ctx.close()
    del model
    mean_ctx = P + warmup + (steps - 1) / 2.0
    ms = 1000.0 * t_dec / steps
    step_bytes = decode_bytes(cfg, mean_ctx)
    flops = prefill_flops(cfg, P, U)
    return {"decode": {"tok_s": round(steps / t_dec, 2), "ms_per_step": round(ms, 4), "mean_ctx": mean_ctx,
                       "algorithmic_bytes_per_step": int(step_bytes),
                       "frac_hbm_peak": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "prefill": {"tok_s": round(P / t_pre, 1), "ms": round(1000 * t_pre, 3),
                        "frac_mfma_peak": round(flops / t_pre / 1e12 / MFMA_BF16_PEAK_TFS, 4)}}


def run_70b(args, cfg):
    """70B-class model on one GPU: 4096-token prompt in ubatches of 512, then
    decode windows at positions 4096, 16384 and 32752 (the cache filled up to
    each window start with synthetic N(0,1) post-RoPE K/V), 16 steps each."""
    import torch
    import tdf_synth
    import transformer_decode_forward_amd as tdf
    from transformer_decode_forward_amd.device import to_device
    P, U, L = cfg["prompt_len"], cfg["n_ubatch"], cfg["n_layer"]
    log("generating and uploading 70B weights (host copies dropped)")
    model, _ = build_model(cfg, keep_host=False)
    ctx = tdf.Context(model, n_ctx=cfg["n_ctx"], n_ubatch=U, kv_dtype=cfg["kv_dtype"])
    prompt = tdf_synth.prompt(cfg, 0, P)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    assert ctx.decode(prompt) == 0, tdf.tdf_last_error()
    t_pre = time.perf_counter() - t0
    pre_flops = prefill_flops(cfg, P, U)
    log(f"prefill {P / t_pre:.0f} tok/s ({pre_flops / t_pre / 1e12:.0f} TFLOP/s)")
    tok = ctx.argmax_ith(P - 1)
    windows = []
    steps = cfg["window_steps"]
    for w0 in cfg["decode_windows"]:
        have = ctx.seq_pos_max(0) + 1
        if w0 > have:
            ks = [to_device(tdf_synth.kv_fill(cfg, l, "k", have, w0, "bf16")) for l in range(L)]
            vs = [to_device(tdf_synth.kv_fill(cfg, l, "v", have, w0, "bf16")) for l in range(L)]
            assert ctx.kv_import(0, have, w0 - have, [t.data_ptr() for t in ks], [t.data_ptr() for t in vs]) == 0
            del ks, vs
        for _ in range(2):  # warm-up at the window (positions w0, w0+1)
            assert ctx.decode([tok]) == 0
            tok = ctx.argmax_ith(0)
        n = min(steps, cfg["n_ctx"] - (ctx.seq_pos_max(0) + 1))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            assert ctx.decode([tok]) == 0, tdf.tdf_last_error()
            tok = ctx.argmax_ith(0)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        c_mean = w0 + 2 + (n - 1) / 2.0
        b = decode_bytes(cfg, c_mean)
        windows.append({"window_start": w0, "steps": n, "tok_s": round(n / dt, 2),
                        "ms_per_step": round(1000 * dt / n, 3), "algorithmic_bytes_per_step": int(b),
                        "frac_hbm_peak": round(b / (dt / n) / 1e9 / HBM_PEAK_GBS, 4)})
        log(f"window {w0}: {n / dt:.2f} tok/s")
    ctx.close()
    first = windows[0]
    return {
        "metric": "decode tok/s (% HBM peak) + prefill tok/s (% MFMA peak), 70B-shape bf16",
        "value": first["tok_s"], "unit": "tok/s", "n_gpus": 1, "steps": first["steps"], "warmup": 2,
        "ms_per_step": first["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"llama70b: batch 1, {P}-token prompt in ubatches of {U}, decode windows at "
                               f"{list(cfg['decode_windows'])} (cache filled with synthetic K/V), KV bf16 "
                               f"{cfg['n_ctx']} cells"},
        "decode_windows": windows,
        "prefill": {"tok_s": round(P / t_pre, 1), "s": round(t_pre, 3),
                    "algorithmic_tflop": round(pre_flops / 1e12, 3),
                    "achieved_TFLOPs": round(pre_flops / t_pre / 1e12, 2),
                    "frac_mfma_peak": round(pre_flops / t_pre / 1e12 / MFMA_BF16_PEAK_TFS, 4)},
        "roofline": None, "cpu_baseline": None,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--prefill-reps", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--config", default="llama8b")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--no-multiseq", action="store_true",
                    help="skip the 32-sequence and 1B-shape sections of the default (8B) run")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--weights", choices=["bf16", "q8_0"], default=None,
                    help="weight storage of the single-sequence workload (default: the config's, bf16)")
    ap.add_argument("--kv", choices=["bf16", "f16", "q8_0"], default=None,
                    help="KV cache element type (default: the config's)")
    ap.add_argument("--swa", type=int, default=0,
                    help="sliding-window attention of this many positions on every layer (0: none)")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import tdf_synth
    import transformer_decode_forward_amd as tdf
    assert torch.cuda.is_available(), "no GPU"
    cfg = dict(tdf_synth.CONFIGS[args.config])
    if args.swa:
        cfg["n_swa"] = args.swa
    if args.weights:
        cfg["weight_dtype"] = args.weights
    if args.kv:
        cfg["kv_dtype"] = args.kv
    q8 = cfg["weight_dtype"] == "q8_0"
    if args.config == "llama8b_multiseq":
        print(json.dumps(run_multiseq(args, cfg)), flush=True)
        return
    if args.config == "llama70b":
        print(json.dumps(run_70b(args, cfg)), flush=True)
        return
    P, U, n_ctx = cfg["prompt_len"], cfg["n_ubatch"], cfg["n_ctx"]
    assert P + args.warmup + args.steps < n_ctx, "steps exceed the KV capacity"

    log(f"generating and uploading {args.config} weights")
    model, host = build_model(cfg)
    prompt = tdf_synth.prompt(cfg, 0, P)

    def run(ctx, steps, warm, on_prefilled=None, on_warm=None):
        # prefill: repeated on a cleared cache, the last repetition timed
        for _ in range(args.prefill_reps + 1):
            ctx.kv_clear()
            if on_prefilled:
                on_prefilled(None)  # drop the earlier repetitions' records
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            assert ctx.decode(prompt) == 0, tdf.tdf_last_error()
            t_pre = time.perf_counter() - t0
        if on_prefilled:
            on_prefilled(ctx)
        tok = ctx.argmax_ith(P - 1)
        for _ in range(warm):
            assert ctx.decode([tok]) == 0, tdf.tdf_last_error()
            tok = ctx.argmax_ith(0)
        torch.cuda.synchronize()
        if on_warm:
            on_warm()
        t0 = time.perf_counter()
        for _ in range(steps):
            assert ctx.decode([tok]) == 0, tdf.tdf_last_error()
            tok = ctx.argmax_ith(0)
        torch.cuda.synchronize()
        return t_pre, time.perf_counter() - t0

    log("timed run")
    ctx = tdf.Context(model, n_ctx=n_ctx, n_ubatch=U, kv_dtype=cfg["kv_dtype"])
    t_pre, t_dec = run(ctx, args.steps, args.warmup)
    # decode with the full fp32 logits row copied to the host every step
    n_d2h = 32
    tok = ctx.argmax_ith(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_d2h):
        assert ctx.decode([tok]) == 0, tdf.tdf_last_error()
        row = ctx.logits_ith(0)
        tok = int(np.argmax(row))
    t_d2h = time.perf_counter() - t0
    # the dominant kernels, back to back on the library's stream (HIP events)
    d, F = cfg["n_embd"], cfg["n_ff"]
    gu_us = ctx.time_op("gate_up", 1, 64)
    gg_us = ctx.time_op("gate_up", U, 16)
    # sampling chain on the last step's logits row (tdf_sample), per call
    samp = {}
    rng = np.random.default_rng(0)
    for name, (t, k, tp, mp) in {"k40": (0.8, 40, 0.9, 0.05), "k1024": (1.0, 1024, 0.95, 0.0)}.items():
        ts = []
        for _ in range(20):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            rc, _ = ctx.sample(t, k, tp, mp, rng.random(1))
            ts.append(time.perf_counter() - t0)
            assert rc == 0, tdf.tdf_last_error()
        samp[name] = {"temperature": t, "top_k": k, "top_p": tp, "min_p": mp,
                      "us_per_call_median": round(1e6 * float(np.median(ts)), 1)}
    # one slide of the context window: drop the oldest half, shift the rest
    # down (re-rotating their cached keys in every layer)
    top = ctx.seq_pos_max(0)
    half = (top + 1) // 2
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    assert ctx.kv_seq_rm(0, 0, half) == 0
    t1 = time.perf_counter()
    assert ctx.kv_seq_shift(0, half, -1, -half) == 0
    t2 = time.perf_counter()
    n_shift = top + 1 - half
    shift_bytes = 2 * n_shift * cfg["n_layer"] * cfg["n_head_kv"] * cfg["head_dim"] * 2  # K read + written
    slide = {"cells_dropped": half, "cells_shifted": n_shift, "rm_ms": round(1000 * (t1 - t0), 3),
             "shift_ms": round(1000 * (t2 - t1), 3),
             "shift_GBs": round(shift_bytes / (t2 - t1) / 1e9, 1)}
    ctx.close()
    ms_step = 1000.0 * t_dec / args.steps
    decode_tps = args.steps / t_dec
    prefill_tps = P / t_pre
    mean_ctx = P + args.warmup + (args.steps + 1) / 2.0
    step_bytes = decode_bytes(cfg, min(mean_ctx, args.swa) if args.swa else mean_ctx)
    pre_flops = prefill_flops(cfg, P, U)
    log(f"prefill {prefill_tps:.0f} tok/s, decode {decode_tps:.1f} tok/s ({ms_step:.3f} ms/step)")

    log("profiled run (HIP events per launch)")
    pctx = tdf.Context(model, n_ctx=n_ctx, n_ubatch=U, kv_dtype=cfg["kv_dtype"], profile=True)
    prof_phase = {}

    def prefilled(c):
        if c is not None:
            prof_phase["prefill"] = c.profile()
        pctx.profile_reset()

    run(pctx, args.steps, args.warmup, on_prefilled=prefilled, on_warm=pctx.profile_reset)
    prof_phase["decode"] = pctx.profile()
    pctx.close()
    # per decode launch: the gate and up matrices once, the normed input, the output
    gu_bytes = int(2 * F * d * weight_bytes_per_element(cfg)) + d * 4 + F * 4
    gu_gbs = gu_bytes / (gu_us * 1e-6) / 1e9
    gg_flops = 2.0 * U * (2 * F) * d
    gg_tfs = gg_flops / (gg_us * 1e-6) / 1e12
    peaks = None if args.no_peaks else measured_peaks()
    breakdown = {phase: {f"{k[0]}/{k[1]}": {"launches": v[0], "avg_us": round(1000.0 * v[1] / v[0], 2),
                                            "total_ms": round(v[1], 3)}
                         for k, v in sorted(pr.items())}
                 for phase, pr in prof_phase.items()}

    # the multi-sequence workload on the same weights: 32 sequences' prompts,
    # then a few lock-step steps of 32 tokens
    multi = None
    if args.config == "llama8b" and not args.no_multiseq and not args.swa:
        mcfg = dict(tdf_synth.CONFIGS["llama8b_multiseq"], weight_dtype=cfg["weight_dtype"],
                    kv_dtype=cfg["kv_dtype"])
        log("multi-sequence section (32 sequences)")
        multi = run_multiseq(args, mcfg, model=model, steps=8, warmup=2)

    # the 1B shape, compactly (its own weights; the 8B model's are freed first
    # only in the sense that both fit: 16 GB and 2.5 GB)
    small = None
    if args.config == "llama8b" and not args.no_multiseq and not args.swa:
        scfg = dict(tdf_synth.CONFIGS["llama1b"])
        log("1B-shape section (512-token prompt, 64 decode steps)")
        small = run_small(scfg)
        log(f"1B: prefill {small['prefill']['tok_s']:.0f} tok/s, decode {small['decode']['tok_s']:.1f} tok/s")

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(cfg, host, P)

    # the counter records cover the 8B shape's kernels
    is8b = args.config == "llama8b" and not args.swa
    busy = mfma_busy("prefill_q8_0" if q8 else "prefill") if is8b and cfg["kv_dtype"] == "bf16" else None
    shape = {"llama8b": "8B", "llama1b": "1B", "tiny": "tiny"}.get(args.config, args.config)
    out = {
        "metric": (f"decode tok/s (% HBM peak) + prefill tok/s (% MFMA peak), {shape}-shape bf16" if not q8 else
                   f"decode tok/s (% HBM peak) + prefill tok/s, {shape}-shape Q8_0 weights"),
        "value": round(decode_tps, 3),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (q8_0 weights)" if q8 else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: batch 1, {P}-token prompt in ubatches of {U} "
                               f"(last-position logits), then greedy decode steps; KV {cfg['kv_dtype']} {n_ctx} cells"
                               + ("; Q8_0 weights" if q8 else ""),
                   "d_model": d, "n_layer": cfg["n_layer"], "n_ff": F, "n_vocab": cfg["n_vocab"],
                   "attention_window": args.swa or None},
        "decode": {"tok_s": round(decode_tps, 3), "mean_ctx": mean_ctx,
                   "tok_s_with_logits_d2h": round(n_d2h / t_d2h, 3),
                   "algorithmic_bytes_per_step": int(step_bytes),
                   "achieved_GBs": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
                   "frac_hbm_peak": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "prefill": {"tok_s": round(prefill_tps, 1), "ms": round(1000 * t_pre, 3),
                    "algorithmic_tflop": round(pre_flops / 1e12, 4),
                    "achieved_TFLOPs": round(pre_flops / t_pre / 1e12, 2),
                    "frac_mfma_peak": round(pre_flops / t_pre / 1e12 / MFMA_BF16_PEAK_TFS, 4)},
        # the dominant decode kernel; the whole step's fraction (every kernel
        # of the step, launch gaps included) is step_frac_hbm_peak
        "roofline": {"bound": "hbm", "kernel": "gate/up GEMV + SwiGLU (decode), dominant kernel only",
                     "achieved": round(gu_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / HBM_PEAK_GBS, 4), "traffic": traffic("decode_q8_0" if q8 else "decode") if is8b else None,
                     "avg_launch_us": round(gu_us, 2), "bytes_per_launch": gu_bytes,
                     "step_frac_hbm_peak": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline_prefill": {"bound": "mfma", "kernel": "gate/up GEMM + SwiGLU (prefill ubatch 512)",
                             "achieved": round(gg_tfs, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                             "frac": round(gg_tfs / MFMA_BF16_PEAK_TFS, 4), "traffic": traffic("prefill_q8_0" if q8 else "prefill") if is8b else None,
                             "avg_launch_us": round(gg_us, 2), "flops_per_launch": gg_flops,
                             "executed_flops_per_launch": 2 * gg_flops,
                             "mfma_busy": (busy or {}).get("gate_up"),
                             "mfma_busy_by_kernel": busy},
        "measured_peaks": peaks,
        "kv_slide": slide,
        "sampling": samp,
        "kernels": breakdown,
        "cpu_baseline": cpu,
    }
    if multi is not None:
        out["multiseq"] = {k: multi[k] for k in ("config", "decode", "prefill", "steps", "warmup", "ms_per_step")}
    if small is not None:
        out["llama1b"] = dict(small, config={"workload": "llama1b: batch 1, 512-token prompt in one ubatch "
                                                         "(last-position logits), then greedy decode steps; KV f16 4096 cells",
                                             "d_model": 2048, "n_layer": 16})
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
