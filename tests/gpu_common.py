"""Shared helpers of the GPU parity tests: seeded weights on both sides, and
the tolerance checks stated for the decoder forward pass."""
import sys
import time

import numpy as np

import tdf_synth

# logits tolerance against the float64 oracle: bf16 weights (max-abs, rel-L2)
TOL_BF16 = (3e-2, 1e-2)
# float32 weights: derived from float32 accumulation over <= a few thousand terms
TOL_F32 = (1e-4, 1e-5)
GAP = 5e-2  # greedy tokens must agree where the oracle's top-2 gap exceeds this


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def make_weights(cfg, layers=None):
    """numpy tensors of every weight of cfg (layers: optional subset count)."""
    c = dict(cfg)
    if layers is not None:
        c["n_layer"] = layers
    return c, tdf_synth.make_all(c)


def device_model(cfg, tensors):
    import transformer_decode_forward_amd as tdf
    from transformer_decode_forward_amd.device import to_device
    dev = {k: to_device(v) for k, v in tensors.items()}
    return tdf.Model(tdf_synth.hparams(cfg), dev)


def oracle_model(cfg, tensors, cache=True):
    from oracle import OracleModel
    return OracleModel(tdf_synth.hparams(cfg), tensors, cache=cache)


def check_logits(got, ref, tol, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    maxabs = float(np.max(np.abs(got - ref)))
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    assert maxabs <= tol[0] and rel <= tol[1], f"{what}: max-abs {maxabs:.3e} rel-L2 {rel:.3e}"
    return maxabs, rel


def check_token(got_tok, ref_row, what=""):
    order = np.argsort(ref_row)[::-1]
    gap = ref_row[order[0]] - ref_row[order[1]]
    if gap > GAP:
        assert got_tok == int(order[0]), f"{what}: token {got_tok} vs oracle {int(order[0])} (gap {gap:.3f})"
    return gap
