"""GPU parity at the 70B-class model's widths (d_model 8192, 64 query heads
over 8 KV heads of 128, FFN 28672, vocabulary 128256) on two layers, the
subset of the 70B workload the float64 oracle can follow step by step:

* the workload's prompt: 4096 uniform-random tokens in 8 ubatches of 512
  (matrix-core projections with K = 8192 and 28672, 8-head query groups in
  the prefill attention), logits for the last position only;
* decode at the workload's three context points (llama.cpp walkthrough,
  "KV-cache and the Prefill / Decode stages": a decode step reads the K/V of
  every earlier position): right after the prompt (position 4096), then with
  the cache filled by synthetic post-RoPE K/V up to 16384 and to 32752, two
  teacher-forced steps each.  The longest context splits the decode
  attention into 32 chunks of 1024 cells and merges them.

Cells, positions and rows bit-exact; logits within max-abs 3e-2 and rel-L2
1e-2 of the oracle; greedy tokens equal where the oracle's top-2 gap exceeds
5e-2.
"""
import numpy as np
import pytest

import tdf_synth
from oracle import OracleContext

from gpu_common import TOL_BF16, check_logits, check_token, device_model, log, make_weights, oracle_model

pytestmark = pytest.mark.gpu


def test_llama70b_width_two_layers_prompt_and_long_context():
    import transformer_decode_forward_amd as tdf
    from transformer_decode_forward_amd.device import to_device
    cfg = dict(tdf_synth.CONFIGS["llama70b"])
    cfg, w = make_weights(cfg, layers=2)
    L, P, n_ctx = cfg["n_layer"], cfg["prompt_len"], cfg["n_ctx"]
    log("70b-width weights generated")
    gm = device_model(cfg, w)
    gc = tdf.Context(gm, n_ctx=n_ctx, n_ubatch=cfg["n_ubatch"], kv_dtype="bf16")
    oc = OracleContext(oracle_model(cfg, w), n_ctx=n_ctx, n_ubatch=cfg["n_ubatch"], kv_dtype="bf16")
    prompt = tdf_synth.prompt(cfg, 0, P)
    assert gc.decode(prompt) == 0, tdf.tdf_last_error()
    ro = oc.decode(prompt)
    log("70b-width prompt (8 x 512) done on both sides")
    assert [len(u) for u in ro.ubatches] == [512] * 8
    assert gc.last_slots() == ro.slots == list(range(P))
    errs = [check_logits(gc.logits_ith(P - 1), ro.logits[0], TOL_BF16, "70b-width prefill")]
    check_token(gc.argmax_ith(P - 1), ro.logits[0], "70b-width prefill")
    nxt = int(ro.tokens[0])
    for w0 in cfg["decode_windows"]:
        have = gc.seq_pos_max(0) + 1
        assert have == oc.seq_pos_max(0) + 1
        if w0 > have:
            ks = [tdf_synth.kv_fill(cfg, l, "k", have, w0, "bf16") for l in range(L)]
            vs = [tdf_synth.kv_fill(cfg, l, "v", have, w0, "bf16") for l in range(L)]
            kd, vd = [to_device(k) for k in ks], [to_device(v) for v in vs]
            assert gc.kv_import(0, have, w0 - have, [t.data_ptr() for t in kd], [t.data_ptr() for t in vd]) == 0
            assert oc.kv_import(0, have, w0, ks, vs) == 0
            assert gc.last_slots() == list(oc.last_import_cells)
            del kd, vd, ks, vs
        for step in range(2):
            assert gc.decode([nxt]) == 0, tdf.tdf_last_error()
            ro = oc.decode([nxt])
            assert ro.positions == [w0 + step]
            assert gc.last_slots() == ro.slots and gc.seq_pos_max(0) == oc.seq_pos_max(0)
            errs.append(check_logits(gc.logits_ith(0), ro.logits[0], TOL_BF16, f"70b-width step at {w0 + step}"))
            check_token(gc.argmax_ith(0), ro.logits[0], f"70b-width step at {w0 + step}")
            nxt = int(ro.tokens[0])
        log(f"70b-width decode at {w0}: max-abs {errs[-1][0]:.2e}, rel-L2 {errs[-1][1]:.2e}")
    assert gc.seq_pos_max(0) == n_ctx - 15
    log(f"70b-width: prefill max-abs {errs[0][0]:.2e} rel-L2 {errs[0][1]:.2e}; worst step max-abs "
        f"{max(e[0] for e in errs[1:]):.2e} rel-L2 {max(e[1] for e in errs[1:]):.2e}")
    gc.close()
    gm.close()
