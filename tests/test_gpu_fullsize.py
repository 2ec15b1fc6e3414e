"""GPU parity at the workloads' full sizes.

The 8B workload's prefill runs as the benchmark runs it: a 2048-token prompt
in ubatches of 512 through all 32 layers (last-row logits), then
teacher-forced decode steps, against the float64 oracle over the same
4 ubatches.  Where the oracle cannot replay a prompt of thousands of tokens
in seconds (the multi-sequence workload's 32 prompts, contexts beyond the
prompt), the cache is restored from the same synthetic post-RoPE K/V on both
sides (tdf_kv_import / OracleContext.kv_import, values drawn by tdf_synth)
and the outputs the oracle can compute one by one are compared: matrix-core
ubatches and decode steps on top of the restored contexts.  The
multi-sequence workload is checked in full for its bookkeeping (cells,
positions, rows), at full depth for a lock-step step of 32 tokens over 4 of
its sequences (the shortest, the longest and two others, restored at their
workload lengths; sequences are independent), and on a two-layer
full-width model with the prompts themselves.  Tolerances as in
test_gpu_parity.
"""
import os

import numpy as np
import pytest

import tdf_synth
from oracle import OracleContext

from gpu_common import TOL_BF16, check_logits, check_token, device_model, log, make_weights, oracle_model

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def llama8b():
    """The 8B-class model of the workload (bf16, all 32 layers): host tensors,
    the device model and an oracle model holding the float64 weights, shared
    by the tests of this module."""
    cfg = dict(tdf_synth.CONFIGS["llama8b"])
    cfg, w = make_weights(cfg)
    log("8b weights generated")
    gm = device_model(cfg, w)
    om = oracle_model(cfg, w, cache=True)
    log("8b weights uploaded")
    yield cfg, w, gm, om
    gm.close()


def test_llama8b_prefill_as_benched_full_depth(llama8b):
    """The 8B workload's prefill as the benchmark runs it: 2048 uniform-random
    tokens in 4 ubatches of 512 (matrix-core projections and attention)
    through all 32 layers, logits for the last position only; then 4
    teacher-forced decode steps on the prompt's cache."""
    import transformer_decode_forward_amd as tdf
    cfg, w, gm, om = llama8b
    gc = tdf.Context(gm, n_ctx=cfg["n_ctx"], n_ubatch=cfg["n_ubatch"], kv_dtype="bf16")
    oc = OracleContext(om, n_ctx=cfg["n_ctx"], n_ubatch=cfg["n_ubatch"], kv_dtype="bf16")
    prompt = tdf_synth.prompt(cfg, 0, cfg["prompt_len"])
    assert gc.decode(prompt) == 0, tdf.tdf_last_error()
    ro = oc.decode(prompt)
    log("8b prefill (4 x 512) done on both sides")
    assert [len(u) for u in ro.ubatches] == [512] * 4
    assert gc.last_slots() == ro.slots == list(range(2048))
    assert gc.output_ids() == ro.out_index == [2047]
    errs = [check_logits(gc.logits_ith(2047), ro.logits[0], TOL_BF16, "8b prefill")]
    check_token(gc.argmax_ith(2047), ro.logits[0], "8b prefill")
    nxt = int(ro.tokens[0])
    for step in range(4):
        assert gc.decode([nxt]) == 0
        ro = oc.decode([nxt])
        assert gc.last_slots() == ro.slots and gc.seq_pos_max(0) == oc.seq_pos_max(0) == 2048 + step
        errs.append(check_logits(gc.logits_ith(0), ro.logits[0], TOL_BF16, f"8b step {step}"))
        check_token(gc.argmax_ith(0), ro.logits[0], f"8b step {step}")
        nxt = int(ro.tokens[0])
    log(f"8b prefill as benched: prefill max-abs {errs[0][0]:.2e} rel-L2 {errs[0][1]:.2e}; "
        f"steps worst max-abs {max(e[0] for e in errs[1:]):.2e} rel-L2 {max(e[1] for e in errs[1:]):.2e}")
    gc.close()


def test_multisequence_lockstep_full_depth(llama8b):
    """The multi-sequence workload at full depth over 4 of its 32 sequences
    (the shortest, the longest and two others), each restored at its
    workload length from its own synthetic K/V; then one lock-step step of
    32 tokens (8 per sequence at consecutive positions: the 9..32-token
    matrix-core path) and one of 4 tokens (one per sequence: the GEMV path),
    every row's logits."""
    import transformer_decode_forward_amd as tdf
    from transformer_decode_forward_amd.device import to_device
    cfg, w, gm, om = llama8b
    mcfg = tdf_synth.CONFIGS["llama8b_multiseq"]
    lens = tdf_synth.seq_lengths(mcfg)
    order = np.argsort(lens)
    picks = [int(order[0]), int(order[len(order) // 3]), int(order[2 * len(order) // 3]), int(order[-1])]
    n_ctx = int(sum(lens[p] for p in picks)) + 64
    L = cfg["n_layer"]
    gc = tdf.Context(gm, n_ctx=n_ctx, n_batch=512, n_ubatch=512, n_seq_max=4, kv_dtype="bf16")
    oc = OracleContext(om, n_ctx=n_ctx, n_batch=512, n_ubatch=512, n_seq_max=4, kv_dtype="bf16")
    base = 0
    for j, s in enumerate(picks):
        n = int(lens[s])
        # sequence j's rows come from its own stretch of the fill streams
        ks = [tdf_synth.kv_fill(cfg, l, "k", base, base + n, "bf16") for l in range(L)]
        vs = [tdf_synth.kv_fill(cfg, l, "v", base, base + n, "bf16") for l in range(L)]
        kd, vd = [to_device(k) for k in ks], [to_device(v) for v in vs]
        assert gc.kv_import(j, 0, n, [t.data_ptr() for t in kd], [t.data_ptr() for t in vd]) == 0
        assert oc.kv_import(j, 0, n, ks, vs) == 0
        assert gc.last_slots() == list(oc.last_import_cells)
        del kd, vd, ks, vs
        base += n
    log(f"4 sequences restored: lengths {[int(lens[p]) for p in picks]}")
    calls = [dict(tokens=tdf_synth.prompt(mcfg, 400, 32), seq_ids=[[j // 8] for j in range(32)],
                  logits=np.ones(32, np.int8)),
             dict(tokens=tdf_synth.prompt(mcfg, 401, 4), seq_ids=[[0], [1], [2], [3]],
                  logits=np.ones(4, np.int8))]
    errs = []
    for k, call in enumerate(calls):
        assert gc.decode(**call) == 0, tdf.tdf_last_error()
        r = oc.decode(**call)
        assert gc.last_slots() == r.slots and gc.output_ids() == r.out_index
        for row, i in enumerate(r.out_index):
            errs.append(check_logits(gc.logits_ith(i), r.logits[row], TOL_BF16, f"lock-step call {k} row {i}"))
            check_token(gc.argmax_ith(i), r.logits[row], f"lock-step call {k} row {i}")
        log(f"lock-step call {k} ({len(call['tokens'])} tokens) done")
    for j, s in enumerate(picks):
        assert gc.seq_pos_max(j) == oc.seq_pos_max(j) == int(lens[s]) + 8
    log(f"multi-sequence full depth: worst max-abs {max(e[0] for e in errs):.2e}, "
        f"rel-L2 {max(e[1] for e in errs):.2e}")
    gc.close()


def _fill(cfg, P):
    L = cfg["n_layer"]
    return ([tdf_synth.kv_fill(cfg, l, "k", 0, P, "bf16") for l in range(L)],
            [tdf_synth.kv_fill(cfg, l, "v", 0, P, "bf16") for l in range(L)])


def _restored_pair(cfg, w, P, n_ctx, cache, gm=None, om=None):
    """GPU and oracle contexts with positions [0, P) of sequence 0 restored
    (the device and oracle models are made here unless given)."""
    import transformer_decode_forward_amd as tdf
    from transformer_decode_forward_amd.device import to_device
    ks, vs = _fill(cfg, P)
    gm = gm if gm is not None else device_model(cfg, w)
    gc = tdf.Context(gm, n_ctx=n_ctx, n_ubatch=512, kv_dtype="bf16")
    kd = [to_device(k) for k in ks]
    vd = [to_device(v) for v in vs]
    assert gc.kv_import(0, 0, P, [t.data_ptr() for t in kd], [t.data_ptr() for t in vd]) == 0
    del kd, vd
    oc = OracleContext(om if om is not None else oracle_model(cfg, w, cache=cache), n_ctx=n_ctx, kv_dtype="bf16")
    assert oc.kv_import(0, 0, P, ks, vs) == 0
    assert gc.last_slots() == list(oc.last_import_cells)
    return gm, gc, oc


@pytest.mark.parametrize("kv_dtype", ["f16", "q8_0"])
def test_llama1b_full_workload_shape(kv_dtype):
    """1B-class model at full depth: 512-token prompt in one ubatch (last-row
    logits), then 12 teacher-forced greedy steps (of the workload's 128).
    With the Q8_0 cache both sides quantize their own K/V rows, so a code may
    differ by one at a rounding boundary in any of the 16 layers; the bf16
    tolerance still applies."""
    cfg = tdf_synth.CONFIGS["llama1b"]
    cfg, w = make_weights(cfg)
    import transformer_decode_forward_amd as tdf
    gm = device_model(cfg, w)
    gc = tdf.Context(gm, n_ctx=cfg["n_ctx"], n_ubatch=512, kv_dtype=kv_dtype)
    oc = OracleContext(oracle_model(cfg, w), n_ctx=cfg["n_ctx"], kv_dtype=kv_dtype)
    prompt = tdf_synth.prompt(cfg, 0, cfg["prompt_len"])
    assert gc.decode(prompt) == 0
    ro = oc.decode(prompt)
    assert gc.last_slots() == ro.slots
    errs = [check_logits(gc.logits_ith(511), ro.logits[0], TOL_BF16, "1b prefill")]
    check_token(gc.argmax_ith(511), ro.logits[0], "1b prefill")
    nxt = int(ro.tokens[0])
    for step in range(12):
        assert gc.decode([nxt]) == 0
        ro = oc.decode([nxt])
        assert gc.last_slots() == ro.slots
        errs.append(check_logits(gc.logits_ith(0), ro.logits[0], TOL_BF16, f"1b step {step}"))
        check_token(gc.argmax_ith(0), ro.logits[0], f"1b step {step}")
        nxt = int(ro.tokens[0])
    log(f"1b full kv={kv_dtype}: worst max-abs {max(e[0] for e in errs):.2e}, rel-L2 {max(e[1] for e in errs):.2e}")


@pytest.mark.parametrize("weight_dtype", ["bf16", "q8_0"])
def test_llama8b_full_depth(weight_dtype, llama8b):
    """8B-class model, all 32 layers (bf16 or Q8_0 weights): context 2048
    restored, then a 64-token ubatch (matrix-core path; logits for 3 rows) and
    2 decode steps."""
    if weight_dtype == "bf16":
        cfg, w, gm, om = llama8b
        gm, gc, oc = _restored_pair(cfg, w, 2048, 4096, cache=False, gm=gm, om=om)
    else:
        cfg = dict(tdf_synth.CONFIGS["llama8b"], weight_dtype=weight_dtype)
        cfg, w = make_weights(cfg)
        log(f"8b {weight_dtype} weights generated")
        gm, gc, oc = _restored_pair(cfg, w, 2048, 4096, cache=False)
    toks = tdf_synth.prompt(cfg, 3, 64)
    flags = np.zeros(64, dtype=np.int8)
    flags[[0, 31, 63]] = 1
    assert gc.decode(toks, logits=flags) == 0
    ro = oc.decode(toks, logits=flags)
    log("8b ubatch done")
    assert gc.last_slots() == ro.slots and gc.output_ids() == ro.out_index == [0, 31, 63]
    errs = []
    for r, i in enumerate(ro.out_index):
        errs.append(check_logits(gc.logits_ith(i), ro.logits[r], TOL_BF16, f"8b ubatch row {i}"))
        check_token(gc.argmax_ith(i), ro.logits[r], f"8b ubatch row {i}")
    nxt = int(ro.tokens[-1])
    for step in range(2):
        assert gc.decode([nxt]) == 0
        ro = oc.decode([nxt])
        assert gc.last_slots() == ro.slots
        errs.append(check_logits(gc.logits_ith(0), ro.logits[0], TOL_BF16, f"8b step {step}"))
        check_token(gc.argmax_ith(0), ro.logits[0], f"8b step {step}")
        nxt = int(ro.tokens[0])
        log(f"8b step {step} done")
    log(f"8b {weight_dtype} full depth: worst max-abs {max(e[0] for e in errs):.2e}, "
        f"rel-L2 {max(e[1] for e in errs):.2e}")


def test_multisequence_bookkeeping_full():
    """All 32 sequences of the multi-sequence workload (lengths uniform on
    [1024, 8192]): prefill calls in sequence order, then lock-step steps of 32
    tokens; cells, positions and output rows bit-exact (bookkeeping-only
    contexts on both sides)."""
    import transformer_decode_forward_amd as tdf
    cfg = tdf_synth.CONFIGS["llama8b_multiseq"]
    hp = tdf_synth.hparams(cfg)
    lens = tdf_synth.seq_lengths(cfg)
    gm = tdf.Model(hp, dry_run=True)
    gc = tdf.Context(gm, n_ctx=cfg["n_ctx"], n_batch=8192, n_ubatch=512, n_seq_max=32, dry_run=True)
    from oracle import OracleModel
    oc = OracleContext(OracleModel(hp, {}), n_ctx=cfg["n_ctx"], n_batch=8192, n_ubatch=512, n_seq_max=32,
                       compute=False)
    for s in range(32):
        toks = tdf_synth.prompt(cfg, s, int(lens[s]))
        assert gc.decode(toks, seq_ids=[[s]] * len(toks)) == 0
        r = oc.decode(toks, seq_ids=[[s]] * len(toks))
        assert gc.last_slots() == r.slots
    for step in range(4):
        toks = tdf_synth.prompt(cfg, 100 + step, 32)
        assert gc.decode(toks, seq_ids=[[s] for s in range(32)], logits=np.ones(32, np.int8)) == 0
        r = oc.decode(toks, seq_ids=[[s] for s in range(32)], logits=np.ones(32, np.int8))
        assert gc.last_slots() == r.slots and gc.output_ids() == list(range(32))
        assert r.positions == [int(lens[s]) + step for s in range(32)]
    for s in range(32):
        assert gc.seq_pos_max(s) == oc.seq_pos_max(s) == int(lens[s]) + 3


def test_multisequence_math_two_layers():
    """Multi-sequence decode at full width on a two-layer model: 4 sequences
    (the shortest and the longest of the workload's lengths, and two others)
    prefilled in their own calls, then 3 lock-step steps with one token per
    sequence and logits for every row (ubatch of 4 tokens, GEMV path), and one
    step of 32 tokens spread over the 4 sequences (matrix-core path)."""
    cfg = dict(tdf_synth.CONFIGS["llama8b_multiseq"])
    lens = tdf_synth.seq_lengths(cfg)
    order = np.argsort(lens)
    picks = [int(order[0]), int(order[1]), int(order[-2]), int(order[-1])]
    cfg, w = make_weights(cfg, layers=2)
    import transformer_decode_forward_amd as tdf
    gm = device_model(cfg, w)
    n_ctx = int(sum(lens[p] for p in picks)) + 128
    gc = tdf.Context(gm, n_ctx=n_ctx, n_batch=8192, n_ubatch=512, n_seq_max=4, kv_dtype="bf16")
    oc = OracleContext(oracle_model(cfg, w), n_ctx=n_ctx, n_batch=8192, n_ubatch=512, n_seq_max=4,
                       kv_dtype="bf16")
    for j, s in enumerate(picks):
        toks = tdf_synth.prompt(cfg, s, int(lens[s]))
        assert gc.decode(toks, seq_ids=[[j]] * len(toks)) == 0
        r = oc.decode(toks, seq_ids=[[j]] * len(toks))
        assert gc.last_slots() == r.slots
        check_logits(gc.logits_ith(len(toks) - 1), r.logits[0], TOL_BF16, f"seq {s} prefill")
        log(f"seq {s} (length {lens[s]}) prefill ok")
    calls = [dict(tokens=tdf_synth.prompt(cfg, 200 + k, 4), seq_ids=[[0], [1], [2], [3]],
                  logits=np.ones(4, np.int8)) for k in range(3)]
    calls.append(dict(tokens=tdf_synth.prompt(cfg, 300, 32), seq_ids=[[j % 4] for j in range(32)],
                      logits=np.ones(32, np.int8)))
    for k, call in enumerate(calls):
        assert gc.decode(**call) == 0
        r = oc.decode(**call)
        assert gc.last_slots() == r.slots and gc.output_ids() == r.out_index
        for row, i in enumerate(r.out_index):
            check_logits(gc.logits_ith(i), r.logits[row], TOL_BF16, f"lock-step call {k} row {i}")
            check_token(gc.argmax_ith(i), r.logits[row], f"lock-step call {k} row {i}")


@pytest.mark.slow
@pytest.mark.skipif(not os.environ.get("TDF_RUN_70B"),
                    reason="needs ~141 GB of device weights and ~10 minutes; set TDF_RUN_70B=1 to run")
def test_llama70b_decode_at_context_4096():
    """70B-class model (141 GB resident): positions [0, 4096) restored, then one
    decode step at position 4096, all 80 layers.  Weights are generated tensor
    by tensor on both sides (uploaded and dropped for the GPU, regenerated on
    demand for the oracle), so host memory holds one layer at a time."""
    import transformer_decode_forward_amd as tdf
    from oracle import OracleModel
    from transformer_decode_forward_amd.device import to_device
    cfg = dict(tdf_synth.CONFIGS["llama70b"])
    L, P = cfg["n_layer"], 4096
    shapes = dict(tdf_synth.tensor_shapes(cfg))
    for l in range(L):
        shapes.update(tdf_synth.tensor_shapes(cfg, l))
    dev = {}
    for i, (name, shape) in enumerate(shapes.items()):
        dev[name] = to_device(tdf_synth.make_tensor(cfg, name, shape))
        if i % 45 == 0:
            log(f"70b upload {i}/{len(shapes)}")
    gm = tdf.Model(tdf_synth.hparams(cfg), dev)
    gc = tdf.Context(gm, n_ctx=P + 128, n_ubatch=512, kv_dtype="bf16")
    for l0 in range(0, L, 16):
        ks = [to_device(tdf_synth.kv_fill(cfg, l, "k", 0, P, "bf16")) for l in range(l0, min(L, l0 + 16))]
        vs = [to_device(tdf_synth.kv_fill(cfg, l, "v", 0, P, "bf16")) for l in range(l0, min(L, l0 + 16))]
        if l0 == 0:
            kd, vd = ks, vs
        else:
            kd += ks
            vd += vs
    assert gc.kv_import(0, 0, P, [t.data_ptr() for t in kd], [t.data_ptr() for t in vd]) == 0
    del kd, vd
    log("70b cache restored")
    seen = set()

    def provider(name):
        layer = name.split(".")[1] if name.startswith("blk.") else name
        if layer not in seen:
            seen.add(layer)
            log(f"70b oracle at {layer}")
        return tdf_synth.make_tensor(cfg, name, shapes[name])
    oc = OracleContext(OracleModel(tdf_synth.hparams(cfg), provider, cache=False), n_ctx=P + 128,
                       kv_dtype="bf16")
    assert oc.kv_import(0, 0, P, lambda l: tdf_synth.kv_fill(cfg, l, "k", 0, P, "bf16"),
                        lambda l: tdf_synth.kv_fill(cfg, l, "v", 0, P, "bf16")) == 0
    assert gc.last_slots() == list(oc.last_import_cells)
    tok = int(tdf_synth.prompt(cfg, 5, 1)[0])
    assert gc.decode([tok]) == 0
    ro = oc.decode([tok])
    assert gc.last_slots() == ro.slots
    e = check_logits(gc.logits_ith(0), ro.logits[0], TOL_BF16, "70b step")
    check_token(gc.argmax_ith(0), ro.logits[0], "70b step")
    log(f"70b decode at 4096: max-abs {e[0]:.2e}, rel-L2 {e[1]:.2e}")
