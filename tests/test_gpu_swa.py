"""GPU parity of sliding-window attention (Ollama engine page, "KV Cache:
memory for causal attention": a windowed layer's mask keeps only the most
recent positions) against the float64 oracle, same seeded inputs and
tolerances as test_gpu_parity.  The windows are chosen to cut through query
tiles, attention splits and ubatch boundaries; one of the two layers is
windowed and the other global, so both paths run in one forward pass."""
import numpy as np
import pytest

import tdf_synth

from gpu_common import TOL_BF16, TOL_F32, make_weights
from test_gpu_parity import SMALL, run_pair, teacher_forced

pytestmark = pytest.mark.gpu

# head_dim 64: the matrix-core prefill attention runs (it takes 64 and 128)
SMALL64 = dict(SMALL, n_embd=256, n_head=4, n_head_kv=2, head_dim=64, n_ff=256, seed=12)


@pytest.mark.parametrize("kv_dtype", ["bf16", "f16", "q8_0"])
def test_window_prefill_tiles_and_decode(kv_dtype):
    """150 tokens in ubatches of 64, 64, 22 with a 37-position window on layer
    0 (query tiles of 32 whose first visible entries differ), every row's
    logits, then 4 decode steps."""
    cfg = dict(SMALL64, n_swa=37, swa_layers=[1, 0])
    cfg, w = make_weights(cfg)
    prompt = tdf_synth.prompt(cfg, 0, 150)
    calls = [dict(tokens=prompt)] + [dict(tokens=[int(t)]) for t in tdf_synth.prompt(cfg, 1, 4)]
    run_pair(cfg, w, dict(n_ctx=256, n_ubatch=64, output_all=True), calls, TOL_BF16, kv_dtype, "swa tiles")


def test_window_long_context_splits():
    """600-token prompt in ubatches of 128 with a 300-position window on both
    layers (split cell ranges in the prefill attention and its merge), then
    decode steps whose windowed attention is split and merged."""
    cfg = dict(SMALL64, n_swa=300)
    cfg, w = make_weights(cfg)
    prompt = tdf_synth.prompt(cfg, 2, 600)
    teacher_forced(cfg, w, 1024, prompt, 5, TOL_BF16, "bf16", n_ubatch=128, label="swa long")


def test_window_gemv_attention_path_and_multi_sequence():
    """head_dim 32 (the split-K attention kernel for every ubatch size):
    three interleaved sequences with a 9-position window on layer 1, then
    lock-step steps of one token per sequence."""
    cfg = dict(SMALL, n_swa=9, swa_layers=[0, 1])
    cfg, w = make_weights(cfg)
    rng = np.random.default_rng(5)
    seqs = [int(s) for s in rng.integers(0, 3, size=90)]
    toks = tdf_synth.prompt(cfg, 3, 90)
    calls = [dict(tokens=toks, seq_ids=[[s] for s in seqs], logits=np.ones(90, dtype=np.int8))]
    for step in range(4):
        calls.append(dict(tokens=tdf_synth.prompt(cfg, 20 + step, 3), seq_ids=[[0], [1], [2]],
                          logits=np.ones(3, dtype=np.int8)))
    run_pair(cfg, w, dict(n_ctx=200, n_ubatch=40, n_seq_max=4), calls, TOL_BF16, "bf16", "swa multiseq")


def test_window_fp32_tiny():
    """The float32 model with a 5-position window on both layers: prompt of
    16, then 10 steps (the window slides past the prompt)."""
    cfg = dict(tdf_synth.CONFIGS["tiny"], n_swa=5)
    cfg, w = make_weights(cfg)
    prompt = tdf_synth.prompt(cfg, 0, cfg["prompt_len"])
    teacher_forced(cfg, w, cfg["n_ctx"], prompt, 10, TOL_F32, "f32", label="swa tiny")


def test_window_graph_replay_matches_eager(monkeypatch):
    """Graph-replayed decode with a window equals plain launches while the
    context grows past the window."""
    import transformer_decode_forward_amd as tdf
    from gpu_common import device_model
    cfg = dict(SMALL64, n_swa=70, swa_layers=[1, 0])
    cfg, w = make_weights(cfg)
    gm = device_model(cfg, w)
    monkeypatch.setenv("TDF_NO_GRAPH", "1")
    eager = tdf.Context(gm, n_ctx=512, n_ubatch=64, kv_dtype="bf16")
    monkeypatch.delenv("TDF_NO_GRAPH")
    graphed = tdf.Context(gm, n_ctx=512, n_ubatch=64, kv_dtype="bf16")
    prompt = tdf_synth.prompt(cfg, 4, 40)
    assert eager.decode(prompt) == 0 and graphed.decode(prompt) == 0
    for i, t in enumerate(tdf_synth.prompt(cfg, 5, 60)):
        assert eager.decode([int(t)]) == 0 and graphed.decode([int(t)]) == 0
        a, b = eager.logits_ith(0), graphed.logits_ith(0)
        assert np.array_equal(a, b), (i, float(np.max(np.abs(a - b))))
    assert graphed.graph_counts()[1] >= 50
