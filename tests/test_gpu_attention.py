"""GPU parity of the decode attention kernels for every query-group size and
both 16-bit cache types against the float64 oracle (tolerances as in
test_gpu_parity).  Decode steps (ubatches of up to 32 tokens) run the
split-K attention over the cached cells: with head_dim 64 or 128 and a
16-bit cache on the matrix cores, otherwise on the vector units.  Each case
prefills a prompt long enough for several splits and 16-cell tiles with a
ragged last tile, then decodes single tokens and a multi-sequence step."""
import numpy as np
import pytest

import tdf_synth

from gpu_common import TOL_BF16, make_weights
from test_gpu_parity import SMALL, run_pair

pytestmark = pytest.mark.gpu

# (head_dim, n_head, n_head_kv): query groups of 1, 2, 4 and 8 heads
SHAPES = [(64, 4, 4), (64, 4, 2), (128, 8, 2), (128, 16, 2), (32, 8, 1)]


@pytest.mark.parametrize("kv_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("hd,H,Hkv", SHAPES)
def test_decode_attention_group_sizes(hd, H, Hkv, kv_dtype):
    # weights scaled with the width (0.08 at d = 128, 0.02 at d = 2048) so that
    # the logits keep the magnitude of the other small models
    d = H * hd
    cfg = dict(SMALL, n_embd=d, n_head=H, n_head_kv=Hkv, head_dim=hd, n_ff=256, n_vocab=300,
               seed=30 + H + hd, weight_std=0.08 * (128 / d) ** 0.5)
    cfg, w = make_weights(cfg)
    calls = []
    # two sequences: 1187 and 413 positions (last tiles ragged), prefilled in
    # ubatches of 256, then three single-token steps on sequence 0 and one
    # step with a token of each sequence
    for s, n in ((0, 1187), (1, 413)):
        toks = tdf_synth.prompt(cfg, 60 + s, n)
        calls.append(dict(tokens=toks, seq_ids=[[s]] * n))
    for k in range(3):
        calls.append(dict(tokens=tdf_synth.prompt(cfg, 70 + k, 1), seq_ids=[[0]]))
    calls.append(dict(tokens=tdf_synth.prompt(cfg, 80, 2), seq_ids=[[0], [1]], logits=np.ones(2, np.int8)))
    run_pair(cfg, w, dict(n_ctx=2048, n_ubatch=256, n_seq_max=2), calls, TOL_BF16, kv_dtype,
             f"attn hd{hd} G{H // Hkv}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "q8_0"])
def test_decode_split_list_unequal_sequences(kv_dtype):
    """Five sequences whose step tokens see 128, 256, 301, 1001 and 65 cells.
    At this size the host splits every token's cells into chunks of 128, so
    the matrix-core kernel's dense (token, chunk) list holds in one launch a
    token with a single whole chunk (written directly), one with whole chunks
    only, one with whole chunks and a partial last one, a long one, and one
    with a single partial chunk; a second step moves every count by one."""
    hd, H, Hkv = 128, 8, 2
    d = H * hd
    cfg = dict(SMALL, n_embd=d, n_head=H, n_head_kv=Hkv, head_dim=hd, n_ff=256, n_vocab=300,
               seed=91, weight_std=0.08 * (128 / d) ** 0.5)
    cfg, w = make_weights(cfg)
    lens = (127, 255, 300, 1000, 64)
    calls = []
    for s, n in enumerate(lens):
        calls.append(dict(tokens=tdf_synth.prompt(cfg, 100 + s, n), seq_ids=[[s]] * n))
    for k in range(2):
        calls.append(dict(tokens=tdf_synth.prompt(cfg, 120 + k, len(lens)), seq_ids=[[s] for s in range(len(lens))],
                          logits=np.ones(len(lens), np.int8)))
    run_pair(cfg, w, dict(n_ctx=2048, n_ubatch=256, n_seq_max=len(lens)), calls, TOL_BF16, kv_dtype,
             f"split list {kv_dtype}")
