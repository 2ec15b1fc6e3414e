"""GPU parity of the sampling chain (Ollama engine page, "Token sampling
pipeline") with the oracle's chain, both reading the same float32 logits
rows (those the GPU decode left in its buffer), over many parameter sets and
uniform numbers.  Tokens must be equal wherever every floating-point
decision of the draw is further than 1e-5 from its boundary
(oracle.sampling.sample_margin); the two sides compute the probabilities in
different precision and summation order, as the greedy tokens are compared
only where the top-2 gap is clear."""
import numpy as np
import pytest

import tdf_synth
from oracle.sampling import sample, sample_margin

from gpu_common import device_model, make_weights
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

PARAMS = [(0.8, 40, 0.9, 0.05), (1.0, 1024, 1.0, 0.0), (0.5, 1, 1.0, 0.0), (1.5, 200, 0.5, 0.1),
          (1.0, 7, 0.3, 0.0), (2.0, 600, 0.95, 0.02)]
MARGIN = 1e-5


def _run(cfg, w, n_rows, label):
    import transformer_decode_forward_amd as tdf
    gc = tdf.Context(device_model(cfg, w), n_ctx=256, n_ubatch=64, kv_dtype="bf16")
    toks = tdf_synth.prompt(cfg, 0, n_rows)
    assert gc.decode(toks, logits=np.ones(n_rows, np.int8)) == 0
    rows = [gc.logits_ith(i).astype(np.float64) for i in range(n_rows)]
    rc, greedy = gc.sample(0.0)
    assert rc == 0 and greedy == [gc.argmax_ith(i) for i in range(n_rows)]
    rng = np.random.default_rng(7)
    compared = total = 0
    for (t, k, p, mp) in PARAMS:
        for rep in range(6):
            u = rng.random(n_rows).astype(np.float32)
            rc, got = gc.sample(t, k, p, mp, u)
            assert rc == 0, tdf.tdf_last_error()
            for i in range(n_rows):
                total += 1
                if sample_margin(rows[i], t, k, p, mp, float(u[i])) <= MARGIN:
                    continue
                compared += 1
                want = sample(rows[i], t, k, p, mp, float(u[i]))
                assert got[i] == want, (label, t, k, p, mp, float(u[i]), i, got[i], want)
    assert compared >= 0.7 * total, (compared, total)


def test_sampling_small_vocab():
    cfg, w = make_weights(SMALL)
    _run(cfg, w, 6, "small")


def test_sampling_full_vocab():
    """128,256-token rows (1B-class widths, two layers)."""
    cfg, w = make_weights(dict(tdf_synth.CONFIGS["llama1b"]), layers=2)
    _run(cfg, w, 4, "1b")


def test_sampling_rejects_bad_parameters():
    import transformer_decode_forward_amd as tdf
    cfg, w = make_weights(SMALL)
    gc = tdf.Context(device_model(cfg, w), n_ctx=64, kv_dtype="bf16")
    assert gc.decode([1, 2, 3]) == 0
    for args in ((1.0, 0, 1.0, 0.0, [0.5]), (1.0, 2000, 1.0, 0.0, [0.5]), (1.0, 40, 1.0, 1.5, [0.5]),
                 (1.0, 40, 1.0, 0.0, [1.0])):
        rc, _ = gc.sample(*args[:4], u=args[4])
        assert rc == tdf.TDF_E_INVALID


def _run_rows(kind, n_vocab, params, n_rows=3, seed=5):
    """tdf_sample_logits on synthetic rows of a given structure against the
    oracle's chain, token by token, where the decisions are clear."""
    import transformer_decode_forward_amd as tdf
    from transformer_decode_forward_amd.device import to_device
    cfg, w = make_weights(SMALL)
    gc = tdf.Context(device_model(cfg, w), n_ctx=64, kv_dtype="bf16")
    rows = tdf_synth.logit_rows(seed, kind, n_rows, n_vocab)
    d = to_device(rows)
    rc, greedy = gc.sample_logits(d.data_ptr(), n_rows, n_vocab, 0.0)
    assert rc == 0 and greedy == [int(np.argmax(r)) for r in rows]
    rng = np.random.default_rng(11)
    compared = total = 0
    for (t, k, p, mp) in params:
        for rep in range(4):
            u = rng.random(n_rows).astype(np.float32)
            rc, got = gc.sample_logits(d.data_ptr(), n_rows, n_vocab, t, k, p, mp, u)
            assert rc == 0, tdf.tdf_last_error()
            for i in range(n_rows):
                z = rows[i].astype(np.float64)
                total += 1
                if sample_margin(z, t, k, p, mp, float(u[i])) <= MARGIN:
                    continue
                compared += 1
                want = sample(z, t, k, p, mp, float(u[i]))
                assert got[i] == want, (kind, n_vocab, t, k, p, mp, float(u[i]), i, got[i], want)
    assert compared >= 0.6 * total, (compared, total)


ROW_PARAMS = [(1.0, 1024, 1.0, 0.0), (0.8, 40, 0.9, 0.05), (1.0, 1, 1.0, 0.0), (3.0, 500, 0.98, 0.0)]


@pytest.mark.parametrize("kind,n_vocab", [("normal", 128256), ("normal", 5000), ("normal", 8193),
                                          ("masked", 128256), ("coarse", 128256), ("comb", 128256),
                                          ("coarse", 3000)])
def test_sampling_structured_rows(kind, n_vocab):
    """Rows that take every path of the Top-K gather: whole rows that fit the
    candidate list (5000, 3000), the sampled threshold (normal, masked, just
    above the list size), heavy ties that overflow it or tie at the K-th place
    (coarse: whole-number logits), and a comb of large values on evenly spaced
    ids that a strided sample sees all of, so the gather falls short of K."""
    _run_rows(kind, n_vocab, ROW_PARAMS)


def test_sample_logits_rejects_bad_arguments():
    import transformer_decode_forward_amd as tdf
    from transformer_decode_forward_amd.device import to_device
    cfg, w = make_weights(SMALL)
    gc = tdf.Context(device_model(cfg, w), n_ctx=64, kv_dtype="bf16")
    d = to_device(tdf_synth.logit_rows(1, "normal", 2, 100))
    assert gc.sample_logits(d.data_ptr(), 2, 0, 1.0, 10, 1.0, 0.0, [0.5, 0.5])[0] == tdf.TDF_E_INVALID
    assert gc.sample_logits(d.data_ptr(), -1, 100, 1.0, 10, 1.0, 0.0, [0.5])[0] == tdf.TDF_E_INVALID
    assert gc.sample_logits(d.data_ptr(), 2, 100, 1.0, 0, 1.0, 0.0, [0.5, 0.5])[0] == tdf.TDF_E_INVALID
    assert gc.sample_logits(0, 2, 100, 1.0, 10, 1.0, 0.0, [0.5, 0.5])[0] == tdf.TDF_E_INVALID
    assert gc.sample_logits(d.data_ptr(), 0, 100, 1.0, 10)[0] == tdf.TDF_OK
