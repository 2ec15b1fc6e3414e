"""tdf_sample_logits_static (the allocation-free variant of
tdf_sample_logits) against tdf_sample_logits on the same device rows: greedy
(its partial maxima in the library's static device array) and the sampling
chain, two calls in a row on a caller's stream, the second with fewer rows
than the first (the array still holds the first call's partials), and the
size limit of the static array."""
import ctypes

import numpy as np
import pytest

import tdf_synth

pytestmark = pytest.mark.gpu

V = 128256


def _ctx():
    import transformer_decode_forward_amd as tdf
    hp = dict(n_vocab=64, n_embd=64, n_layer=0, n_head=1, n_head_kv=1, head_dim=64, n_ff=64,
              rms_eps=1e-5, rope_theta=1e4, tied=True, weight_dtype="f32")
    import torch
    emb = torch.zeros(64, 64, device="cuda")
    gain = torch.ones(64, device="cuda")
    m = tdf.Model(hp, {"token_embd.weight": emb, "output_norm.weight": gain})
    return m, tdf.Context(m, n_ctx=8, kv_dtype="f32"), (emb, gain)


def _static(rows_dev, n, params, u_dev, stream):
    import torch
    import transformer_decode_forward_amd as tdf
    out = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    p = tdf.tdf_sampling(*params)
    rc = tdf.tdf_sample_logits_static(rows_dev.data_ptr(), n, V, p, u_dev.data_ptr() if u_dev is not None else 0,
                                      out.data_ptr(), stream.cuda_stream)
    assert rc == 0, tdf.tdf_last_error()
    stream.synchronize()
    return out.cpu().numpy().tolist()


@pytest.mark.parametrize("params", [(0.0, 40, 1.0, 0.0), (0.8, 40, 0.9, 0.05), (1.0, 1024, 0.95, 0.0)])
def test_static_variant_matches_existing_entry_point(params):
    import torch
    m, ctx, keep = _ctx()
    stream = torch.cuda.Stream()
    for n, seed in ((64, 21), (5, 22)):
        rows = torch.from_numpy(tdf_synth.logit_rows(seed, "normal", n, V).astype(np.float32)).cuda()
        u = np.random.default_rng(seed).random(n).astype(np.float32)
        u_dev = torch.from_numpy(u).cuda()
        torch.cuda.synchronize()
        got = _static(rows, n, params, u_dev, stream)
        rc, ref = ctx.sample_logits(rows.data_ptr(), n, V, *params, u=u.tolist())
        assert rc == 0
        assert got == ref, (n, params)
        if params[0] <= 0:
            assert got == np.argmax(rows.cpu().numpy(), axis=1).tolist()
    ctx.close()
    m.close()


def test_static_variant_rejects_oversize_and_bad_arguments():
    import torch
    import transformer_decode_forward_amd as tdf
    rows = torch.zeros(4, V, device="cuda")
    out = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    greedy = tdf.tdf_sampling(0.0, 40, 1.0, 0.0)
    # 2081 rows of 128256 logits need more partials than the static array holds
    assert tdf.tdf_sample_logits_static(rows.data_ptr(), 2081, V, greedy, 0, out.data_ptr(), 0) == tdf.TDF_E_INVALID
    assert "static scratch" in tdf.tdf_last_error()
    assert tdf.tdf_sample_logits_static(rows.data_ptr(), -1, V, greedy, 0, out.data_ptr(), 0) == tdf.TDF_E_INVALID
    bad = tdf.tdf_sampling(1.0, 4096, 1.0, 0.0)
    assert tdf.tdf_sample_logits_static(rows.data_ptr(), 4, V, bad, rows.data_ptr(), out.data_ptr(), 0) \
        == tdf.TDF_E_INVALID
    torch.cuda.synchronize()
    assert out.cpu().tolist() == [-7] * 4  # nothing was enqueued
    # zero rows: nothing to do
    assert tdf.tdf_sample_logits_static(rows.data_ptr(), 0, V, greedy, 0, out.data_ptr(), 0) == tdf.TDF_OK
