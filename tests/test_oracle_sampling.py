"""Pins of the oracle's sampling chain (Ollama engine page, "Token sampling
pipeline").  The draw is inverse-CDF sampling, so on a uniform grid of N
draws each surviving token is chosen about N times its renormalised
probability; the filters are checked on distributions with known
probabilities (logits = log p reproduce p through the softmax)."""
import numpy as np
import pytest

from oracle.sampling import rank, sample, sample_margin

N = 20000
GRID = (np.arange(N) + 0.5) / N


def counts(z, t, k, p, mp):
    out = np.zeros(len(z), dtype=np.int64)
    for u in GRID:
        out[sample(z, t, k, p, mp, u)] += 1
    return out


def softmax(x):
    e = np.exp(x - np.max(x))
    return e / e.sum()


def test_greedy_cases():
    rng = np.random.default_rng(0)
    z = rng.normal(size=50)
    best = int(np.argmax(z))
    for u in (0.0, 0.3, 0.999):
        assert sample(z, 0.0, 50, 1.0, 0.0, u) == best       # temperature 0
        assert sample(z, -1.0, 50, 1.0, 0.0, u) == best
        assert sample(z, 0.8, 1, 1.0, 0.0, u) == best        # top-k 1
        assert sample(z, 1e-6, 50, 1.0, 0.0, u) == best      # vanishing temperature
        assert sample(z, 1.0, 50, 1e-9, 0.0, u) == best      # top-p keeps the first only
        assert sample(z, 1.0, 50, 1.0, 1.0, u) == best       # min-p 1 keeps the maximum only


def test_ties_go_to_the_lower_id():
    z = np.array([2.0, 5.0, 5.0, 1.0])
    assert list(rank(z)) == [1, 2, 0, 3]
    assert sample(z, 1.0, 1, 1.0, 0.0, 0.9) == 1
    assert sample(z, 0.0, 4, 1.0, 0.0, 0.9) == 1


@pytest.mark.parametrize("t", [1.0, 0.5, 2.0])
def test_frequencies_follow_the_tempered_softmax(t):
    z = np.array([0.3, -1.2, 2.0, 0.0, 1.1, -0.4])
    c = counts(z, t, 6, 1.0, 0.0)
    assert np.all(np.abs(c - N * softmax(z / t)) <= 1.0)


def test_top_k_renormalises_the_kept_tokens():
    z = np.array([0.3, -1.2, 2.0, 0.0, 1.1, -0.4])
    c = counts(z, 1.0, 2, 1.0, 0.0)
    p = np.zeros(6)
    p[[2, 4]] = softmax(z[[2, 4]])
    assert np.all(np.abs(c - N * p) <= 1.0)


def test_top_p_keeps_cumulative_at_most_p():
    p = np.array([0.05, 0.5, 0.15, 0.3])
    z = np.log(p)
    # ranking 1, 3, 2, 0 with cumulative 0.5, 0.8, 0.95, 1.0
    assert np.array_equal(counts(z, 1.0, 4, 0.75, 0.0), [0, N, 0, 0])
    c = counts(z, 1.0, 4, 0.9, 0.0)
    assert c[0] == c[2] == 0 and abs(c[1] - N * 0.5 / 0.8) <= 1 and abs(c[3] - N * 0.3 / 0.8) <= 1
    c = counts(z, 1.0, 4, 0.97, 0.0)
    assert c[0] == 0 and abs(c[2] - N * 0.15 / 0.95) <= 1


def test_min_p_threshold_relative_to_the_top():
    p = np.array([0.05, 0.5, 0.15, 0.3])
    z = np.log(p)
    c = counts(z, 1.0, 4, 1.0, 0.25)   # threshold 0.125: drops 0.05
    assert c[0] == 0 and abs(c[2] - N * 0.15 / 0.95) <= 1
    c = counts(z, 1.0, 4, 1.0, 0.61)   # threshold 0.305: keeps 0.5 only
    assert np.array_equal(c, [0, N, 0, 0])


def test_margin_flags_boundaries():
    p = np.array([0.5, 0.3, 0.2])
    z = np.log(p)
    assert sample_margin(z, 1.0, 3, 1.0, 0.0, 0.5) < 1e-9        # u * total on a cumulative boundary
    assert sample_margin(z, 1.0, 3, 1.0, 0.0, 0.25) > 0.1


def test_margin_values_on_hand_cases():
    """The margin of each decision, written out from its definition on a
    distribution with known probabilities (0.5, 0.3, 0.2)."""
    p = np.array([0.5, 0.3, 0.2])
    z = np.log(p)
    # greedy: the top-2 logit gap
    assert sample_margin(np.array([1.0, 3.0, 2.5]), 0.0, 3, 1.0, 0.0, 0.3) == 0.5
    # Top-P 0.75: cumulative 0.5 | 0.8, 1.0 -> nearest cut distance 0.05; the
    # draw over the single survivor is 0.5 (1 - u) = 0.45 away
    np.testing.assert_allclose(sample_margin(z, 1.0, 3, 0.75, 0.0, 0.1), 0.05, rtol=1e-12)
    # Min-P 0.5: threshold 0.25, relative distances |0.3 - 0.25| / 0.25 = |0.2 - 0.25| / 0.25 = 0.2;
    # the draw over the two survivors at u = 0.3 is min(|0.5 - 0.24|, |0.8 - 0.24|) = 0.26
    np.testing.assert_allclose(sample_margin(z, 1.0, 3, 1.0, 0.5, 0.3), 0.2, rtol=1e-12)
    # the draw alone: |cumulative - u| = 0.01 at u = 0.49
    np.testing.assert_allclose(sample_margin(z, 1.0, 3, 1.0, 0.0, 0.49), 0.01, rtol=1e-9)
    # temperature enters before the softmax: T = 2 on log p gives p^(1/2) renormalised
    q = np.sqrt(p) / np.sqrt(p).sum()
    np.testing.assert_allclose(sample_margin(z, 2.0, 3, 1.0, 0.0, 0.2), abs(q[0] - 0.2), rtol=1e-9)


def test_margin_locates_real_boundaries():
    """Brute force: wherever the margin is small the token changes under a
    tiny move of u, and a move of u below the margin never changes it."""
    rng = np.random.default_rng(5)
    for _ in range(200):
        z = rng.normal(size=12) * 2
        t, k, tp, mp = 0.9, 8, 0.9, 0.05
        u = float(rng.uniform())
        m = sample_margin(z, t, k, tp, mp, u)
        tok = sample(z, t, k, tp, mp, u)
        # the draw's cumulative moves by at most |du| * total <= |du| when u moves by du
        for du in (-0.5 * m, 0.5 * m):
            if 0.0 <= u + du < 1.0:
                assert sample(z, t, k, tp, mp, u + du) == tok
    # u set exactly on a cumulative boundary: the two sides differ
    p = np.array([0.5, 0.3, 0.2])
    z = np.log(p)
    assert sample_margin(z, 1.0, 3, 1.0, 0.0, 0.8) < 1e-9
    assert sample(z, 1.0, 3, 1.0, 0.0, 0.8 - 1e-6) != sample(z, 1.0, 3, 1.0, 0.0, 0.8 + 1e-6)
