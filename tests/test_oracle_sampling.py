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
