"""Token sampling chain of the oracle (Ollama engine page, "Token sampling
pipeline"; llama.cpp walkthrough, "Steps 14-15" sampler chain).

TEST INFRASTRUCTURE: imported only by tests, smoke() and bench.py's
cpu_baseline leg.

Order of the chain on one row of logits: temperature 0 means greedy
(argmax); otherwise Top-K (keep the K highest logits) -> temperature (divide
the logits by it) -> softmax -> Top-P (keep tokens while the cumulative
probability is <= p) -> Min-P (keep tokens above a threshold) -> weighted
random draw.  The uniform random number of the draw is an input, so that a
seeded caller reproduces the same tokens.

Readings where the pages leave a step open:
* Ordering: candidates are ranked by logit, larger first, ties to the lower
  token id; Top-K keeps the first K of that ranking (K in [1, V]).
* Top-P: token i of the ranking survives when the cumulative probability of
  tokens 0..i is <= p; the first token always survives; p >= 1 keeps every
  token (the cumulative never exceeds 1, whatever the rounding).
* Min-P: the threshold is min_p times the largest probability; tokens with
  probability >= threshold survive.
* Draw: over the survivors in ranking order, the first token whose
  cumulative probability exceeds u times the survivors' total; the last
  survivor if rounding leaves none.
"""
from __future__ import annotations

import numpy as np


def rank(logits: np.ndarray) -> np.ndarray:
    """Token ids ordered by logit (larger first), ties to the lower id."""
    z = np.asarray(logits, dtype=np.float64)
    return np.lexsort((np.arange(z.size), -z))


def sample(logits: np.ndarray, temperature: float, top_k: int, top_p: float, min_p: float,
           u: float) -> int:
    """One token from one row of logits; see the module docstring."""
    z = np.asarray(logits, dtype=np.float64)
    if temperature <= 0:
        return int(np.argmax(z))
    order = rank(z)[: max(1, min(int(top_k), z.size))]
    s = z[order] / float(temperature)
    e = np.exp(s - s[0])
    p = e / e.sum()
    cum = np.cumsum(p)
    keep = cum <= top_p
    keep[0] = True
    if top_p >= 1:
        keep[:] = True
    n = int(np.argmin(keep)) if not keep.all() else keep.size  # survivors form a prefix
    n = min(n, int(np.count_nonzero(p >= min_p * p[0])))
    total = cum[n - 1]
    hit = np.flatnonzero(cum[:n] > u * total)
    return int(order[hit[0]] if hit.size else order[n - 1])


def sample_margin(logits: np.ndarray, temperature: float, top_k: int, top_p: float, min_p: float,
                  u: float) -> float:
    """Smallest distance of a floating-point decision of the chain from its
    boundary: the Top-P cut (|cumulative - p|), the Min-P cut (relative
    |probability - threshold| / threshold), the draw (|cumulative - u total|)
    and, for greedy, the top-2 logit gap.  Two implementations that compute
    the probabilities in different precision or order may disagree only
    where this is tiny."""
    z = np.asarray(logits, dtype=np.float64)
    if temperature <= 0:
        top2 = np.sort(z)[-2:]
        return float(top2[1] - top2[0]) if z.size > 1 else np.inf
    order = rank(z)[: max(1, min(int(top_k), z.size))]
    s = z[order] / float(temperature)
    e = np.exp(s - s[0])
    p = e / e.sum()
    cum = np.cumsum(p)
    m = np.inf
    if cum.size > 1 and top_p < 1:
        m = min(m, float(np.min(np.abs(cum[1:] - top_p))))
    if p.size > 1 and min_p > 0:
        thr = min_p * p[0]
        m = min(m, float(np.min(np.abs(p[1:] - thr))) / thr)
    keep = cum <= top_p
    keep[0] = True
    if top_p >= 1:
        keep[:] = True
    n = int(np.argmin(keep)) if not keep.all() else keep.size
    n = min(n, int(np.count_nonzero(p >= min_p * p[0])))
    m = min(m, float(np.min(np.abs(cum[:n] - u * cum[n - 1]))))
    return m
