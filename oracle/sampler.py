"""Float64 oracle of the article's sampler (test infrastructure only).

Source: "Inside an LLM: Pure Python Inference for Qwen3-0.6B on MLX", Step 8
(LM head and sampling). Steps, in the article's order:

1. temperature 0 -> greedy argmax;
2. divide the logits by the temperature;
3. softmax;
4. order the tokens by descending probability;
5. cumulative sum; keep the first ``#{k : cum_k < top_p} + 1`` tokens (the
   smallest prefix whose mass reaches top_p);
6. renormalise the kept probabilities;
7. draw one of them.

Readings of what the article leaves open:
* argmax ties and equal probabilities are ordered by ascending token id (the
  article does not say whether its sort is stable);
* the kept count is capped at the vocabulary size (guards rounding when
  top_p is at or near 1);
* the categorical draw of step 7 takes a supplied uniform u in [0, 1) and
  returns the first kept token whose renormalised cumulative probability
  exceeds u (inverse CDF); if rounding leaves no such token, the last kept one;
* masses, sums and prefix sums are float64; the division by the temperature is
  done in float64 on the float32 logits.
"""
from __future__ import annotations

import numpy as np


def _order(logits: np.ndarray) -> np.ndarray:
    """Token ids by descending logit, ties by ascending id."""
    ids = np.arange(logits.shape[0])
    return np.lexsort((ids, -logits.astype(np.float64)))


def sample(logits: np.ndarray, temperature: float, top_p: float, u: float) -> int:
    logits = np.asarray(logits, dtype=np.float32)
    if temperature == 0:
        return int(np.argmax(logits))          # first (lowest) id among equal maxima
    z = logits.astype(np.float64) / np.float64(temperature)
    e = np.exp(z - z.max())
    probs = e / e.sum()
    order = _order(logits)
    sorted_p = probs[order]
    cum = np.cumsum(sorted_p)
    cutoff = min(len(sorted_p), int(np.sum(cum < top_p)) + 1)
    kept = sorted_p[:cutoff]
    kept = kept / kept.sum()
    cdf = np.cumsum(kept)
    k = int(np.searchsorted(cdf, np.float64(u), side="right"))   # first cdf_k > u
    return int(order[min(k, cutoff - 1)])


def sample_margin(logits: np.ndarray, temperature: float, top_p: float, u: float) -> float:
    """Relative distance of the two sampler decisions from their nearest boundary.

    Returns min(|cum_k - top_p| over k, |cdf_k - u| over kept k), in units of
    probability. A differently-ordered float64 summation can change a decision
    only when this margin is within a few ulps of zero.
    """
    if temperature == 0:
        top2 = np.sort(np.asarray(logits, dtype=np.float64))[-2:]
        return float(top2[1] - top2[0])
    z = np.asarray(logits, dtype=np.float64) / np.float64(temperature)
    e = np.exp(z - z.max())
    probs = e / e.sum()
    order = _order(np.asarray(logits, dtype=np.float32))
    cum = np.cumsum(probs[order])
    cutoff = min(len(cum), int(np.sum(cum < top_p)) + 1)
    kept = probs[order][:cutoff]
    cdf = np.cumsum(kept / kept.sum())
    m1 = float(np.min(np.abs(cum - top_p)))
    m2 = float(np.min(np.abs(cdf - u)))
    return min(m1, m2)
