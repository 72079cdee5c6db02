"""Float64 numpy definition of next-token selection from logits (test infrastructure only).

Follows the linkmax.top LLaMA walkthrough, section 3.3 "generate": with a
positive temperature the logits are divided by it and turned into
probabilities with a softmax, and the token is drawn by nucleus (top-p)
sampling; with temperature 0 the token is the argmax.

Readings taken where the page leaves a step open:

* Order of equal probabilities: the page sorts descending without fixing the
  order of ties; here ties are ordered by ascending token id, which makes
  the kept set and the draw unique.
* The draw: the page calls a multinomial sampler on the renormalised kept
  probabilities.  Here the random number is an input: one u in [0, 1) per
  row, and the token is the first one in sorted order whose inclusive
  cumulative kept probability exceeds u (inverse-CDF sampling, which draws
  from exactly that distribution when u is uniform).

Nothing here is imported by the GPU path; only tests and the benchmark's CPU
leg call it.
"""
from __future__ import annotations

import numpy as np


def softmax_temperature(logits: np.ndarray, temperature: float) -> np.ndarray:
    """Probabilities softmax(logits / temperature) over the last axis (float64)."""
    z = np.asarray(logits, dtype=np.float64) / float(temperature)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def sorted_order(probs: np.ndarray) -> np.ndarray:
    """Token ids of one row in descending probability, ties by ascending id."""
    ids = np.arange(probs.shape[-1])
    return np.lexsort((ids, -probs))


def top_p_keep(probs: np.ndarray, top_p: float):
    """Kept token ids of one row, in sorted order.

    A token is dropped when the probability mass strictly before it in the
    sorted order (the cumulative sum minus its own probability) exceeds
    top_p; the first token is therefore always kept.
    """
    order = sorted_order(probs)
    ps = probs[order]
    before = np.cumsum(ps) - ps
    return order[before <= top_p]


def sample_row(logits: np.ndarray, temperature: float, top_p: float, u: float) -> int:
    """Next token of one row: argmax at temperature <= 0, else top-p sampling driven by u."""
    logits = np.asarray(logits, dtype=np.float64)
    if temperature <= 0:
        return int(np.argmax(logits))           # first index among equal maxima
    probs = softmax_temperature(logits, temperature)
    kept = top_p_keep(probs, top_p)
    q = probs[kept] / probs[kept].sum()         # renormalised kept probabilities
    cdf = np.cumsum(q)
    j = int(np.searchsorted(cdf, u, side="right"))
    return int(kept[min(j, len(kept) - 1)])


def sample(logits: np.ndarray, temperature: float, top_p: float, uniforms: np.ndarray) -> np.ndarray:
    """Next token of every row of [rows, vocab] logits; uniforms holds one u per row."""
    logits = np.asarray(logits)
    return np.array([sample_row(logits[r], temperature, top_p, float(uniforms[r]))
                     for r in range(logits.shape[0])], dtype=np.int64)


def decision_margins(logits: np.ndarray, temperature: float, top_p: float, u: float):
    """How close one row's draw is to a tie in the arithmetic (for comparing a float32 implementation).

    Returns (margin_p, margin_u): the distance, in probability units, from top_p
    to the nearest exclusive cumulative sum around the cut, and from u to the
    nearest boundary of the renormalised cumulative distribution.
    """
    probs = softmax_temperature(logits, temperature)
    order = sorted_order(probs)
    ps = probs[order]
    before = np.cumsum(ps) - ps
    margin_p = float(np.min(np.abs(before - top_p)))
    kept = order[before <= top_p]
    q = probs[kept] / probs[kept].sum()
    cdf = np.cumsum(q)
    margin_u = float(np.min(np.abs(cdf - u)))
    return margin_p, margin_u
