"""Top-k score-gap enforcement for generated activations -- TEST INFRASTRUCTURE.

A token's expert selection is only well defined across precisions when the
k-th and (k+1)-th router logits are apart; a token whose fp64 logit gap at
rank k is below ``gap`` gets its activation row redrawn from the next
sub-stream.  Logits come from the oracle (``oracle.router_logits``), so the
generator module itself holds no layer arithmetic.
"""
from __future__ import annotations

import numpy as np

from . import router_logits


def kth_gaps(z: np.ndarray, k: int) -> np.ndarray:
    """z_(k) - z_(k+1) per row (fp64 logit space, after any bias)."""
    s = -np.sort(-z, axis=1)
    if k >= z.shape[1]:
        return np.full(z.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


def enforce_gap(shape, x: np.ndarray, wr: np.ndarray, bias, redraw, gap: float = 1e-3,
                max_redraws: int = 64):
    """Redraw rows of ``x`` until every token's gap is >= ``gap``.

    ``redraw(t, r)`` returns the r-th redraw of token t as bf16 bits.
    Returns (x, number_of_redraws).
    """
    x = np.array(x, copy=True)
    n = 0
    for _ in range(max_redraws):
        z = router_logits(shape, x, wr, bias)
        bad = np.nonzero(kth_gaps(z, shape.top_k) < gap)[0]
        if len(bad) == 0:
            return x, n
        for t in bad:
            n += 1
            x[t] = redraw(int(t), n)
    raise RuntimeError("could not reach a top-k gap of %g after %d redraws" % (gap, n))
