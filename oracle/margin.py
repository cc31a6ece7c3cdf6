"""Margin audit of the block selection (fp64), used to keep floating-point ties
from flipping a block between the oracle and any other implementation.

A row of pooled scores passes when, in fp64 on the final bf16 data:

* at every selection boundary r (the first r blocks of the descending order
  are on one side), the scores on either side differ by at least ``gap``
  (2e-4: each score is at least 1e-4 from the midpoint);
* for the NABLA cut with K kept blocks, the cumulative softmax masses c_K and
  c_(K-1) both differ from 1 - thr by at least ``mass_gap`` (1e-4).

TEST INFRASTRUCTURE ONLY (see the package header).
"""

import numpy as np

from . import sla


def row_ok(s_row, boundaries=(), thr=None, gap=2e-4, mass_gap=1e-4):
    s = np.asarray(s_row, dtype=np.float64)
    order = sla.descending_order(s)
    ss = s[order]
    nkb = len(ss)
    cuts = [r for r in boundaries if 0 < r < nkb]
    if thr is not None:
        K = sla.cdf_count(s, thr)
        if K < nkb:
            cuts.append(K)
        p = sla.softmax(s)[order]
        c = np.concatenate([[0.0], np.cumsum(p)])
        target = 1.0 - thr
        if abs(c[K] - target) < mass_gap or abs(c[K - 1] - target) < mass_gap:
            return False
    for r in cuts:
        if ss[r - 1] - ss[r] < gap:
            return False
    return True


def failing_rows(scores, boundaries=(), thr=None, gap=2e-4, mass_gap=1e-4):
    """Indices (as tuples over the leading axes) of rows that fail the audit."""
    lead = scores.shape[:-1]
    flat = scores.reshape(-1, scores.shape[-1])
    bad = [r for r in range(flat.shape[0]) if not row_ok(flat[r], boundaries, thr, gap, mass_gap)]
    return [np.unravel_index(r, lead) for r in bad]
