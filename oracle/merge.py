"""fp64 log-sum-exp merge of two partial attention results (oracle).

The pages only add partial outputs together ([RAF] section 3, step 5, which
its own comment calls a simplification).  The exact rule follows from the
definition: if a query's keys are split into two disjoint sets with partial
results (O1, L1) and (O2, L2), where O is the softmax-weighted mean of V over
that set and L its natural-log sum of exp(scores), then

    L = ln(e^L1 + e^L2)
    O = e^(L1 - L) * O1 + e^(L2 - L) * O2

An empty set has L = -inf and O = 0; merging with it returns the other
operand unchanged, and two empty sets give (0, -inf).
"""
from __future__ import annotations

import numpy as np


def lse_merge(o1, l1, o2, l2):
    o1 = np.asarray(o1, np.float64)
    o2 = np.asarray(o2, np.float64)
    l1 = np.asarray(l1, np.float64)
    l2 = np.asarray(l2, np.float64)
    l = np.logaddexp(l1, l2)
    empty = np.isneginf(l)
    safe = np.where(empty, 0.0, l)
    w1 = np.where(np.isneginf(l1), 0.0, np.exp(np.where(np.isneginf(l1), 0.0, l1) - safe))
    w2 = np.where(np.isneginf(l2), 0.0, np.exp(np.where(np.isneginf(l2), 0.0, l2) - safe))
    o = w1[..., None] * o1 + w2[..., None] * o2
    o = np.where(empty[..., None], 0.0, o)
    return o, l
