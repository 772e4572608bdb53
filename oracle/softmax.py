"""Row softmax and its top-k in plain fp64 numpy.

TEST INFRASTRUCTURE ONLY (like the rest of this package): the test suite,
the smoke check and the benchmark's CPU-baseline leg are the only callers;
the GPU library shares nothing with it.

What it computes, for each row x of n values:

    y_j = exp(x_j - max x) / sum_k exp(x_k - max x),
    lse = max x + log sum_k exp(x_k - max x),

the classical softmax with the maximum subtracted first (the notebook
"Online Softmax Without the Attention Matrix", code cell: the dense
weighted form; "Online normalizer calculation for softmax", abstract: the
same classical softmax, computed with fewer memory passes).  The online
normaliser is the GPU's way of reaching this result and is not used here.

Top-k: the k largest probabilities of a row with their column indices, in
descending order.  Softmax is increasing in x, so this is the order of x;
equal values come lower index first (a reading: the pages give no rule for
ties).
"""
from __future__ import annotations

import numpy as np


def softmax(x):
    """y [rows, n] and lse [rows] of x [rows, n] (any float dtype), in fp64."""
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=-1, keepdims=True)
    e = np.exp(x - m)
    s = e.sum(axis=-1, keepdims=True)
    return e / s, (m + np.log(s))[..., 0]


def topk(x, k: int):
    """Column indices [rows, k] of the k largest values of each row of x,
    descending, equal values lower index first."""
    x = np.asarray(x, dtype=np.float64)
    rows, n = x.shape
    if not 1 <= k <= n:
        raise ValueError("need 1 <= k <= n")
    cols = np.broadcast_to(np.arange(n), x.shape)
    order = np.lexsort((cols, -x), axis=-1)  # primary key -x, then the index
    return order[:, :k]


def softmax_topk(x, k: int):
    """(probabilities [rows, k], indices [rows, k], lse [rows]): the k largest
    softmax probabilities of each row and where they are."""
    y, lse = softmax(x)
    idx = topk(x, k)
    return np.take_along_axis(y, idx, axis=-1), idx, lse
