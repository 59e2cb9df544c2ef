"""Oracle softmax over vocabulary rows, in fp64 (test infrastructure).

The target's and the draft's distributions are the softmax of their logits
("Speculative Decoding: Two Models, One Voice", Implementing it against a
real model: p = softmax(target logits), q = softmax(draft logits)); the rule
needs properly normalised distributions over the same vocabulary
("Speculative Decoding: The Algebra and the Proof", Where it breaks). No
temperature is applied (T = 1).
"""

import numpy as np


def softmax_rows(logits):
    """Softmax of every row of float32 logits, computed in float64.

    Returns (p, row_max, row_sumexp) where, per row, row_max = max_v l[v],
    row_sumexp = sum_v exp(l[v] - row_max) and p[v] = exp(l[v] - row_max) /
    row_sumexp. Subtracting the maximum leaves p unchanged and keeps exp in
    range.
    """
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    m = l.max(axis=-1, keepdims=True)
    e = np.exp(l - m)
    s = e.sum(axis=-1, keepdims=True)
    return e / s, m[..., 0], s[..., 0]
