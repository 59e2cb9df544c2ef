"""Oracle softmax over vocabulary rows, in fp64 (test infrastructure).

The target's and the draft's distributions are the softmax of their logits
("Speculative Decoding: Two Models, One Voice", Implementing it against a
real model: p = softmax(target logits), q = softmax(draft logits)); the rule
needs properly normalised distributions over the same vocabulary
("Speculative Decoding: The Algebra and the Proof", Where it breaks).

Temperature warps the logits before the softmax, p = softmax(l / T); the
rule is then exact with respect to the warped distributions ("Two Models,
One Voice", Three remarks worth internalizing; "Speculative Decoding: Guess
Several Tokens, Check Them in One Pass", What happens to the rejected
tokens). At T = 0 the distribution puts all its mass on the most probable
token, which turns the rule into greedy verification ("Two Models", the same
remarks). Reading: among equal maxima the smallest token id is the argmax.
"""

import numpy as np


def softmax_rows(logits, temperature=1.0):
    """Softmax of every row of float32 logits at temperature T, in float64.

    Returns (p, row_max, row_sumexp) where, per row, row_max = max_v l[v],
    row_sumexp = sum_v exp((l[v] - row_max) / T) and p[v] = exp((l[v] -
    row_max) / T) / row_sumexp. Subtracting the maximum leaves p unchanged
    and keeps exp in range. T = 0 gives the one-hot distribution of the
    first maximum (row_sumexp = 1).
    """
    T = float(temperature)
    if not (T >= 0.0) or not np.isfinite(T):
        raise ValueError("temperature must be finite and >= 0")
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    m = l.max(axis=-1, keepdims=True)
    if T == 0.0:
        p = np.zeros_like(l)
        idx = np.argmax(l, axis=-1)  # first maximum
        np.put_along_axis(p, idx[..., None], 1.0, axis=-1)
        return p, m[..., 0], np.ones(m.shape[:-1])
    e = np.exp((l - m) / T)
    s = e.sum(axis=-1, keepdims=True)
    return e / s, m[..., 0], s[..., 0]
