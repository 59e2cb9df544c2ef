"""Comparison of the GPU's verify decisions with the oracle's.

Accept decisions and accepted-prefix lengths must be bit-exact wherever the
oracle's margin |u - p/q| exceeds the tie band (1e-5) at every decision up to
the first rejection; at least MIN_COMPARED of the sequences must be outside
such ties, so a case cannot pass by excluding what it was meant to compare.

The token that ends a round is drawn by inverse CDF: the smallest y with
C[y] > T, T = u * Z. Where T lies farther than band * Z from both edges of
the oracle's cell, the GPU's token must equal the oracle's. Inside that band
the two computations may round to different sides of an edge, so the GPU's
token must lie in the set of tokens whose cells meet [T - band Z, T + band Z]:
what any sampler whose cumulative weights are within band * Z of the exact
ones could return (a few tokens of the vocabulary). At V = 128256 a token's
cell is often narrower than the band, so many draws are checked this way;
every sequence is checked one way or the other.
"""

import numpy as np

from oracle import speculative as spec

MIN_COMPARED = 0.9


def tie_masks(ref, band=spec.TIE_BAND):
    """(n_tie, tok_tie) per sequence of an oracle verify_batch result:
    the prefix length depends on a decision within the band, and the
    emitted tokens do (the prefix, the draw's margin, or the empty-residual
    fallback)."""
    K = ref["accept"].shape[1]
    upto = np.arange(K)[None, :] <= np.minimum(ref["n_accepted"], K - 1)[:, None]
    n_tie = ref["n_tie"] | np.any((ref["accept_margin"] <= band) & upto, axis=1)
    tok_tie = n_tie | ref["token_tie"] | (ref["sample_margin"] <= band)
    return n_tie, tok_tie


def band_tokens(weights, u, band=spec.TIE_BAND):
    """Tokens whose inverse-CDF cell [C[y-1], C[y]) meets
    [T - band Z, T + band Z], T = u Z, for unnormalised weights."""
    w = np.asarray(weights, dtype=np.float64)
    c = np.cumsum(w)
    z = float(c[-1])
    t = float(u) * z
    prev = np.concatenate([[0.0], c[:-1]])
    return np.flatnonzero((w > 0) & (c > t - band * z) & (prev < t + band * z))


def compare_rounds(out, n, ref, what, u_sample, P=None, Q=None, band=spec.TIE_BAND,
                   min_compared=MIN_COMPARED):
    """Asserts GPU (out_tokens [B][K+1], n_emitted [B]) against the oracle's
    verify result `ref` on probabilities P [B][K+1][V], Q [B][K][V] (by
    default those the result carries) and the sample uniforms. Returns
    (sequences, prefix ties, draws checked within the band)."""
    P = ref["P"] if P is None else P
    Q = ref["Q"] if Q is None else Q
    n_tie, tok_tie = tie_masks(ref, band)
    B, K = len(n), ref["accept"].shape[1]
    assert B - int(n_tie.sum()) >= min_compared * B, f"{what}: prefix ties {int(n_tie.sum())}/{B}"
    assert np.array_equal(n[~n_tie], ref["n_emitted"][~n_tie]), what
    exact = ~tok_tie
    assert np.array_equal(out[exact], ref["out_tokens"][exact]), what
    in_band = np.flatnonzero(tok_tie & ~n_tie)
    widths = []
    for b in in_band:
        k = int(ref["n_accepted"][b])
        assert np.array_equal(out[b, :k], ref["out_tokens"][b, :k]), (what, b)
        w = spec.residual_weights(P[b][k], Q[b][k])[0] if k < K else P[b][K]
        allowed = band_tokens(w, u_sample[b][k], band)
        widths.append(len(allowed))
        assert int(out[b, k]) in allowed, (what, b, int(out[b, k]), allowed[:8])
    for b in range(B):
        assert (out[b, n[b]:] == -1).all() and (out[b, :n[b]] >= 0).all(), what
    print(f"{what}: {B} sequences, {int(n_tie.sum())} prefix ties, {int(exact.sum())} tokens "
          f"exact, {len(in_band)} within the band (at most {max(widths, default=0)} candidates), "
          f"mean emitted {float(np.mean(n)):.3f}", flush=True)
    return B, int(n_tie.sum()), len(in_band)


def floor_over_rounds(total, prefix_ties, what, min_compared=MIN_COMPARED):
    """The floor on prefix ties applied to counts gathered over rounds."""
    assert total > 0 and total - prefix_ties >= min_compared * total, \
        f"{what}: {prefix_ties} of {total} prefixes tie"
