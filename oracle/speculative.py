"""Oracle for speculative sampling over the K+1 verified positions (fp64).

TEST INFRASTRUCTURE (see the package docstring for who may import it).

Row convention, per sequence. The drafter proposes K tokens x_1..x_K, x_i
drawn from q_i; the one target pass yields p_1..p_{K+1}, where p_{i+1} is the
target's distribution for the slot after x_1..x_i ("Speculative Decoding: Two
Models, One Voice", The idea, step 2, and the pseudocode's
``logits[:, n-1:]`` slice). Arrays are 0-based:

    P[j] = p_{j+1}  (j = 0..K),   Q[j] = q_{j+1}  (j = 0..K-1),
    tokens[j] = x_{j+1}.

The pages draw the random numbers inside the sampler. Here they are inputs,
so that the GPU path and this oracle consume the same draws (the method only
fixes the law of the output, "Speculative Decoding: The Algebra and the
Proof", The proof):

    u_accept[j]  drives the accept test of tokens[j];
    u_sample[j]  drives the sample that ends the round at row j (the first
                 rejection, or j = K for the bonus token). Only that one
                 sample uniform is consumed per round.

Readings where the pages disagree or are silent (each also listed in the
design notes of the repository):

* strict ``u < ratio`` and no epsilon in the ratio (the "Two Models" and
  "Guess Several Tokens" code and the wiki pseudocode; the wpnews sampler's
  ``<=`` and ``q + 1e-10`` differ only on ties);
* q(x) = 0 for a proposed token: ratio = +inf if p(x) > 0, else 0;
* zero residual mass: fall back to p itself and flag it (the wpnews
  sampler's guard; "The Algebra and the Proof" warns of the division by zero
  when p = q);
* invalid inputs: a draft token outside the vocabulary is rejected (it
  cannot have been proposed), a row with no positive weight draws token -1,
  and a number of accepted drafts outside [0, K] draws token -1;
* inverse-CDF sampling in ascending token id: the token is the smallest y
  whose cumulative weight exceeds u * Z. The pages fix only the law of the
  sampled token, not this map from u to a token id: parity unpinned by the
  pages; it is a convention shared with the GPU path.
"""

import math

import numpy as np

from .softmax import softmax_rows

# Decisions whose margin to the rounding-sensitive threshold is at most this
# are reported as ties and excluded from bit-exact comparison.
TIE_BAND = 1e-5


# --------------------------------------------------------------------------
# One position
# --------------------------------------------------------------------------

def accept_ratio(p_x, q_x):
    """p(x)/q(x) with the q(x) = 0 convention (+inf if p(x) > 0, else 0)."""
    p_x = float(p_x)
    q_x = float(q_x)
    if q_x > 0.0:
        return p_x / q_x
    return math.inf if p_x > 0.0 else 0.0


def accept_test(P, Q, tokens, u_accept):
    """Accept test at every draft position.

    A proposal x drawn from q is kept with probability min(1, p(x)/q(x))
    ("Two Models, One Voice", The idea, step 3; "Guess Several Tokens",
    Step 3). With u uniform on [0, 1), ``u < p(x)/q(x)`` happens with exactly
    that probability (u < 1 makes the min(1, .) automatic).

    Returns (accept bool[K], ratio float64[K], margin float64[K]) with
    margin = |u - ratio| (inf when the ratio is inf).
    """
    K = len(tokens)
    accept = np.zeros(K, dtype=bool)
    ratio = np.zeros(K, dtype=np.float64)
    margin = np.zeros(K, dtype=np.float64)
    for j in range(K):
        x = int(tokens[j])
        V = len(P[j])
        # a token outside the vocabulary cannot have been proposed: rejected
        r = accept_ratio(P[j][x], Q[j][x]) if 0 <= x < V else 0.0
        u = float(u_accept[j])
        ratio[j] = r
        accept[j] = u < r
        margin[j] = math.inf if math.isinf(r) else abs(u - r)
    return accept, ratio, margin


def first_rejection(accept):
    """Number of accepted drafts: the index of the first rejection, or K.

    Drafts after the first rejection were conditioned on a prefix that no
    longer exists and are discarded, so the accepted tokens are a prefix
    ("Two Models, One Voice", The rule that makes it exact, second remark).
    """
    for j, ok in enumerate(accept):
        if not ok:
            return j
    return len(accept)


def residual_weights(p, q):
    """Unnormalised residual max(0, p - q) and a zero-mass flag.

    After a rejection the replacement is drawn from norm(max(0, p - q))
    ("Two Models, One Voice", The rule that makes it exact). If the residual
    has no mass, the weights fall back to p and the flag is set.
    """
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    r = np.maximum(p - q, 0.0)
    if not (r.sum() > 0.0):
        return p.copy(), True
    return r, False


def inverse_cdf(weights, u):
    """Sample a token from unnormalised weights with the uniform u.

    With C the running sum of the weights in ascending token id and
    Z = C[V-1], the token is the smallest y with C[y] > u * Z. If rounding
    leaves no such y, it is the largest y with a positive weight.

    Returns (token, margin) where margin = min(T - C[y-1], C[y] - T) / Z is
    the distance of T = u * Z to the nearest edge of the chosen cell,
    relative to the total mass. Weights with no positive entry give -1.
    """
    w = np.asarray(weights, dtype=np.float64)
    if not np.any(w > 0.0):
        return -1, 0.0  # nothing to draw from
    c = np.cumsum(w)
    z = float(c[-1])
    t = float(u) * z
    y = int(np.searchsorted(c, t, side="right"))
    if y >= len(w):
        y = int(np.flatnonzero(w > 0.0)[-1])
    lo = float(c[y - 1]) if y > 0 else 0.0
    margin = min(t - lo, float(c[y]) - t) / z if z > 0.0 else 0.0
    return y, margin


# --------------------------------------------------------------------------
# One round (one sequence)
# --------------------------------------------------------------------------

def sample_row(P, Q, n, u_sample):
    """The token that ends the round after n accepted drafts.

    n < K: draw from the residual of row n with u_sample[n].
    n = K: every draft survived; draw the bonus token from p_{K+1} = P[K]
    with u_sample[K] ("Two Models, One Voice", The idea, step 3).
    Returns (token, margin, zero_residual).
    """
    K = len(Q)
    if n < K:
        w, zero = residual_weights(P[n], Q[n])
    else:
        w, zero = np.asarray(P[K], dtype=np.float64), False
    y, margin = inverse_cdf(w, u_sample[n])
    return y, margin, zero


def verify_round(P, Q, tokens, u_accept, u_sample):
    """One speculative round on probabilities: accept, first rejection,
    resample or bonus, emit.

    The round emits the n accepted drafts followed by one sampled token, so
    between 1 and K+1 tokens ("Two Models, One Voice", Appendix tool 2: the
    round emits N + 1 tokens in every case).
    """
    K = len(tokens)
    accept, ratio, amargin = accept_test(P, Q, tokens, u_accept)
    n = first_rejection(accept)
    y, smargin, zero = sample_row(P, Q, n, u_sample)
    out = np.full(K + 1, -1, dtype=np.int64)
    out[:n] = np.asarray(tokens[:n], dtype=np.int64)
    out[n] = y
    # n depends on the decisions at positions 0..min(n, K-1).
    n_tie = bool(np.any(amargin[:min(n, K - 1) + 1] <= TIE_BAND)) if K > 0 else False
    return {
        "out_tokens": out,
        "n_emitted": n + 1,
        "n_accepted": n,
        "accept": accept,
        "ratio": ratio,
        "accept_margin": amargin,
        "token": y,
        "sample_margin": smargin,
        "zero_residual": zero,
        "n_tie": n_tie,
        "token_tie": n_tie or smargin <= TIE_BAND or zero,
    }


# --------------------------------------------------------------------------
# Batches
# --------------------------------------------------------------------------

_BATCH_KEYS = ("out_tokens", "n_emitted", "n_accepted", "accept", "ratio",
               "accept_margin", "token", "sample_margin", "zero_residual",
               "n_tie", "token_tie")


def verify_batch_probs(P, Q, tokens, u_accept, u_sample):
    """verify_round for every sequence b of P[B][K+1][V], Q[B][K][V]."""
    rounds = [verify_round(P[b], Q[b], tokens[b], u_accept[b], u_sample[b])
              for b in range(len(tokens))]
    return {k: np.array([r[k] for r in rounds]) for k in _BATCH_KEYS}


def verify_batch(target_logits, draft_logits, tokens, u_accept, u_sample, t_target=1.0,
                 t_draft=1.0):
    """The whole sampling stage from float32 logits.

    target_logits [B][K+1][V], draft_logits [B][K][V] -> softmax in fp64 at
    temperatures t_target (the requested law) and t_draft (the law the
    drafts were drawn from) -> verify_round per sequence. Also returns the
    probabilities. t_target = 0 is greedy verification: the warped target is
    one-hot at its argmax, so a draft is kept iff it is that argmax and the
    round ends with the argmax ("Two Models, One Voice", Three remarks worth
    internalizing).
    """
    P, _, _ = softmax_rows(target_logits, t_target)
    Q, _, _ = softmax_rows(draft_logits, t_draft)
    res = verify_batch_probs(P, Q, tokens, u_accept, u_sample)
    res["P"] = P
    res["Q"] = Q
    return res


def accept_batch(P, Q, tokens, u_accept):
    """Accept stage alone: (n_accepted int[B], accept bool[B][K],
    accept_margin float64[B][K], n_tie bool[B])."""
    B = len(tokens)
    K = len(tokens[0]) if B else 0
    n_acc = np.zeros(B, dtype=np.int64)
    acc = np.zeros((B, K), dtype=bool)
    mar = np.zeros((B, K), dtype=np.float64)
    tie = np.zeros(B, dtype=bool)
    for b in range(B):
        a, _, m = accept_test(P[b], Q[b], tokens[b], u_accept[b])
        n = first_rejection(a)
        n_acc[b], acc[b], mar[b] = n, a, m
        tie[b] = bool(np.any(m[:min(n, K - 1) + 1] <= TIE_BAND))
    return n_acc, acc, mar, tie


def sample_batch(P, Q, n_accepted, u_sample):
    """Sample stage alone, given n_accepted per sequence: (token int[B],
    sample_margin float64[B], zero_residual bool[B])."""
    B = len(n_accepted)
    tok = np.zeros(B, dtype=np.int64)
    mar = np.zeros(B, dtype=np.float64)
    zero = np.zeros(B, dtype=bool)
    for b in range(B):
        n = int(n_accepted[b])
        if not 0 <= n <= len(Q[b]):
            tok[b] = -1  # not a number of accepted drafts
            continue
        tok[b], mar[b], zero[b] = sample_row(P[b], Q[b], n, u_sample[b])
    return tok, mar, zero


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------

def acceptance_rate(p, q):
    """alpha = sum_x min(p(x), q(x)), the probability that a proposal from q
    is accepted ("Two Models, One Voice", Appendix tool 1 (a))."""
    return float(np.minimum(np.asarray(p, np.float64), np.asarray(q, np.float64)).sum())


def total_variation(p, q):
    """TV(p, q) = 1/2 sum_x |p(x) - q(x)|; alpha = 1 - TV ("The Algebra and
    the Proof", The proof)."""
    return 0.5 * float(np.abs(np.asarray(p, np.float64) - np.asarray(q, np.float64)).sum())


def emitted_law(p, q):
    """Exact law of the token emitted at one position, and the acceptance
    probability, from the two events of the rule.

    A proposal x comes from q and is kept with probability
    a(x) = min(1, p(x)/q(x)); a token with q(x) = 0 is never proposed. So x
    is emitted by acceptance with probability q(x) a(x). Otherwise -- with
    probability sum_x q(x) (1 - a(x)) -- the token comes from the normalised
    residual (p - q)_+ ("The Algebra and the Proof", The proof; "Two Models,
    One Voice", The rule that makes it exact). The law is the sum of the two
    parts; the second is zero when the residual has no mass (then nothing is
    ever rejected). Returns (law, alpha) with alpha = sum_x q(x) a(x).
    """
    p = np.asarray(p, np.float64)
    q = np.asarray(q, np.float64)
    keep = np.zeros_like(q)
    proposed = q > 0.0
    keep[proposed] = np.minimum(1.0, p[proposed] / q[proposed])
    by_acceptance = q * keep
    alpha = float(by_acceptance.sum())
    rejected = float((q * (1.0 - keep)).sum())
    resid = np.maximum(p - q, 0.0)
    mass = float(resid.sum())
    by_resample = rejected * resid / mass if mass > 0.0 else np.zeros_like(p)
    return by_acceptance + by_resample, alpha


def expected_tokens(alpha, K):
    """E[tokens per round] = (1 - alpha^{K+1}) / (1 - alpha) for i.i.d.
    acceptance ("Two Models, One Voice", Appendix tool 2); K+1 at alpha = 1."""
    if alpha == 1.0:
        return float(K + 1)
    return (1.0 - alpha ** (K + 1)) / (1.0 - alpha)


def expected_tokens_general(alphas):
    """E[N] = 1 + sum_{i=1}^{K} prod_{j<=i} alpha_j with position-dependent
    conditional acceptance alpha_j ("The Algebra and the Proof", The algebra)."""
    total, prod = 1.0, 1.0
    for a in alphas:
        prod *= float(a)
        total += prod
    return total
