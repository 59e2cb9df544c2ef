"""GPU parity of the sampling stage calls against the fp64 oracle.

Both sides receive the same fp32 inputs (logits, or fp32 probabilities that
the oracle's softmax produced and rounded) and the same uniforms. Softmax:
within 1e-6 absolute. Accept decisions, accepted-prefix lengths and sampled
token ids: bit-exact wherever the oracle's margin to the threshold exceeds
1e-5; a token drawn inside that band must be one the band allows; ties are
counted and printed, and at least 90 % of the prefixes must be outside them.
"""

import numpy as np
import pytest

import oracle
import synth
from oracle import speculative as spec
from parity import compare_rounds, tie_masks

pytestmark = pytest.mark.gpu


def to_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


# ---------------------------------------------------------------------------
# softmax
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rows,V,std", [(5, 1000, 2.0), (9, 128256, 1.28), (17, 128256, 3.0),
                                        (3, 1001, 3.0), (2, 1, 1.0), (4, 3, 1.0),
                                        (3, 4097, 8.0)])
def test_softmax(sv, dev, rows, V, std):
    import torch
    l = synth.normals(rows * V, "sm", (rows, V), std)
    p, mx, se = sv.softmax(to_dev(l, dev))
    torch.cuda.synchronize()
    P, M, S = oracle.softmax_rows(l)
    err = float(np.max(np.abs(p.cpu().numpy() - P)))
    print(f"softmax {rows}x{V}: max abs err {err:.2e}", flush=True)
    assert err <= 1e-6
    assert np.array_equal(mx.cpu().numpy().astype(np.float64), M)
    assert np.max(np.abs(se.cpu().numpy() / S - 1)) <= 1e-6


def test_softmax_peaked_row(sv, dev):
    import torch
    V = 128256
    l = synth.normals(5, "peak", (2, V), 1.0)
    l[0, 77] = 40.0   # p ~ 1
    l[1, :] = -3.0
    l[1, V - 1] = 25.0
    p, _, _ = sv.softmax(to_dev(l, dev))
    torch.cuda.synchronize()
    P, _, _ = oracle.softmax_rows(l)
    assert float(np.max(np.abs(p.cpu().numpy() - P))) <= 1e-6


# ---------------------------------------------------------------------------
# accept scan + residual sample on probabilities
# ---------------------------------------------------------------------------

def probs_inputs(seed, B, K, V, std, sigma):
    d = synth.sampling_inputs(seed, B, K, V, std, sigma)
    P, _, _ = oracle.softmax_rows(d["target_logits"])
    Q, _, _ = oracle.softmax_rows(d["draft_logits"])
    d["P32"] = P.astype(np.float32)
    d["Q32"] = Q.astype(np.float32)
    return d


def run_stage(sv, dev, P32, Q32, toks, ua, us):
    import torch
    p, q = to_dev(P32, dev), to_dev(Q32, dev)
    n, mask = sv.accept_scan(p, q, to_dev(toks.astype(np.int32), dev), to_dev(ua, dev))
    tok, zero = sv.residual_sample(p, q, n, to_dev(us, dev))
    torch.cuda.synchronize()
    return n.cpu().numpy(), mask.cpu().numpy(), tok.cpu().numpy(), zero.cpu().numpy()


def compare_stage(gpu, P, Q, toks, ua, us, what):
    """The stage calls' outputs against the oracle's round on the same
    probabilities: accept decisions outside ties, then the round they
    define (accepted drafts and the drawn token) through the shared
    comparison, and the empty-residual flags."""
    n, mask, tok, zero = gpu
    ref = oracle.verify_batch_probs(P, Q, toks, ua, us)
    clear = ref["accept_margin"] > spec.TIE_BAND
    assert np.array_equal(mask.astype(bool)[clear], ref["accept"][clear]), what
    B, K = toks.shape
    out = np.full((B, K + 1), -1, np.int64)
    for b in range(B):
        k = int(n[b])
        out[b, :k] = toks[b, :k]
        out[b, k] = tok[b]
    compare_rounds(out, n + 1, ref, what, us, P=P, Q=Q)
    n_tie, _ = tie_masks(ref)
    assert np.array_equal(zero.astype(bool)[~n_tie], ref["zero_residual"][~n_tie]), what
    return ref["n_accepted"]


@pytest.mark.parametrize("seed", range(8))
def test_stage_tiny_many_seeds(sv, dev, seed):
    d = probs_inputs(seed, 128, 4, 1000, 2.0, 0.5)
    P, Q = d["P32"].astype(np.float64), d["Q32"].astype(np.float64)
    gpu = run_stage(sv, dev, d["P32"], d["Q32"], d["draft_tokens"], d["u_accept"], d["u_sample"])
    n_ref = compare_stage(gpu, P, Q, d["draft_tokens"], d["u_accept"], d["u_sample"], f"tiny s{seed}")
    assert 0 < n_ref.mean() < 4  # both rejections and full accepts occur


@pytest.mark.parametrize("alpha", [0.6, 0.81, 0.9])
def test_stage_stress_shape(sv, dev, alpha):
    sigma = synth.draft_noise_sigma("stress_std3", alpha)
    d = probs_inputs(int(alpha * 100), 64, 8, 128256, 3.0, sigma)
    P, Q = d["P32"].astype(np.float64), d["Q32"].astype(np.float64)
    gpu = run_stage(sv, dev, d["P32"], d["Q32"], d["draft_tokens"], d["u_accept"], d["u_sample"])
    compare_stage(gpu, P, Q, d["draft_tokens"], d["u_accept"], d["u_sample"], f"stress a={alpha}")


@pytest.mark.parametrize("K,V", [(1, 50), (64, 300), (7, 4096), (3, 4097), (2, 1)])
def test_stage_edge_k_and_v(sv, dev, K, V):
    d = probs_inputs(K * 1000 + V, 16, K, V, 2.0, 0.7)
    P, Q = d["P32"].astype(np.float64), d["Q32"].astype(np.float64)
    gpu = run_stage(sv, dev, d["P32"], d["Q32"], d["draft_tokens"], d["u_accept"], d["u_sample"])
    compare_stage(gpu, P, Q, d["draft_tokens"], d["u_accept"], d["u_sample"], f"K={K} V={V}")


def test_stage_degenerate_inputs(sv, dev):
    """Out-of-range drafts are rejected; q(x) = 0 accepts; an empty residual
    falls back to p and is flagged; n_accepted outside [0, K] yields -1."""
    import torch
    B, K, V = 4, 2, 6
    P = np.zeros((B, K + 1, V), np.float32)
    Q = np.zeros((B, K, V), np.float32)
    P[:] = [0.3, 0.2, 0.2, 0.1, 0.1, 0.1]
    Q[:] = [0.3, 0.2, 0.2, 0.1, 0.1, 0.1]
    Q[1, 0] = [0.0, 0.4, 0.2, 0.2, 0.1, 0.1]     # q(x=0) = 0 < p(0)
    toks = np.array([[-1, 0], [0, 6], [2, 2], [3, 3]], np.int32)
    ua = np.array([[0.5, 0.5], [0.99, 0.5], [1.0, 0.5], [0.2, 0.2]], np.float32)
    us = np.full((B, K + 1), 0.5, np.float32)
    n, mask, tok, zero = run_stage(sv, dev, P, Q, toks, ua, us)
    n_ref, acc_ref, _, _ = spec.accept_batch(P.astype(np.float64), Q.astype(np.float64), toks, ua)
    tok_ref, _, zero_ref = spec.sample_batch(P.astype(np.float64), Q.astype(np.float64), n_ref, us)
    assert list(n) == [0, 1, 0, 2] and list(n_ref) == [0, 1, 0, 2]
    assert mask[0, 0] == 0 and mask[1, 0] == 1 and mask[1, 1] == 0
    assert bool(zero[2]) and zero_ref[2]       # p == q, rejected by u = 1
    assert np.array_equal(tok, tok_ref) and np.array_equal(zero.astype(bool), zero_ref)
    p, q = to_dev(P, dev), to_dev(Q, dev)
    bad = to_dev(np.array([-1, 3, 2, 0], np.int32), dev)
    t2, _ = sv.residual_sample(p, q, bad, to_dev(us, dev))
    torch.cuda.synchronize()
    t2 = t2.cpu().numpy()
    assert t2[0] == -1 and t2[1] == -1 and t2[2] >= 0 and t2[3] >= 0


def test_stage_deterministic(sv, dev):
    d = probs_inputs(9, 64, 8, 128256, 3.0, 0.48)
    a = run_stage(sv, dev, d["P32"], d["Q32"], d["draft_tokens"], d["u_accept"], d["u_sample"])
    b = run_stage(sv, dev, d["P32"], d["Q32"], d["draft_tokens"], d["u_accept"], d["u_sample"])
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
