"""Statistics of the verify step at the sampling-stress shape: B = 64
sequences, K = 8 drafts, V = 128256, target logits N(0, 3^2).

The method guarantees two things over many rounds with fixed logits
("Speculative Decoding: Two Models, One Voice", How much faster and Appendix;
"Speculative Decoding: The Algebra and the Proof", The proof):

* the number of tokens a round emits has mean 1 + sum_i prod_{j<=i} alpha_j,
  alpha_j = sum_x min(p_j(x), q_j(x)) the acceptance rate of draft row j;
* every emitted token at slot j, given the round reached slot j, is
  distributed as the target's p_j.

Each draft row's noise scale is bisected so that its alpha equals the target
value (0.6, 0.81, 0.9), and the expectation uses the rows' exact alphas. The
GPU runs ROUNDS rounds per alpha, each with fresh drafts x_j ~ q_j (inverse
CDF of q with a uniform), fresh accept and sample uniforms. Checks:

* mean emitted tokens within 4 standard errors of the expectation;
* the randomized probability integral transform F_j(y - 1) + v p_j(y) of
  every emitted token y (v uniform) is uniform on [0, 1): Kolmogorov-Smirnov
  distance and a 100-bin chi-square at p = 1e-4;
* the first rounds are also compared with the fp64 oracle, bit-exact outside
  ties.

The draft sampling, the probabilities for the expectation and the transform
are plain torch fp64 (test harness); the verify step is the HIP library.
"""

import math

import numpy as np
import pytest

import oracle
import synth
from parity import compare_rounds

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

B, K, V = 64, 8, 128256
ROUNDS = 20000
SEED = 2027


def calibrate(tl, z, alpha):
    """Per-row sigma (torch fp64 bisection on device) with
    sum min(p, softmax(fp32(l + sigma z))) = alpha."""
    import torch
    p = torch.softmax(tl[:, :K].double(), dim=-1)
    lo = torch.zeros((B, K), dtype=torch.float64, device=tl.device)
    hi = torch.full((B, K), 8.0, dtype=torch.float64, device=tl.device)
    for _ in range(44):
        mid = 0.5 * (lo + hi)
        d = (tl[:, :K] + mid.float()[..., None] * z)
        a = torch.minimum(p, torch.softmax(d.double(), dim=-1)).sum(-1)
        above = a > alpha  # alpha falls as the noise grows
        lo = torch.where(above, mid, lo)
        hi = torch.where(above, hi, mid)
    return (0.5 * (lo + hi)).float()


@pytest.mark.parametrize("alpha", [0.6, 0.81, 0.9])
def test_stress_statistics(sv, dev, alpha):
    import torch
    from scipy import stats

    tl = torch.from_numpy(synth.normals(SEED, "stress.target", (B, K + 1, V), 3.0)).to(dev)
    z = torch.from_numpy(synth.normals(SEED, "stress.noise", (B, K, V))).to(dev)
    sigma = calibrate(tl, z, alpha)
    dl = (tl[:, :K] + sigma[..., None] * z).contiguous()
    del z

    P = torch.softmax(tl.double(), dim=-1)          # [B][K+1][V]
    Q = torch.softmax(dl.double(), dim=-1)          # [B][K][V]
    a = torch.minimum(P[:, :K], Q).sum(-1)          # exact alpha per draft row
    assert float((a - alpha).abs().max()) < 1e-5, "calibration"
    expect = float((1.0 + torch.cumprod(a, dim=1).sum(1)).mean())
    cq = torch.cumsum(Q, dim=-1).reshape(B * K, V)
    del Q
    cp = torch.cumsum(P, dim=-1)

    gen = torch.Generator(device=dev)
    gen.manual_seed(SEED + int(alpha * 100))
    ws = sv.new_workspace(B, K, V, dev)
    out = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    n = torch.empty(B, dtype=torch.int32, device=dev)
    slots = torch.arange(K + 1, device=dev)[None, :]
    tot = torch.zeros((), dtype=torch.float64, device=dev)
    tot2 = torch.zeros((), dtype=torch.float64, device=dev)
    pits = []
    n_ties = 0
    for r in range(ROUNDS):
        u_draft = torch.rand((B * K, 1), generator=gen, device=dev)
        tok = torch.searchsorted(cq, u_draft.double() * cq[:, -1:], right=True)
        tok = tok.clamp_(max=V - 1).reshape(B, K).int()
        u_acc = torch.rand((B, K), generator=gen, device=dev)
        u_smp = torch.rand((B, K + 1), generator=gen, device=dev)
        sv.verify(tl, dl, tok, u_acc, u_smp, workspace=ws, out_tokens=out, n_emitted=n)
        nd = n.double()
        tot += nd.sum()
        tot2 += (nd * nd).sum()
        # transform of every emitted token under its slot's target law
        y = out.long().clamp(min=0)
        py = torch.gather(P, 2, y[..., None])[..., 0]
        fy = torch.gather(cp, 2, y[..., None])[..., 0]
        v = torch.rand((B, K + 1), generator=gen, device=dev, dtype=torch.float64)
        pit = fy - py + v * py
        pits.append(torch.where(slots < n[:, None].long(), pit, -1.0))  # -1: slot not emitted
        if r < 2:  # bit-exact against the oracle on the first rounds, 8 sequences
            s = slice(0, 8)
            ref = oracle.verify_batch(tl[s].cpu().numpy(), dl[s].cpu().numpy(),
                                      tok[s].cpu().numpy(), u_acc[s].cpu().numpy(),
                                      u_smp[s].cpu().numpy())
            n_ties += compare_rounds(out[s].cpu().numpy(), n[s].cpu().numpy(), ref,
                                     f"alpha={alpha} round {r}", u_smp[s].cpu().numpy())[1]
    cnt = ROUNDS * B
    mean = float(tot) / cnt
    var = float(tot2) / cnt - mean * mean
    se = math.sqrt(var / cnt)
    closed = (1 - alpha ** (K + 1)) / (1 - alpha)
    u = torch.cat(pits).flatten()
    u = u[u >= 0].clamp_(0.0, 1.0)
    m = u.numel()
    us = torch.sort(u).values
    i = torch.arange(1, m + 1, device=dev, dtype=torch.float64)
    ks = float(torch.maximum(i / m - us, us - (i - 1) / m).max())
    hist = torch.histc(u.float(), bins=100, min=0.0, max=1.0).double()
    chi2 = float(((hist - m / 100) ** 2 / (m / 100)).sum())
    chi2_crit = float(stats.chi2.ppf(1 - 1e-4, 99))
    ks_crit = 2.23 / math.sqrt(m)  # Kolmogorov distribution, p = 1e-4
    print(f"alpha={alpha}: tokens/round {mean:.5f} expected {expect:.5f} "
          f"(closed form {closed:.5f}) se {se:.5f}; {m} emitted tokens: KS {ks:.2e} "
          f"(crit {ks_crit:.2e}) chi2 {chi2:.1f} (crit {chi2_crit:.1f}); "
          f"oracle prefix ties {n_ties}", flush=True)
    assert abs(expect - closed) < 1e-3
    assert abs(mean - expect) < 4 * se
    assert ks < ks_crit
    assert chi2 < chi2_crit
