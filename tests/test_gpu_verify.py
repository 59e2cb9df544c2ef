"""GPU parity of spec_verify (the fused step after the stack) against the
fp64 oracle.

Both sides see the same fp32 logits and uniforms: emitted tokens and counts
are bit-exact outside the oracle's ties (margin <= 1e-5), and at least 90 %
of the sequences must be outside every tie. With the lm-head computed on the
GPU, the oracle decides on the GPU's own fp32 logits (read back after the
call), and those logits are held to the GEMM tolerance against the fp64
oracle GEMM.
"""

import numpy as np
import pytest

import oracle
import synth
from parity import compare_rounds as compare, floor_over_rounds

pytestmark = pytest.mark.gpu


def to_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def run_verify(sv, dev, d, hidden=None, lm_head=None):
    import torch
    tl = to_dev(d["target_logits"], dev) if hidden is None else \
        torch.empty((d["B"], d["K"] + 1, d["V"]), dtype=torch.float32, device=dev)
    out, n = sv.verify(tl, to_dev(d["draft_logits"], dev),
                       to_dev(d["draft_tokens"].astype(np.int32), dev),
                       to_dev(d["u_accept"], dev), to_dev(d["u_sample"], dev),
                       hidden=hidden, lm_head=lm_head)
    torch.cuda.synchronize()
    return out.cpu().numpy(), n.cpu().numpy(), tl


def lm_head_rounds(sv, dev, hidden, lm, dl, B, K, V, seed, rounds, what):
    """spec_verify with the lm-head on the GPU, `rounds` times with fresh
    drafts (x ~ q) and uniforms. The oracle decides on the GPU's own fp32
    logits, read back after the first call (every call recomputes them and
    must reproduce them bit for bit); the logits themselves are held to the
    GEMM tolerance against the fp64 oracle GEMM."""
    import torch
    from synth import device as sd
    tl = torch.empty((B, K + 1, V), dtype=torch.float32, device=dev)
    gpu_logits, P, Q = None, None, None
    seqs = ties = 0
    for r in range(rounds):
        tok = synth.gumbel_max_tokens(dl, seed + r)
        ua = synth.uniforms(seed, f"ua{r}", (B, K))
        us = synth.uniforms(seed, f"us{r}", (B, K + 1))
        out, n = sv.verify(tl, to_dev(dl, dev), to_dev(tok.astype(np.int32), dev),
                           to_dev(ua, dev), to_dev(us, dev), hidden=hidden, lm_head=lm)
        torch.cuda.synchronize()
        logits = tl.cpu().numpy()
        if gpu_logits is None:
            gpu_logits = logits
            ref_logits = oracle.linear(sd.to_bits(hidden), sd.to_bits(lm)).reshape(B, K + 1, V)
            rms = np.sqrt(np.mean(ref_logits ** 2, axis=-1, keepdims=True))
            err = float(np.max(np.abs(gpu_logits - ref_logits) / np.maximum(np.abs(ref_logits),
                                                                            rms)))
            assert err <= 2e-2, (what, err)
            P, _, _ = oracle.softmax_rows(gpu_logits)
            Q, _, _ = oracle.softmax_rows(dl)
        assert np.array_equal(logits, gpu_logits), what
        ref = oracle.verify_batch_probs(P, Q, tok, ua, us)
        b, t, _ = compare(out.cpu().numpy(), n.cpu().numpy(), ref, f"{what} round {r}", us,
                          P=P, Q=Q, min_compared=0.0)
        seqs += b
        ties += t
    floor_over_rounds(seqs, ties, what)
    print(f"{what}: {rounds} rounds, {seqs} sequences, {ties} prefix ties", flush=True)


@pytest.mark.parametrize("seed", range(4))
def test_verify_tiny_logits_many_seeds(sv, dev, seed):
    d = synth.sampling_inputs(seed, 256, 4, 1000, 2.0, 0.5)
    out, n, _ = run_verify(sv, dev, d)
    ref = oracle.verify_batch(d["target_logits"], d["draft_logits"], d["draft_tokens"],
                              d["u_accept"], d["u_sample"])
    compare(out, n, ref, f"tiny seed {seed}", d["u_sample"])
    assert (n >= 1).all() and (n <= 5).all()
    for b in range(len(n)):
        assert (out[b, n[b]:] == -1).all() and (out[b, :n[b]] >= 0).all()


def test_verify_tiny_with_lm_head(sv, dev):
    """The tiny workload end to end: its 256 -> 1000 linear as the lm-head,
    draft logits = the oracle GEMM's logits + N(0, 0.5^2) (alpha about 0.8),
    64 rounds."""
    from synth import device as sd
    d = synth.tiny(11)
    hidden = sd.from_bits(d["x_bits"], dev)
    lm = sd.from_bits(d["w_bits"], dev)
    ref_logits = oracle.linear(d["x_bits"], d["w_bits"]).astype(np.float32)[None]
    dl = (ref_logits[:, :4] + synth.normals(11, "lmh.noise", (1, 4, 1000), 0.5)).astype(np.float32)
    lm_head_rounds(sv, dev, hidden, lm, dl, 1, 4, 1000, 11, 64, "tiny lm-head")


def test_verify_llama8b_sampling_shape(sv, dev):
    """B = 1, K = 4, V = 128256 with synthetic logits of the lm-head's scale
    and draft noise calibrated to alpha = 0.8; several seeds batched."""
    sigma = synth.draft_noise_sigma("llama8b_lm_head", 0.8)
    d = synth.sampling_inputs(8, 16, 4, 128256, 0.02 * 4096 ** 0.5, sigma)
    out, n, _ = run_verify(sv, dev, d)
    ref = oracle.verify_batch(d["target_logits"], d["draft_logits"], d["draft_tokens"],
                              d["u_accept"], d["u_sample"])
    compare(out, n, ref, "8B sampling", d["u_sample"])


@pytest.mark.parametrize("alpha", [0.6, 0.9])
def test_verify_stress_shape(sv, dev, alpha):
    sigma = synth.draft_noise_sigma("stress_std3", alpha)
    d = synth.sampling_inputs(40, 64, 8, 128256, 3.0, sigma)
    out, n, _ = run_verify(sv, dev, d)
    ref = oracle.verify_batch(d["target_logits"], d["draft_logits"], d["draft_tokens"],
                              d["u_accept"], d["u_sample"])
    compare(out, n, ref, f"stress alpha={alpha}", d["u_sample"])


@pytest.mark.parametrize("B", [1, 2])
def test_verify_llama8b_with_lm_head(sv, dev, B):
    """The 8B lm-head 4096 -> 128256 on the GPU, then sampling, over 64
    rounds. B = 1 (M = 5) runs the lm-head on the streaming kernel with the
    statistics in its epilogue, B = 2 (M = 10) on the tile kernel followed
    by the statistics pass."""
    import torch
    from synth import device as sd
    K, V, dm = 4, 128256, 4096
    lm = sd.normal_bf16((V, dm), synth.WEIGHT_STD, 1234, dev)
    hidden = sd.normal_bf16((B * (K + 1), dm), 1.0, 1235, dev)
    base = oracle.linear(sd.to_bits(hidden), sd.to_bits(lm)).astype(np.float32)
    sigma = synth.draft_noise_sigma("llama8b_lm_head", 0.8)
    dl = (base.reshape(B, K + 1, V)[:, :K]
          + synth.normals(3, "lm8b.noise", (B, K, V), sigma)).astype(np.float32)
    lm_head_rounds(sv, dev, hidden, lm, dl, B, K, V, 3, 64, f"8B lm-head B={B}")
    del lm
    torch.cuda.empty_cache()


def test_verify_edge_k(sv, dev):
    for K, V in [(1, 7), (64, 200), (3, 4097)]:
        d = synth.sampling_inputs(K + V, 8, K, V, 2.0, 0.6)
        out, n, _ = run_verify(sv, dev, d)
        ref = oracle.verify_batch(d["target_logits"], d["draft_logits"], d["draft_tokens"],
                                  d["u_accept"], d["u_sample"])
        compare(out, n, ref, f"K={K} V={V}", d["u_sample"])


def test_verify_deterministic(sv, dev):
    d = synth.sampling_inputs(5, 32, 8, 128256, 3.0, 0.48)
    a = run_verify(sv, dev, d)
    b = run_verify(sv, dev, d)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
