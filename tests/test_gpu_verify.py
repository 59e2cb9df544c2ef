"""GPU parity of spec_verify (the fused step after the stack) against the
fp64 oracle.

With target logits supplied, both sides see the same fp32 logits and
uniforms: emitted tokens and counts are bit-exact outside the oracle's ties
(margin <= 1e-5). With the lm-head computed on the GPU, the GPU's fp32
logits differ from the oracle's fp64 logits by the GEMM's rounding delta;
decisions are then compared outside a band widened to 1e-5 + 8 * delta
(a logit shift delta moves p/q by a factor within exp(+-2 delta)), and the
logits themselves are checked to the GEMM tolerance.
"""

import numpy as np
import pytest

import oracle
import synth
from oracle import speculative as spec

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


def compare(out, n, ref, what, band=spec.TIE_BAND):
    n_tie = ref["n_tie"] | np.any(
        (ref["accept_margin"] <= band) &
        (np.arange(ref["accept"].shape[1])[None, :] <= np.minimum(ref["n_accepted"], ref["accept"].shape[1] - 1)[:, None]),
        axis=1)
    tok_tie = n_tie | ref["token_tie"] | (ref["sample_margin"] <= band)
    ok = ~n_tie
    assert np.array_equal(n[ok], ref["n_emitted"][ok]), what
    ok_t = ~tok_tie
    assert np.array_equal(out[ok_t], ref["out_tokens"][ok_t]), what
    # accepted prefixes are the drafts themselves even where the token ties
    print(f"{what}: {len(n)} seqs, {int(n_tie.sum())} prefix ties, {int(tok_tie.sum())} token "
          f"ties, mean emitted {n.mean():.3f}", flush=True)


@pytest.mark.parametrize("seed", range(4))
def test_verify_tiny_logits_many_seeds(sv, dev, seed):
    d = synth.sampling_inputs(seed, 256, 4, 1000, 2.0, 0.5)
    out, n, _ = run_verify(sv, dev, d)
    ref = oracle.verify_batch(d["target_logits"], d["draft_logits"], d["draft_tokens"],
                              d["u_accept"], d["u_sample"])
    compare(out, n, ref, f"tiny seed {seed}")
    assert (n >= 1).all() and (n <= 5).all()
    for b in range(len(n)):
        assert (out[b, n[b]:] == -1).all() and (out[b, :n[b]] >= 0).all()


def test_verify_tiny_with_lm_head(sv, dev):
    from synth import device as sd
    d = synth.tiny(11)
    hidden = sd.from_bits(d["x_bits"], dev)
    lm = sd.from_bits(d["w_bits"], dev)
    # draft logits follow the GEMM's logits so that alpha is about 0.8
    ref_logits = oracle.linear(d["x_bits"], d["w_bits"]).astype(np.float32)[None]
    d["draft_logits"] = (ref_logits[:, :4] + synth.normals(11, "lmh.noise", (1, 4, 1000), 0.5)
                         ).astype(np.float32)
    d["draft_tokens"] = synth.gumbel_max_tokens(d["draft_logits"], 11)
    out, n, tl = run_verify(sv, dev, d, hidden=hidden, lm_head=lm)
    gpu_logits = tl.cpu().numpy()
    delta = float(np.max(np.abs(gpu_logits - ref_logits)))
    rms = float(np.sqrt(np.mean(ref_logits.astype(np.float64) ** 2)))
    assert delta / rms <= 2e-2
    ref = oracle.verify_batch(ref_logits, d["draft_logits"], d["draft_tokens"],
                              d["u_accept"], d["u_sample"])
    compare(out, n, ref, "tiny lm-head", band=spec.TIE_BAND + 8 * delta)


def test_verify_llama8b_sampling_shape(sv, dev):
    """B = 1, K = 4, V = 128256 with synthetic logits of the lm-head's scale
    and draft noise calibrated to alpha = 0.8; several seeds batched."""
    sigma = synth.draft_noise_sigma("llama8b_lm_head", 0.8)
    d = synth.sampling_inputs(8, 16, 4, 128256, 0.02 * 4096 ** 0.5, sigma)
    out, n, _ = run_verify(sv, dev, d)
    ref = oracle.verify_batch(d["target_logits"], d["draft_logits"], d["draft_tokens"],
                              d["u_accept"], d["u_sample"])
    compare(out, n, ref, "8B sampling")


@pytest.mark.parametrize("alpha", [0.6, 0.9])
def test_verify_stress_shape(sv, dev, alpha):
    sigma = synth.draft_noise_sigma("stress_std3", alpha)
    d = synth.sampling_inputs(40, 64, 8, 128256, 3.0, sigma)
    out, n, _ = run_verify(sv, dev, d)
    ref = oracle.verify_batch(d["target_logits"], d["draft_logits"], d["draft_tokens"],
                              d["u_accept"], d["u_sample"])
    compare(out, n, ref, f"stress alpha={alpha}")


@pytest.mark.parametrize("B", [1, 2])
def test_verify_llama8b_with_lm_head(sv, dev, B):
    """The 8B lm-head 4096 -> 128256 on the GPU, then sampling; the oracle
    computes its own logits from the same bf16 inputs. B = 1 (M = 5) runs the
    lm-head on the streaming kernel with the statistics in its epilogue,
    B = 2 (M = 10) on the tile kernel followed by the statistics pass."""
    import torch
    from synth import device as sd
    K, V, dm = 4, 128256, 4096
    lm = sd.normal_bf16((V, dm), synth.WEIGHT_STD, 1234, dev)
    hidden = sd.normal_bf16((B * (K + 1), dm), 1.0, 1235, dev)
    ref_logits = oracle.linear(sd.to_bits(hidden), sd.to_bits(lm)).astype(np.float32)
    ref_logits = ref_logits.reshape(B, K + 1, V)
    sigma = synth.draft_noise_sigma("llama8b_lm_head", 0.8)
    dl = (ref_logits[:, :K] + synth.normals(3, "lm8b.noise", (B, K, V), sigma)).astype(np.float32)
    d = {"B": B, "K": K, "V": V, "draft_logits": dl,
         "draft_tokens": synth.gumbel_max_tokens(dl, 3),
         "u_accept": synth.uniforms(3, "ua", (B, K)), "u_sample": synth.uniforms(3, "us", (B, K + 1))}
    out, n, tl = run_verify(sv, dev, d, hidden=hidden, lm_head=lm)
    gpu_logits = tl.cpu().numpy()
    delta = float(np.max(np.abs(gpu_logits - ref_logits)))
    assert delta / float(np.sqrt(np.mean(ref_logits.astype(np.float64) ** 2))) <= 2e-2
    ref = oracle.verify_batch(ref_logits, dl, d["draft_tokens"], d["u_accept"], d["u_sample"])
    compare(out, n, ref, "8B lm-head", band=spec.TIE_BAND + 8 * delta)
    del lm
    torch.cuda.empty_cache()


def test_verify_edge_k(sv, dev):
    for K, V in [(1, 7), (64, 200), (3, 4097)]:
        d = synth.sampling_inputs(K + V, 8, K, V, 2.0, 0.6)
        out, n, _ = run_verify(sv, dev, d)
        ref = oracle.verify_batch(d["target_logits"], d["draft_logits"], d["draft_tokens"],
                                  d["u_accept"], d["u_sample"])
        compare(out, n, ref, f"K={K} V={V}")


def test_verify_deterministic(sv, dev):
    d = synth.sampling_inputs(5, 32, 8, 128256, 3.0, 0.48)
    a = run_verify(sv, dev, d)
    b = run_verify(sv, dev, d)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
