"""GPU parity of spec_verify with the lm-head on the streaming kernel and the
target rows' softmax statistics fused into its epilogue. spec_verify streams
the lm-head where spec_verify_gemm would: B*(K+1) <= 8 with at least 2^26
weights (V*d), or up to 16 positions when d is not a multiple of 64; the
cases below all take that path.

Each workgroup of the lm-head launch folds its logits into a running
(max, fp64 sum of exp) per position, or the first index of the maximum for a
greedy row; the accept kernel merges those partials, so the logits are never
re-read for the statistics. The oracle is run on the GPU's own fp32 logits,
read back after the call, so every accept decision, prefix length and token
must be bit-exact outside the oracle's ties (margin <= 1e-5); a draw inside
the band must land on one of the tokens the band allows, and at least 90 %
of the prefixes must be outside ties over the case's rounds. The logits
themselves are checked against the fp64 oracle GEMM to the GEMM tolerance,
and the fused path against the same call with those logits given as input.
"""

import numpy as np
import pytest

import oracle
import synth
from parity import compare_rounds, floor_over_rounds

pytestmark = pytest.mark.gpu

# B, K, V, d, t_target, t_draft
CASES = [
    (1, 4, 1000, 264, 1.0, 1.0),      # 63 row blocks: most workgroups hold no rows
    (1, 4, 4097, 264, 1.0, 1.0),      # last row block holds a single row
    (1, 4, 128256, 4096, 1.0, 1.0),   # the Llama-3.1-8B lm-head at M = 5
    (2, 4, 128256, 4104, 1.0, 1.0),   # M = 10
    (3, 4, 32000, 520, 0.7, 1.3),     # M = 15, temperature-warped
    (1, 4, 32000, 520, 0.0, 1.0),     # greedy target
    (2, 3, 5000, 264, 1.0, 0.0),      # greedy draft
    (1, 1, 7, 72, 1.0, 1.0),          # V below one row block, M = 2
    (8, 1, 2000, 264, 1.0, 1.0),      # M = 16, the most positions of the fused path
]


def to_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def drafts_at(dl, t_draft, seed):
    if t_draft == 0.0:
        return np.argmax(dl, axis=-1).astype(np.int32)   # numpy: first maximum
    return synth.gumbel_max_tokens((dl / np.float32(t_draft)).astype(np.float32), seed)


@pytest.mark.parametrize("B,K,V,dm,t_target,t_draft", CASES)
def test_fused_lm_head_statistics(sv, dev, B, K, V, dm, t_target, t_draft):
    import torch
    from synth import device as sd
    seed = 7 * V + 13 * dm + B
    M = B * (K + 1)
    w_std = 2.0 / dm ** 0.5 if V < 100000 else synth.WEIGHT_STD
    lm = sd.normal_bf16((V, dm), w_std, seed, dev)
    hidden = sd.normal_bf16((M, dm), 1.0, seed + 1, dev)
    ref_logits = oracle.linear(sd.to_bits(hidden), sd.to_bits(lm)).astype(np.float32)
    dl = (ref_logits.reshape(B, K + 1, V)[:, :K]
          + synth.normals(seed, "fused.noise", (B, K, V), 0.5)).astype(np.float32)
    tok = drafts_at(dl, t_draft, seed)
    ua = synth.uniforms(seed, "ua", (B, K))
    us = synth.uniforms(seed, "us", (B, K + 1))
    tl = torch.empty((B, K + 1, V), dtype=torch.float32, device=dev)
    args = (to_dev(dl, dev), to_dev(tok, dev), to_dev(ua, dev), to_dev(us, dev))
    out, n = sv.verify(tl, *args, hidden=hidden, lm_head=lm, t_target=t_target, t_draft=t_draft)
    torch.cuda.synchronize()
    out, n = out.cpu().numpy(), n.cpu().numpy()
    gpu_logits = tl.cpu().numpy()

    # the logits: GEMM tolerance against the fp64 oracle
    ref2 = ref_logits.reshape(M, V).astype(np.float64)
    rms = np.sqrt(np.mean(ref2 ** 2, axis=1, keepdims=True))
    err = np.abs(gpu_logits.reshape(M, V) - ref2) / np.maximum(np.abs(ref2), rms)
    assert float(err.max()) <= 2e-2

    # the decisions: the oracle on the GPU's own logits, bit-exact outside ties
    ref = oracle.verify_batch(gpu_logits, dl, tok, ua, us, t_target=t_target, t_draft=t_draft)
    P, Q = ref["P"], ref["Q"]
    seqs, ties, _ = compare_rounds(out, n, ref, f"fused B={B} K={K} V={V}", us, min_compared=0.0)
    # more decisions on the same logits: fresh drafts and uniforms, each call
    # fused again (at least 64 sequence-rounds per case)
    for r in range(max(6, 64 // B)):
        tok_r = drafts_at(dl, t_draft, seed + 1000 + r)
        ua_r = synth.uniforms(seed, f"ua{r}", (B, K))
        us_r = synth.uniforms(seed, f"us{r}", (B, K + 1))
        out_r, n_r = sv.verify(tl, args[0], to_dev(tok_r, dev), to_dev(ua_r, dev),
                               to_dev(us_r, dev), hidden=hidden, lm_head=lm, t_target=t_target,
                               t_draft=t_draft)
        torch.cuda.synchronize()
        ref_r = oracle.verify_batch_probs(P, Q, tok_r, ua_r, us_r)
        b_r, t_r, _ = compare_rounds(out_r.cpu().numpy(), n_r.cpu().numpy(), ref_r,
                                     f"fused round {r}", us_r, P=P, Q=Q, min_compared=0.0)
        seqs += b_r
        ties += t_r
    floor_over_rounds(seqs, ties, f"fused B={B} K={K} V={V}")

    # the same call with those logits as input (statistics from the logits)
    out2, n2 = sv.verify(tl, *args, t_target=t_target, t_draft=t_draft)
    torch.cuda.synchronize()
    assert np.array_equal(n2.cpu().numpy(), n) and np.array_equal(out2.cpu().numpy(), out)

    # deterministic: a second fused call repeats every output bit for bit
    tl3 = torch.empty_like(tl)
    out3, n3 = sv.verify(tl3, *args, hidden=hidden, lm_head=lm, t_target=t_target,
                         t_draft=t_draft)
    torch.cuda.synchronize()
    assert torch.equal(tl3, tl)
    assert np.array_equal(out3.cpu().numpy(), out) and np.array_equal(n3.cpu().numpy(), n)
    print(f"fused B={B} K={K} V={V} T=({t_target},{t_draft}): {seqs} sequence-rounds, "
          f"{ties} prefix ties, mean emitted {n.mean():.3f}", flush=True)
    del lm
    torch.cuda.empty_cache()
