"""GPU parity of spec_verify_warped (temperature-warped and greedy
verification) against the fp64 oracle.

The target's law is softmax(l / t_target) and the draft's softmax(l /
t_draft); the accept test and the residual draw are the unchanged exact rule
applied to those laws ("Speculative Decoding: Two Models, One Voice", Three
remarks worth internalizing). Drafts are drawn at the draft's temperature
(Gumbel-max on l / t_draft, or the argmax when t_draft = 0). Decisions are
compared bit-exact outside the oracle's tie band. With t_target = 0 every
decision is exact (the ratio is 0 or at least 1), so the comparison there
has no band at all.
"""

import numpy as np
import pytest

import oracle
import synth
from parity import compare_rounds

pytestmark = pytest.mark.gpu


def to_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def drafts_at(dl, t_draft, seed):
    if t_draft == 0.0:
        return np.argmax(dl, axis=-1).astype(np.int32)   # numpy: first maximum
    return synth.gumbel_max_tokens((dl / np.float32(t_draft)).astype(np.float32), seed)


def run(sv, dev, tl, dl, tok, ua, us, t_target, t_draft):
    import torch
    out, n = sv.verify(to_dev(tl, dev), to_dev(dl, dev), to_dev(tok.astype(np.int32), dev),
                       to_dev(ua, dev), to_dev(us, dev), t_target=t_target, t_draft=t_draft)
    torch.cuda.synchronize()
    return out.cpu().numpy(), n.cpu().numpy()


def compare(out, n, ref, what, u_sample):
    compare_rounds(out, n, ref, what, u_sample)


def inputs(seed, B, K, V, std, sigma, t_draft):
    d = synth.sampling_inputs(seed, B, K, V, std, sigma)
    d["draft_tokens"] = drafts_at(d["draft_logits"], t_draft, seed)
    return d


@pytest.mark.parametrize("t_target,t_draft", [(0.6, 0.6), (1.7, 1.7), (0.6, 1.7), (1.0, 0.5),
                                              (1.3, 1.0)])
def test_warped_tiny(sv, dev, t_target, t_draft):
    d = inputs(21, 256, 4, 1000, 2.0, 0.5, t_draft)
    out, n = run(sv, dev, d["target_logits"], d["draft_logits"], d["draft_tokens"],
                 d["u_accept"], d["u_sample"], t_target, t_draft)
    ref = oracle.verify_batch(d["target_logits"], d["draft_logits"], d["draft_tokens"],
                              d["u_accept"], d["u_sample"], t_target=t_target, t_draft=t_draft)
    compare(out, n, ref, f"tiny T=({t_target}, {t_draft})", d["u_sample"])


@pytest.mark.parametrize("t", [0.7, 1.5])
def test_warped_llama8b_sampling_shape(sv, dev, t):
    """V = 128256 (many chunks per row), logits of the lm-head's scale."""
    sigma = synth.draft_noise_sigma("llama8b_lm_head", 0.8)
    d = inputs(31, 16, 4, 128256, 0.02 * 4096 ** 0.5, sigma, t)
    out, n = run(sv, dev, d["target_logits"], d["draft_logits"], d["draft_tokens"],
                 d["u_accept"], d["u_sample"], t, t)
    ref = oracle.verify_batch(d["target_logits"], d["draft_logits"], d["draft_tokens"],
                              d["u_accept"], d["u_sample"], t_target=t, t_draft=t)
    compare(out, n, ref, f"8B T={t}", d["u_sample"])


@pytest.mark.parametrize("V,t_draft", [(1000, 1.0), (128256, 1.0), (4097, 0.0), (128256, 0.8)])
def test_greedy_target_exact(sv, dev, V, t_draft):
    """t_target = 0: emitted tokens and counts equal the oracle's everywhere
    (no tie band), and every emitted token is its row's first argmax."""
    B, K = (64, 4) if V < 100000 else (8, 8)
    d = inputs(41 + V, B, K, V, 3.0, 0.6, t_draft)
    tl = d["target_logits"]
    # plant exact ties of the maximum in some rows: the first index wins
    tl[0, :, 7] = tl[0].max(axis=-1)
    tl[1, :, V - 1] = tl[1].max(axis=-1)
    # and make some drafts the target's argmax so that rounds accept
    am = np.argmax(tl, axis=-1)
    tok = d["draft_tokens"].copy()
    tok[::2] = am[::2, :K]
    out, n = run(sv, dev, tl, d["draft_logits"], tok, d["u_accept"], d["u_sample"], 0.0, t_draft)
    ref = oracle.verify_batch(tl, d["draft_logits"], tok, d["u_accept"], d["u_sample"],
                              t_target=0.0, t_draft=t_draft)
    assert np.array_equal(n, ref["n_emitted"])
    assert np.array_equal(out, ref["out_tokens"])
    for b in range(B):
        assert np.array_equal(out[b, :n[b]], am[b, :n[b]])
        assert (out[b, n[b]:] == -1).all()
    assert (n[::2] == K + 1).all()
    print(f"greedy target V={V} t_draft={t_draft}: mean emitted {n.mean():.3f}", flush=True)


def test_greedy_both_ignores_uniforms(sv, dev):
    d = inputs(51, 32, 6, 50000, 3.0, 1.0, 0.0)
    tl, dl, tok = d["target_logits"], d["draft_logits"], d["draft_tokens"]
    a = run(sv, dev, tl, dl, tok, d["u_accept"], d["u_sample"], 0.0, 0.0)
    ua2 = synth.uniforms(52, "u_accept", d["u_accept"].shape)
    us2 = synth.uniforms(52, "u_sample", d["u_sample"].shape)
    b = run(sv, dev, tl, dl, tok, ua2, us2, 0.0, 0.0)
    ref = oracle.verify_batch(tl, dl, tok, d["u_accept"], d["u_sample"], t_target=0.0,
                              t_draft=0.0)
    for out, n in (a, b):
        assert np.array_equal(out, ref["out_tokens"]) and np.array_equal(n, ref["n_emitted"])


@pytest.mark.parametrize("t_target", [1.0, 0.8, 2.0])
def test_greedy_draft(sv, dev, t_target):
    """t_draft = 0: q is one-hot at the draft's argmax, the kept-probability
    is p(x) and the residual is p with the draft token removed."""
    d = inputs(61, 128, 4, 3000, 2.0, 0.3, 0.0)
    out, n = run(sv, dev, d["target_logits"], d["draft_logits"], d["draft_tokens"],
                 d["u_accept"], d["u_sample"], t_target, 0.0)
    ref = oracle.verify_batch(d["target_logits"], d["draft_logits"], d["draft_tokens"],
                              d["u_accept"], d["u_sample"], t_target=t_target, t_draft=0.0)
    compare(out, n, ref, f"greedy draft T_target={t_target}", d["u_sample"])
    # a rejected slot never re-emits the rejected draft token
    for b in range(len(n)):
        j = n[b] - 1
        if j < d["K"]:
            assert out[b, j] != d["draft_tokens"][b, j]


@pytest.mark.parametrize("case", ["printed", "all_match"])
def test_greedy_worked_example_gpu(sv, dev, golden, case):
    """The greedy worked example: three kept guesses and the target's
    correction, or all four kept and the bonus token, for any uniforms
    ("Speculative Decoding: Guess Several Tokens, Check Them in One Pass",
    A worked example with greedy decoding)."""
    g = golden("guess_several_greedy.json")
    draft = g["draft"] if case == "printed" else g["all_match_draft"]
    want = g["printed_result"] if case == "printed" else g["all_match_result"]
    vocab = sorted(set(g["draft"]) | set(g["target_picks"]) | {" the", " city"})
    rng = np.random.default_rng(7)
    tl = rng.standard_normal((1, len(g["target_picks"]), len(vocab))).astype(np.float32)
    for i, t in enumerate(g["target_picks"]):
        tl[0, i, vocab.index(t)] = np.float32(6.0)
    dl = rng.standard_normal((1, len(draft), len(vocab))).astype(np.float32)
    toks = np.array([[vocab.index(t) for t in draft]], np.int32)
    for trial in range(4):
        ua = rng.random((1, len(draft)), dtype=np.float32)
        us = rng.random((1, len(draft) + 1), dtype=np.float32)
        out, n = run(sv, dev, tl, dl, toks, ua, us, 0.0, 1.0)
        assert [vocab[t] for t in out[0][:n[0]]] == want
        assert (out[0][n[0]:] == -1).all()
