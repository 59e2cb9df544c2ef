"""CPU checks of the shared GPU-vs-oracle comparison (tests/parity.py):
the oracle's own rounds pass it, and planted mistakes fail it -- a wrong
prefix length, a wrong token outside the band, a token far from the band
in a tied draw, and too many tied prefixes. The mistakes are planted in a
copy of the oracle's outputs, on the CPU."""

import numpy as np
import pytest

import oracle
import synth
from parity import band_tokens, compare_rounds, tie_masks


@pytest.fixture(scope="module")
def case():
    # V = 128256 so that many draws fall inside the tie band
    d = synth.sampling_inputs(8, 16, 4, 128256, 0.02 * 4096 ** 0.5, 0.5)
    ref = oracle.verify_batch(d["target_logits"], d["draft_logits"], d["draft_tokens"],
                              d["u_accept"], d["u_sample"])
    return d, ref


def test_oracle_passes_itself(case):
    d, ref = case
    B, n_tie, in_band = compare_rounds(ref["out_tokens"].copy(), ref["n_emitted"].copy(), ref,
                                       "oracle", d["u_sample"])
    assert B == 16 and n_tie == 0 and in_band > 0   # the band check is exercised


def test_band_tokens_is_small_and_holds_the_draw(case):
    d, ref = case
    P, Q = ref["P"], ref["Q"]
    for b in range(16):
        k = int(ref["n_accepted"][b])
        w = oracle.residual_weights(P[b][k], Q[b][k])[0] if k < 4 else P[b][4]
        allowed = band_tokens(w, d["u_sample"][b][k])
        assert ref["token"][b] in allowed and 1 <= len(allowed) <= 64


def test_wrong_prefix_fails(case):
    d, ref = case
    n = ref["n_emitted"].copy()
    n[3] = n[3] % 5 + 1
    with pytest.raises(AssertionError):
        compare_rounds(ref["out_tokens"].copy(), n, ref, "planted", d["u_sample"])


def test_wrong_token_fails_exact_and_band(case):
    d, ref = case
    _, tok_tie = tie_masks(ref)
    for b in (int(np.flatnonzero(~tok_tie)[0]), int(np.flatnonzero(tok_tie)[0])):
        out = ref["out_tokens"].copy()
        k = int(ref["n_accepted"][b])
        out[b, k] = (out[b, k] + 5000) % 128256
        with pytest.raises(AssertionError):
            compare_rounds(out, ref["n_emitted"].copy(), ref, "planted", d["u_sample"])


def test_too_many_prefix_ties_fail(case):
    d, ref = case
    tied = dict(ref)
    tied["n_tie"] = np.ones_like(ref["n_tie"])
    with pytest.raises(AssertionError):
        compare_rounds(ref["out_tokens"].copy(), ref["n_emitted"].copy(), tied, "ties",
                       d["u_sample"])
