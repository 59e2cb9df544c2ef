"""Pins for the fp64 oracle: what the pages and the mathematics fix.

CPU only. Each test ties an oracle function to something other than itself:
values printed on the pages (tests/golden/, each with its citation), exact
rational enumeration, IEEE facts, closed forms and statistical checks with
stated standard errors.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle
import synth
from oracle import speculative as spec


# ---------------------------------------------------------------------------
# bf16 decode and the linear layers
# ---------------------------------------------------------------------------

def test_bf16_decode_ieee_values():
    # IEEE bfloat16: sign, 8 exponent bits (bias 127), 7 fraction bits.
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x3FC0, 0x4049,
                     0x7F7F, 0x0001, 0x0080], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, 1.5, 3.140625,
            (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** -133, 2.0 ** -126]
    got = oracle.bf16_to_f64(bits)
    for g, w in zip(got, want):
        assert g == w and math.copysign(1, g) == math.copysign(1, w)


def test_round_to_bf16_ties_to_even_and_spacing():
    # 8 significant bits: between 1 and 2 the spacing is 2^-7
    vals = [1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -30, -(1 + 2 ** -8),
            3.0 + 2 ** -7, 2 ** -130 + 2 ** -134, 0.0, 448.0, 1e-3]
    want = [1.0, 1.0, 1 + 2 ** -6, 1 + 2 ** -7, -1.0, 3.0, 2 ** -130, 0.0, 448.0,
            0.0009994506835937500]
    got = oracle.round_to_bf16(np.array(vals))
    assert got.tolist() == want
    bits = oracle.to_bf16_bits(np.array([1.0, -2.0, 3.140625, 1 + 2 ** -8]))
    assert bits.tolist() == [0x3F80, 0xC000, 0x4049, 0x3F80]


def test_round_to_bf16_matches_torch_on_float32_values():
    import torch
    v = np.random.default_rng(8).standard_normal(20000).astype(np.float32) * np.float32(37)
    t = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_to_bf16(v.astype(np.float64)), t)


def _one_bits(shape):
    return np.zeros(shape, dtype=np.uint16)


def test_linear_one_hot_weight_rows_select_activation_columns():
    rng = np.random.default_rng(1)
    M, d_in, d_out = 5, 48, 33
    x = synth.bf16_normal_bits(3, "pin.x", (M, d_in))
    w = _one_bits((d_out, d_in))
    cols = rng.integers(0, d_in, d_out)
    w[np.arange(d_out), cols] = 0x3F80  # 1.0
    y = oracle.linear(x, w)
    assert np.array_equal(y, oracle.bf16_to_f64(x)[:, cols])


def test_linear_one_hot_activation_rows_select_weight_columns():
    rng = np.random.default_rng(2)
    M, d_in, d_out = 7, 40, 29
    w = synth.bf16_normal_bits(4, "pin.w", (d_out, d_in), 0.02)
    x = _one_bits((M, d_in))
    cols = rng.integers(0, d_in, M)
    x[np.arange(M), cols] = 0x3F80
    y = oracle.linear(x, w)
    assert np.array_equal(y, oracle.bf16_to_f64(w)[:, cols].T)


def test_linear_all_ones_gives_row_length():
    x = np.full((3, 24), 0x3F80, dtype=np.uint16)
    w = np.full((5, 24), 0x3F80, dtype=np.uint16)
    assert np.array_equal(oracle.linear(x, w), np.full((3, 5), 24.0))


def test_linear_matches_exact_rational_sum_within_fp64_bound():
    # bf16 values are dyadic rationals, so the exact dot product is a
    # Fraction; the fp64 result must lie within d_in * 2^-53 * sum|x||w|.
    M, d_in, d_out = 3, 72, 11
    x = synth.bf16_normal_bits(5, "pin.x2", (M, d_in))
    w = synth.bf16_normal_bits(6, "pin.w2", (d_out, d_in), 0.02)
    # a tiny block size exercises several ragged row blocks
    y = oracle.linear(x, w, block_bytes=8 * d_in * 4)
    xf = oracle.bf16_to_f64(x)
    wf = oracle.bf16_to_f64(w)
    for m in range(M):
        for n in range(d_out):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xf[m], wf[n]))
            bound = d_in * 2.0 ** -53 * float(np.abs(xf[m]) @ np.abs(wf[n]))
            assert abs(Fraction(float(y[m, n])) - exact) <= Fraction(bound)


def test_linear_rejects_mismatched_shapes():
    with pytest.raises(ValueError):
        oracle.linear(np.zeros((2, 8), np.uint16), np.zeros((3, 16), np.uint16))


# ---------------------------------------------------------------------------
# FP8 E4M3 weights (weight-only 8-bit storage)
# ---------------------------------------------------------------------------

def test_e4m3_decode_format_values():
    # OCP FP8 E4M3: bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN.
    codes = [0x38, 0xB8, 0x00, 0x80, 0x7E, 0xFE, 0x08, 0x07, 0x01, 0x3C, 0x40, 0x77, 0x30]
    want = [1.0, -1.0, 0.0, -0.0, 448.0, -448.0, 2.0 ** -6, 7 * 2.0 ** -9, 2.0 ** -9, 1.5, 2.0,
            240.0, 0.5]
    got = oracle.e4m3_to_f64(np.array(codes, dtype=np.uint8))
    for g, w in zip(got, want):
        assert g == w and math.copysign(1, g) == math.copysign(1, w)
    v = oracle.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    assert np.flatnonzero(np.isnan(v)).tolist() == [0x7F, 0xFF]
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                       # codes 0x00..0x7E ascend
    assert np.array_equal(v[0x80:0xFF], -pos)             # the sign bit only negates


def test_e4m3_decode_matches_torch_float8():
    import torch
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    v = oracle.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    nan = np.isnan(v)
    assert np.array_equal(nan, np.isnan(t)) and np.array_equal(v[~nan], t[~nan])


def test_linear_w8_one_hot_activation_selects_scaled_weight_column():
    rng = np.random.default_rng(12)
    M, d_in, d_out = 6, 64, 37
    w = synth.e4m3_normal_codes(12, "pin.w8", (d_out, d_in))
    s = synth.w8_row_scales(12, "pin.s8", d_out)
    x = _one_bits((M, d_in))
    cols = rng.integers(0, d_in, M)
    x[np.arange(M), cols] = 0x3F80
    y = oracle.linear_w8(x, w, s)
    want = oracle.e4m3_to_f64(w)[:, cols].T * s.astype(np.float64)[None, :]
    assert np.array_equal(y, want)


def test_linear_w8_matches_exact_rational_sum():
    # E4M3 and bf16 values are dyadic rationals: the exact result is a
    # Fraction; fp64 lies within (d_in + 1) * 2^-53 * scale * sum|x||w|.
    M, d_in, d_out = 3, 56, 9
    x = synth.bf16_normal_bits(13, "pin.x8", (M, d_in))
    w = synth.e4m3_normal_codes(13, "pin.w8b", (d_out, d_in))
    s = synth.w8_row_scales(13, "pin.s8b", d_out)
    y = oracle.linear_w8(x, w, s, block_bytes=8 * d_in * 4)  # ragged row blocks
    xf = oracle.bf16_to_f64(x)
    wf = oracle.e4m3_to_f64(w)
    for m in range(M):
        for n in range(d_out):
            exact = Fraction(float(s[n])) * sum(
                Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xf[m], wf[n]))
            bound = (d_in + 1) * 2.0 ** -53 * float(s[n]) * float(np.abs(xf[m]) @ np.abs(wf[n]))
            assert abs(Fraction(float(y[m, n])) - exact) <= Fraction(bound)


def test_linear_w8_unit_scale_is_the_bf16_linear_of_the_decoded_weights():
    # every E4M3 value is exact in bf16 (3 mantissa bits, exponents within
    # range), so with unit scales the product is the bf16 linear of them
    x = synth.bf16_normal_bits(14, "pin.x8c", (4, 40))
    w = synth.e4m3_normal_codes(14, "pin.w8c", (21, 40))
    wb = synth.bf16_bits(oracle.e4m3_to_f64(w).astype(np.float32))
    assert np.array_equal(oracle.bf16_to_f64(wb), oracle.e4m3_to_f64(w))
    y = oracle.linear_w8(x, w, np.ones(21, np.float32))
    assert np.array_equal(y, oracle.linear(x, wb))


def test_linear_w8_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.linear_w8(np.zeros((2, 8), np.uint16), np.zeros((3, 16), np.uint8), np.ones(3))
    with pytest.raises(ValueError):
        oracle.linear_w8(np.zeros((2, 8), np.uint16), np.zeros((3, 8), np.uint8), np.ones(4))


# ---------------------------------------------------------------------------
# Verify attention (causal K+1 queries over the KV cache)
# ---------------------------------------------------------------------------

def _attn_inputs(seed, B, K1, H, Hkv, T, D):
    q = synth.bf16_normal_bits(seed, "pin.aq", (B, K1, H, D))
    k = synth.bf16_normal_bits(seed, "pin.ak", (B, T, Hkv, D))
    v = synth.bf16_normal_bits(seed, "pin.av", (B, T, Hkv, D))
    return q, k, v


def test_attention_equal_keys_average_the_visible_values():
    # equal scores: the softmax is uniform over the positions a query sees,
    # so position i averages values 0 .. T-K1+i exactly
    B, K1, H, Hkv, T, D = 2, 5, 4, 2, 37, 8
    q, _, v = _attn_inputs(1, B, K1, H, Hkv, T, D)
    k = np.zeros((B, T, Hkv, D), np.uint16)
    o = oracle.verify_attention(q, k, v, 0.3)
    vf = oracle.bf16_to_f64(v)
    for i in range(K1):
        want = vf[:, :T - K1 + i + 1].mean(axis=1)          # [B][Hkv][D]
        for h in range(H):
            assert np.allclose(o[:, i, h], want[:, h // (H // Hkv)], rtol=0, atol=1e-15)


def test_attention_dominant_key_selects_its_value_when_visible():
    B, K1, H, Hkv, T, D = 1, 4, 2, 1, 20, 8
    q = np.full((B, K1, H, D), 0x3F80, np.uint16)            # all ones
    k = np.zeros((B, T, Hkv, D), np.uint16)
    j = T - 2                                                 # seen by the last two queries
    k[0, j, 0, :] = 0x4200                                    # 32.0: score 256 * scale
    v = synth.bf16_normal_bits(2, "pin.av2", (B, T, Hkv, D))
    o = oracle.verify_attention(q, k, v, 4.0)                 # score gap 1024: exp underflows
    vf = oracle.bf16_to_f64(v)
    for i in range(K1):
        last = T - K1 + i
        want = vf[0, j, 0] if j <= last else vf[0, :last + 1, 0].mean(axis=0)
        for h in range(H):
            assert np.array_equal(o[0, i, h], want) or np.allclose(o[0, i, h], want, atol=1e-15)


def test_attention_matches_masked_scipy_softmax():
    B, K1, H, Hkv, T, D = 2, 5, 8, 2, 29, 16
    q, k, v = _attn_inputs(3, B, K1, H, Hkv, T, D)
    scale = 1 / math.sqrt(D)
    o = oracle.verify_attention(q, k, v, scale)
    qf, kf, vf = (oracle.bf16_to_f64(a) for a in (q, k, v))
    mask = np.arange(T)[None, :] > (T - K1 + np.arange(K1))[:, None]   # [K1][T] future keys
    for b in range(B):
        for h in range(H):
            g = h // (H // Hkv)
            s = scale * np.einsum("id,td->it", qf[b, :, h], kf[b, :, g])
            s[mask] = -np.inf
            p = scipy.special.softmax(s, axis=-1)
            assert np.abs(o[b, :, h] - p @ vf[b, :, g]).max() < 1e-13


def test_attention_is_causal_and_grouped():
    B, K1, H, Hkv, T, D = 1, 5, 6, 2, 16, 8
    q, k, v = _attn_inputs(4, B, K1, H, Hkv, T, D)
    o = oracle.verify_attention(q, k, v, 0.5)
    # changing the last key/value changes only the last query's output
    k2, v2 = k.copy(), v.copy()
    k2[0, T - 1] ^= 0x0100
    v2[0, T - 1] ^= 0x0100
    o2 = oracle.verify_attention(q, k2, v2, 0.5)
    assert np.array_equal(o[:, :K1 - 1], o2[:, :K1 - 1])
    assert not np.array_equal(o[:, K1 - 1], o2[:, K1 - 1])
    # heads of one group with the same query give the same output; swapping
    # the two key/value heads swaps the outputs of the two groups
    q3 = q.copy()
    q3[:, :, 1] = q3[:, :, 0]
    o3 = oracle.verify_attention(q3, k, v, 0.5)
    assert np.array_equal(o3[:, :, 0], o3[:, :, 1])
    q4 = np.concatenate([q[:, :, 3:], q[:, :, :3]], axis=2)
    o4 = oracle.verify_attention(q4, k[:, :, ::-1], v[:, :, ::-1], 0.5)
    assert np.array_equal(o4, np.concatenate([o[:, :, 3:], o[:, :, :3]], axis=2))


def test_attention_single_query_is_decode_attention_over_everything():
    B, K1, H, Hkv, T, D = 1, 1, 2, 2, 9, 4
    q, k, v = _attn_inputs(5, B, K1, H, Hkv, T, D)
    o = oracle.verify_attention(q, k, v, 1.0)
    qf, kf, vf = (oracle.bf16_to_f64(a) for a in (q, k, v))
    for h in range(H):
        p = scipy.special.softmax(kf[0, :, h] @ qf[0, 0, h])
        assert np.abs(o[0, 0, h] - p @ vf[0, :, h]).max() < 1e-14


# ---------------------------------------------------------------------------
# Softmax
# ---------------------------------------------------------------------------

def test_softmax_constant_row_is_uniform():
    V = 1000
    p, m, s = oracle.softmax_rows(np.full((2, V), 3.25, np.float32))
    assert np.all(m == 3.25) and np.all(s == V)
    assert np.max(np.abs(p - 1.0 / V)) < 1e-18


def test_softmax_two_token_closed_form():
    # p_1 = e^l / (1 + e^l) for logits (0, l): also pins the sign of the
    # exponent (the larger logit gets the larger probability).
    l = np.float32(np.log(3.0))
    p, m, s = oracle.softmax_rows(np.array([[0.0, l]], np.float32))
    e = math.exp(float(l))
    assert abs(p[0, 1] - e / (1 + e)) < 4e-16 and abs(p[0, 0] - 1 / (1 + e)) < 4e-16
    assert m[0] == float(l) and abs(s[0] - (1 + math.exp(-float(l)))) < 1e-15


def test_softmax_shift_invariance_and_normalisation():
    rng = np.random.default_rng(7)
    l = rng.integers(-40, 40, size=(6, 777)).astype(np.float32)
    p1, _, _ = oracle.softmax_rows(l)
    p2, _, _ = oracle.softmax_rows(l + np.float32(64.0))  # exact in fp32
    assert np.max(np.abs(p1 - p2)) < 1e-16
    assert np.max(np.abs(p1.sum(axis=1) - 1.0)) < 1e-15


def test_softmax_matches_scipy():
    l = synth.normals(8, "pin.sm", (4, 128256), 3.0)
    p, _, _ = oracle.softmax_rows(l)
    ref = scipy.special.softmax(l.astype(np.float64), axis=-1)
    assert np.max(np.abs(p - ref)) < 1e-15


# ---------------------------------------------------------------------------
# The accept test, the residual and the sampler
# ---------------------------------------------------------------------------

def test_six_token_example_alpha_tv_and_residual(golden):
    g = golden("two_models_six_token.json")
    P, Q = np.array(g["P"]), np.array(g["Q"])
    alpha = oracle.acceptance_rate(P, Q)
    assert abs(alpha - 0.81) < 1e-15 and round(alpha, 3) == g["alpha_printed"]
    assert abs(oracle.total_variation(P, Q) - (1 - alpha)) < 1e-15
    r, zero = oracle.residual_weights(P, Q)
    assert not zero
    rn = r / r.sum()
    want = [Fraction(0), Fraction(10, 19), Fraction(2, 19), Fraction(7, 19), Fraction(0), Fraction(0)]
    assert np.max(np.abs(rn - np.array([float(v) for v in want]))) < 1e-15
    nz = g["residual_nonzero_tokens"]
    assert list(np.flatnonzero(rn)) == nz
    assert [round(float(v), 2) for v in rn[nz]] == g["residual_printed_2dp"]


def test_three_token_example(golden):
    g = golden("guess_several_three_token.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    assert abs(oracle.acceptance_rate(p, q) - g["alpha_printed"]) < 1e-15
    grey = 1
    _, ratio, _ = oracle.accept_test([p], [q], [grey], [0.0])
    assert abs(ratio[0] - float(Fraction(g["grey_survival_exact"]))) < 1e-15
    # u on the float32 grid just below / above 2/5
    lo = math.floor(0.4 * 2 ** 24) / 2 ** 24
    hi = math.ceil(0.4 * 2 ** 24) / 2 ** 24
    assert oracle.accept_test([p], [q], [grey], [lo])[0][0]
    assert not oracle.accept_test([p], [q], [grey], [hi])[0][0]
    r, _ = oracle.residual_weights(p, q)
    a, b = g["residual_ratio_blue_to_clear"]
    assert r[1] == 0 and abs(r[0] / r[2] - a / b) < 1e-14


def test_accept_is_strict_and_handles_zero_q():
    P = [np.array([0.25, 0.75])]
    Q = [np.array([0.5, 0.5])]
    # ratio exactly 1/2: u = 1/2 is rejected, the largest grid value below accepts
    assert not oracle.accept_test(P, Q, [0], [0.5])[0][0]
    assert oracle.accept_test(P, Q, [0], [0.5 - 2 ** -24])[0][0]
    # q(x) = 0: accepted whenever p(x) > 0, rejected when p(x) = 0 too
    Pz = [np.array([0.0, 0.4, 0.6])]
    Qz = [np.array([0.5, 0.0, 0.5])]
    acc, ratio, margin = oracle.accept_test(Pz, Qz, [1], [1 - 2 ** -24])
    assert acc[0] and math.isinf(ratio[0]) and math.isinf(margin[0])
    Qz2 = [np.array([0.0, 0.5, 0.5])]
    acc, ratio, _ = oracle.accept_test(Pz, Qz2, [0], [0.0])
    assert not acc[0] and ratio[0] == 0.0


def test_identical_draft_has_alpha_one_and_no_division_by_zero(golden):
    p = np.array([1.0, 0.0])
    law, alpha = oracle.emitted_law(p, p)
    assert alpha == 1.0 and np.array_equal(law, p)
    w, zero = oracle.residual_weights(p, p)
    assert zero and np.array_equal(w, p)
    # every draft (only token 0 has mass) is accepted for every u < 1
    assert oracle.accept_test([p], [p], [0], [1 - 2 ** -24])[0][0]


def test_inverse_cdf_edges_and_zero_weights():
    w = np.array([0.0, 0.0, 2.0, 0.0, 1.0, 1.0, 0.0])
    assert oracle.inverse_cdf(w, 0.0)[0] == 2             # first positive weight
    assert oracle.inverse_cdf(w, 1 - 2 ** -24)[0] == 5    # last positive weight
    assert oracle.inverse_cdf(w, 0.5)[0] == 4             # T = C[2] = 2 -> next cell
    assert oracle.inverse_cdf(w, 0.5 - 2 ** -24)[0] == 2
    rng = np.random.default_rng(11)
    for _ in range(200):
        y, margin = oracle.inverse_cdf(w, float(rng.random()))
        assert w[y] > 0 and 0 <= margin <= 0.5


def _grid(n):
    return [(k + 0.5) / n for k in range(n)]


def _exact_one_position_law(p_exact, q_exact, N):
    """Drive the oracle's accept test and residual sampler with uniforms at
    the midpoints of an N-cell grid; N is a multiple of every denominator of
    the decision thresholds (the ratios p/q and the residual CDF), so each
    cell's decision is the exact-arithmetic one and the count per cell is an
    exact probability. Returns the law of the emitted token as Fractions."""
    V = len(p_exact)
    p = np.array([float(v) for v in p_exact])
    q = np.array([float(v) for v in q_exact])
    P, Q = [p, p], [q]
    grid = _grid(N)
    law = [Fraction(0)] * V
    reject_mass = Fraction(0)
    for x in range(V):
        if q_exact[x] == 0:
            continue
        n_acc = sum(1 for u in grid if oracle.accept_test(P, Q, [x], [u])[0][0])
        a = Fraction(n_acc, N)
        law[x] += q_exact[x] * a
        reject_mass += q_exact[x] * (1 - a)
    counts = [0] * V
    for u in grid:
        y, _, _ = spec.sample_row(P, Q, 0, [u, 0.0])
        counts[y] += 1
    for y in range(V):
        law[y] += reject_mass * Fraction(counts[y], N)
    return law


def test_exact_law_six_token_example(golden):
    # thresholds: ratios 15/22, 5/6, 5/8 and residual CDF 10/19, 12/19:
    # every denominator divides 5016
    g = golden("two_models_six_token.json")
    p = [Fraction(v) for v in g["P_exact"]]
    q = [Fraction(v) for v in g["Q_exact"]]
    assert _exact_one_position_law(p, q, 5016) == p


def test_exact_law_three_token_example(golden):
    g = golden("guess_several_three_token.json")
    p = [Fraction(v) for v in g["p_exact"]]
    q = [Fraction(v) for v in g["q_exact"]]
    assert _exact_one_position_law(p, q, 15) == p


def test_exact_law_reversed_roles():
    # Swapping p and q of the six-token example: thresholds 22/15 (>=1),
    # 3/5, 8/9, 5/12, 6/5, 8/5 and residual CDF 14/19, 16/19 -> N = 4*9*5*19
    q = [Fraction(v) for v in ["3/10", "1/4", "9/50", "3/25", "1/10", "1/20"]]
    p = [Fraction(v) for v in ["11/25", "3/20", "4/25", "1/20", "3/25", "2/25"]]
    assert _exact_one_position_law(p, q, 4 * 9 * 5 * 19 * 2) == p


def _random_pair(rng):
    """A target law p and a draft law q over 2..64 tokens: softmax of
    Gaussian logits at a random scale; q is p's logits plus noise, and in
    some pairs q or p is zero on a random subset (tokens the draft never
    proposes, tokens the target never wants)."""
    V = int(rng.integers(2, 65))
    lp = rng.standard_normal(V) * rng.uniform(0.3, 4.0)
    lq = lp + rng.standard_normal(V) * rng.uniform(0.0, 3.0)
    p, q = np.exp(lp - lp.max()), np.exp(lq - lq.max())
    kind = int(rng.integers(0, 3))
    if kind == 1 and V > 2:
        q[rng.random(V) < 0.3] = 0.0
        q[int(rng.integers(0, V))] = 1.0
    elif kind == 2 and V > 2:
        p[rng.random(V) < 0.3] = 0.0
        p[int(rng.integers(0, V))] = 1.0
    return p / p.sum(), q / q.sum()


def test_random_pairs_law_is_p_and_alpha_is_one_minus_tv(golden):
    """The rule's emitted law equals p and its acceptance equals 1 - TV(p, q)
    for random pairs ("The Algebra and the Proof", The proof, which states
    both and checks them on random pairs to 1e-12 and about 3e-16). Pairs
    come from a Philox stream with the shapes of _random_pair, including
    q = 0 and p = 0 on subsets."""
    g = golden("closed_forms.json")
    rng = synth.stream(2026, "pins.random_pairs")
    worst_law = worst_alpha = 0.0
    for _ in range(g["random_pairs"]):
        p, q = _random_pair(rng)
        law, alpha = oracle.emitted_law(p, q)
        worst_alpha = max(worst_alpha, abs(alpha - (1 - oracle.total_variation(p, q))))
        assert abs(alpha - oracle.acceptance_rate(p, q)) < 1e-14
        worst_law = max(worst_law, float(np.abs(law - p).max()))
    assert worst_alpha < g["random_pairs_alpha_bound"]
    assert worst_law <= 2e-15   # the page printed 3.3e-16 for its own pairs


# ---------------------------------------------------------------------------
# Rounds: first rejection, row and uniform indices, emit
# ---------------------------------------------------------------------------

def _indexed_rows(K=3, V=5):
    """Row j's residual puts all its mass on token j; the bonus row puts all
    its mass on token K; every draft is token V-1 with ratio 1/2."""
    P, Q = [], []
    for j in range(K):
        p = np.full(V, 0.1)
        p[j] = 1.0 - 0.1 * (V - 1)
        P.append(p)
        Q.append(np.full(V, 1.0 / V))
    bonus = np.zeros(V)
    bonus[K] = 1.0
    P.append(bonus)
    return P, Q, [V - 1] * K


@pytest.mark.parametrize("u_acc,want", [
    ([0.9, 0.9, 0.9], [0, -1, -1, -1]),
    ([0.1, 0.9, 0.1], [4, 1, -1, -1]),
    ([0.1, 0.1, 0.9], [4, 4, 2, -1]),
    ([0.1, 0.1, 0.1], [4, 4, 4, 3]),
])
def test_round_uses_row_of_first_rejection(u_acc, want):
    P, Q, toks = _indexed_rows()
    r = oracle.verify_round(P, Q, toks, u_acc, [0.5] * 4)
    assert list(r["out_tokens"]) == want
    n = want.index(-1) - 1 if -1 in want else len(want) - 1
    assert r["n_accepted"] == n and r["n_emitted"] == n + 1


def test_round_uses_sample_uniform_of_terminating_row():
    # row j's residual splits evenly between tokens 0 and 1
    K, V = 3, 4
    P = [np.array([0.35, 0.35, 0.15, 0.15])] * K + [np.array([0.5, 0.5, 0.0, 0.0])]
    Q = [np.array([0.25, 0.25, 0.25, 0.25])] * K
    toks = [3] * K  # ratio 0.6
    u_s = [0.1, 0.9, 0.1, 0.9]
    for n in range(K + 1):
        u_a = [0.1] * n + [0.9] * (K - n)
        r = oracle.verify_round(P, Q, toks, u_a, u_s)
        assert r["n_accepted"] == n
        assert r["token"] == (0 if u_s[n] < 0.5 else 1)


def test_round_reports_ties():
    P, Q, toks = _indexed_rows()
    r = oracle.verify_round(P, Q, toks, [0.5 - 1e-6, 0.9, 0.9], [0.5] * 4)
    assert r["n_tie"] and r["token_tie"]
    r = oracle.verify_round(P, Q, toks, [0.1, 0.9, 0.5 + 1e-6], [0.5] * 4)
    assert not r["n_tie"]  # the tie sits after the first rejection


def test_batch_from_logits_matches_rounds_on_oracle_probs():
    d = synth.sampling_inputs(5, 3, 4, 300, 2.0, 0.5)
    res = oracle.verify_batch(d["target_logits"], d["draft_logits"], d["draft_tokens"],
                              d["u_accept"], d["u_sample"])
    P, _, _ = oracle.softmax_rows(d["target_logits"])
    Q, _, _ = oracle.softmax_rows(d["draft_logits"])
    for b in range(3):
        r = oracle.verify_round(P[b], Q[b], d["draft_tokens"][b], d["u_accept"][b], d["u_sample"][b])
        assert np.array_equal(r["out_tokens"], res["out_tokens"][b])
    assert res["out_tokens"].shape == (3, 5)
    n_acc, acc, _, _ = spec.accept_batch(P, Q, d["draft_tokens"], d["u_accept"])
    assert np.array_equal(n_acc, res["n_accepted"]) and np.array_equal(acc, res["accept"])
    tok, _, _ = spec.sample_batch(P, Q, n_acc, d["u_sample"])
    assert np.array_equal(tok, res["token"])


# ---------------------------------------------------------------------------
# Closed forms and statistics
# ---------------------------------------------------------------------------

def test_expected_tokens_printed_values(golden):
    g = golden("closed_forms.json")
    for c in g["cases"]:
        e = oracle.expected_tokens(c["alpha"], c["K"])
        assert round(e, c["decimals"]) == c["printed"], c
        # the general per-position form with equal alphas gives the same value
        assert abs(oracle.expected_tokens_general([c["alpha"]] * c["K"]) - e) < 1e-12
    assert abs(oracle.expected_tokens_general([0.8] * 4) - 3.3616) < 1e-12
    for K in range(1, 60):  # 0.6^(K+1) stays above fp64 resolution here
        assert oracle.expected_tokens(0.6, K) < g["cap_alpha_0_6_below"]
    for c in g["k1_cases"]:
        assert abs(oracle.expected_tokens(c["alpha"], 1) - c["printed"]) < 1e-12
    assert oracle.expected_tokens(1.0, 4) == 5.0


def _draw(q, u):
    """Drafter stand-in for the statistical pins: inverse-CDF draw from q."""
    return np.minimum(np.searchsorted(np.cumsum(q), u * np.sum(q), side="right"), len(q) - 1)


def test_monte_carlo_tokens_per_round_and_emitted_law(golden):
    # The page's simulation setting: the same p and q at every position,
    # K = 4, 200k rounds.
    g = golden("two_models_six_token.json")
    P, Q = np.array(g["P"]), np.array(g["Q"])
    K, R = g["K"], g["rounds"]
    alpha = oracle.acceptance_rate(P, Q)
    ud = synth.uniforms(1, "pin.mc.draft", (R, K)).astype(np.float64)
    ua = synth.uniforms(1, "pin.mc.accept", (R, K))
    us = synth.uniforms(1, "pin.mc.sample", (R, K + 1))
    toks = _draw(Q, ud)
    Pr, Qr = [P] * (K + 1), [Q] * K
    counts = np.zeros(len(P))
    n_hist = np.zeros(K + 1)
    total = 0
    for i in range(R):
        r = oracle.verify_round(Pr, Qr, toks[i], ua[i], us[i])
        e = r["out_tokens"][:r["n_emitted"]]
        total += len(e)
        np.add.at(counts, e, 1)
        n_hist[r["n_accepted"]] += 1
    mean = total / R
    # exact law of N: truncated geometric (Appendix tool 2)
    pn = np.array([alpha ** n * (1 - alpha) for n in range(K)] + [alpha ** K])
    var = float(np.sum(pn * (np.arange(K + 1) + 1) ** 2) - oracle.expected_tokens(alpha, K) ** 2)
    se = math.sqrt(var / R)
    assert abs(mean - oracle.expected_tokens(alpha, K)) < 4 * se
    assert abs(mean - g["tokens_per_round_measured_printed"]) < 4 * se + 5e-4
    emp = counts / counts.sum()
    sd = np.sqrt(P * (1 - P) / counts.sum())
    assert np.all(np.abs(emp - P) < 4 * sd + 1e-4)
    assert np.all(np.abs(n_hist / R - pn) < 4 * np.sqrt(pn * (1 - pn) / R))


def test_monte_carlo_three_token_acceptance(golden):
    g = golden("guess_several_three_token.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    R = 100_000
    x = _draw(q, synth.uniforms(2, "pin.mc3.draft", R).astype(np.float64))
    ua = synth.uniforms(2, "pin.mc3.accept", (R, 1))
    us = synth.uniforms(2, "pin.mc3.sample", (R, 2))
    out = np.zeros(R, dtype=np.int64)
    acc = np.zeros(R, dtype=bool)
    for i in range(R):
        r = oracle.verify_round([p, p], [q], [x[i]], ua[i], us[i])
        out[i] = r["out_tokens"][0]
        acc[i] = r["n_accepted"] == 1
    a = g["acceptance_printed"]
    assert abs(acc.mean() - a) < 4 * math.sqrt(a * (1 - a) / R)
    emp = np.bincount(out, minlength=3) / R
    assert np.all(np.abs(emp - p) < 4 * np.sqrt(p * (1 - p) / R))


def test_invalid_inputs_have_defined_results():
    P = [np.array([0.5, 0.5])] * 2
    Q = [np.array([0.5, 0.5])]
    for bad in (-1, 2):
        acc, ratio, _ = oracle.accept_test(P, Q, [bad], [0.0])
        assert not acc[0] and ratio[0] == 0.0
    assert oracle.inverse_cdf(np.zeros(4), 0.3)[0] == -1
    tok, _, _ = spec.sample_batch(np.array([P]), np.array([Q]), [2], [[0.5, 0.5]])
    assert tok[0] == -1


# ---------------------------------------------------------------------------
# Temperature and greedy verification
# ---------------------------------------------------------------------------

def _greedy_logits(picks, vocab, rng):
    """Logits whose argmax at row i is picks[i] (clear margin)."""
    l = rng.standard_normal((len(picks), len(vocab))).astype(np.float32)
    for i, t in enumerate(picks):
        l[i, vocab.index(t)] = np.float32(6.0)
    return l


@pytest.mark.parametrize("case", ["printed", "all_match"])
def test_greedy_worked_example(golden, case):
    """Greedy verification (target temperature 0) reproduces the printed
    verify_greedy call, for every choice of uniforms: three accepted guesses
    plus the target's correction, or four plus the bonus token."""
    g = golden("guess_several_greedy.json")
    draft = g["draft"] if case == "printed" else g["all_match_draft"]
    want = g["printed_result"] if case == "printed" else g["all_match_result"]
    vocab = sorted(set(g["draft"]) | set(g["target_picks"]) | {" the", " city"})
    rng = np.random.default_rng(5)
    tl = _greedy_logits(g["target_picks"], vocab, rng)[None]
    dl = rng.standard_normal((1, len(draft), len(vocab))).astype(np.float32)
    toks = np.array([[vocab.index(t) for t in draft]])
    for trial in range(20):
        ua = rng.random((1, len(draft)), dtype=np.float32)
        us = rng.random((1, len(draft) + 1), dtype=np.float32)
        r = oracle.verify_batch(tl, dl, toks, ua, us, t_target=0.0)
        n = int(r["n_emitted"][0])
        got = [vocab[t] for t in r["out_tokens"][0][:n]]
        assert got == want, (trial, got)
        assert (r["out_tokens"][0][n:] == -1).all()


def test_temperature_two_token_closed_form():
    # p1 = sigmoid(d / T) for logits (0, d); T = 1 is the plain softmax
    for d in (0.5, 2.0, -3.0):
        for T in (0.25, 0.7, 1.0, 3.0):
            p, _, _ = oracle.softmax_rows(np.array([[0.0, d]], np.float32), T)
            assert abs(p[0, 1] - 1.0 / (1.0 + math.exp(-d / T))) < 1e-15
    l = np.random.default_rng(1).standard_normal((3, 50)).astype(np.float32)
    assert np.array_equal(oracle.softmax_rows(l, 1.0)[0], oracle.softmax_rows(l)[0])
    # scipy reference at T: softmax of l / T
    for T in (0.3, 2.5):
        ref = scipy.special.softmax(l.astype(np.float64) / T, axis=-1)
        assert np.abs(oracle.softmax_rows(l, T)[0] - ref).max() < 1e-15


def test_temperature_zero_is_first_argmax_and_the_cold_limit():
    l = np.array([[0.5, 2.0, 2.0, -1.0], [3.0, 1.0, 0.0, 2.9]], np.float32)
    p0, _, s0 = oracle.softmax_rows(l, 0.0)
    assert np.array_equal(p0, [[0, 1, 0, 0], [1, 0, 0, 0]]) and np.array_equal(s0, [1, 1])
    # a clear maximum: T -> 0 approaches the one-hot law
    pc, _, _ = oracle.softmax_rows(l[1:], 1e-3)
    assert abs(pc[0, 0] - 1.0) < 1e-12
    with pytest.raises(ValueError):
        oracle.softmax_rows(l, -1.0)


def test_warped_law_is_the_warped_target():
    """The rule applied to warped p and q emits exactly the warped target
    (its law does not depend on how p and q were produced)."""
    rng = np.random.default_rng(2)
    for T_t, T_d in ((0.6, 0.6), (0.6, 1.4), (2.0, 1.0)):
        lt = rng.standard_normal((1, 40)).astype(np.float32) * 2
        ld = lt + rng.standard_normal((1, 40)).astype(np.float32)
        p = oracle.softmax_rows(lt, T_t)[0][0]
        q = oracle.softmax_rows(ld, T_d)[0][0]
        law, alpha = oracle.emitted_law(p, q)
        assert np.abs(law - p).max() < 1e-15
        assert abs(alpha - (1 - oracle.total_variation(p, q))) < 1e-14


def test_greedy_expected_tokens_monte_carlo():
    """Greedy target, drafts sampled from q: position j is accepted with
    probability alpha_j = q_j(argmax p_j), so tokens per round have mean
    1 + sum_i prod_{j<=i} alpha_j. 40000 rounds, within 4 standard errors."""
    rng = np.random.default_rng(3)
    K, V, R = 4, 12, 40000
    lt = (rng.standard_normal((1, K + 1, V)) * 1.5).astype(np.float32)
    ld = (lt[:, :K] + rng.standard_normal((1, K, V)).astype(np.float32) * 0.8).astype(np.float32)
    P, _, _ = oracle.softmax_rows(lt, 0.0)
    Q, _, _ = oracle.softmax_rows(ld, 1.0)
    a = [Q[0, j, int(np.argmax(lt[0, j]))] for j in range(K)]
    want = oracle.expected_tokens_general(a)
    cq = np.cumsum(Q[0], axis=-1)
    n_tot = np.zeros(R)
    for r in range(R):
        u = rng.random(K)
        toks = np.array([[min(int(np.searchsorted(cq[j], u[j] * cq[j, -1], side="right")), V - 1)
                          for j in range(K)]])
        res = spec.verify_batch_probs(P, Q, toks, rng.random((1, K)), rng.random((1, K + 1)))
        n_tot[r] = res["n_emitted"][0]
    se = n_tot.std() / math.sqrt(R)
    assert abs(n_tot.mean() - want) < 4 * se, (n_tot.mean(), want, se)
