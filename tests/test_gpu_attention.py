"""GPU parity of spec_verify_attention against the fp64 oracle
(oracle.verify_attention): the K+1 verify positions attending causally over
the KV cache, grouped-query heads.

Tolerance, derived from the arithmetic: the probabilities enter the value
product rounded to bf16 (relative error at most 2^-9 each) and the row sums
add the same rounded values, so the output is a convex combination of the
values with weights off by at most that factor: |o - o_ref| <= 2^-9 *
max_t |v_t - o_ref| <= 2^-8 * max |v|. fp32 scores, exp2 and sums add far
less; the test allows 1.1 * 2^-8 * max|v|, plus half a bf16 ulp of the
output for bf16 outputs. A wrong mask, head mapping or split merge misses it
by orders of magnitude.
"""

import math

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def inputs(seed, B, K1, H, Hkv, T, D=128):
    q = synth.bf16_normal_bits(seed, "att.q", (B, K1, H, D))
    k = synth.bf16_normal_bits(seed, "att.k", (B, T, Hkv, D))
    v = synth.bf16_normal_bits(seed, "att.v", (B, T, Hkv, D))
    return q, k, v


def run(sv, dev, q, k, v, scale, out_dtype):
    import torch
    from synth import device as sd
    o = sv.verify_attention(sd.from_bits(q, dev), sd.from_bits(k, dev), sd.from_bits(v, dev),
                            scale=scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64)


def check(o, ref, v_bits, bf16_out, what):
    vmax = float(np.abs(oracle.bf16_to_f64(v_bits)).max())
    tol = 1.1 * 2.0 ** -8 * vmax + (2.0 ** -9 * np.abs(ref) if bf16_out else 0.0)
    err = np.abs(o - ref)
    print(f"{what}: max err {err.max():.2e} (tolerance {np.max(tol):.2e})", flush=True)
    assert np.all(err <= tol), what


CASES = [  # B, K, T, H, Hkv
    (1, 4, 37, 8, 2),
    (2, 4, 300, 32, 8),
    (3, 0, 129, 4, 4),        # one query: decode attention
    (1, 7, 1000, 32, 8),      # 32 query rows per kv head
    (2, 3, 77, 16, 2),        # 8 query heads per kv head
    (1, 4, 5, 32, 8),         # no context: T = K+1
    (1, 4, 4096, 32, 8),      # the Llama-3.1-8B layer shape, context splits
    (1, 3, 4096, 32, 8),      # 16 rows: eight waves in single-wave teams, 16 splits
    (40, 4, 300, 32, 8),      # 320 (sequence, kv head) groups: four waves, two splits
    (40, 3, 300, 32, 8),      # the same with 16 rows (single-wave teams)
    (64, 3, 200, 32, 8),      # 512 groups of 16 rows: four waves, one split
]


@pytest.mark.parametrize("B,K,T,H,Hkv", CASES)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_attention_matches_oracle(sv, dev, B, K, T, H, Hkv, out):
    import torch
    q, k, v = inputs(B * 1000 + T + K, B, K + 1, H, Hkv, T)
    scale = 1 / math.sqrt(128)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    o = run(sv, dev, q, k, v, scale, dt)
    ref = oracle.verify_attention(q, k, v, scale)
    check(o, ref, v, out == "bf16", f"B={B} K={K} T={T} H={H}/{Hkv} out={out}")


def test_attention_sharp_scores(sv, dev):
    """A large scale makes every softmax nearly one-hot."""
    import torch
    q, k, v = inputs(7, 2, 5, 32, 8, 700)
    o = run(sv, dev, q, k, v, 1.5, torch.float32)
    check(o, oracle.verify_attention(q, k, v, 1.5), v, False, "scale 1.5")


def test_attention_long_context_and_batch(sv, dev):
    """Many splits (B=1, T=16384) and no splits (B=64, T=4096); the oracle
    checks a few sequences of the batch."""
    import torch
    from synth import device as sd
    for B, T, idx in [(1, 16384, [0]), (64, 4096, [0, 37, 63])]:
        q = sd.normal_bf16((B, 5, 32, 128), 1.0, 11 + B, dev)
        k = sd.normal_bf16((B, T, 8, 128), 1.0, 12 + B, dev)
        v = sd.normal_bf16((B, T, 8, 128), 1.0, 13 + B, dev)
        o = sv.verify_attention(q, k, v, out_dtype=torch.float32)
        torch.cuda.synchronize()
        sel = torch.tensor(idx, device=dev)
        qb, kb, vb = (sd.to_bits(t.index_select(0, sel)) for t in (q, k, v))
        ref = oracle.verify_attention(qb, kb, vb, 1 / math.sqrt(128))
        got = o.index_select(0, sel).cpu().numpy().astype(np.float64)
        check(got, ref, vb, False, f"B={B} T={T}")


def test_attention_deterministic(sv, dev):
    import torch
    from synth import device as sd
    q = sd.normal_bf16((1, 5, 32, 128), 1.0, 21, dev)
    k = sd.normal_bf16((1, 8192, 8, 128), 1.0, 22, dev)
    v = sd.normal_bf16((1, 8192, 8, 128), 1.0, 23, dev)
    a = sv.verify_attention(q, k, v, out_dtype=torch.float32)
    b = sv.verify_attention(q, k, v, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
