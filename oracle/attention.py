"""Oracle for the verify pass's attention, in fp64 (test infrastructure).

The K+1 verify positions of a sequence go through the target like a tiny
prefill, attention included: each position attends, through the causal
mask, only to the tokens before it and itself, and the keys and values of
the earlier context are read once for all K+1 positions ("Speculative
Decoding: Guess Several Tokens, Check Them in One Pass", Step 1).

Layouts (bf16 bit patterns, uint16):

* q        [B][K+1][H][D]    queries of the K+1 verify positions;
* k_cache  [B][T][Hkv][D]    keys of all T = ctx + K + 1 positions, the K+1
  verify positions last (they were appended by the same pass);
* v_cache  [B][T][Hkv][D]    values, same layout.

Query position i (0..K) sits at absolute position T - K - 1 + i and attends
to keys 0 .. T - K - 1 + i. Query head h reads key/value head h // (H / Hkv)
(grouped-query attention). Output [B][K+1][H][D]:

    o = sum_t softmax_t(scale * q . k_t) v_t.

Readings (the pages give no more detail): the new positions' keys and values
are already in the cache, and scale is the caller's (1/sqrt(D) as usual).
"""

import numpy as np

from .linear import bf16_to_f64


def verify_attention(q_bits, k_bits, v_bits, scale):
    """Attention of the K+1 verify positions over the cache, float64 [B][K+1][H][D]."""
    q = bf16_to_f64(q_bits)
    k = bf16_to_f64(k_bits)
    v = bf16_to_f64(v_bits)
    if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape:
        raise ValueError(f"shapes q {q.shape}, k {k.shape}, v {v.shape}")
    B, K1, H, D = q.shape
    _, T, Hkv, Dk = k.shape
    if k.shape[0] != B or Dk != D or H % Hkv != 0 or T < K1:
        raise ValueError(f"shapes q {q.shape}, k {k.shape} disagree")
    G = H // Hkv
    out = np.empty((B, K1, H, D), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            kh = k[b, :, h // G, :]            # [T][D]
            vh = v[b, :, h // G, :]
            for i in range(K1):
                last = T - K1 + i              # the last key position i may see
                s = scale * (kh[:last + 1] @ q[b, i, h])
                s -= s.max()
                p = np.exp(s)
                out[b, i, h] = (p @ vh[:last + 1]) / p.sum()
    return out
