"""Plain fp64 CPU oracle for the verification step of speculative decoding.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package. The HIP library never calls it, it never calls the HIP library, and
the two share no code, headers, tables or helpers. The only code both sides
use is the seeded input generator in ``synth/``, which holds none of the
method's arithmetic.

What it computes, and where the pages define it:

* ``linear``   -- ``y = x . W^T`` over the K+1 verify positions, the one
  weight-streaming pass of the target ("Speculative Decoding: Guess Several
  Tokens, Check Them in One Pass", Step 1; "What Actually Happens During
  Speculative Decoding in LLMs", the 5-candidate pass).
* ``linear_w8`` -- the same pass with FP8 E4M3 weights and a per-row scale
  (weight-only 8-bit storage, "Speculative Decoding: The Algebra and the
  Proof", Where it breaks).
* ``verify_attention`` -- the K+1 verify positions attending causally over
  the KV cache, grouped-query heads ("Speculative Decoding: Guess Several
  Tokens, Check Them in One Pass", Step 1: the pass works like a tiny
  prefill and reads the cache once).
* ``softmax_rows`` -- p and q from logits ("Speculative Decoding: Two Models,
  One Voice", Implementing it against a real model).
* ``speculative`` -- the accept test min(1, p/q), the first rejection, the
  residual norm(max(0, p-q)) resample, the bonus token from p_{K+1}, and the
  closed forms alpha = sum min(p, q) = 1 - TV and E[N] = (1-a^{K+1})/(1-a)
  ("Two Models, One Voice", The rule that makes it exact and Appendix tools
  1-2; "Speculative Decoding: The Algebra and the Proof", The algebra / The
  proof).

Every function is pinned by ``tests/test_oracle_pins.py`` against values the
pages print, closed forms, exact rational enumeration and brute force. The
one convention no page fixes -- which token id a given uniform maps to under
inverse-CDF sampling -- is "parity unpinned": only the law of the sampled
token is pinned, the id map is a convention shared with the GPU path.
"""

from .attention import verify_attention
from .linear import bf16_to_f64, e4m3_to_f64, linear, linear_w8, round_to_bf16, to_bf16_bits
from .softmax import softmax_rows
from .speculative import (
    TIE_BAND,
    accept_batch,
    acceptance_rate,
    accept_test,
    emitted_law,
    expected_tokens,
    expected_tokens_general,
    first_rejection,
    inverse_cdf,
    residual_weights,
    sample_batch,
    sample_row,
    total_variation,
    verify_batch,
    verify_batch_probs,
    verify_round,
)

__all__ = [
    "TIE_BAND", "accept_batch", "sample_batch", "sample_row", "verify_batch_probs",
    "bf16_to_f64", "e4m3_to_f64", "linear", "linear_w8", "round_to_bf16", "to_bf16_bits",
    "softmax_rows", "verify_attention", "acceptance_rate", "accept_test",
    "emitted_law", "expected_tokens", "expected_tokens_general",
    "first_rejection", "inverse_cdf", "residual_weights", "total_variation",
    "verify_batch", "verify_round",
]
