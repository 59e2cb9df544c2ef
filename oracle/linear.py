"""Oracle for the verify pass's linear layers, in fp64 (test infrastructure).

The verify pass feeds the K+1 positions of every sequence through each target
linear in one read of the weights: the activations form an [M x d_in] tile
with M = B*(K+1) rows, and each linear computes y = x . W^T with W stored as
[d_out][d_in] ("What Actually Happens During Speculative Decoding in LLMs":
a [5 x d] matrix multiplied against the weights instead of a [1 x d] vector;
"Speculative Decoding: Guess Several Tokens, Check Them in One Pass", Step 1).

Inputs are bfloat16 bit patterns (uint16). Widening bf16 -> fp64 is exact and
every bf16*bf16 product is exact in fp64, so the only error is the fp64
summation (relative error below d_in * 2^-53).

``linear_w8`` is the same product with weight-only 8-bit storage: the
weights are FP8 E4M3 codes with one float32 scale per output row, the
activations stay bf16 ("Speculative Decoding: The Algebra and the Proof",
Where it breaks: weight-only 8-bit storage with BF16 compute halves the bytes
per weight and so doubles the verify pass's FLOPs per byte).
"""

import numpy as np


def bf16_to_f64(bits):
    """Exact value of bfloat16 bit patterns, as float64.

    A bfloat16 is the upper half of an IEEE float32: placing the 16 bits in
    the high half of a 32-bit word gives the float32 with the same value.
    """
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_to_bf16(values):
    """Nearest bfloat16 value of finite float64 values, ties to even, as
    float64 (round-to-nearest-even is the IEEE default the format uses).

    bfloat16 keeps 8 significant bits: for |v| in [2^(e-1), 2^e) the spacing
    is 2^(e-8); below 2^-126 the subnormal spacing 2^-133 applies. Values
    beyond the largest bfloat16 are not expected here.
    """
    v = np.asarray(values, dtype=np.float64)
    _, e = np.frexp(v)
    step = np.maximum(e - 8, -133)
    return np.ldexp(np.rint(np.ldexp(v, -step)), step)


def to_bf16_bits(values):
    """bfloat16 bit patterns (uint16) of round_to_bf16(values)."""
    r = round_to_bf16(values).astype(np.float32)  # exact: r is a bfloat16 value
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def linear(x_bits, w_bits, block_bytes=64 << 20):
    """y[m][n] = sum_k x[m][k] * w[n][k] in float64.

    x_bits: uint16 [M][d_in] bf16 activations (one row per verify position).
    w_bits: uint16 [d_out][d_in] bf16 weights (nn.Linear layout).
    Returns float64 [M][d_out].

    The weights are widened one block of rows at a time so that a 1 GB bf16
    matrix never becomes a 4 GB fp64 copy; each block is a plain fp64 matrix
    product (a library primitive), with no other reordering.
    """
    x_bits = np.asarray(x_bits)
    w_bits = np.asarray(w_bits)
    if x_bits.ndim != 2 or w_bits.ndim != 2 or x_bits.shape[1] != w_bits.shape[1]:
        raise ValueError(f"shape mismatch: x {x_bits.shape}, w {w_bits.shape}")
    x = bf16_to_f64(x_bits)
    m, d_in = x.shape
    d_out = w_bits.shape[0]
    y = np.empty((m, d_out), dtype=np.float64)
    rows = max(1, block_bytes // (8 * max(d_in, 1)))
    for n0 in range(0, d_out, rows):
        w = bf16_to_f64(w_bits[n0:n0 + rows])
        y[:, n0:n0 + rows] = x @ w.T
    return y


def e4m3_to_f64(codes):
    """Exact value of FP8 E4M3 codes (uint8), as float64.

    The OCP 8-bit floating-point format E4M3: one sign bit, a 4-bit exponent
    with bias 7, a 3-bit mantissa. Exponent field 0 holds the subnormals
    (m / 8) * 2^-6; otherwise the value is (1 + m / 8) * 2^(e - 7). The
    format has no infinities: S.1111.111 is NaN, so the largest finite
    magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


def linear_w8(x_bits, w_codes, w_scale, block_bytes=64 << 20):
    """y[m][n] = w_scale[n] * sum_k x[m][k] * e4m3(w[n][k]) in float64.

    x_bits: uint16 [M][d_in] bf16 activations.
    w_codes: uint8 [d_out][d_in] FP8 E4M3 weight codes (nn.Linear layout).
    w_scale: float32 [d_out], the dequantisation scale of each output row.
    Returns float64 [M][d_out]. Blocked over rows of w like ``linear``.
    """
    x_bits = np.asarray(x_bits)
    w_codes = np.asarray(w_codes)
    w_scale = np.asarray(w_scale, dtype=np.float32)
    if x_bits.ndim != 2 or w_codes.ndim != 2 or x_bits.shape[1] != w_codes.shape[1]:
        raise ValueError(f"shape mismatch: x {x_bits.shape}, w {w_codes.shape}")
    if w_scale.shape != (w_codes.shape[0],):
        raise ValueError(f"w_scale shape {w_scale.shape}, expected ({w_codes.shape[0]},)")
    x = bf16_to_f64(x_bits)
    m, d_in = x.shape
    d_out = w_codes.shape[0]
    y = np.empty((m, d_out), dtype=np.float64)
    rows = max(1, block_bytes // (8 * max(d_in, 1)))
    for n0 in range(0, d_out, rows):
        w = e4m3_to_f64(w_codes[n0:n0 + rows])
        y[:, n0:n0 + rows] = (x @ w.T) * w_scale[n0:n0 + rows].astype(np.float64)
    return y
