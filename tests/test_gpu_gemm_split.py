"""GPU parity of spec_verify_gemm_ws (the tile kernel with its reduction
split over workgroups, fp32 partial outputs added by a second kernel)
against the fp64 oracle.

Tolerances as for spec_verify_gemm: max |y - y_ref| / max(|y_ref|, rms of
the reference row) <= 2e-2 for bf16 outputs and 1e-3 for fp32 outputs (fp32
accumulation in every split, then a sum of at most 16 fp32 partials); a
split that skipped or repeated its k-tiles would miss 1e-3 by far.
"""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 2e-2
TOL_F32 = 1e-3


def rel_err(y, ref):
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    return float(np.max(np.abs(y - ref) / np.maximum(np.abs(ref), rms)))


def check(y, ref, out_dtype, what):
    import torch
    e = rel_err(y, ref)
    print(f"{what}: rel err {e:.3e}", flush=True)
    assert e <= TOL, what
    if out_dtype == torch.float32:
        assert e <= TOL_F32, what


def splits(sv, M, d_in, d_out):
    """Number of splits the plan takes (0: none)."""
    return sv.gemm_workspace_bytes(M, d_in, d_out) // (M * d_out * 4)


# Shapes the plan splits, one per split tile shape reachable at sizes the
# oracle finishes in seconds: ragged M and d_out tails, and k-tile counts
# (d_in / 64) that the splits do not divide evenly (94 over 16, 128 over 15,
# 94 over 10, 128 over 10) as well as ones they do (80 over 16).
SMALL = [
    (9, 5120, 300),      # 32x64 tiles, 16 splits
    (9, 6016, 300),      # 32x64, 16 splits of 94 k-tiles
    (37, 6016, 777),     # 64x64, 16 splits
    (37, 8192, 2050),    # 64x128, 15 splits
    (77, 6016, 3000),    # 128x128, 10 splits
    (517, 8192, 300),    # 128x64, 10 splits
]


@pytest.mark.parametrize("M,d_in,d_out", SMALL)
def test_split_parity(sv, dev, M, d_in, d_out):
    import torch
    from synth import device as sd
    assert splits(sv, M, d_in, d_out) >= 2, (M, d_in, d_out)
    xb, wb = synth.linear_inputs(500 + M, f"split{d_in}.{d_out}", M, d_in, d_out)
    ref = oracle.linear(xb, wb)
    x, w = sd.from_bits(xb, dev), sd.from_bits(wb, dev)
    for od in (torch.float32, torch.bfloat16):
        y = sv.verify_gemm_ws(x, w, out_dtype=od)
        torch.cuda.synchronize()
        check(y.float().cpu().numpy().astype(np.float64), ref, od,
              f"split M={M} {d_in}->{d_out} {od}")


def test_split_workspace_reuse_and_determinism(sv, dev):
    """One workspace serves calls of different shapes in stream order; a
    repeated call gives bitwise equal outputs (the partials are added in
    split order)."""
    import torch
    from synth import device as sd
    shapes = [(77, 6016, 3000), (37, 8192, 2050), (77, 6016, 3000)]
    need = max(sv.gemm_workspace_bytes(*s) for s in shapes)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    outs = []
    for i, (M, d_in, d_out) in enumerate(shapes):
        x = sd.normal_bf16((M, d_in), 1.0, 10 + M, dev)
        w = sd.normal_bf16((d_out, d_in), synth.WEIGHT_STD, 20 + d_in, dev)
        outs.append(sv.verify_gemm_ws(x, w, out_dtype=torch.float32, workspace=ws))
        if i == 1:
            xb, wb = sd.to_bits(x), sd.to_bits(w)
            torch.cuda.synchronize()
            check(outs[1].cpu().numpy().astype(np.float64), oracle.linear(xb, wb),
                  torch.float32, "reused workspace 37x8192->2050")
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("M,d_in,d_out", [(5, 4096, 4096), (320, 4096, 28672),
                                           (5, 8192, 57344), (40, 1032, 777)])
def test_no_split_is_spec_verify_gemm(sv, dev, M, d_in, d_out):
    """Where the plan does not split (workspace size 0) the call is
    spec_verify_gemm: bitwise equal outputs, no workspace needed (the tile
    kernel, the streaming kernel, and d_in not a multiple of 64)."""
    import torch
    from synth import device as sd
    assert sv.gemm_workspace_bytes(M, d_in, d_out) == 0
    x = sd.normal_bf16((M, d_in), 1.0, 30 + M, dev)
    w = sd.normal_bf16((d_out, d_in), synth.WEIGHT_STD, 40 + d_in, dev)
    a = sv.verify_gemm(x, w, out_dtype=torch.bfloat16)
    b = sv.verify_gemm_ws(x, w, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def sampled_full_size(sv, dev, M, d_in, d_out, seed, out_dtype, n_cols=48):
    """Full-size linear through spec_verify_gemm_ws; the oracle checks a
    sample of output columns (first and last 8 plus random ones)."""
    import torch
    from synth import device as sd
    w = sd.normal_bf16((d_out, d_in), synth.WEIGHT_STD, seed, dev)
    x = sd.normal_bf16((M, d_in), 1.0, seed + 1, dev)
    y = sv.verify_gemm_ws(x, w, out_dtype=out_dtype)
    rng = np.random.default_rng(seed)
    cols = np.unique(np.concatenate([np.arange(8), np.arange(d_out - 8, d_out),
                                     rng.integers(0, d_out, n_cols)]))
    idx = torch.from_numpy(cols).to(dev)
    w_rows = sd.to_bits(w.index_select(0, idx))
    x_bits = sd.to_bits(x)
    y_s = y.index_select(1, idx).float().cpu().numpy().astype(np.float64)
    del w, y
    torch.cuda.empty_cache()
    return y_s, oracle.linear(x_bits, w_rows)


# Full-size linears the plan splits: the Llama-3.1-8B down projection at
# every swept M (32x64, 128x128, 256x128, 320x128 and 320x256 tiles), a
# ragged 320-row tile (M = 301) and 256x256 tiles (M = 1000), the O
# projection at M = 1100 (320x128 tiles, two splits; at M = 1280 an
# exact-fill 160x128 tile runs unsplit), and the Llama-3.1-70B down
# projection (128x256 and 256x256 tiles).
FULL = [(5, 14336, 4096), (20, 14336, 4096), (80, 14336, 4096), (160, 14336, 4096),
        (301, 14336, 4096), (320, 14336, 4096), (1000, 14336, 4096), (1280, 14336, 4096),
        (1100, 4096, 4096), (80, 28672, 8192), (160, 28672, 8192), (640, 8192, 10240),
        # partial tiles stored through the LDS staging block with d_out not
        # a multiple of 4 (element by element at every row): 256x128,
        # 256x256, 320x128, 320x256 and 128x256 tiles
        (160, 8192, 8191), (160, 14336, 8191), (320, 14336, 4095), (320, 14336, 10239),
        (640, 14336, 2047)]


@pytest.mark.parametrize("M,d_in,d_out", FULL)
def test_split_full_size(sv, dev, M, d_in, d_out):
    import torch
    assert splits(sv, M, d_in, d_out) >= 2, (M, d_in, d_out)
    for od in (torch.bfloat16, torch.float32):
        y, ref = sampled_full_size(sv, dev, M, d_in, d_out, 7 * M + d_in, od)
        check(y, ref, od, f"split full M={M} {d_in}->{d_out} {od}")


# ---------------------------------------------------------------------------
# FP8 E4M3 weights with per-row scales (spec_verify_gemm_w8_ws): the partials
# are unscaled sums, the split-sum kernel applies the row scale once.
# ---------------------------------------------------------------------------

def w8_splits(sv, M, d_in, d_out):
    return sv.gemm_w8_workspace_bytes(M, d_in, d_out) // (M * d_out * 4)


@pytest.mark.parametrize("M,d_in,d_out", [(17, 6016, 300), (100, 4160, 4100)])
def test_w8_split_parity(sv, dev, M, d_in, d_out):
    """64x128 tiles in 16 splits of 94 k-tiles, 128x128 in 7 splits of 65
    (both widened once per workgroup), ragged M and d_out."""
    import torch
    from synth import device as sd
    assert w8_splits(sv, M, d_in, d_out) >= 2
    xb = synth.bf16_normal_bits(M, "w8split.x", (M, d_in))
    codes = synth.e4m3_normal_codes(M, "w8split.w", (d_out, d_in))
    scale = synth.w8_row_scales(M, "w8split.s", d_out)
    ref = oracle.linear_w8(xb, codes, scale)
    x = sd.from_bits(xb, dev)
    w = torch.from_numpy(np.ascontiguousarray(codes)).to(dev)
    s = torch.from_numpy(np.ascontiguousarray(scale)).to(dev)
    for od in (torch.float32, torch.bfloat16):
        y = sv.verify_gemm_w8_ws(x, w, s, out_dtype=od)
        torch.cuda.synchronize()
        check(y.float().cpu().numpy().astype(np.float64), ref, od,
              f"w8 split M={M} {d_in}->{d_out} {od}")


def test_w8_split_one_hot_exact(sv, dev):
    """One-hot activations through a split plan: each output is a single
    product in one split and exact zeros in the others, so y equals
    fp32(scale * e4m3(code)) bit for bit for every finite code."""
    import torch
    from synth import device as sd
    M, d_in = 17, 6016
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    d_out = 300
    assert w8_splits(sv, M, d_in, d_out) >= 2
    rng = np.random.default_rng(8)
    cols = rng.permutation(d_in)[:M]
    w = np.zeros((d_out, d_in), dtype=np.uint8)
    for j, k in enumerate(cols):
        w[:, k] = np.resize(np.roll(codes, 13 * j), d_out)
    s = synth.w8_row_scales(9, "w8.special.split", d_out)
    x = np.zeros((M, d_in), dtype=np.uint16)
    x[np.arange(M), cols] = 0x3F80  # 1.0
    y = sv.verify_gemm_w8_ws(sd.from_bits(x, dev), torch.from_numpy(w).to(dev),
                             torch.from_numpy(s).to(dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = (oracle.e4m3_to_f64(w[:, cols].T) * s.astype(np.float64)[None, :]).astype(np.float32)
    assert np.array_equal(y.cpu().numpy(), want)


# Full-size FP8 linears the plan splits: the Llama-3.1-8B down projection at
# M = 20 to 1280 (64x128, 128x256 with 128-element stages, 320x128,
# 320x256, 256x256 tiles, a ragged 320-row tile at M = 301), d_in = 14400 (a
# multiple of 64 but not 128: the 64-element 128x256 form), the O
# projection at M = 320, gate/up at M = 80, and the Llama-3.1-70B down
# projection at M = 160.
W8_FULL = [(20, 14336, 4096), (80, 14336, 4096), (160, 14336, 4096), (301, 14336, 4096),
           (320, 14336, 4096), (1000, 14336, 4096), (1280, 14336, 4096), (80, 14400, 4096),
           (333, 14400, 4096), (320, 4096, 4096), (80, 4096, 28672), (160, 28672, 8192),
           # staged partial tiles with d_out not a multiple of 4: 128x256
           # (128-element stages), 256x256, 320x128 and 320x256
           (160, 8192, 4095), (160, 14336, 8191), (320, 8192, 8191), (320, 8192, 10239)]


@pytest.mark.parametrize("M,d_in,d_out", W8_FULL)
def test_w8_split_full_size(sv, dev, M, d_in, d_out):
    import torch
    from synth import device as sd
    assert w8_splits(sv, M, d_in, d_out) >= 2, (M, d_in, d_out)
    seed = 43 * M + d_in
    w = sd.e4m3_normal_codes((d_out, d_in), synth.W8_CODE_STD, seed, dev)
    s = sd.w8_row_scales(d_out, synth.WEIGHT_STD / synth.W8_CODE_STD, seed + 1, dev)
    x = sd.normal_bf16((M, d_in), 1.0, seed + 2, dev)
    rng = np.random.default_rng(seed)
    cols = np.unique(np.concatenate([np.arange(8), np.arange(d_out - 8, d_out),
                                     rng.integers(0, d_out, 48)]))
    idx = torch.from_numpy(cols).to(dev)
    ref = oracle.linear_w8(sd.to_bits(x), w.index_select(0, idx).cpu().numpy(),
                           s.index_select(0, idx).cpu().numpy())
    for od in (torch.bfloat16, torch.float32):
        y = sv.verify_gemm_w8_ws(x, w, s, out_dtype=od)
        got = y.index_select(1, idx).float().cpu().numpy().astype(np.float64)
        check(got, ref, od, f"w8 split full M={M} {d_in}->{d_out} {od}")
    a = sv.verify_gemm_w8_ws(x, w, s, out_dtype=torch.float32)
    b = sv.verify_gemm_w8_ws(x, w, s, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b), "split FP8 launches differ"
    del w, a, b
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M,d_in,d_out", [(16, 14336, 4096), (320, 4096, 28672), (20, 4096, 4096)])
def test_w8_no_split_is_spec_verify_gemm_w8(sv, dev, M, d_in, d_out):
    """No split planned (the streaming kernel at M <= 16; the tile kernel for
    gate/up at M = 320 and O at M = 20): bitwise spec_verify_gemm_w8."""
    import torch
    from synth import device as sd
    assert sv.gemm_w8_workspace_bytes(M, d_in, d_out) == 0
    w = sd.e4m3_normal_codes((d_out, d_in), synth.W8_CODE_STD, 3, dev)
    s = sd.w8_row_scales(d_out, synth.WEIGHT_STD / synth.W8_CODE_STD, 4, dev)
    x = sd.normal_bf16((M, d_in), 1.0, 5, dev)
    a = sv.verify_gemm_w8(x, w, s, out_dtype=torch.bfloat16)
    b = sv.verify_gemm_w8_ws(x, w, s, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_split_in_graph_replays(sv, dev):
    """The split path (tile kernel, then the split-sum kernel) captured in a
    HIP graph, as the step benchmark runs it: every replay, with eager work
    and synchronizations between them, equals the eager call bit for bit."""
    import torch
    from synth import device as sd
    M, d_in, d_out = 320, 14336, 4096
    assert splits(sv, M, d_in, d_out) >= 2
    x = sd.normal_bf16((M, d_in), 1.0, 61, dev)
    w = sd.normal_bf16((d_out, d_in), synth.WEIGHT_STD, 62, dev)
    ws = torch.empty(sv.gemm_workspace_bytes(M, d_in, d_out), dtype=torch.uint8, device=dev)
    eager = sv.verify_gemm_ws(x, w, out_dtype=torch.bfloat16, workspace=ws)
    torch.cuda.synchronize()
    y = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sv.verify_gemm_ws(x, w, out=y, workspace=ws)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        sv.verify_gemm_ws(x, w, out=y, workspace=ws)
    for r in range(4):
        y.fill_(0.0)
        ws.fill_(0xFF)  # the partials must be rewritten by every replay
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), f"replay {r}"
        # eager work between replays, on the same workspace
        sv.verify_gemm_ws(x[:80].contiguous(), w, out_dtype=torch.bfloat16, workspace=ws)
        torch.cuda.synchronize()
