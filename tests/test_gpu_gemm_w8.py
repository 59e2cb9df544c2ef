"""GPU parity of the weight-only FP8 verify linear (spec_verify_gemm_w8 and
the FP8 chain) against the fp64 oracle (oracle.linear_w8): the streaming
kernel up to 16 positions, the MFMA tile kernel above.

Weights are FP8 E4M3 codes with one float32 scale per output row,
activations bf16 ("Speculative Decoding: The Algebra and the Proof", Where it
breaks: weight-only 8-bit storage with BF16 compute). Every E4M3 value is
exact in bf16 and every product exact in fp32, so the GPU result differs from
the fp64 oracle only by fp32 accumulation and the final scaling: the same
tolerances as the bf16 linear (2e-2, and 1e-3 for fp32 outputs), and
bit-exact where a single product is summed.
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


def host_inputs(seed, M, d_in, d_out):
    x = synth.bf16_normal_bits(seed, "w8.x", (M, d_in))
    w = synth.e4m3_normal_codes(seed, "w8.w", (d_out, d_in))
    s = synth.w8_row_scales(seed, "w8.s", d_out)
    return x, w, s


def run(sv, dev, x_bits, codes, scale, out_dtype):
    import torch
    from synth import device as sd
    x = sd.from_bits(x_bits, dev)
    w = torch.from_numpy(np.ascontiguousarray(codes)).to(dev)
    s = torch.from_numpy(np.ascontiguousarray(scale)).to(dev)
    y = sv.verify_gemm_w8(x, w, s, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def check(y, ref, f32, what):
    e = rel_err(y, ref)
    print(f"{what}: rel err {e:.3e}", flush=True)
    assert e <= TOL, what
    if f32:
        assert e <= TOL_F32, what


@pytest.mark.parametrize("M", list(range(1, 17)))
@pytest.mark.parametrize("d_in,d_out", [(1040, 777), (9008, 300), (1024, 1024), (528, 4104)])
def test_w8_every_m(sv, dev, M, d_in, d_out):
    """Every M of the streaming kernel; ragged reduction (d_in not a multiple
    of a stage), several activation chunks at larger M (9008), ragged row
    blocks (777, 300) and more row blocks than workgroups (4104)."""
    import torch
    x, w, s = host_inputs(M * 7 + d_in, M, d_in, d_out)
    y = run(sv, dev, x, w, s, torch.float32)
    check(y, oracle.linear_w8(x, w, s), True, f"w8 M={M} {d_in}->{d_out}")


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M", [5, 16])
def test_w8_output_dtypes(sv, dev, out, M):
    import torch
    dt = torch.float32 if out == "f32" else torch.bfloat16
    x, w, s = host_inputs(31 + M, M, 4096, 1536)
    y = run(sv, dev, x, w, s, dt)
    check(y, oracle.linear_w8(x, w, s), out == "f32", f"w8 out={out} M={M}")


def test_w8_special_codes_one_hot_exact(sv, dev):
    """One-hot activations select single products: y = fp32(scale * e4m3),
    bit-exact, over every finite code (subnormals, +-448, +-0)."""
    import torch
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)  # 254
    d_in, d_out = 256, len(codes)
    rng = np.random.default_rng(3)
    w = np.zeros((d_out, d_in), dtype=np.uint8)
    cols = rng.permutation(d_in)[:16]
    for j, k in enumerate(cols):
        w[:, k] = np.roll(codes, 17 * j)
    s = synth.w8_row_scales(4, "w8.special", d_out)
    x = np.zeros((16, d_in), dtype=np.uint16)
    x[np.arange(16), cols] = 0x3F80  # 1.0
    y = run(sv, dev, x, w, s, torch.float32)
    want = (oracle.e4m3_to_f64(w[:, cols].T) * s.astype(np.float64)[None, :]).astype(np.float32)
    assert np.array_equal(y.astype(np.float32), want)


LLAMA8B = [(4096, 6144), (4096, 4096), (4096, 28672), (14336, 4096), (4096, 128256)]


# Above 16 positions the tile kernel: one case per FP8 tile form the
# dispatcher can pick -- 256x256, 128x256, 128x128, 64x128, 64x64 in two
# k-groups, 64x32 in four; 32x32 in one round (eight waves, four k-groups)
# and in several (four waves, two); 32x16 (eight waves, eight k-groups);
# 32x64 in one round (eight waves, two k-groups) and in several (four
# waves); 320x128 and 320x256 -- with ragged M and N tails, d_in of one
# stage (64 or 128: some k-groups get no k-tile) up to many. Where d_in is
# a multiple of 128, 128x256, 128x128, 64x64, 64x32, 32x16 and the
# one-round 32x32 and 32x64 run with 128-element stages; each of those
# shapes appears here with such a d_in and with one that is not. The
# 320-row tiles, and 64x128 and 128x128 from M = 256, widen each stage's
# codes once per workgroup in LDS: each of those appears with d_in a
# multiple of 128 and not.
W8_TILE_CASES = [(513, 256, 16400), (200, 192, 16400), (130, 384, 24000), (513, 1024, 4104),
                 (300, 192, 8200), (80, 320, 16400), (80, 256, 16400), (33, 128, 16400),
                 (1280, 320, 777), (301, 256, 6150), (130, 64, 4095), (47, 640, 8200),
                 (611, 128, 792), (611, 192, 792), (17, 1024, 4104), (20, 192, 6150),
                 (193, 128, 2334), (20, 4096, 777), (17, 320, 1000), (20, 256, 12288),
                 (20, 192, 12300), (17, 512, 16400), (301, 192, 24000), (257, 128, 24000),
                 (301, 64, 60000), (513, 128, 60000),
                 # 320x256 over two to four rounds, split by columns: the
                 # rest on 320x192 tiles (whose 52 load instructions per
                 # stage leave four spare ones for the eight waves)
                 (1250, 64, 28000), (1900, 128, 28000), (1280, 64, 57344),
                 # the forms that store through the LDS staging block
                 # (256x256, 128x256 with 64- and 128-element stages, the
                 # widen-once 320x128 and 320x256, the column split) with
                 # d_out not a multiple of 8
                 (480, 64, 28675), (1280, 64, 6147), (1280, 128, 6147), (301, 64, 24001),
                 (640, 64, 28675), (1250, 64, 28003)]


@pytest.mark.parametrize("M,d_in,d_out", W8_TILE_CASES)
def test_w8_tile_kernel(sv, dev, M, d_in, d_out):
    import torch
    x, w, s = host_inputs(M + 3 * d_in + d_out, M, d_in, d_out)
    ref = oracle.linear_w8(x, w, s)
    for od in (torch.float32, torch.bfloat16):
        y = run(sv, dev, x, w, s, od)
        check(y, ref, od == torch.float32, f"w8 tile M={M} {d_in}->{d_out} {od}")


@pytest.mark.parametrize("M,d_in", [(32, 256), (320, 512)])
def test_w8_tile_special_codes_one_hot_exact(sv, dev, M, d_in):
    """As the one-hot test below, through the tile kernel: every finite code
    times its row scale, bit-exact -- with the codes widened per wave at
    every fragment read (M = 32) and once per workgroup in LDS (M = 320, a
    320-row tile)."""
    import torch
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    d_out = len(codes)
    rng = np.random.default_rng(5)
    w = np.zeros((d_out, d_in), dtype=np.uint8)
    cols = rng.permutation(d_in)[:M]
    for j, k in enumerate(cols):
        w[:, k] = np.roll(codes, 11 * j)
    s = synth.w8_row_scales(6, "w8.special.tile", d_out)
    x = np.zeros((M, d_in), dtype=np.uint16)
    x[np.arange(M), cols] = 0x3F80  # 1.0
    y = run(sv, dev, x, w, s, torch.float32)
    want = (oracle.e4m3_to_f64(w[:, cols].T) * s.astype(np.float64)[None, :]).astype(np.float32)
    assert np.array_equal(y.astype(np.float32), want)


@pytest.mark.parametrize("M", [20, 80, 320, 1280])
@pytest.mark.parametrize("d_in,d_out", LLAMA8B)
def test_w8_batch_sweep_shapes(sv, dev, M, d_in, d_out):
    """The Llama-3.1-8B linears with FP8 weights at every swept batch (B = 4,
    16, 64, 256 at K = 4), as the FP8 batch sweep runs them; the oracle
    checks sampled output columns (first and last 8 plus random ones)."""
    import torch
    from synth import device as sd
    seed = 41 * M + d_out
    w = sd.e4m3_normal_codes((d_out, d_in), synth.W8_CODE_STD, seed, dev)
    s = sd.w8_row_scales(d_out, synth.WEIGHT_STD / synth.W8_CODE_STD, seed + 1, dev)
    x = sd.normal_bf16((M, d_in), 1.0, seed + 2, dev)
    od = torch.float32 if d_out == 128256 else torch.bfloat16
    y = sv.verify_gemm_w8(x, w, s, out_dtype=od)
    rng = np.random.default_rng(seed)
    cols = np.unique(np.concatenate([np.arange(8), np.arange(d_out - 8, d_out),
                                     rng.integers(0, d_out, 48)]))
    idx = torch.from_numpy(cols).to(dev)
    ref = oracle.linear_w8(sd.to_bits(x), w.index_select(0, idx).cpu().numpy(),
                           s.index_select(0, idx).cpu().numpy())
    got = y.index_select(1, idx).float().cpu().numpy().astype(np.float64)
    check(got, ref, od == torch.float32, f"w8 sweep M={M} {d_in}->{d_out}")
    del w, y
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M", [20, 320])
def test_w8_tile_deterministic(sv, dev, M):
    import torch
    from synth import device as sd
    w = sd.e4m3_normal_codes((6144, 4096), synth.W8_CODE_STD, 5, dev)
    s = sd.w8_row_scales(6144, synth.WEIGHT_STD / synth.W8_CODE_STD, 6, dev)
    x = sd.normal_bf16((M, 4096), 1.0, 7, dev)
    a = sv.verify_gemm_w8(x, w, s)
    b = sv.verify_gemm_w8(x, w, s)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("d_in,d_out", LLAMA8B)
def test_w8_llama8b_shapes_sampled_rows(sv, dev, d_in, d_out):
    """Full Llama-8B-shaped linears at M = 5 (the launch the FP8 chain runs
    per linear); the oracle checks 96 sampled output columns, including the
    first and last row blocks."""
    import torch
    from synth import device as sd
    M = 5
    w = sd.e4m3_normal_codes((d_out, d_in), synth.W8_CODE_STD, 900 + d_out, dev)
    s = sd.w8_row_scales(d_out, synth.WEIGHT_STD / synth.W8_CODE_STD, 901 + d_out, dev)
    x = sd.normal_bf16((M, d_in), 1.0, 902 + d_out, dev)
    y = sv.verify_gemm_w8(x, w, s, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(d_out)
    rows = np.unique(np.concatenate([[0, 1, 15, 16, d_out - 17, d_out - 1],
                                     rng.integers(0, d_out, 90)]))
    ref = oracle.linear_w8(sd.to_bits(x), w[rows].cpu().numpy(), s[rows].cpu().numpy())
    got = y[:, rows].cpu().numpy().astype(np.float64)
    check(got, ref, True, f"w8 8B {d_in}->{d_out}")
    del w
    torch.cuda.empty_cache()


def _w8_chain_linears(dev, M, shapes, seed):
    import torch
    from synth import device as sd
    out = []
    for i, (d_in, d_out, dt) in enumerate(shapes):
        x = sd.normal_bf16((M, d_in), 1.0, seed + 3 * i, dev)
        w = sd.e4m3_normal_codes((d_out, d_in), synth.W8_CODE_STD, seed + 3 * i + 1, dev)
        s = sd.w8_row_scales(d_out, synth.WEIGHT_STD / synth.W8_CODE_STD, seed + 3 * i + 2, dev)
        y = torch.empty((M, d_out), dtype=dt, device=dev)
        out.append((x, w, s, y))
    return out


@pytest.mark.parametrize("M", [1, 5, 16])
def test_w8_chain_matches_single_launches(sv, dev, M):
    import torch
    shapes = [(1040, 777, torch.bfloat16), (4096, 6144, torch.bfloat16),
              (8192, 256, torch.float32), (14336, 4096, torch.bfloat16),
              (272, 3000, torch.float32)]
    lin = _w8_chain_linears(dev, M, shapes, 300 + M)
    ch = sv.Chain(lin, dev)
    ch.run()
    torch.cuda.synchronize()
    assert ch.error() == 0
    for x, w, s, y in lin:
        ref = sv.verify_gemm_w8(x, w, s, out_dtype=y.dtype)
        torch.cuda.synchronize()
        assert torch.equal(ref, y)
    # and the oracle on the first linear
    x, w, s, y = lin[0]
    from synth import device as sd
    ref = oracle.linear_w8(sd.to_bits(x), w.cpu().numpy(), s.cpu().numpy())
    check(y.float().cpu().numpy().astype(np.float64), ref, False, f"w8 chain M={M}")


def test_w8_chain_plan_mismatch_is_reported(sv, dev):
    """A workspace prepared for an FP8 chain, run as a bf16 chain (and the
    reverse), computes nothing and reports bit 1."""
    import torch
    lin8 = _w8_chain_linears(dev, 5, [(1024, 512, torch.float32)], 77)
    ch8 = sv.Chain(lin8, dev)
    lin8[0][3].fill_(7.0)
    assert sv.lib.spec_verify_gemm_chain(1, 5, ch8.workspace.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert ch8.error() == 2
    assert bool((lin8[0][3] == 7.0).all())
    from synth import device as sd
    x = sd.normal_bf16((5, 1024), 1.0, 78, dev)
    w = sd.normal_bf16((512, 1024), 0.02, 79, dev)
    y = torch.full((5, 512), 7.0, dtype=torch.float32, device=dev)
    ch = sv.Chain([(x, w, y)], dev)
    assert sv.lib.spec_verify_gemm_chain_w8(1, 5, ch.workspace.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert ch.error() == 2
    assert bool((y == 7.0).all())


def test_w8_chain_full_8b_stack_sampled(sv, dev):
    """The whole Llama-8B-shaped stack with FP8 weights in one chain launch,
    as the FP8 step benchmark runs it (every linear, then the fp32 lm-head,
    M = 5); the oracle checks 32 sampled output columns of every linear."""
    import torch
    stack = synth.LLAMA_8B
    shapes = [(d_in, d_out, torch.bfloat16) for _, d_in, d_out in stack.all_linears()]
    shapes[-1] = (shapes[-1][0], shapes[-1][1], torch.float32)
    lin = _w8_chain_linears(dev, 5, shapes, 7000)
    ch = sv.Chain(lin, dev)
    ch.run()
    torch.cuda.synchronize()
    assert ch.error() == 0
    from synth import device as sd
    rng = np.random.default_rng(2)
    worst = 0.0
    for i, (x, w, s, y) in enumerate(lin):
        n = w.shape[0]
        rows = np.unique(np.concatenate([np.arange(4), np.arange(n - 4, n), rng.integers(0, n, 24)]))
        idx = torch.from_numpy(rows).to(dev)
        ref = oracle.linear_w8(sd.to_bits(x), w.index_select(0, idx).cpu().numpy(),
                               s.index_select(0, idx).cpu().numpy())
        got = y.index_select(1, idx).float().cpu().numpy().astype(np.float64)
        e = rel_err(got, ref)
        worst = max(worst, e)
        assert e <= TOL, (i, e)
    print(f"w8 8B stack: {len(lin)} linears, worst sampled rel err {worst:.2e}", flush=True)
    del lin, ch
    torch.cuda.empty_cache()
