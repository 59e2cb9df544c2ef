"""GPU parity of spec_verify_gemm against the fp64 oracle.

Tolerance: max |y - y_ref| / max(|y_ref|, rms of the reference row) <= 2e-2
(bf16 inputs, fp32 accumulation). fp32 outputs must also meet 1e-3, a bound
derived from fp32 accumulation (a few d_in^(1/2) * 2^-24 of the row scale);
a dropped segment of the reduction (1/32 of d_in) would miss it by far.
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


def run_host(sv, dev, x_bits, w_bits, out_dtype):
    import torch
    from synth import device as sd
    x = sd.from_bits(x_bits, dev)
    w = sd.from_bits(w_bits, dev)
    y = sv.verify_gemm(x, w, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def check(y, ref, out_dtype, what):
    import torch
    e = rel_err(y, ref)
    print(f"{what}: rel err {e:.3e}", flush=True)
    assert e <= TOL, what
    if out_dtype == torch.float32:
        assert e <= TOL_F32, what


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_tiny_linear(sv, dev, out):
    import torch
    d = synth.tiny(1)
    od = torch.float32 if out == "f32" else torch.bfloat16
    y = run_host(sv, dev, d["x_bits"], d["w_bits"], od)
    check(y, oracle.linear(d["x_bits"], d["w_bits"]), od, f"tiny {out}")


# ragged d_in (not a multiple of the 128-element segment) and d_out (not a
# multiple of the rows per workgroup); 9000 spans several activation chunks
# at the larger M. d_out 1024 (whole 16-row blocks) and 4104 (24 rows per
# workgroup: a whole and a half block) take the 8-outputs-per-store path,
# 777 and 300 (not multiples of 8) the one-output-per-store path.
@pytest.mark.parametrize("M", list(range(1, 17)))
@pytest.mark.parametrize("d_in,d_out", [(1032, 777), (9000, 300), (1032, 1024), (520, 4104)])
def test_stream_kernel_every_m(sv, dev, M, d_in, d_out):
    import torch
    x, w = synth.linear_inputs(100 + M, f"stream{d_in}", M, d_in, d_out)
    y = run_host(sv, dev, x, w, torch.float32)
    check(y, oracle.linear(x, w), torch.float32, f"stream M={M} {d_in}->{d_out}")


# 17..128 positions: the weight-streaming MFMA kernel. d_in = 1032 leaves a
# ragged 64-element segment, d_out = 777 a partial 16-row tile; every count
# of 16-row position tiles (2..8) and partial position tiles are covered.
@pytest.mark.parametrize("M", [17, 20, 31, 32, 33, 48, 63, 64, 65, 80, 96, 97, 112, 127, 128])
def test_skinny_kernel(sv, dev, M):
    import torch
    x, w = synth.linear_inputs(300 + M, "skinny", M, 1032, 777)
    for od in (torch.float32, torch.bfloat16):
        y = run_host(sv, dev, x, w, od)
        check(y, oracle.linear(x, w), od, f"skinny M={M} {od}")


# d_out >= 16384 switches to two 16-row weight tiles per workgroup; 16400
# ends in a partial tile, d_in = 520 in a partial segment.
@pytest.mark.parametrize("M", [17, 40, 64])
def test_skinny_kernel_wide(sv, dev, M):
    import torch
    x, w = synth.linear_inputs(400 + M, "skinny_wide", M, 520, 16400)
    y = run_host(sv, dev, x, w, torch.float32)
    check(y, oracle.linear(x, w), torch.float32, f"skinny wide M={M}")


@pytest.mark.parametrize("M", [17, 20, 33, 64, 80, 130, 320])
def test_mfma_kernel(sv, dev, M):
    import torch
    x, w = synth.linear_inputs(200 + M, "mfma", M, 1032, 777)
    for od in (torch.float32, torch.bfloat16):
        y = run_host(sv, dev, x, w, od)
        check(y, oracle.linear(x, w), od, f"mfma M={M} {od}")


@pytest.mark.parametrize("M,d_in,d_out", [(9, 512, 4095), (16, 256, 28672), (17, 512, 4095),
                                           (20, 4096, 4096), (20, 256, 28672),
                                           (31, 128, 20000), (47, 256, 5000),
                                           (65, 512, 4097), (129, 64, 777), (200, 1024, 777),
                                           (256, 512, 4112), (320, 1024, 300), (513, 128, 1000),
                                           (1280, 1024, 777), (301, 256, 24000),
                                           (640, 192, 28672), (1250, 64, 28000),
                                           (1900, 128, 28600), (1100, 64, 57344),
                                           (480, 64, 28675), (1280, 64, 6147), (80, 64, 50001),
                                           (301, 64, 24001), (640, 64, 28675), (1250, 64, 28003),
                                           (1250, 64, 28004), (300, 128, 4095), (1250, 64, 4095),
                                           (320, 192, 4096), (1280, 128, 4096), (300, 64, 28600),
                                           (320, 128, 28672), (1250, 64, 6100),
                                           (100, 64, 6143), (128, 128, 6144)])
def test_tile_kernel(sv, dev, M, d_in, d_out):
    """The pipelined tile kernel (d_in a multiple of 64, M above 8): ragged
    M and N tails, one or many stages (d_in 64 leaves k-groups without a
    k-tile), the two-, four- and eight-wave tile shapes the dispatcher picks
    (32x16, 32x32, 32x64, 64x32, 64x64, 128x64), with and without k-groups,
    the 320x128 tile (M = 301: a ragged 320-row tile; M = 640: two), and
    320x256 tiles split over two launches by columns, the rest on 320x192
    tiles (M = 1250, 1900, 1100: ragged rows, a ragged last column tile of
    either launch, two to four rounds). The tiles that store through the
    LDS staging block (256x256, 256x128, 128x256, 320x128, 320x256 and the
    column split: M = 480, 1280, 80, 301, 640, 1250 with d_out not a
    multiple of 8) also meet output rows whose 16-byte stores do not line
    up, stored element by element (d_out = 28004: bf16 rows element by
    element, fp32 rows in 16-byte stores). The exact-fill tiles, taken where
    their tiles number one per CU: 80x64 in two k-groups of five waves (M =
    300, 320 with d_out = 4095, 4096), 160x128 (M = 1250, 1280), 160x224
    on fourteen waves (M = 300, 320 with d_out = 28600, 28672), 160x192
    (M = 1250, d_out = 6100) and 64x48 in two k-groups of four waves (M =
    100, 128 with d_out = 6143, 6144)."""
    import torch
    x, w = synth.linear_inputs(300 + M, f"tile{d_in}.{d_out}", M, d_in, d_out)
    ref = oracle.linear(x, w)
    for od in (torch.float32, torch.bfloat16):
        y = run_host(sv, dev, x, w, od)
        check(y, ref, od, f"tile M={M} {d_in}->{d_out} {od}")


def test_edge_shapes(sv, dev):
    import torch
    for M, d_in, d_out in [(1, 8, 1), (5, 8, 3), (16, 16, 1), (17, 8, 1), (2, 2048 + 8, 65)]:
        x, w = synth.linear_inputs(7, f"edge{M}.{d_in}.{d_out}", M, d_in, d_out)
        y = run_host(sv, dev, x, w, torch.float32)
        check(y, oracle.linear(x, w), torch.float32, f"edge {M}x{d_in}->{d_out}")


def sampled_full_size(sv, dev, M, d_in, d_out, seed, out_dtype, n_rows=48):
    """Full-size linear on the device; the oracle checks a sample of output
    columns (first and last 8 plus random ones)."""
    import torch
    from synth import device as sd
    w = sd.normal_bf16((d_out, d_in), synth.WEIGHT_STD, seed, dev)
    x = sd.normal_bf16((M, d_in), 1.0, seed + 1, dev)
    y = sv.verify_gemm(x, w, out_dtype=out_dtype)
    rng = np.random.default_rng(seed)
    cols = np.unique(np.concatenate([np.arange(8), np.arange(d_out - 8, d_out),
                                     rng.integers(0, d_out, n_rows)]))
    idx = torch.from_numpy(cols).to(dev)
    w_rows = sd.to_bits(w.index_select(0, idx))
    x_bits = sd.to_bits(x)
    y_s = y.index_select(1, idx).float().cpu().numpy().astype(np.float64)
    del w, y
    torch.cuda.empty_cache()
    return y_s, oracle.linear(x_bits, w_rows)


LLAMA8B = [(4096, 6144), (4096, 4096), (4096, 28672), (14336, 4096)]
LLAMA70B = [(8192, 10240), (8192, 8192), (8192, 57344), (28672, 8192)]


@pytest.mark.parametrize("d_in,d_out", LLAMA8B + LLAMA70B)
def test_full_size_stack_linears_m5(sv, dev, d_in, d_out):
    import torch
    y, ref = sampled_full_size(sv, dev, 5, d_in, d_out, d_in + d_out, torch.bfloat16)
    check(y, ref, torch.bfloat16, f"M=5 {d_in}->{d_out} bf16")


@pytest.mark.parametrize("d_in", [4096, 8192])
def test_full_size_lm_head_m5(sv, dev, d_in):
    import torch
    y, ref = sampled_full_size(sv, dev, 5, d_in, 128256, 77 + d_in, torch.float32, n_rows=200)
    check(y, ref, torch.float32, f"lm-head {d_in}->128256")


# The batch sweep of the Llama-3.1-8B shapes (B = 4, 16, 64, 256 at K = 4):
# every linear at every swept M, so every tile instantiation the dispatcher
# picks for that workload (64x128 for QKV at M = 320, 128x256 for the
# lm-head at M = 80, the k-group small tiles at M = 20 and 80, ...) is held
# to the oracle, in the output type the step uses and in the other one.
SWEEP_M = [20, 80, 320, 1280]
SWEEP_LINEARS = LLAMA8B + [(4096, 128256)]


@pytest.mark.parametrize("M", SWEEP_M)
@pytest.mark.parametrize("d_in,d_out", SWEEP_LINEARS)
def test_batch_sweep_shapes(sv, dev, M, d_in, d_out):
    import torch
    step_dtype = torch.float32 if d_out == 128256 else torch.bfloat16
    for od in (step_dtype, torch.bfloat16 if step_dtype == torch.float32 else torch.float32):
        y, ref = sampled_full_size(sv, dev, M, d_in, d_out, 31 * M + d_in + d_out, od)
        check(y, ref, od, f"sweep M={M} {d_in}->{d_out} {od}")


@pytest.mark.parametrize("M,d_out", [(5, 6144), (5, 16400), (80, 6144), (320, 6144)])
def test_deterministic(sv, dev, M, d_out):
    """Two launches give bitwise equal outputs: the tile kernel with and
    without k-groups (M = 5, 80, 320 on a 6144-row linear) and the streaming
    kernel (M = 5 on a linear of 2^26 weights or more)."""
    import torch
    from synth import device as sd
    w = sd.normal_bf16((d_out, 4096), 0.02, 3, dev)
    x = sd.normal_bf16((M, 4096), 1.0, 4, dev)
    a = sv.verify_gemm(x, w)
    b = sv.verify_gemm(x, w)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("loads", [1, 2, 4, 8])
def test_read_probes_run(sv, dev, loads):
    """The read probes (into registers, and straight to LDS) sweep a buffer
    with a ragged tail (not a whole number of grid sweeps) and write nothing:
    the sink keeps its value, and the buffer is unchanged."""
    import torch
    n = (48 << 20) + 16 * 37
    buf = torch.arange(n // 4, dtype=torch.int32, device=dev)
    sink = torch.full((4,), 7, dtype=torch.int32, device=dev)
    sv.probe_read(buf, sink, loads, 1)
    sv.probe_read_lds(buf, sink, loads)
    torch.cuda.synchronize()
    assert torch.equal(sink.cpu(), torch.full((4,), 7, dtype=torch.int32))
    assert torch.equal(buf[-5:].cpu(), torch.arange(n // 4 - 5, n // 4, dtype=torch.int32))
