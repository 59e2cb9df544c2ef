"""GPU tests of spec_verify_gemm_chain: the stack of linears in one launch.

Each linear of a chain must equal what spec_verify_gemm computes for it
(bitwise: same kernel arithmetic) and the fp64 oracle within the GEMM
tolerance. A chain whose linear i+1 reads linear i's output checks that the
device-side barrier orders the layers.
"""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def rel_err(y, ref):
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    return float(np.max(np.abs(y - ref) / np.maximum(np.abs(ref), rms)))


def make_linears(dev, M, shapes, seed, chained=False):
    import torch
    from synth import device as sd
    out, x = [], None
    for i, (d_in, d_out, dt) in enumerate(shapes):
        if x is None or not chained:
            x = sd.normal_bf16((M, d_in), 1.0, seed + 2 * i, dev)
        # chained layers keep activations O(1): w ~ N(0, 1/d_in)
        std = (1.0 / d_in) ** 0.5 if chained else synth.WEIGHT_STD
        w = sd.normal_bf16((d_out, d_in), std, seed + 2 * i + 1, dev)
        y = torch.empty((M, d_out), dtype=dt, device=dev)
        out.append((x, w, y))
        x = y
    return out


@pytest.mark.parametrize("M", [1, 5, 8, 16])
def test_chain_matches_single_launches(sv, dev, M):
    """A chain computes what single launches of the streaming kernel
    compute, bit for bit. A single launch with d_in a multiple of 64 runs the
    tile kernel instead (different summation order) above 8 positions, or on
    a linear of fewer than 2^26 weights; there the chain is held to the
    oracle."""
    import torch
    from synth import device as sd
    shapes = [(1032, 777, torch.bfloat16), (4096, 6144, torch.bfloat16), (8192, 256, torch.float32),
              (14336, 4096, torch.bfloat16), (264, 3000, torch.float32),
              (4096, 16400, torch.bfloat16)]
    lin = make_linears(dev, M, shapes, 100 + M)
    ch = sv.Chain(lin, dev)
    ch.run()
    torch.cuda.synchronize()
    assert ch.error() == 0
    for x, w, y in lin:
        d_in, d_out = x.shape[1], w.shape[0]
        if d_in % 64 != 0 or (M <= 8 and d_in * d_out >= 1 << 26):
            ref = sv.verify_gemm(x, w, out_dtype=y.dtype)
            torch.cuda.synchronize()
            assert torch.equal(ref, y)
        else:
            ref = oracle.linear(sd.to_bits(x), sd.to_bits(w))
            assert rel_err(y.float().cpu().numpy().astype(np.float64), ref) <= 2e-2


def test_chain_of_dependent_layers(sv, dev):
    """y_i feeds x_{i+1}. The oracle runs the same dependent chain on its
    own, from the seeded first input only: each layer in fp64, rounded to
    bf16 (nearest, ties to even) as the next layer's input. Every GPU layer
    must match it within the GEMM tolerance; a layer that read its input
    before the previous layer's output was complete and visible (the outputs
    are zeroed before every launch) would miss by far."""
    import torch
    from synth import device as sd
    M = 5
    dims = [4096, 6144, 4096, 14336, 4096, 4096, 1000]
    shapes = [(dims[i], dims[i + 1], torch.bfloat16) for i in range(len(dims) - 1)]
    lin = make_linears(dev, M, shapes, 7, chained=True)
    for i in range(1, len(lin)):
        assert lin[i][0].data_ptr() == lin[i - 1][2].data_ptr()
    refs, cur = [], sd.to_bits(lin[0][0])
    for _, w, _ in lin:
        r = oracle.linear(cur, sd.to_bits(w))
        refs.append(r)
        cur = oracle.to_bf16_bits(r)
    ch = sv.Chain(lin, dev)
    for _ in range(3):  # repeated launches reuse the counters (generations)
        for _, _, y in lin:
            y.zero_()
        ch.run()
        torch.cuda.synchronize()
        assert ch.error() == 0
        for i, ((_, _, y), ref) in enumerate(zip(lin, refs)):
            e = rel_err(y.float().cpu().numpy().astype(np.float64), ref)
            assert e <= 2e-2, (i, e)


def test_chain_oracle_llama_layer(sv, dev):
    import torch
    from synth import device as sd
    M = 5
    shapes = [(4096, 6144, torch.bfloat16), (4096, 4096, torch.bfloat16),
              (4096, 28672, torch.bfloat16), (14336, 4096, torch.bfloat16),
              (4096, 128256, torch.float32)]
    lin = make_linears(dev, M, shapes, 55)
    ch = sv.Chain(lin, dev)
    ch.run()
    torch.cuda.synchronize()
    assert ch.error() == 0
    rng = np.random.default_rng(0)
    for x, w, y in lin:
        cols = np.unique(np.concatenate([np.arange(4), np.arange(w.shape[0] - 4, w.shape[0]),
                                         rng.integers(0, w.shape[0], 64)]))
        idx = torch.from_numpy(cols).to(dev)
        ref = oracle.linear(sd.to_bits(x), sd.to_bits(w.index_select(0, idx)))
        got = y.index_select(1, idx).float().cpu().numpy().astype(np.float64)
        assert rel_err(got, ref) <= 2e-2


def test_chain_plan_mismatch_is_reported(sv, dev):
    import torch
    lin = make_linears(dev, 5, [(512, 256, torch.float32), (256, 128, torch.float32)], 3)
    ch = sv.Chain(lin, dev)
    for _, _, y in lin:
        y.fill_(7.0)
    sv.check(sv.lib.spec_verify_gemm_chain(2, 4, sv._ptr(ch.workspace), sv._stream()))
    torch.cuda.synchronize()
    assert ch.error() == 2
    assert all(bool((y == 7.0).all()) for _, _, y in lin)  # nothing computed
    ch.run()
    torch.cuda.synchronize()
    assert ch.error() == 0


def test_chain_graph_replay(sv, dev):
    import torch
    shapes = [(4096, 4096, torch.bfloat16), (4096, 6144, torch.bfloat16)]
    lin = make_linears(dev, 5, shapes, 9)
    ch = sv.Chain(lin, dev)
    ch.run()
    torch.cuda.synchronize()
    want = [y.clone() for _, _, y in lin]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ch.run()
    for _ in range(3):
        for _, _, y in lin:
            y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, y) for a, (_, _, y) in zip(want, lin))
    assert ch.error() == 0


@pytest.mark.parametrize("stack_name", ["LLAMA_8B", "LLAMA_70B_16L"])
def test_chain_full_stack_every_column(sv, dev, stack_name):
    """The whole stack in one chain launch, as the step benchmark runs it:
    every linear of every layer, then the fp32 lm-head, at M = 5 with the
    workload's weight distribution. Every output of every linear against
    the fp64 oracle (the weights are copied back one linear at a time)."""
    import time

    import torch
    from synth import device as sd
    stack = getattr(synth, stack_name)
    M = 5
    lin = []
    for i, (_, d_in, d_out) in enumerate(stack.all_linears()):
        last = i == len(stack.all_linears()) - 1
        x = sd.normal_bf16((M, d_in), 1.0, 9000 + 2 * i, dev)
        w = sd.normal_bf16((d_out, d_in), synth.WEIGHT_STD, 9001 + 2 * i, dev)
        y = torch.empty((M, d_out), dtype=torch.float32 if last else torch.bfloat16, device=dev)
        lin.append((x, w, y))
    ch = sv.Chain(lin, dev)
    for _ in range(2):  # a second launch reuses the counters (generations)
        ch.run()
        torch.cuda.synchronize()
        assert ch.error() == 0
    worst, outputs, t0 = 0.0, 0, time.time()
    for i, (x, w, y) in enumerate(lin):
        ref = oracle.linear(sd.to_bits(x), sd.to_bits(w))
        got = y.float().cpu().numpy().astype(np.float64)
        e = rel_err(got, ref)
        worst = max(worst, e)
        outputs += got.size
        assert e <= 2e-2, (i, e)
    print(f"{stack_name}: {len(lin)} linears, {outputs} outputs, worst rel err {worst:.2e} "
          f"(oracle {time.time() - t0:.1f} s)", flush=True)
    del lin, ch
    torch.cuda.empty_cache()


def _header(ch):
    """The chain workspace's 64-byte header as 16 int32 words: gen at word 0,
    exit count 1, error 2, magic 3, n 4, M 5, grid 6, spin limit 7."""
    import torch
    return ch.workspace[:64].view(torch.int32)


def _dependent_chain(sv, dev, seed):
    import torch
    from synth import device as sd
    M = 5
    dims = [4096, 4096, 6144, 1000]
    shapes = [(dims[i], dims[i + 1], torch.bfloat16) for i in range(len(dims) - 1)]
    lin = make_linears(dev, M, shapes, seed, chained=True)
    refs, cur = [], sd.to_bits(lin[0][0])
    for _, w, _ in lin:
        r = oracle.linear(cur, sd.to_bits(w))
        refs.append(r)
        cur = oracle.to_bf16_bits(r)
    return lin, refs


def _run_and_check(ch, lin, refs, what):
    import torch
    for _, _, y in lin:
        y.zero_()
    ch.run()
    torch.cuda.synchronize()
    assert ch.error() == 0, what
    for i, ((_, _, y), ref) in enumerate(zip(lin, refs)):
        e = rel_err(y.float().cpu().numpy().astype(np.float64), ref)
        assert e <= 2e-2, (what, i, e)


def test_chain_counters_across_the_32bit_wrap(sv, dev):
    """Every barrier counter is cumulative over launches and compared modulo
    2^32. Reset to a few launches before (launches * workgroups) wraps, and
    before the launch count itself wraps, then run dependent launches
    through both points: every barrier must release (no error) and every
    layer must match the oracle."""
    lin, refs = _dependent_chain(sv, dev, 21)
    ch = sv.Chain(lin, dev)
    G = int(_header(ch)[6])
    assert G >= 1
    for gen0 in ((1 << 32) // G - 2, (1 << 32) - 2):
        ch.reset(gen0)
        assert int(_header(ch)[0]) & 0xFFFFFFFF == gen0
        for k in range(4):
            _run_and_check(ch, lin, refs, f"G={G} gen0={gen0} launch {k}")
        assert (int(_header(ch)[0]) & 0xFFFFFFFF) == (gen0 + 4) & 0xFFFFFFFF


def test_chain_barrier_give_up_is_reported(sv, dev):
    """Forced from the host: the header claims more completed launches than
    the counters record, so no barrier of the next launch can release. With
    a spin limit of 64 polls every wait gives up, the launch still runs to
    its end, and bit 0 of the error word is set. A reset to the header's own
    count (and the default spin limit) makes the next launch correct."""
    import torch
    lin, refs = _dependent_chain(sv, dev, 23)
    ch = sv.Chain(lin, dev)
    hdr = _header(ch)
    default_limit = int(hdr[7])
    hdr[7] = 64
    hdr[0] = 5
    torch.cuda.synchronize()
    ch.run()
    torch.cuda.synchronize()
    assert ch.error() & 1
    # the same, reported by the binding's checked launch
    ch.reset(5)
    hdr[7] = 64
    hdr[0] = 9
    torch.cuda.synchronize()
    with pytest.raises(RuntimeError, match="error word 1"):
        ch.run(check_error=True)
    hdr[7] = default_limit
    ch.reset(5)
    _run_and_check(ch, lin, refs, "after reset")
    ch.run(check_error=True)
