"""The split plans of the benchmarked linears, pinned (no GPU: the plan
depends on the shape only and the workspace-size calls make no device call).

The numbers are the reduction splits spec_verify_gemm_ws and
spec_verify_gemm_w8_ws take for the Llama-3.1-8B linears at the batch
sweep's M = B (K + 1), K = 4. Each plan was chosen by the library's time
models and checked against forced alternatives on MI355X; a change to the
models or the tile tables that moves any of them should be measured again
before this table is updated.
"""

import ctypes

import pytest

LINEARS = [(4096, 6144), (4096, 4096), (4096, 28672), (14336, 4096), (4096, 128256)]
# M -> splits for QKV, O, gate/up, down, lm-head (0: no split)
BF16 = {5: [0, 0, 0, 4, 0], 20: [0, 0, 0, 4, 0], 80: [0, 0, 0, 8, 0],
        320: [0, 0, 0, 8, 0], 1280: [0, 0, 0, 4, 0]}
FP8 = {5: [0, 0, 0, 0, 0], 20: [0, 0, 0, 8, 0], 80: [5, 0, 2, 16, 0],
       320: [0, 3, 0, 8, 0], 1280: [0, 2, 0, 4, 0]}


def splits(fn, M, d_in, d_out):
    return fn(M, d_in, d_out) // (M * d_out * 4)


@pytest.mark.parametrize("w8", [False, True])
def test_split_plans_of_the_sweep(sv, w8):
    fn = sv.lib.spec_verify_gemm_w8_workspace_bytes if w8 else sv.lib.spec_verify_gemm_workspace_bytes
    want = FP8 if w8 else BF16
    got = {M: [splits(fn, M, d_in, d_out) for d_in, d_out in LINEARS] for M in want}
    assert got == want


def test_workspace_is_whole_splits(sv):
    """A plan's workspace is exactly S x M x d_out fp32 partials."""
    for fn in (sv.lib.spec_verify_gemm_workspace_bytes, sv.lib.spec_verify_gemm_w8_workspace_bytes):
        for M in (20, 80, 320, 1280):
            for d_in, d_out in LINEARS:
                n = fn(M, d_in, d_out)
                assert n % (M * d_out * 4) == 0
                assert ctypes.c_size_t(n).value == n
