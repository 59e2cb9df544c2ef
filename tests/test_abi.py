"""The C-ABI library loads, exports every call include/spec_verify.h
declares, and rejects bad arguments before any HIP call (CPU only: no call
here reaches the device)."""

import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "spec_verify.h")

A = 0x10000          # a 256-byte aligned stand-in address; never dereferenced
MIS = 0x10001        # misaligned stand-in


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported(sv):
    names = declared_functions()
    assert len(names) == 28
    for n in names:
        assert hasattr(sv.lib, n), n


def test_binding_covers_exactly_the_header(sv):
    assert sorted(sv.SIGNATURES) == declared_functions()


def test_version_and_status_strings(sv):
    assert sv.abi_version() == 8
    for code, name in [(0, b"SPEC_OK"), (-1, b"SPEC_ERR_INVALID_ARGUMENT"),
                       (-2, b"SPEC_ERR_ALIGNMENT"), (-3, b"SPEC_ERR_UNSUPPORTED"),
                       (-4, b"SPEC_ERR_WORKSPACE"), (-5, b"SPEC_ERR_HIP")]:
        assert sv.lib.spec_status_string(code) == name


GEMM_BAD = [
    ((None, A, A, 0, 5, 4096, 4096), -1),
    ((A, None, A, 0, 5, 4096, 4096), -1),
    ((A, A, None, 0, 5, 4096, 4096), -1),
    ((A, A, A, 7, 5, 4096, 4096), -1),
    ((A, A, A, 0, 0, 4096, 4096), -1),
    ((A, A, A, 0, 65537, 4096, 4096), -1),
    ((A, A, A, 0, 5, 4100, 4096), -1),
    ((A, A, A, 0, 5, 0, 4096), -1),
    ((A, A, A, 0, 5, (1 << 20) + 8, 4096), -1),
    ((A, A, A, 0, 5, 4096, 0), -1),
    ((A, A, A, 0, 5, 4096, (1 << 24) + 1), -1),
    ((A + 8, A, A, 0, 5, 4096, 4096), -2),
    ((A, A + 8, A, 0, 5, 4096, 4096), -2),
    ((A, A, A + 2, 0, 5, 4096, 4096), -2),
    ((A, A, MIS, 1, 5, 4096, 4096), -2),
]


@pytest.mark.parametrize("args,code", GEMM_BAD)
def test_gemm_rejects(sv, args, code):
    assert sv.lib.spec_verify_gemm(*args, None) == code
    assert sv.lib.spec_last_error()


@pytest.mark.parametrize("args,code", GEMM_BAD)
def test_gemm_ws_rejects_as_gemm(sv, args, code):
    assert sv.lib.spec_verify_gemm_ws(*args, A, 1 << 30, None) == code
    assert sv.lib.spec_last_error()


def test_gemm_workspace_bytes(sv):
    f = sv.lib.spec_verify_gemm_workspace_bytes
    # out of range, or d_in not a multiple of 64: no split
    assert f(0, 14336, 4096) == 0 and f(65537, 14336, 4096) == 0
    assert f(320, 14336 + 8, 4096) == 0 and f(320, 14336, 0) == 0
    # the streaming kernel's shapes (M <= 8 on 2^26 weights or more): no split
    assert f(5, 8192, 57344) == 0
    # the 14336 -> 4096 down projection splits at every batch of the sweep,
    # into whole fp32 copies of the output, at most 16
    for M in (20, 80, 320, 1280):
        n = f(M, 14336, 4096)
        assert n > 0 and n % (M * 4096 * 4) == 0 and 2 <= n // (M * 4096 * 4) <= 16
    # the gate/up projection (d_in 4096 into 28672) never does
    for M in (20, 80, 320, 1280):
        assert f(M, 4096, 28672) == 0


def test_gemm_ws_rejects_workspace(sv):
    f = sv.lib.spec_verify_gemm_ws
    need = sv.lib.spec_verify_gemm_workspace_bytes(320, 14336, 4096)
    assert need > 0
    # checked before any device call
    assert f(A, A, A, 1, 320, 14336, 4096, None, need, None) == -4
    assert f(A, A, A, 1, 320, 14336, 4096, A, need - 1, None) == -4
    assert b"smaller" in sv.lib.spec_last_error()
    assert f(A, A, A, 1, 320, 14336, 4096, A + 8, need, None) == -4
    assert b"aligned" in sv.lib.spec_last_error()


def test_softmax_rejects(sv):
    f = sv.lib.spec_softmax
    assert f(None, 1, 10, A, A, A, None) == -1
    assert f(A, 0, 10, A, A, A, None) == -1
    assert f(A, 1, 0, A, A, A, None) == -1
    assert f(A, 1, (1 << 26) + 1, A, A, A, None) == -1
    assert f(MIS, 1, 10, A, A, A, None) == -2
    assert f(A, 1, 10, MIS, None, None, None) == -2
    # nothing requested: a no-op that succeeds without touching the device
    assert f(A, 3, 10, None, None, None, None) == 0


@pytest.mark.parametrize("B,K,V,code", [(0, 4, 10, -1), (1, 0, 10, -1), (1, 65, 10, -1),
                                        (1, 4, 0, -1), ((1 << 20) + 1, 4, 10, -1)])
def test_accept_and_sample_reject_sizes(sv, B, K, V, code):
    assert sv.lib.spec_accept_scan(A, A, A, A, B, K, V, A, None, None) == code
    assert sv.lib.spec_residual_sample(A, A, A, A, B, K, V, A, None, None) == code


def test_accept_and_sample_reject_pointers(sv):
    assert sv.lib.spec_accept_scan(A, A, None, A, 1, 4, 10, A, None, None) == -1
    assert sv.lib.spec_accept_scan(A, A, A, A, 1, 4, 10, None, None, None) == -1
    assert sv.lib.spec_accept_scan(A, MIS, A, A, 1, 4, 10, A, None, None) == -2
    assert sv.lib.spec_residual_sample(A, A, None, A, 1, 4, 10, A, None, None) == -1
    assert sv.lib.spec_residual_sample(A, A, A, A, 1, 4, 10, None, None, None) == -1
    assert sv.lib.spec_residual_sample(A, A, A, MIS, 1, 4, 10, A, None, None) == -2


def test_workspace_bytes(sv):
    f = sv.lib.spec_verify_workspace_bytes
    assert f(0, 4, 10) == 0 and f(1, 0, 10) == 0 and f(1, 65, 10) == 0 and f(1, 4, 0) == 0
    a, b = f(1, 4, 128256), f(64, 8, 128256)
    assert 0 < a < b and a % 256 == 0 and b % 256 == 0


def _verify(sv, hidden=None, lm=None, d=0, B=1, K=4, V=1000, ws=A, wsb=None, tl=A):
    if wsb is None:
        wsb = sv.lib.spec_verify_workspace_bytes(B, K, V)
    return sv.lib.spec_verify(hidden, lm, d, tl, A, A, A, A, B, K, V, A, A, ws, wsb, None)


def test_verify_rejects(sv):
    assert _verify(sv, tl=None) == -1
    assert _verify(sv, ws=None) == -1
    assert _verify(sv, hidden=A) == -1                       # lm_head missing
    assert _verify(sv, lm=A) == -1                           # hidden missing
    assert _verify(sv, K=65) == -1
    assert _verify(sv, hidden=A, lm=A, d=12) == -1           # d % 8 != 0
    assert _verify(sv, hidden=A + 8, lm=A, d=256) == -2
    assert _verify(sv, B=20000, K=4, V=1000, hidden=A, lm=A, d=256) == -1  # M > 65536
    assert _verify(sv, B=1 << 20, K=64, V=1 << 20) == -1     # grid bound
    assert _verify(sv, wsb=100) == -4
    assert _verify(sv, ws=A + 16) == -4


def test_probe_rejects(sv):
    import ctypes
    f = ctypes.c_double()
    assert sv.lib.spec_probe_read(None, 1024, 4, 1, A, None) == -1
    assert sv.lib.spec_probe_read(A, 0, 4, 1, A, None) == -1
    assert sv.lib.spec_probe_read(A, 1000, 4, 1, A, None) == -1
    assert sv.lib.spec_probe_read(A, 1024, 3, 1, A, None) == -1
    assert sv.lib.spec_probe_read(A, 1024, 4, 0, A, None) == -1
    assert sv.lib.spec_probe_read(A + 8, 1024, 4, 1, A, None) == -2
    assert sv.lib.spec_probe_read_lds(None, 1024, 4, A, None) == -1
    assert sv.lib.spec_probe_read_lds(A, 1024, 4, None, None) == -1
    assert sv.lib.spec_probe_read_lds(A, 1000, 4, A, None) == -1
    assert sv.lib.spec_probe_read_lds(A, 1024, 3, A, None) == -1
    assert sv.lib.spec_probe_read_lds(A + 8, 1024, 4, A, None) == -2
    assert sv.lib.spec_probe_read_lds(A, 1024, 4, A + 2, None) == -2
    assert sv.lib.spec_probe_mfma(8, 10, A, ctypes.byref(f), None) == -1
    assert sv.lib.spec_probe_mfma(16, 0, A, ctypes.byref(f), None) == -1
    assert sv.lib.spec_probe_mfma(32, 10, None, ctypes.byref(f), None) == -1
    assert sv.lib.spec_probe_mfma(32, 10, A + 2, ctypes.byref(f), None) == -2


def test_verify_noalloc_rejects(sv):
    f = sv.lib.spec_verify_noalloc

    def call(B=1, K=4, V=1000, tl=A, hidden=None, lm=None, d=0, out=A):
        return f(hidden, lm, d, tl, A, A, A, A, B, K, V, out, A, None)
    assert call(tl=None) == -1
    assert call(out=None) == -1
    assert call(hidden=A) == -1
    assert call(K=65) == -1
    assert call(tl=MIS) == -2
    # beyond the 4 MiB static scratch: rejected on the host, with the sizes
    assert sv.lib.spec_verify_workspace_bytes(512, 8, 128256) > 4 << 20
    assert call(B=512, K=8, V=128256) == -4
    assert b"scratch" in sv.lib.spec_last_error()


def test_verify_warped_rejects(sv):
    wsb = sv.lib.spec_verify_workspace_bytes(1, 4, 1000)

    def call(t_t, t_d, **kw):
        args = dict(hidden=None, lm=None, tl=A, ws=A, wsb=wsb)
        args.update(kw)
        return sv.lib.spec_verify_warped(args["hidden"], args["lm"], 0, args["tl"], A, A, A, A,
                                         1, 4, 1000, t_t, t_d, A, A, args["ws"], args["wsb"], None)
    for t_t, t_d in ((-1.0, 1.0), (1.0, -0.5), (float("inf"), 1.0), (1.0, float("nan"))):
        assert call(t_t, t_d) == -1
        assert b"temperature" in sv.lib.spec_last_error()
    assert call(0.0, 1.0, tl=None) == -1       # other checks still apply
    assert call(0.7, 0.0, wsb=100) == -4


def test_gemm_w8_rejects(sv):
    f = sv.lib.spec_verify_gemm_w8
    cases = [
        ((A, A, None, A, 0, 5, 4096, 4096), -1),     # null w_scale
        ((None, A, A, A, 0, 5, 4096, 4096), -1),     # null x
        ((A, A, A, A, 2, 5, 4096, 4096), -1),        # bad y_dtype
        ((A, A, A, A, 0, 5, 4104, 4096), -1),        # d_in a multiple of 8 but not of 16
        ((A, A, A, A, 0, 5, 0, 4096), -1),
        ((A, A, A, A, 0, 0, 4096, 4096), -1),
        ((A, A, A, A, 0, 5, 4096, 0), -1),
        ((A, A, A + 2, A, 0, 5, 4096, 4096), -2),    # misaligned scales
        ((A, A + 8, A, A, 0, 5, 4096, 4096), -2),    # misaligned weights
        ((A, A, A, A, 0, 17, 4112, 4096), -3),       # tile kernel: d_in not a multiple of 64
    ]
    for args, code in cases:
        assert f(*args, None) == code, args
        assert sv.lib.spec_last_error()


def test_gemm_w8_workspace_bytes_and_rejects(sv):
    f = sv.lib.spec_verify_gemm_w8_workspace_bytes
    # the streaming kernel's positions, d_in not a multiple of 64, out of range
    assert f(16, 14336, 4096) == 0 and f(320, 14336 + 16, 4096) == 0 and f(0, 4096, 4096) == 0
    for M in (20, 80, 320, 1280):
        n = f(M, 14336, 4096)
        assert n > 0 and n % (M * 4096 * 4) == 0 and 2 <= n // (M * 4096 * 4) <= 16
    g = sv.lib.spec_verify_gemm_w8_ws
    need = f(320, 14336, 4096)
    assert g(A, A, A, A, 1, 320, 14336, 4096, None, need, None) == -4
    assert g(A, A, A, A, 1, 320, 14336, 4096, A, need - 1, None) == -4
    assert g(A, A, A, A, 1, 320, 14336, 4096, A + 8, need, None) == -4
    # argument checks as spec_verify_gemm_w8
    assert g(A, A, None, A, 0, 320, 14336, 4096, A, need, None) == -1
    assert g(A, A, A, A, 0, 17, 4112, 4096, A, 1 << 30, None) == -3


def test_attention_rejects(sv):
    wsb = sv.lib.spec_verify_attention_workspace_bytes
    f = sv.lib.spec_verify_attention
    # B=1, K=4, T=4096, 32/8 heads, D=128: splits, so a workspace is needed
    nb = wsb(1, 4, 4096, 32, 8, 128)
    assert nb > 0 and nb % 256 == 0
    assert wsb(64, 4, 4096, 32, 8, 128) == 0          # enough workgroups without splits
    assert wsb(1, 4, 4096, 32, 8, 64) == 0             # unsupported head_dim
    assert wsb(1, 8, 4096, 32, 8, 128) == 0            # 36 query rows per kv head
    assert wsb(1, 4, 4, 32, 8, 128) == 0               # T < K+1

    def call(**kw):
        args = dict(q=A, k=A, v=A, out=A, dt=1, B=1, K=4, T=4096, H=32, Hkv=8, D=128,
                    scale=0.088, ws=A, wsb=nb)
        args.update(kw)
        return f(args["q"], args["k"], args["v"], args["out"], args["dt"], args["B"], args["K"],
                 args["T"], args["H"], args["Hkv"], args["D"], args["scale"], args["ws"],
                 args["wsb"], None)
    for kw, code in [(dict(q=None), -1), (dict(out=None), -1), (dict(dt=2), -1),
                     (dict(B=0), -1), (dict(K=-1), -1), (dict(K=65), -1), (dict(T=4), -1),
                     (dict(Hkv=5), -1), (dict(D=64), -3), (dict(K=8), -3),
                     (dict(scale=float("nan")), -1), (dict(k=A + 8), -2), (dict(out=A + 1), -2),
                     (dict(wsb=nb - 1), -4), (dict(ws=None), -4), (dict(ws=A + 16), -4)]:
        assert call(**kw) == code, kw
        assert sv.lib.spec_last_error()


def test_chain_w8_rejects(sv):
    L = sv.SpecLinearW8
    good = (L * 2)(L(A, A, A, A, 4096, 4096, 1, 0), L(A, A, A, A, 4096, 128, 0, 0))
    nb = sv.lib.spec_chain_workspace_bytes(2)
    f = sv.lib.spec_chain_prepare_w8
    assert f(None, 2, 5, A, nb) == -1
    assert f(good, 2, 5, None, nb) == -1
    assert f(good, 2, 17, A, nb) == -1
    assert f(good, 2, 5, A, nb - 1) == -4
    for bad, code in [(L(A, A, None, A, 4096, 8, 1, 0), -1), (L(A, A, A, A, 4104, 8, 1, 0), -1),
                      (L(A, A, A, A, 4096, 8, 1, 1), -1), (L(A, A, A + 2, A, 4096, 8, 1, 0), -2)]:
        arr = (L * 2)(good[0], bad)
        assert f(arr, 2, 5, A, nb) == code
        assert b"linear 1" in sv.lib.spec_last_error()
    g = sv.lib.spec_verify_gemm_chain_w8
    assert g(0, 5, A, None) == -1 and g(2, 17, A, None) == -1 and g(2, 5, None, None) == -1
    assert g(2, 5, A + 8, None) == -4


def test_chain_rejects(sv):
    L = sv.SpecLinear
    good = (L * 2)(L(A, A, A, 4096, 4096, 1, 0), L(A, A, A, 4096, 128, 0, 0))
    nb = sv.lib.spec_chain_workspace_bytes(2)
    assert nb > 0 and nb % 256 == 0 and sv.lib.spec_chain_workspace_bytes(0) == 0
    assert sv.lib.spec_chain_workspace_bytes(4097) == 0
    f = sv.lib.spec_chain_prepare
    assert f(None, 2, 5, A, nb) == -1
    assert f(good, 2, 5, None, nb) == -1
    assert f(good, 0, 5, A, nb) == -1
    assert f(good, 2, 17, A, nb) == -1            # beyond the streaming regime
    assert f(good, 2, 0, A, nb) == -1
    assert f(good, 2, 5, A, nb - 1) == -4
    assert f(good, 2, 5, A + 64, nb) == -4
    for bad, code in [(L(A, A, A, 4100, 8, 1, 0), -1), (L(A, A, A, 8, 8, 3, 0), -1),
                      (L(A, A, A, 8, 8, 1, 1), -1), (L(A + 8, A, A, 8, 8, 1, 0), -2),
                      (L(A, A, None, 8, 8, 1, 0), -1)]:
        arr = (L * 2)(good[0], bad)
        assert f(arr, 2, 5, A, nb) == code
        assert b"linear 1" in sv.lib.spec_last_error()
    g = sv.lib.spec_verify_gemm_chain
    assert g(0, 5, A, None) == -1 and g(2, 17, A, None) == -1 and g(2, 5, None, None) == -1
    assert g(2, 5, A + 8, None) == -4
    import ctypes
    assert sv.lib.spec_chain_error(None, ctypes.byref(ctypes.c_int())) == -1
    assert sv.lib.spec_chain_reset(None, 0) == -1
    assert sv.lib.spec_chain_reset(A + 8, 0) == -4
