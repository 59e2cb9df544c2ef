"""Canary guard bands: every output buffer and workspace of a call sits
inside a larger allocation whose bytes before and after it hold a sentinel,
and after the call those bands must be unchanged. A write past either end of
a buffer (a ragged tile edge, a row stride, a split partial, a sampler index)
changes a sentinel byte. Each guarded result is also compared bitwise with
the same call into a plain tensor, so the bands sit next to real work.
"""

import ctypes

import pytest

import synth

pytestmark = pytest.mark.gpu

PAD = 4096          # bytes of sentinel on each side (keeps 256-byte alignment)
SENTINEL = 0xA5


class Guarded:
    """`nbytes` of device memory between two sentinel bands."""

    def __init__(self, nbytes, dev):
        import torch
        self.nbytes = int(nbytes)
        self.buf = torch.full((self.nbytes + 2 * PAD,), SENTINEL, dtype=torch.uint8, device=dev)
        self.inner = self.buf[PAD:PAD + self.nbytes]

    def tensor(self, shape, dtype):
        return self.inner.view(dtype).view(shape)

    def check(self, what):
        import torch
        torch.cuda.synchronize()
        before = self.buf[:PAD]
        after = self.buf[PAD + self.nbytes:]
        bad_b = int((before != SENTINEL).sum())
        bad_a = int((after != SENTINEL).sum())
        assert bad_b == 0 and bad_a == 0, f"{what}: {bad_b} bytes before, {bad_a} after changed"


def guarded_like(shape, dtype, dev):
    import torch
    n = 1
    for s in shape:
        n *= s
    g = Guarded(n * torch.empty((), dtype=dtype).element_size(), dev)
    return g, g.tensor(shape, dtype)


def ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


# (M, d_in, d_out): the streaming kernel (M <= 16), the skinny and two-buffer
# MFMA kernels (d_in not a multiple of 64), the tile kernel with direct
# stores, in k-groups, with the LDS staging epilogue at a ragged width, split
# by columns (a row stride wider than each launch's columns), and the
# exact-fill 80x64 (ten waves), 160x128, 160x224 (fourteen waves), 160x192 and 64x48 tiles
GEMM = [(5, 4096, 777), (16, 1032, 300), (40, 1032, 777), (200, 1032, 777),
        (20, 512, 4095), (20, 4096, 4096), (301, 64, 24001), (1250, 64, 28003),
        (300, 128, 4095), (1250, 64, 4095), (300, 64, 28600), (1250, 64, 6100),
        (90, 64, 6120)]


@pytest.mark.parametrize("M,d_in,d_out", GEMM)
def test_gemm_guard_bands(sv, dev, M, d_in, d_out):
    import torch
    from synth import device as sd
    x = sd.normal_bf16((M, d_in), 1.0, 3 + M, dev)
    w = sd.normal_bf16((d_out, d_in), synth.WEIGHT_STD, 4 + d_in, dev)
    for od in (torch.float32, torch.bfloat16):
        g, y = guarded_like((M, d_out), od, dev)
        sv.verify_gemm(x, w, out=y)
        g.check(f"gemm M={M} {d_in}->{d_out} {od}")
        assert torch.equal(y, sv.verify_gemm(x, w, out_dtype=od))


# shapes the split plan splits: staged fp32 partials at a ragged width
# (320x128 and 256x256 tiles), 64x128 tiles, and the split-sum kernel's
# scalar tail (M * d_out not a multiple of 4)
SPLIT = [(320, 14336, 4095), (160, 14336, 8191), (37, 8192, 2050), (9, 5120, 301)]


@pytest.mark.parametrize("M,d_in,d_out", SPLIT)
def test_gemm_split_guard_bands(sv, dev, M, d_in, d_out):
    import torch
    from synth import device as sd
    need = sv.gemm_workspace_bytes(M, d_in, d_out)
    assert need > 0, (M, d_in, d_out)
    x = sd.normal_bf16((M, d_in), 1.0, 5 + M, dev)
    w = sd.normal_bf16((d_out, d_in), synth.WEIGHT_STD, 6 + d_in, dev)
    gw = Guarded(need, dev)
    for od in (torch.float32, torch.bfloat16):
        g, y = guarded_like((M, d_out), od, dev)
        sv.verify_gemm_ws(x, w, out=y, workspace=gw.inner)
        g.check(f"split M={M} {d_in}->{d_out} {od} output")
        gw.check(f"split M={M} {d_in}->{d_out} {od} workspace")
        assert torch.equal(y, sv.verify_gemm_ws(x, w, out_dtype=od))


# FP8 weights: the streaming kernel, widen-once and staged tile forms, the
# column split, and a split plan with its workspace
W8 = [(5, 4096, 777), (80, 256, 16401), (301, 64, 24001), (1250, 64, 28003), (320, 8192, 8191)]


@pytest.mark.parametrize("M,d_in,d_out", W8)
def test_gemm_w8_guard_bands(sv, dev, M, d_in, d_out):
    import torch
    from synth import device as sd
    w = sd.e4m3_normal_codes((d_out, d_in), synth.W8_CODE_STD, 7 + d_in, dev)
    s = sd.w8_row_scales(d_out, synth.WEIGHT_STD / synth.W8_CODE_STD, 8 + d_out, dev)
    x = sd.normal_bf16((M, d_in), 1.0, 9 + M, dev)
    need = sv.gemm_w8_workspace_bytes(M, d_in, d_out)
    gw = Guarded(max(need, 256), dev)
    for od in (torch.float32, torch.bfloat16):
        g, y = guarded_like((M, d_out), od, dev)
        if need > 0:
            sv.verify_gemm_w8_ws(x, w, s, out=y, workspace=gw.inner)
            gw.check(f"w8 split M={M} {d_in}->{d_out} {od} workspace")
            ref = sv.verify_gemm_w8_ws(x, w, s, out_dtype=od)
        else:
            sv.verify_gemm_w8(x, w, s, out=y)
            ref = sv.verify_gemm_w8(x, w, s, out_dtype=od)
        g.check(f"w8 M={M} {d_in}->{d_out} {od}")
        assert torch.equal(y, ref)


@pytest.mark.parametrize("w8", [False, True])
def test_chain_guard_bands(sv, dev, w8):
    """A dependent chain of three linears with every output guarded."""
    import torch
    from synth import device as sd
    M = 5
    dims = [(1032, 777), (777 + 7, 4104), (4104, 300)]  # d_in multiples of 8 (16 for FP8)
    if w8:
        dims = [(1040, 784), (784, 4112), (4112, 304)]
    lin, guards, plain = [], [], []
    for i, (d_in, d_out) in enumerate(dims):
        x = sd.normal_bf16((M, d_in), 1.0, 20 + i, dev)
        g, y = guarded_like((M, d_out), torch.bfloat16 if i < 2 else torch.float32, dev)
        yp = torch.empty_like(y)
        guards.append(g)
        if w8:
            w = sd.e4m3_normal_codes((d_out, d_in), synth.W8_CODE_STD, 30 + i, dev)
            s = sd.w8_row_scales(d_out, synth.WEIGHT_STD / synth.W8_CODE_STD, 40 + i, dev)
            lin.append((x, w, s, y))
            plain.append((x, w, s, yp))
        else:
            w = sd.normal_bf16((d_out, d_in), synth.WEIGHT_STD, 30 + i, dev)
            lin.append((x, w, y))
            plain.append((x, w, yp))
    chain = sv.Chain(lin, dev)
    for _ in range(2):
        chain.run(check_error=True)
    for i, g in enumerate(guards):
        g.check(f"chain w8={w8} linear {i}")
    sv.Chain(plain, dev).run(check_error=True)
    torch.cuda.synchronize()
    for (a, b) in zip(lin, plain):
        assert torch.equal(a[-1], b[-1])


def test_sampling_guard_bands(sv, dev):
    """spec_softmax, spec_accept_scan, spec_residual_sample and spec_verify
    (with the lm-head, so the logits are an output too) into guarded
    buffers, at a vocabulary that is not a multiple of the kernels' chunks."""
    import torch
    from synth import device as sd
    B, K, V, d = 3, 4, 50021, 256
    lib = sv.lib
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    tl = sd.normal_f32((B, K + 1, V), 3.0, 50, dev)
    dl = (tl[:, :K] + sd.normal_f32((B, K, V), 1.0, 51, dev)).contiguous()
    toks = sd.gumbel_max_tokens(dl, 52)
    ua = sd.uniform_f32((B, K), 53, dev)
    us = sd.uniform_f32((B, K + 1), 54, dev)

    # softmax: probabilities and row statistics
    rows = B * (K + 1)
    gp, p = guarded_like((B, K + 1, V), torch.float32, dev)
    gm, mx = guarded_like((rows,), torch.float32, dev)
    gs, se = guarded_like((rows,), torch.float32, dev)
    sv.check(lib.spec_softmax(ptr(tl), rows, V, ptr(p), ptr(mx), ptr(se), st))
    for g, nm in ((gp, "probs"), (gm, "row_max"), (gs, "row_sumexp")):
        g.check(f"softmax {nm}")
    p_ref, mx_ref, se_ref = sv.softmax(tl)
    assert torch.equal(p, p_ref) and torch.equal(mx, mx_ref.reshape(-1)) \
        and torch.equal(se, se_ref.reshape(-1))
    q = sv.softmax(dl, stats=False)[0]

    # accept scan
    gn, n_acc = guarded_like((B,), torch.int32, dev)
    gk, mask = guarded_like((B, K), torch.uint8, dev)
    sv.check(lib.spec_accept_scan(ptr(p), ptr(q), ptr(toks), ptr(ua), B, K, V, ptr(n_acc),
                                  ptr(mask), st))
    gn.check("accept n_accepted")
    gk.check("accept mask")
    n_ref, m_ref = sv.accept_scan(p, q, toks, ua)
    assert torch.equal(n_acc, n_ref) and torch.equal(mask, m_ref)

    # residual / bonus sample
    gt, tok = guarded_like((B,), torch.int32, dev)
    gz, zero = guarded_like((B,), torch.uint8, dev)
    sv.check(lib.spec_residual_sample(ptr(p), ptr(q), ptr(n_acc), ptr(us), B, K, V, ptr(tok),
                                      ptr(zero), st))
    gt.check("residual token")
    gz.check("residual zero_residual")
    t_ref, z_ref = sv.residual_sample(p, q, n_acc, us)
    assert torch.equal(tok, t_ref) and torch.equal(zero, z_ref)

    # the whole step with the lm-head: logits, tokens, counts and workspace
    hidden = sd.normal_bf16((B * (K + 1), d), 1.0, 55, dev)
    lm = sd.normal_bf16((V, d), synth.WEIGHT_STD, 56, dev)
    gl, logits = guarded_like((B, K + 1, V), torch.float32, dev)
    go, out = guarded_like((B, K + 1), torch.int32, dev)
    ge, n_em = guarded_like((B,), torch.int32, dev)
    gw = Guarded(sv.workspace_bytes(B, K, V), dev)
    for t_target, t_draft in ((1.0, 1.0), (0.7, 1.3), (0.0, 0.0)):
        sv.verify(logits, dl, toks, ua, us, hidden=hidden, lm_head=lm, workspace=gw.inner,
                  out_tokens=out, n_emitted=n_em, t_target=t_target, t_draft=t_draft)
        for g, nm in ((gl, "logits"), (go, "out_tokens"), (ge, "n_emitted"), (gw, "workspace")):
            g.check(f"verify T=({t_target}, {t_draft}) {nm}")
        o_ref, e_ref = sv.verify(torch.empty_like(logits), dl, toks, ua, us, hidden=hidden,
                                 lm_head=lm, t_target=t_target, t_draft=t_draft)
        assert torch.equal(out, o_ref) and torch.equal(n_em, e_ref)


# (B, K, T): context splits with a merge (B = 1, the 8B layer's cache), two
# splits (B = 40), and no split (B = 64)
ATT = [(1, 4, 4101), (40, 4, 300), (64, 3, 200)]


@pytest.mark.parametrize("B,K,T", ATT)
def test_attention_guard_bands(sv, dev, B, K, T):
    import torch
    from synth import device as sd
    H, Hkv, D = 32, 8, 128
    q = sd.normal_bf16((B, K + 1, H, D), 1.0, 60 + B, dev)
    k = sd.normal_bf16((B, T, Hkv, D), 1.0, 61 + B, dev)
    v = sd.normal_bf16((B, T, Hkv, D), 1.0, 62 + B, dev)
    need = sv.lib.spec_verify_attention_workspace_bytes(B, K, T, H, Hkv, D)
    gw = Guarded(max(need, 256), dev) if need > 0 else None
    for od in (torch.float32, torch.bfloat16):
        g, o = guarded_like((B, K + 1, H, D), od, dev)
        sv.verify_attention(q, k, v, out=o, workspace=gw.inner if gw else None)
        g.check(f"attention B={B} T={T} {od} out")
        if gw:
            gw.check(f"attention B={B} T={T} {od} workspace")
        assert torch.equal(o, sv.verify_attention(q, k, v, out_dtype=od))
