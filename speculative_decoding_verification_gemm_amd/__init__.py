"""Python binding of libspecverify.so, the MI355X verify step of speculative
decoding.

Argument marshalling only: every call passes device pointers of caller-owned
torch tensors and torch's current HIP stream to the C ABI declared in
include/spec_verify.h; all computation runs in the library's HIP kernels.
Importing this package fails if the library has not been built
(``python speculative_decoding_verification_gemm_amd/build.py``); there is no
fallback.
"""

import ctypes
import os

# torch ships its own HIP runtime under the same soname (libamdhip64.so.7) as
# the system one this library links against; whichever is loaded first serves
# the whole process. Device pointers and streams come from torch, so torch's
# runtime must be the one loaded: import torch before opening the library.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing; build it with "
        "`python speculative_decoding_verification_gemm_amd/build.py`")

lib = ctypes.CDLL(LIB_PATH)

SPEC_OK = 0
SPEC_ERR_INVALID_ARGUMENT = -1
SPEC_ERR_ALIGNMENT = -2
SPEC_ERR_UNSUPPORTED = -3
SPEC_ERR_WORKSPACE = -4
SPEC_ERR_HIP = -5
SPEC_F32 = 0
SPEC_BF16 = 1

_p = ctypes.c_void_p
_i = ctypes.c_int
_z = ctypes.c_size_t
_f = ctypes.c_float

# name -> (restype, argtypes), exactly as declared in include/spec_verify.h
SIGNATURES = {
    "spec_abi_version": (_i, []),
    "spec_status_string": (ctypes.c_char_p, [_i]),
    "spec_last_error": (ctypes.c_char_p, []),
    "spec_verify_gemm": (_i, [_p, _p, _p, _i, _i, _i, _i, _p]),
    "spec_verify_gemm_workspace_bytes": (_z, [_i, _i, _i]),
    "spec_verify_gemm_ws": (_i, [_p, _p, _p, _i, _i, _i, _i, _p, _z, _p]),
    "spec_softmax": (_i, [_p, _i, _i, _p, _p, _p, _p]),
    "spec_accept_scan": (_i, [_p, _p, _p, _p, _i, _i, _i, _p, _p, _p]),
    "spec_residual_sample": (_i, [_p, _p, _p, _p, _i, _i, _i, _p, _p, _p]),
    "spec_verify_workspace_bytes": (_z, [_i, _i, _i]),
    "spec_chain_workspace_bytes": (_z, [_i]),
    "spec_chain_prepare": (_i, [_p, _i, _i, _p, _z]),
    "spec_verify_gemm_chain": (_i, [_i, _i, _p, _p]),
    "spec_verify_gemm_w8": (_i, [_p, _p, _p, _p, _i, _i, _i, _i, _p]),
    "spec_verify_gemm_w8_workspace_bytes": (_z, [_i, _i, _i]),
    "spec_verify_gemm_w8_ws": (_i, [_p, _p, _p, _p, _i, _i, _i, _i, _p, _z, _p]),
    "spec_chain_prepare_w8": (_i, [_p, _i, _i, _p, _z]),
    "spec_verify_gemm_chain_w8": (_i, [_i, _i, _p, _p]),
    "spec_verify_attention_workspace_bytes": (_z, [_i, _i, _i, _i, _i, _i]),
    "spec_verify_attention": (_i, [_p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _p, _z, _p]),
    "spec_chain_error": (_i, [_p, ctypes.POINTER(ctypes.c_int)]),
    "spec_chain_reset": (_i, [_p, ctypes.c_uint]),
    "spec_probe_read": (_i, [_p, _z, _i, _i, _p, _p]),
    "spec_probe_read_lds": (_i, [_p, _z, _i, _p, _p]),
    "spec_probe_mfma": (_i, [_i, _i, _p, ctypes.POINTER(ctypes.c_double), _p]),
    "spec_verify": (_i, [_p, _p, _i, _p, _p, _p, _p, _p, _i, _i, _i, _p, _p, _p, _z, _p]),
    "spec_verify_warped": (_i, [_p, _p, _i, _p, _p, _p, _p, _p, _i, _i, _i, _f, _f, _p, _p, _p,
                                _z, _p]),
    "spec_verify_noalloc": (_i, [_p, _p, _i, _p, _p, _p, _p, _p, _i, _i, _i, _p, _p, _p]),
}
for _name, (_res, _args) in SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class SpecLinear(ctypes.Structure):
    """spec_linear of include/spec_verify.h."""
    _fields_ = [("x", ctypes.c_void_p), ("w", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32),
                ("y_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class SpecLinearW8(ctypes.Structure):
    """spec_linear_w8 of include/spec_verify.h."""
    _fields_ = [("x", ctypes.c_void_p), ("w", ctypes.c_void_p), ("w_scale", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32),
                ("y_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class SpecVerifyError(RuntimeError):
    """A libspecverify call returned a non-zero status."""

    def __init__(self, code, message):
        super().__init__(f"{lib.spec_status_string(code).decode()}: {message}")
        self.code = code


def check(status):
    if status != SPEC_OK:
        raise SpecVerifyError(status, lib.spec_last_error().decode())


def abi_version():
    return lib.spec_abi_version()


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, dtype, name, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t


def _gemm_out(x, w, out, out_dtype):
    torch = _torch()
    _need(x, torch.bfloat16, "x", 2)
    _need(w, torch.bfloat16, "w", 2)
    M, d_in = x.shape
    d_out = w.shape[0]
    if w.shape[1] != d_in:
        raise ValueError(f"x {tuple(x.shape)} and w {tuple(w.shape)} disagree on d_in")
    if out is None:
        out = torch.empty((M, d_out), dtype=out_dtype or torch.float32, device=x.device)
    _need(out, out.dtype, "out", 2)
    if tuple(out.shape) != (M, d_out):
        raise ValueError(f"out must be {(M, d_out)}, got {tuple(out.shape)}")
    code = {torch.float32: SPEC_F32, torch.bfloat16: SPEC_BF16}.get(out.dtype)
    if code is None:
        raise TypeError("out must be float32 or bfloat16")
    return out, code, M, d_in, d_out


def verify_gemm(x, w, out=None, out_dtype=None):
    """y[M][d_out] = x[M][d_in] . w[d_out][d_in]^T (bf16 in, fp32 accumulate).

    out_dtype: torch.float32 (default) or torch.bfloat16."""
    out, code, M, d_in, d_out = _gemm_out(x, w, out, out_dtype)
    check(lib.spec_verify_gemm(_ptr(x), _ptr(w), _ptr(out), code, M, d_in, d_out, _stream()))
    return out


def gemm_workspace_bytes(M, d_in, d_out):
    """Workspace bytes verify_gemm_ws needs for this shape (0: none)."""
    return lib.spec_verify_gemm_workspace_bytes(M, d_in, d_out)


def verify_gemm_ws(x, w, out=None, out_dtype=None, workspace=None):
    """verify_gemm with the reduction split over workgroups where that is
    faster; `workspace` is a device tensor of at least
    gemm_workspace_bytes(M, d_in, d_out) bytes (allocated here if None)."""
    out, code, M, d_in, d_out = _gemm_out(x, w, out, out_dtype)
    workspace, n = _workspace(workspace, gemm_workspace_bytes(M, d_in, d_out), x.device)
    check(lib.spec_verify_gemm_ws(_ptr(x), _ptr(w), _ptr(out), code, M, d_in, d_out,
                                  _ptr(workspace), n, _stream()))
    return out


def _gemm_w8_out(x, w, w_scale, out, out_dtype):
    torch = _torch()
    _need(x, torch.bfloat16, "x", 2)
    _need(w, torch.uint8, "w", 2)
    _need(w_scale, torch.float32, "w_scale", 1)
    M, d_in = x.shape
    d_out = w.shape[0]
    if w.shape[1] != d_in or w_scale.shape[0] != d_out:
        raise ValueError(f"x {tuple(x.shape)}, w {tuple(w.shape)}, w_scale "
                         f"{tuple(w_scale.shape)} disagree")
    if out is None:
        out = torch.empty((M, d_out), dtype=out_dtype or torch.float32, device=x.device)
    _need(out, out.dtype, "out", 2)
    if tuple(out.shape) != (M, d_out):
        raise ValueError(f"out must be {(M, d_out)}, got {tuple(out.shape)}")
    code = {torch.float32: SPEC_F32, torch.bfloat16: SPEC_BF16}.get(out.dtype)
    if code is None:
        raise TypeError("out must be float32 or bfloat16")
    return out, code, M, d_in, d_out


def verify_gemm_w8(x, w, w_scale, out=None, out_dtype=None):
    """y[m][n] = w_scale[n] * sum_k x[m][k] * e4m3(w[n][k]) (weight-only FP8).

    x bf16 [M][d_in]; w uint8 FP8 E4M3 codes [d_out][d_in]; w_scale float32
    [d_out]; out_dtype torch.float32 (default) or torch.bfloat16."""
    out, code, M, d_in, d_out = _gemm_w8_out(x, w, w_scale, out, out_dtype)
    check(lib.spec_verify_gemm_w8(_ptr(x), _ptr(w), _ptr(w_scale), _ptr(out), code, M, d_in,
                                  d_out, _stream()))
    return out


def gemm_w8_workspace_bytes(M, d_in, d_out):
    """Workspace bytes verify_gemm_w8_ws needs for this shape (0: none)."""
    return lib.spec_verify_gemm_w8_workspace_bytes(M, d_in, d_out)


def _workspace(workspace, need, dev):
    torch = _torch()
    if workspace is None:
        return (torch.empty(need, dtype=torch.uint8, device=dev) if need else None), need
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
        raise TypeError("workspace must be a device tensor")
    return workspace, workspace.numel() * workspace.element_size()


def verify_gemm_w8_ws(x, w, w_scale, out=None, out_dtype=None, workspace=None):
    """verify_gemm_w8 with the reduction split over workgroups where that is
    faster; `workspace` is a device tensor of at least
    gemm_w8_workspace_bytes(M, d_in, d_out) bytes (allocated here if None)."""
    out, code, M, d_in, d_out = _gemm_w8_out(x, w, w_scale, out, out_dtype)
    workspace, n = _workspace(workspace, gemm_w8_workspace_bytes(M, d_in, d_out), x.device)
    check(lib.spec_verify_gemm_w8_ws(_ptr(x), _ptr(w), _ptr(w_scale), _ptr(out), code, M, d_in,
                                     d_out, _ptr(workspace), n, _stream()))
    return out


def verify_attention(q, k_cache, v_cache, scale=None, out=None, out_dtype=None, workspace=None):
    """The verify positions' attention over the KV cache.

    q bf16 [B][K+1][H][D]; k_cache, v_cache bf16 [B][T][Hkv][D] with the K+1
    verify positions last; scale defaults to 1/sqrt(D). Returns out
    [B][K+1][H][D] (bf16 unless out_dtype / out say otherwise)."""
    torch = _torch()
    _need(q, torch.bfloat16, "q", 4)
    _need(k_cache, torch.bfloat16, "k_cache", 4)
    _need(v_cache, torch.bfloat16, "v_cache", 4)
    B, K1, H, D = q.shape
    T, Hkv = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, T, Hkv, D) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError(f"q {tuple(q.shape)}, k {tuple(k_cache.shape)}, v "
                         f"{tuple(v_cache.shape)} disagree")
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    if out is None:
        out = torch.empty((B, K1, H, D), dtype=out_dtype or torch.bfloat16, device=q.device)
    _need(out, out.dtype, "out", 4)
    if tuple(out.shape) != (B, K1, H, D):
        raise ValueError(f"out must be {(B, K1, H, D)}, got {tuple(out.shape)}")
    code = {torch.float32: SPEC_F32, torch.bfloat16: SPEC_BF16}.get(out.dtype)
    if code is None:
        raise TypeError("out must be float32 or bfloat16")
    nbytes = lib.spec_verify_attention_workspace_bytes(B, K1 - 1, T, H, Hkv, D)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    check(lib.spec_verify_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), code, B,
                                    K1 - 1, T, H, Hkv, D, float(scale), _ptr(workspace),
                                    0 if workspace is None else workspace.numel(), _stream()))
    return out


def softmax(logits, probs=True, stats=True):
    """Row softmax of fp32 logits [..., V]: (probs or None, row_max, row_sumexp)
    (the last two None unless stats)."""
    torch = _torch()
    _need(logits, torch.float32, "logits")
    V = logits.shape[-1]
    rows = logits.numel() // V
    p = torch.empty_like(logits) if probs else None
    mx = torch.empty(logits.shape[:-1], dtype=torch.float32, device=logits.device) if stats else None
    se = torch.empty_like(mx) if stats else None
    check(lib.spec_softmax(_ptr(logits), rows, V, _ptr(p), _ptr(mx), _ptr(se), _stream()))
    return p, mx, se


def accept_scan(p_probs, q_probs, draft_tokens, u_accept, with_mask=True):
    """(n_accepted int32 [B], accept_mask uint8 [B][K] or None)."""
    torch = _torch()
    _need(p_probs, torch.float32, "p_probs", 3)
    _need(q_probs, torch.float32, "q_probs", 3)
    _need(draft_tokens, torch.int32, "draft_tokens", 2)
    _need(u_accept, torch.float32, "u_accept", 2)
    B, K1, V = p_probs.shape
    K = K1 - 1
    if tuple(q_probs.shape) != (B, K, V) or tuple(draft_tokens.shape) != (B, K) \
            or tuple(u_accept.shape) != (B, K):
        raise ValueError("inconsistent shapes")
    n = torch.empty(B, dtype=torch.int32, device=p_probs.device)
    mask = torch.empty((B, K), dtype=torch.uint8, device=p_probs.device) if with_mask else None
    check(lib.spec_accept_scan(_ptr(p_probs), _ptr(q_probs), _ptr(draft_tokens), _ptr(u_accept),
                               B, K, V, _ptr(n), _ptr(mask), _stream()))
    return n, mask


def residual_sample(p_probs, q_probs, n_accepted, u_sample):
    """(token int32 [B], zero_residual uint8 [B])."""
    torch = _torch()
    _need(p_probs, torch.float32, "p_probs", 3)
    _need(q_probs, torch.float32, "q_probs", 3)
    _need(n_accepted, torch.int32, "n_accepted", 1)
    _need(u_sample, torch.float32, "u_sample", 2)
    B, K1, V = p_probs.shape
    K = K1 - 1
    if tuple(q_probs.shape) != (B, K, V) or tuple(n_accepted.shape) != (B,) \
            or tuple(u_sample.shape) != (B, K1):
        raise ValueError("inconsistent shapes")
    tok = torch.empty(B, dtype=torch.int32, device=p_probs.device)
    zero = torch.empty(B, dtype=torch.uint8, device=p_probs.device)
    check(lib.spec_residual_sample(_ptr(p_probs), _ptr(q_probs), _ptr(n_accepted),
                                   _ptr(u_sample), B, K, V, _ptr(tok), _ptr(zero), _stream()))
    return tok, zero


def workspace_bytes(B, K, V):
    return lib.spec_verify_workspace_bytes(B, K, V)


def new_workspace(B, K, V, device="cuda"):
    """A device buffer of spec_verify_workspace_bytes(B, K, V) bytes (torch's
    allocator returns 256-byte aligned blocks)."""
    torch = _torch()
    n = workspace_bytes(B, K, V)
    if n == 0:
        raise ValueError(f"invalid (B, K, V) = {(B, K, V)}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def verify(target_logits, draft_logits, draft_tokens, u_accept, u_sample,
           hidden=None, lm_head=None, workspace=None, out_tokens=None, n_emitted=None,
           t_target=1.0, t_draft=1.0):
    """The verify step after the stack. With hidden [B*(K+1)][d] and lm_head
    [V][d] (bf16), target_logits [B][K+1][V] is written first; otherwise it
    is an input. t_target / t_draft are the temperatures of the target's and
    the draft's distributions (0: greedy, one-hot at the first maximum).
    Returns (out_tokens int32 [B][K+1], n_emitted int32 [B])."""
    torch = _torch()
    _need(target_logits, torch.float32, "target_logits", 3)
    _need(draft_logits, torch.float32, "draft_logits", 3)
    _need(draft_tokens, torch.int32, "draft_tokens", 2)
    _need(u_accept, torch.float32, "u_accept", 2)
    _need(u_sample, torch.float32, "u_sample", 2)
    B, K1, V = target_logits.shape
    K = K1 - 1
    d = 0
    if lm_head is not None:
        _need(lm_head, torch.bfloat16, "lm_head", 2)
        _need(hidden, torch.bfloat16, "hidden", 2)
        d = lm_head.shape[1]
        if tuple(lm_head.shape) != (V, d) or tuple(hidden.shape) != (B * K1, d):
            raise ValueError("hidden / lm_head shapes disagree with the logits")
    if workspace is None:
        workspace = new_workspace(B, K, V, target_logits.device)
    if out_tokens is None:
        out_tokens = torch.empty((B, K1), dtype=torch.int32, device=target_logits.device)
    if n_emitted is None:
        n_emitted = torch.empty(B, dtype=torch.int32, device=target_logits.device)
    if t_target == 1.0 and t_draft == 1.0:
        check(lib.spec_verify(_ptr(hidden), _ptr(lm_head), d, _ptr(target_logits),
                              _ptr(draft_logits), _ptr(draft_tokens), _ptr(u_accept),
                              _ptr(u_sample), B, K, V, _ptr(out_tokens), _ptr(n_emitted),
                              _ptr(workspace), workspace.numel(), _stream()))
    else:
        check(lib.spec_verify_warped(_ptr(hidden), _ptr(lm_head), d, _ptr(target_logits),
                                     _ptr(draft_logits), _ptr(draft_tokens), _ptr(u_accept),
                                     _ptr(u_sample), B, K, V, float(t_target), float(t_draft),
                                     _ptr(out_tokens), _ptr(n_emitted), _ptr(workspace),
                                     workspace.numel(), _stream()))
    return out_tokens, n_emitted


def probe_read(buf, sink, loads_per_lane=4, wgs_per_cu=1):
    """spec_probe_read over the whole of `buf` (a device tensor); `sink` is
    a device tensor of at least 4 bytes."""
    check(lib.spec_probe_read(_ptr(buf), buf.numel() * buf.element_size(), int(loads_per_lane),
                              int(wgs_per_cu), _ptr(sink), _stream()))


def probe_read_lds(buf, sink, loads_per_lane=4):
    """spec_probe_read_lds over the whole of `buf` (a device tensor); `sink`
    is a device tensor of at least 4 bytes."""
    check(lib.spec_probe_read_lds(_ptr(buf), buf.numel() * buf.element_size(),
                                  int(loads_per_lane), _ptr(sink), _stream()))


def probe_mfma(shape, iters, sink):
    """spec_probe_mfma; returns the launch's floating-point operations."""
    flops = ctypes.c_double(0.0)
    check(lib.spec_probe_mfma(int(shape), int(iters), _ptr(sink), ctypes.byref(flops), _stream()))
    return flops.value


def verify_noalloc(target_logits, draft_logits, draft_tokens, u_accept, u_sample,
                   out_tokens, n_emitted, hidden=None, lm_head=None):
    """spec_verify_noalloc: verify() without a workspace (the library's
    static scratch serves instead). The outputs are caller-provided, so this
    call allocates nothing on the device."""
    torch = _torch()
    _need(target_logits, torch.float32, "target_logits", 3)
    _need(draft_logits, torch.float32, "draft_logits", 3)
    _need(draft_tokens, torch.int32, "draft_tokens", 2)
    _need(u_accept, torch.float32, "u_accept", 2)
    _need(u_sample, torch.float32, "u_sample", 2)
    _need(out_tokens, torch.int32, "out_tokens", 2)
    _need(n_emitted, torch.int32, "n_emitted", 1)
    B, K1, V = target_logits.shape
    d = 0
    if lm_head is not None:
        _need(lm_head, torch.bfloat16, "lm_head", 2)
        _need(hidden, torch.bfloat16, "hidden", 2)
        d = lm_head.shape[1]
        if tuple(lm_head.shape) != (V, d) or tuple(hidden.shape) != (B * K1, d):
            raise ValueError("hidden / lm_head shapes disagree with the logits")
    if tuple(out_tokens.shape) != (B, K1) or tuple(n_emitted.shape) != (B,):
        raise ValueError("out_tokens / n_emitted shapes disagree with the logits")
    check(lib.spec_verify_noalloc(_ptr(hidden), _ptr(lm_head), d, _ptr(target_logits),
                                  _ptr(draft_logits), _ptr(draft_tokens), _ptr(u_accept),
                                  _ptr(u_sample), B, K1 - 1, V, _ptr(out_tokens), _ptr(n_emitted),
                                  _stream()))
    return out_tokens, n_emitted


class Chain:
    """A prepared chain of linears (spec_chain_prepare) and its workspace.

    linears: list of (x, w, y) device tensors, x bf16 [M][d_in], w bf16
    [d_out][d_in], y fp32 or bf16 [M][d_out]; or, for a chain of FP8-weight
    linears, (x, w, w_scale, y) with w uint8 E4M3 codes and w_scale float32
    [d_out]. The tensors must stay alive while the chain is used."""

    def __init__(self, linears, device="cuda"):
        torch = _torch()
        if not linears:
            raise ValueError("empty chain")
        M = linears[0][0].shape[0]
        self.w8 = len(linears[0]) == 4
        descs = ((SpecLinearW8 if self.w8 else SpecLinear) * len(linears))()
        for i, lin in enumerate(linears):
            if len(lin) != (4 if self.w8 else 3):
                raise ValueError("a chain is all bf16 (x, w, y) or all FP8 (x, w, w_scale, y)")
            x, w, y = lin[0], lin[1], lin[-1]
            _need(x, torch.bfloat16, f"x[{i}]", 2)
            _need(w, torch.uint8 if self.w8 else torch.bfloat16, f"w[{i}]", 2)
            _need(y, y.dtype, f"y[{i}]", 2)
            code = {torch.float32: SPEC_F32, torch.bfloat16: SPEC_BF16}.get(y.dtype)
            if code is None:
                raise TypeError(f"y[{i}] must be float32 or bfloat16")
            if x.shape[0] != M or tuple(y.shape) != (M, w.shape[0]) or x.shape[1] != w.shape[1]:
                raise ValueError(f"linear {i}: shapes x {tuple(x.shape)}, w {tuple(w.shape)}, "
                                 f"y {tuple(y.shape)} disagree")
            if self.w8:
                _need(lin[2], torch.float32, f"w_scale[{i}]", 1)
                if lin[2].shape[0] != w.shape[0]:
                    raise ValueError(f"linear {i}: w_scale has {lin[2].shape[0]} entries")
                descs[i] = SpecLinearW8(x.data_ptr(), w.data_ptr(), lin[2].data_ptr(),
                                        y.data_ptr(), x.shape[1], w.shape[0], code, 0)
            else:
                descs[i] = SpecLinear(x.data_ptr(), w.data_ptr(), y.data_ptr(), x.shape[1],
                                      w.shape[0], code, 0)
        self.n, self.M = len(linears), M
        self.keep = list(linears)
        nbytes = lib.spec_chain_workspace_bytes(self.n)
        if nbytes == 0:
            raise ValueError(f"chain of {self.n} linears is out of range")
        self.workspace = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        torch.cuda.synchronize()
        prepare = lib.spec_chain_prepare_w8 if self.w8 else lib.spec_chain_prepare
        check(prepare(descs, self.n, self.M, _ptr(self.workspace), nbytes))

    def run(self, check_error=False):
        """One launch of the chain on the current stream (asynchronous). A
        barrier that gives up, or a grid the device could not hold, is only
        known on the device: with check_error=True the call waits for the
        launch and raises RuntimeError if the error word is set (it is then
        read and cleared)."""
        run = lib.spec_verify_gemm_chain_w8 if self.w8 else lib.spec_verify_gemm_chain
        check(run(self.n, self.M, _ptr(self.workspace), _stream()))
        if check_error:
            _torch().cuda.current_stream().synchronize()
            e = self.error()
            if e:
                raise RuntimeError(
                    f"chain launch failed on the device (error word {e}: bit 0, a barrier "
                    "gave up waiting; bit 1, the grid differs from the prepared plan); "
                    "its outputs are not valid")

    def error(self):
        """Read and clear the device-side error word (synchronous)."""
        e = ctypes.c_int(0)
        check(lib.spec_chain_error(_ptr(self.workspace), ctypes.byref(e)))
        return e.value

    def reset(self, generation=0):
        """Counters as after `generation` complete launches, error word
        cleared (synchronous; spec_chain_reset)."""
        _torch().cuda.synchronize()
        check(lib.spec_chain_reset(_ptr(self.workspace), int(generation) & 0xFFFFFFFF))
