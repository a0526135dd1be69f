"""Python binding of libfa, the gfx950 attention library (include/fa.h).

Argument marshalling only: torch tensors supply device memory and the HIP
stream, every step of the computation runs in the library's HIP kernels.
There is no fallback: if libfa.so is missing or fails to load, every call
raises.

Entry points keep the C names:

    fa_fwd(Q, K, V, O, LSE, scale, causal=False, stream=None)
    fa_fwd_ws(Q, K, V, O, LSE, workspace, scale, causal=False, stream=None)
    fa_fwd_workspace_size(B, H, Nq, Nk, d) -> int
    fa_fwd_splitkv(Q, K, V, O, LSE, num_splits, workspace, scale, causal=False, stream=None)
    fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, num_splits) -> int
    fa_fwd_num_splits(B, H, Nq, Nk, d, causal) -> int
    fa_dropout_threshold(dropout_p) -> int
    fa_fwd_dropout(Q, K, V, O, LSE, dropout_p, seed, scale, causal=False, stream=None)
    fa_bwd_dropout(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, dropout_p, seed, scale, causal=False, stream=None)
    fa_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, scale, causal=False, stream=None)
    fa_bwd_workspace_size(B, H, Nq, Nk, d) -> int
    fa_bwd_noalloc(Q, K, V, O, dO, LSE, dQ, dK, dV, scale, causal=False, stream=None)
    fa_bwd_num_stages() -> int
    fa_bwd_stage(stage, <fa_bwd arguments>)
    fa_status_string(status) -> str
    fa_build_info() -> str
    fa_describe(d, dtype, causal) -> str

plus ``forward`` / ``backward`` helpers that allocate the outputs.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# LIBFA_PATH selects another build of the same library (e.g. to compare builds).
LIB_PATH = os.environ.get("LIBFA_PATH") or os.path.join(_HERE, "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
FA_BF16, FA_F16, FA_F32 = 0, 1, 2

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s returned %s (%d)" % (what, fa_status_string(status), status))
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libfa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libfa.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    L.fa_fwd.restype = i
    L.fa_fwd_ws.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, vp]
    L.fa_fwd_ws.restype = i
    L.fa_fwd_workspace_size.argtypes = [i, i, i, i, i]
    L.fa_fwd_workspace_size.restype = sz
    L.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, sz, vp]
    L.fa_fwd_splitkv.restype = i
    L.fa_fwd_splitkv_workspace_size.argtypes = [i, i, i, i, i, i]
    L.fa_fwd_splitkv_workspace_size.restype = sz
    L.fa_fwd_num_splits.argtypes = [i, i, i, i, i, i]
    L.fa_fwd_num_splits.restype = i
    u64 = ctypes.c_ulonglong
    L.fa_dropout_threshold.argtypes = [f]
    L.fa_dropout_threshold.restype = i
    L.fa_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, f, u64, vp]
    L.fa_fwd_dropout.restype = i
    L.fa_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, f, u64, vp, sz, vp]
    L.fa_bwd_dropout.restype = i
    L.fa_bwd_workspace_size.argtypes = [i, i, i, i, i]
    L.fa_bwd_workspace_size.restype = sz
    L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, vp]
    L.fa_bwd.restype = i
    L.fa_build_info.argtypes = []
    L.fa_build_info.restype = ctypes.c_char_p
    L.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    L.fa_bwd_noalloc.restype = i
    L.fa_bwd_num_stages.argtypes = []
    L.fa_bwd_num_stages.restype = i
    L.fa_bwd_stage.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, vp]
    L.fa_bwd_stage.restype = i
    L.fa_status_string.argtypes = [i]
    L.fa_status_string.restype = ctypes.c_char_p
    L.fa_describe.argtypes = [i, i, i]
    L.fa_describe.restype = ctypes.c_char_p
    _lib = L
    return L


def dtype_code(t) -> int:
    import torch
    codes = {torch.bfloat16: FA_BF16, torch.float16: FA_F16, torch.float32: FA_F32}
    if t not in codes:
        raise ValueError("unsupported dtype %s" % t)
    return codes[t]


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _dims(Q, K):
    if Q.dim() != 4 or K.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    B, H, Nq, d = Q.shape
    _need(K.shape[0] == B and K.shape[1] == H and K.shape[3] == d,
          "K must be [B, H, Nk, d] with Q's B, H and d (Q %s, K %s)" % (tuple(Q.shape), tuple(K.shape)))
    return B, H, Nq, K.shape[2], d


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check(Q, K, V, O, LSE, dO=None, dQ=None, dK=None, dV=None, extra=()):
    """Every check the C ABI cannot make on device pointers: shapes (K and V
    [B, H, Nk, d] with Q's B, H and d; O, dO, dQ shaped like Q; dK, dV like K;
    LSE float32 [B, H, Nq]), one shared dtype, contiguous device tensors on one
    device.  Shapes and dtypes are checked first, so a mistake is reported
    before anything touches a device.  Returns (B, H, Nq, Nk, d)."""
    B, H, Nq, Nk, d = _dims(Q, K)
    _need(V.shape == K.shape, "V must have K's shape (K %s, V %s)" % (tuple(K.shape), tuple(V.shape)))
    for name, t in (("O", O), ("dO", dO), ("dQ", dQ)):
        if t is not None:
            _need(t.shape == Q.shape, "%s must have Q's shape (Q %s, %s %s)" % (name, tuple(Q.shape), name,
                                                                                tuple(t.shape)))
    for name, t in (("dK", dK), ("dV", dV)):
        if t is not None:
            _need(t.shape == K.shape, "%s must have K's shape (K %s, %s %s)" % (name, tuple(K.shape), name,
                                                                                tuple(t.shape)))
    _need(tuple(LSE.shape) == (B, H, Nq), "LSE must be [B, H, Nq] = %s, got %s" % ((B, H, Nq), tuple(LSE.shape)))
    _need(str(LSE.dtype) == "torch.float32", "LSE must be float32, got %s" % LSE.dtype)
    tensors = [t for t in (Q, K, V, O, dO, dQ, dK, dV) if t is not None]
    _need(len({t.dtype for t in tensors}) == 1, "Q, K, V, O (and dO, dQ, dK, dV) must share a dtype")
    dtype_code(Q.dtype)
    devs = set()
    for t in tensors + [LSE] + [t for t in extra if t is not None]:
        _need(t.is_cuda and t.is_contiguous(), "tensors must be contiguous device tensors")
        devs.add(t.device)
    _need(len(devs) == 1, "all tensors must be on one device")
    return B, H, Nq, Nk, d


def fa_fwd(Q, K, V, O, LSE, scale=None, causal=False, stream=None) -> None:
    B, H, Nq, Nk, d = _check(Q, K, V, O, LSE)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(LSE), B, H, Nq, Nk, d, float(scale),
                      int(bool(causal)), dtype_code(Q.dtype), _stream_handle(stream))
    if st != FA_OK:
        raise FaError(st, "fa_fwd")


def fa_fwd_workspace_size(B, H, Nq, Nk, d) -> int:
    return int(lib().fa_fwd_workspace_size(B, H, Nq, Nk, d))


def fa_fwd_ws(Q, K, V, O, LSE, workspace, scale=None, causal=False, stream=None) -> None:
    B, H, Nq, Nk, d = _check(Q, K, V, O, LSE, extra=(workspace,))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nbytes = workspace.numel() * workspace.element_size()
    st = lib().fa_fwd_ws(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(LSE), B, H, Nq, Nk, d, float(scale),
                         int(bool(causal)), dtype_code(Q.dtype), _ptr(workspace), nbytes, _stream_handle(stream))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_ws")


def fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, num_splits) -> int:
    return int(lib().fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, int(num_splits)))


def fa_fwd_num_splits(B, H, Nq, Nk, d, causal=False) -> int:
    return int(lib().fa_fwd_num_splits(B, H, Nq, Nk, d, int(bool(causal))))


def fa_fwd_splitkv(Q, K, V, O, LSE, num_splits, workspace, scale=None, causal=False, stream=None) -> None:
    B, H, Nq, Nk, d = _check(Q, K, V, O, LSE, extra=(workspace,))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    wptr = _ptr(workspace) if workspace is not None else ctypes.c_void_p(0)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().fa_fwd_splitkv(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(LSE), B, H, Nq, Nk, d, float(scale),
                              int(bool(causal)), dtype_code(Q.dtype), int(num_splits), wptr, nbytes,
                              _stream_handle(stream))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_splitkv")


def fa_dropout_threshold(dropout_p) -> int:
    return int(lib().fa_dropout_threshold(float(dropout_p)))


def fa_fwd_dropout(Q, K, V, O, LSE, dropout_p, seed, scale=None, causal=False, stream=None) -> None:
    B, H, Nq, Nk, d = _check(Q, K, V, O, LSE)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd_dropout(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(LSE), B, H, Nq, Nk, d, float(scale),
                              int(bool(causal)), dtype_code(Q.dtype), float(dropout_p),
                              ctypes.c_ulonglong(int(seed) & (2 ** 64 - 1)), _stream_handle(stream))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_dropout")


def fa_bwd_dropout(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, dropout_p, seed, scale=None, causal=False,
                   stream=None) -> None:
    args = list(_bwd_args(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, scale, causal, stream))
    # _bwd_args ends with (..., dtype, workspace, nbytes, stream): the rate and seed go before the workspace
    head, tail = args[:17], args[17:]
    st = lib().fa_bwd_dropout(*head, float(dropout_p), ctypes.c_ulonglong(int(seed) & (2 ** 64 - 1)), *tail)
    if st != FA_OK:
        raise FaError(st, "fa_bwd_dropout")


def fa_bwd_workspace_size(B, H, Nq, Nk, d) -> int:
    return int(lib().fa_bwd_workspace_size(B, H, Nq, Nk, d))


def _bwd_args(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, scale, causal, stream):
    B, H, Nq, Nk, d = _check(Q, K, V, O, LSE, dO, dQ, dK, dV, extra=(workspace,))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nbytes = workspace.numel() * workspace.element_size()
    return (_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(LSE), _ptr(dQ), _ptr(dK), _ptr(dV),
            B, H, Nq, Nk, d, float(scale), int(bool(causal)), dtype_code(Q.dtype), _ptr(workspace), nbytes,
            _stream_handle(stream))


def fa_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, scale=None, causal=False, stream=None) -> None:
    st = lib().fa_bwd(*_bwd_args(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, scale, causal, stream))
    if st != FA_OK:
        raise FaError(st, "fa_bwd")


FA_NOALLOC_MAX_ROWS = 4 * 1024 * 1024  # include/fa.h


def fa_bwd_noalloc(Q, K, V, O, dO, LSE, dQ, dK, dV, scale=None, causal=False, stream=None) -> None:
    """fa_bwd without a workspace: D lives in the library's fixed device array
    (calls that overlap on one GPU race; B*H*Nq <= FA_NOALLOC_MAX_ROWS)."""
    B, H, Nq, Nk, d = _check(Q, K, V, O, LSE, dO, dQ, dK, dV)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_bwd_noalloc(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(LSE), _ptr(dQ), _ptr(dK),
                              _ptr(dV), B, H, Nq, Nk, d, float(scale), int(bool(causal)), dtype_code(Q.dtype),
                              _stream_handle(stream))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_noalloc")


def fa_bwd_num_stages() -> int:
    return int(lib().fa_bwd_num_stages())


def fa_bwd_stage(stage, Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, scale=None, causal=False, stream=None) -> None:
    st = lib().fa_bwd_stage(int(stage), *_bwd_args(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, scale, causal,
                                                   stream))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_stage")


def fa_build_info() -> str:
    return lib().fa_build_info().decode()


def fa_status_string(status: int) -> str:
    return lib().fa_status_string(int(status)).decode()


def fa_describe(d: int, dtype: int, causal: bool) -> str:
    return lib().fa_describe(int(d), int(dtype), int(bool(causal))).decode()


# ------------------------------------------------------------------ helpers

def forward(Q, K, V, scale=None, causal=False, stream=None):
    """Allocate O and LSE, run fa_fwd, return (O, LSE)."""
    import torch
    B, H, Nq, Nk, d = _dims(Q, K)
    O = torch.empty_like(Q)
    LSE = torch.empty((B, H, Nq), device=Q.device, dtype=torch.float32)
    fa_fwd(Q, K, V, O, LSE, scale, causal, stream)
    return O, LSE


def forward_splitkv(Q, K, V, scale=None, causal=False, stream=None, num_splits=None):
    """Allocate O, LSE and the split-KV workspace, run fa_fwd_splitkv (with
    fa_fwd_num_splits' choice unless num_splits is given), return (O, LSE)."""
    import torch
    B, H, Nq, Nk, d = _dims(Q, K)
    if num_splits is None:
        num_splits = fa_fwd_num_splits(B, H, Nq, Nk, d, causal)
    O = torch.empty_like(Q)
    LSE = torch.empty((B, H, Nq), device=Q.device, dtype=torch.float32)
    n = fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, num_splits)
    ws = torch.empty(max(n, 1), device=Q.device, dtype=torch.uint8) if n > 0 else None
    fa_fwd_splitkv(Q, K, V, O, LSE, num_splits, ws, scale, causal, stream)
    return O, LSE


def alloc_workspace(Q, K):
    import torch
    B, H, Nq, Nk, d = _dims(Q, K)
    n = fa_bwd_workspace_size(B, H, Nq, Nk, d)
    return torch.empty(n, device=Q.device, dtype=torch.uint8)


def backward(Q, K, V, O, dO, LSE, scale=None, causal=False, stream=None, workspace=None):
    """Allocate dQ, dK, dV (and the workspace unless given), run fa_bwd."""
    import torch
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    if workspace is None:
        workspace = alloc_workspace(Q, K)
    fa_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, scale, causal, stream)
    return dQ, dK, dV
