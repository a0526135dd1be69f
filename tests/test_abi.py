"""The C ABI on the host: the library loads, exports every symbol include/fa.h
declares, and rejects bad arguments before touching the GPU (CPU only; no
call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import tiled_online_softmax_03_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return fa.lib()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert names == ["fa_build_info", "fa_bwd", "fa_bwd_dropout", "fa_bwd_noalloc", "fa_bwd_num_stages", "fa_bwd_stage",
                     "fa_bwd_workspace_size",
                     "fa_describe", "fa_dropout_threshold", "fa_fwd", "fa_fwd_dropout", "fa_fwd_num_splits",
                     "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_size", "fa_fwd_workspace_size", "fa_fwd_ws",
                     "fa_status_string"]
    for n in names:
        assert hasattr(lib, n), n


def test_build_info(lib):
    s = fa.fa_build_info()
    assert s.startswith("HIP ") and "clang" in s and "gfx950" in s


def test_status_strings(lib):
    assert fa.fa_status_string(0) == "FA_OK"
    assert fa.fa_status_string(1) == "FA_ERR_INVALID_ARG"
    assert fa.fa_status_string(2) == "FA_ERR_UNSUPPORTED"
    assert fa.fa_status_string(3) == "FA_ERR_HIP"
    assert fa.fa_status_string(99) == "FA_UNKNOWN_STATUS"


def test_describe(lib):
    # the whole description fits: it names every kernel of a step, the last one included,
    # and ends with the backward's closing clause (a truncated copy would not)
    for d in (64, 128):
        for dt in (0, 1, 2):
            for c in (0, 1):
                s = fa.fa_describe(d, dt, c)
                assert ("d=%d" % d) in s and ("causal=%d" % c) in s
                for k in ("fwd_kernel", "v_pack_kernel", "bwd_pre_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"):
                    assert k in s, (k, s)
                assert s.endswith("no atomics"), s
                assert len(s) < 2047, len(s)
    assert fa.fa_describe(96, 0, 0) == "unsupported"
    assert fa.fa_describe(64, 7, 0) == "unsupported"


def test_workspace_size(lib):
    B, H, Nq, Nk, d = 2, 3, 100, 50, 64
    rows = B * H * Nq
    pad = lambda n: (n + 255) // 256 * 256
    assert fa.fa_bwd_workspace_size(B, H, Nq, Nk, d) == pad(rows * 4)
    assert fa.fa_bwd_workspace_size(0, H, Nq, Nk, d) == 0
    assert fa.fa_bwd_workspace_size(B, H, Nq, -1, d) == 0


# Fake, aligned, never-dereferenced addresses: every case below fails validation.
P = ctypes.c_void_p(0x10000)
MIS = ctypes.c_void_p(0x10008)
NULL = ctypes.c_void_p(0)


def _fwd(lib, Q=P, O=P, B=1, H=1, Nq=8, Nk=8, d=64, scale=0.125, dtype=0):
    return lib.fa_fwd(Q, P, P, O, P, B, H, Nq, Nk, d, scale, 0, dtype, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(Q=NULL), fa.FA_ERR_INVALID_ARG),
    (dict(O=NULL), fa.FA_ERR_INVALID_ARG),
    (dict(Q=MIS), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(H=-1), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-0.5), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=3), fa.FA_ERR_UNSUPPORTED),
    (dict(B=1 << 14, H=1 << 10, Nq=1 << 10), fa.FA_ERR_UNSUPPORTED),
])
def test_fwd_rejects(lib, kw, status):
    assert _fwd(lib, **kw) == status


def _bwd(lib, ws=P, ws_bytes=1 << 40, dQ=P, d=64, dtype=0, Nq=8):
    return lib.fa_bwd(P, P, P, P, P, P, dQ, P, P, 1, 1, Nq, 8, d, 0.125, 0, dtype, ws, ws_bytes, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(ws=NULL), fa.FA_ERR_INVALID_ARG),
    (dict(ws=ctypes.c_void_p(0x10010)), fa.FA_ERR_INVALID_ARG),  # not 256-byte aligned
    (dict(ws_bytes=16), fa.FA_ERR_INVALID_ARG),
    (dict(dQ=NULL), fa.FA_ERR_INVALID_ARG),
    (dict(dQ=MIS), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=-1), fa.FA_ERR_UNSUPPORTED),
])
def test_bwd_rejects(lib, kw, status):
    assert _bwd(lib, **kw) == status


def test_fwd_workspace_size(lib):
    # fp16 V^T tiles of 64 keys (d = 128) or 128 keys (d = 64), the last one padded
    pad = lambda n: (n + 255) // 256 * 256
    assert fa.fa_fwd_workspace_size(2, 3, 100, 130, 128) == pad(2 * 3 * 3 * 64 * 128 * 2)
    assert fa.fa_fwd_workspace_size(2, 3, 100, 130, 64) == pad(2 * 3 * 2 * 128 * 64 * 2)
    assert fa.fa_fwd_workspace_size(1, 1, 1, 1, 64) == 128 * 64 * 2
    assert fa.fa_fwd_workspace_size(0, 3, 100, 130, 64) == 0
    assert fa.fa_fwd_workspace_size(2, 3, 100, 130, 96) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(ws=NULL), fa.FA_ERR_INVALID_ARG),
    (dict(ws=ctypes.c_void_p(0x10010)), fa.FA_ERR_INVALID_ARG),  # not 256-byte aligned
    (dict(ws_bytes=128 * 64 * 2 - 1), fa.FA_ERR_INVALID_ARG),
    (dict(Q=MIS), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=5), fa.FA_ERR_UNSUPPORTED),
])
def test_fwd_ws_rejects(lib, kw, status):
    a = dict(Q=P, ws=P, ws_bytes=1 << 40, Nk=8, d=64, dtype=0)
    a.update(kw)
    assert lib.fa_fwd_ws(a["Q"], P, P, P, P, 1, 1, 8, a["Nk"], a["d"], 0.125, 0, a["dtype"], a["ws"], a["ws_bytes"],
                         NULL) == status


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    Q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device"):
        fa.forward(Q, Q, Q)


def _t(*shape, dtype=None):
    import torch
    return torch.zeros(*shape, dtype=dtype or torch.bfloat16)


@pytest.mark.parametrize("case", ["K_batch", "K_heads", "K_dim", "V_shape", "O_shape", "LSE_shape", "LSE_dtype",
                                  "dtype_mix"])
def test_binding_checks_forward_shapes(case):
    # every shape or dtype mistake is a ValueError raised before any pointer reaches the
    # library (CPU tensors: the check must come before the device check)
    torch = pytest.importorskip("torch")
    B, H, Nq, Nk, d = 2, 3, 8, 5, 64
    t = dict(Q=_t(B, H, Nq, d), K=_t(B, H, Nk, d), V=_t(B, H, Nk, d), O=_t(B, H, Nq, d),
             LSE=_t(B, H, Nq, dtype=torch.float32))
    bad = {"K_batch": ("K", _t(1, H, Nk, d)), "K_heads": ("K", _t(B, 1, Nk, d)), "K_dim": ("K", _t(B, H, Nk, 128)),
           "V_shape": ("V", _t(B, H, Nk + 1, d)), "O_shape": ("O", _t(B, H, Nq - 1, d)),
           "LSE_shape": ("LSE", _t(B, H, Nq + 1, dtype=torch.float32)), "LSE_dtype": ("LSE", _t(B, H, Nq)),
           "dtype_mix": ("V", _t(B, H, Nk, d, dtype=torch.float16))}[case]
    t[bad[0]] = bad[1]
    for call in (lambda: fa.fa_fwd(t["Q"], t["K"], t["V"], t["O"], t["LSE"]),
                 lambda: fa.fa_fwd_ws(t["Q"], t["K"], t["V"], t["O"], t["LSE"], _t(1024, dtype=torch.uint8)),
                 lambda: fa.fa_fwd_splitkv(t["Q"], t["K"], t["V"], t["O"], t["LSE"], 2, _t(1024, dtype=torch.uint8)),
                 lambda: fa.fa_fwd_dropout(t["Q"], t["K"], t["V"], t["O"], t["LSE"], 0.1, 7)):
        with pytest.raises(ValueError) as e:
            call()
        assert "device" not in str(e.value), e.value


@pytest.mark.parametrize("case", ["dO_shape", "dQ_shape", "dK_shape", "dV_shape", "LSE_shape", "LSE_dtype",
                                  "K_batch", "dtype_mix"])
def test_binding_checks_backward_shapes(case):
    torch = pytest.importorskip("torch")
    B, H, Nq, Nk, d = 2, 3, 8, 5, 64
    t = dict(Q=_t(B, H, Nq, d), K=_t(B, H, Nk, d), V=_t(B, H, Nk, d), O=_t(B, H, Nq, d), dO=_t(B, H, Nq, d),
             LSE=_t(B, H, Nq, dtype=torch.float32), dQ=_t(B, H, Nq, d), dK=_t(B, H, Nk, d), dV=_t(B, H, Nk, d))
    bad = {"dO_shape": ("dO", _t(B, H, Nq, 128)), "dQ_shape": ("dQ", _t(B, H, Nk, d)),
           "dK_shape": ("dK", _t(B, H, Nq, d)), "dV_shape": ("dV", _t(B, 1, Nk, d)),
           "LSE_shape": ("LSE", _t(1, H, Nq, dtype=torch.float32)), "LSE_dtype": ("LSE", _t(B, H, Nq)),
           "K_batch": ("K", _t(1, H, Nk, d)), "dtype_mix": ("dK", _t(B, H, Nk, d, dtype=torch.float16))}[case]
    t[bad[0]] = bad[1]
    ws = _t(1 << 16, dtype=torch.uint8)
    a = [t[k] for k in ("Q", "K", "V", "O", "dO", "LSE", "dQ", "dK", "dV")]
    for call in (lambda: fa.fa_bwd(*a, ws), lambda: fa.fa_bwd_stage(1, *a, ws),
                 lambda: fa.fa_bwd_dropout(*a, ws, 0.1, 7)):
        with pytest.raises(ValueError) as e:
            call()
        assert "device" not in str(e.value), e.value


def test_bwd_stages(lib):
    assert fa.fa_bwd_num_stages() == 3
    args = (P, P, P, P, P, P, P, P, P, 1, 1, 8, 8, 64, 0.125, 0, 0, P, 1 << 40, NULL)
    assert lib.fa_bwd_stage(3, *args) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_bwd_stage(-1, *args) == fa.FA_ERR_INVALID_ARG
    bad = (P, P, P, P, P, P, NULL, P, P, 1, 1, 8, 8, 64, 0.125, 0, 0, P, 1 << 40, NULL)
    assert lib.fa_bwd_stage(1, *bad) == fa.FA_ERR_INVALID_ARG


def test_splitkv_workspace_size(lib):
    B, H, Nq, Nk, d = 2, 3, 100, 50, 64
    pad = lambda n: (n + 255) // 256 * 256
    for G in (2, 5, 256):
        rows = B * H * Nq * G
        assert fa.fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, G) == pad(rows * d * 4) + 2 * pad(rows * 4)
    assert fa.fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, 1) == 0  # one range is fa_fwd: no workspace
    for G in (0, -3, 257):
        assert fa.fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, G) == 0
    assert fa.fa_fwd_splitkv_workspace_size(B, 0, Nq, Nk, d, 4) == 0


def _split(lib, G=4, ws=P, ws_bytes=1 << 40, B=1, Q=P, d=64, scale=0.125):
    return lib.fa_fwd_splitkv(Q, P, P, P, P, B, 1, 8, 8, d, scale, 0, 0, G, ws, ws_bytes, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(G=0), fa.FA_ERR_INVALID_ARG),
    (dict(G=-1), fa.FA_ERR_INVALID_ARG),
    (dict(G=257), fa.FA_ERR_INVALID_ARG),
    (dict(G=1, B=0), fa.FA_ERR_INVALID_ARG),          # one range: fa_fwd's own checks
    (dict(ws=NULL), fa.FA_ERR_INVALID_ARG),
    (dict(ws=ctypes.c_void_p(0x10010)), fa.FA_ERR_INVALID_ARG),  # not 256-byte aligned
    (dict(ws_bytes=256), fa.FA_ERR_INVALID_ARG),
    (dict(Q=NULL), fa.FA_ERR_INVALID_ARG),
    (dict(Q=MIS), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
])
def test_splitkv_rejects(lib, kw, status):
    assert _split(lib, **kw) == status


def test_num_splits(lib):
    # one head of 4096 queries: 16 query tiles -> 8 ranges of 8 key tiles
    assert fa.fa_fwd_num_splits(1, 1, 4096, 4096, 64, False) == 8
    # 32 heads of 128 queries against 32768 keys: 32 workgroups -> 8 ranges
    assert fa.fa_fwd_num_splits(1, 32, 128, 32768, 128, False) == 8
    # 4096 query tiles already fill 256 CUs
    assert fa.fa_fwd_num_splits(8, 32, 4096, 4096, 128, False) == 1
    assert fa.fa_fwd_num_splits(4, 16, 1024, 8192, 64, False) == 1
    # a single query row against 8192 keys, 8 heads: 8 workgroups -> 16 ranges (8 tiles each)
    assert fa.fa_fwd_num_splits(1, 8, 1, 8192, 128, False) == 16
    # causal: no row sees keys past Nq - 1, so a long key sequence does not add ranges
    assert fa.fa_fwd_num_splits(1, 8, 1, 8192, 128, True) == 1
    assert fa.fa_fwd_num_splits(1, 1, 4096, 4096, 64, True) == 8
    assert fa.fa_fwd_num_splits(1, 1, 1024, 8192, 128, True) == 2
    # too few keys to split
    assert fa.fa_fwd_num_splits(1, 1, 64, 100, 64, False) == 1
    assert fa.fa_fwd_num_splits(0, 1, 64, 100, 64, False) == 0
    assert fa.fa_fwd_num_splits(1, 1, 64, 100, 80, False) == 0


def test_dropout_threshold(lib):
    # the rate is realised in 1/256 steps, rounded to nearest
    assert fa.fa_dropout_threshold(0.0) == 0
    assert fa.fa_dropout_threshold(0.0019) == 0    # below 1/512: no dropout
    assert fa.fa_dropout_threshold(0.1) == 26      # 25.6 -> 26
    assert fa.fa_dropout_threshold(0.5) == 128
    assert fa.fa_dropout_threshold(0.999) == 255   # capped: 255/256
    for bad in (-0.1, 1.0, 1.5, float("nan"), float("inf")):
        assert fa.fa_dropout_threshold(bad) == -1


def test_dropout_rejects(lib):
    u64 = ctypes.c_ulonglong(7)
    fwd = lambda p, B=1: lib.fa_fwd_dropout(P, P, P, P, P, B, 1, 8, 8, 64, 0.125, 0, 0, p, u64, NULL)
    assert fwd(-0.5) == fa.FA_ERR_INVALID_ARG
    assert fwd(1.0) == fa.FA_ERR_INVALID_ARG
    assert fwd(float("nan")) == fa.FA_ERR_INVALID_ARG
    assert fwd(0.1, B=0) == fa.FA_ERR_INVALID_ARG
    bwd = lambda p, ws=P: lib.fa_bwd_dropout(P, P, P, P, P, P, P, P, P, 1, 1, 8, 8, 64, 0.125, 0, 0, p, u64, ws,
                                             1 << 40, NULL)
    assert bwd(1.2) == fa.FA_ERR_INVALID_ARG
    assert bwd(0.1, ws=NULL) == fa.FA_ERR_INVALID_ARG


def test_noalloc_rejects(lib):
    # argument problems come back before the library looks up its device array
    # (nothing here initialises the GPU)
    ok = (P, P, P, P, P, P, P, P, P, 1, 1, 8, 8, 64, 0.125, 0, 0, NULL)
    bad = lambda i, v: tuple(v if k == i else a for k, a in enumerate(ok))
    assert lib.fa_bwd_noalloc(*bad(6, NULL)) == fa.FA_ERR_INVALID_ARG     # dQ null
    assert lib.fa_bwd_noalloc(*bad(0, MIS)) == fa.FA_ERR_INVALID_ARG      # Q misaligned
    assert lib.fa_bwd_noalloc(*bad(9, 0)) == fa.FA_ERR_INVALID_ARG        # B = 0
    assert lib.fa_bwd_noalloc(*bad(14, float("inf"))) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_bwd_noalloc(*bad(13, 80)) == fa.FA_ERR_UNSUPPORTED      # d
    assert lib.fa_bwd_noalloc(*bad(11, fa.FA_NOALLOC_MAX_ROWS + 1)) == fa.FA_ERR_UNSUPPORTED  # rows past the array
