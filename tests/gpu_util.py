"""Helpers for the GPU parity tests: how the oracle sees the inputs, the
tolerances, and error metrics.  Imported only by tests."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

# Tolerances (attention forward/backward against the fp64 oracle).
O_MAX_ABS = 1e-2      # O, elementwise, against the fp64 oracle
O_REL_L2 = 1e-3       # O, relative L2, against the oracle rounded (RNE) to O's storage dtype
LSE_MAX_ABS = 1e-3    # LSE, natural-log units
GRAD_REL_L2 = 5e-3    # dQ, dK, dV, relative L2 against the fp64 oracle


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_view(t: torch.Tensor) -> np.ndarray:
    """The values the kernels compute with, widened to float64 on the host:
    16-bit tensors exactly; float32 tensors after RNE rounding to bf16 (the
    FA_F32 mode rounds every matrix-core operand to bf16)."""
    t = t.detach().to("cpu")
    if t.dtype == torch.float32:
        t = t.to(torch.bfloat16)
    return t.double().numpy()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def round_like(x: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """The fp64 oracle rounded (RNE) to a storage dtype, back in float64."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).double().numpy()


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))


def max_abs(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.max(np.abs(a - b))) if a.size else 0.0


REL_L2_MIN_ELEMS = 16384  # rel-L2 over fewer outputs is dominated by single rounding flips

_MANT = {torch.bfloat16: (7, -133), torch.float16: (10, -24), torch.float32: (23, -149)}


def half_ulp(x: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Half a unit in the last place of |x| in a storage dtype."""
    mant, min_exp = _MANT[dtype]
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -140)))
    return 0.5 * np.exp2(np.maximum(e - mant, min_exp))


def elementwise_bound(O_ref, A_ref, dtype, n_keys, v_max):
    """A-priori bound on |O_gpu - O_ref| from the kernel's arithmetic: the
    output rounding (half an ulp of the storage dtype), the probabilities
    rounded to fp16 (2^-11 relative, doubled for the fp32 exponential and
    accumulation), and fp16 subnormal probabilities (2^-25 absolute each).
    A_ref = sum_j P_ij |V_jc|, computed by the oracle."""
    return half_ulp(np.abs(O_ref) + 2.0 ** -10 * A_ref, dtype) + 2.0 ** -10 * A_ref \
        + n_keys * 2.0 ** -25 * v_max + 1e-7


def check_forward(O_gpu, LSE_gpu, O_ref, LSE_ref, dtype, label="", A_ref=None, n_keys=0, v_max=0.0,
                  max_abs_bar=True):
    """Assert the forward tolerances; returns the measured errors.

    Always: O max-abs <= 1e-2 and LSE max-abs <= 1e-3 against the fp64
    oracle.  O rel-L2 <= 1e-3 against the oracle rounded (RNE) to O's dtype
    when O has at least REL_L2_MIN_ELEMS elements.  With A_ref, every element
    also within elementwise_bound().  max_abs_bar=False drops the 1e-2
    max-abs bar for stress inputs whose outputs exceed 2 in magnitude, where
    half an ulp of bf16 alone is 7.8e-3 or more; max_abs_bar="auto" applies
    the bar to the elements with |O| < 4 only (dropout scales O by
    1 / (1 - rate), so few-key rows exceed 4, where half a bf16 ulp is 1.6e-2)."""
    assert np.all(np.isfinite(O_gpu)) and np.all(np.isfinite(LSE_gpu)), label
    e = {
        "O_max_abs": max_abs(O_gpu, O_ref),
        "O_rel_l2_vs_rounded": rel_l2(O_gpu, round_like(O_ref, dtype)),
        "O_rel_l2_vs_fp64": rel_l2(O_gpu, O_ref),
        "LSE_max_abs": max_abs(LSE_gpu, LSE_ref),
    }
    if A_ref is not None:
        bound = elementwise_bound(O_ref, A_ref, dtype, n_keys, v_max)
        e["worst_err_over_bound"] = float(np.max(np.abs(O_gpu - O_ref) / bound))
    say("   ", label, "n=%d" % O_gpu.size, " ".join("%s=%.3g" % kv for kv in e.items()))
    if max_abs_bar == "auto":
        # the bar where half an ulp of the storage dtype stays below it (|O| < 4)
        small = np.abs(O_ref) < 4.0
        e["O_max_abs_below_4"] = max_abs(O_gpu[small], O_ref[small]) if np.any(small) else 0.0
        assert e["O_max_abs_below_4"] <= O_MAX_ABS, (label, e)
    elif max_abs_bar:
        assert e["O_max_abs"] <= O_MAX_ABS, (label, e)
    assert e["LSE_max_abs"] <= LSE_MAX_ABS, (label, e)
    if O_gpu.size >= REL_L2_MIN_ELEMS:
        assert e["O_rel_l2_vs_rounded"] <= O_REL_L2, (label, e)
    if A_ref is not None:
        assert e["worst_err_over_bound"] <= 1.0, (label, e)
    return e


def check_grads(got, ref, label="", zero_abs=1e-4):
    """got/ref: dicts name -> array for dQ, dK, dV.  rel-L2 <= 5e-3 against
    the fp64 oracle; a gradient that is identically zero in exact arithmetic
    (e.g. dQ and dK with a single key) must come out within zero_abs of zero
    (1e-4 by default; callers whose stored O is not exact pass the bound that
    O's rounding implies, see zero_grad_bound)."""
    e = {}
    for k in ("dQ", "dK", "dV"):
        assert np.all(np.isfinite(got[k])), (label, k)
        if np.linalg.norm(ref[k]) == 0.0:
            e[k + "_max_abs"] = float(np.max(np.abs(got[k]))) if got[k].size else 0.0
        else:
            e[k + "_rel_l2"] = rel_l2(got[k], ref[k])
    say("   ", label, " ".join("%s=%.3g" % kv for kv in e.items()))
    for k, v in e.items():
        assert v <= (GRAD_REL_L2 if k.endswith("rel_l2") else zero_abs), (label, k, e)
    return e


def zero_grad_bound(O, dO, K, Q, scale, dtype):
    """Bound on dQ and dK where they vanish in exact arithmetic: the kernel's
    D_i = rowsum(dO_i * O_i) uses O as stored, so D_i is off by up to
    sum_c |dO_ic| * half_ulp(O_ic); dS_ij = P_ij (dP_ij - D_i) inherits that,
    and dQ_i = scale sum_j dS_ij K_j, dK_j = scale sum_i dS_ij Q_i (P rows sum
    to at most the keep scale).  Twice that, and never below 1e-4."""
    dD = np.max(np.sum(np.abs(dO) * half_ulp(np.abs(O), dtype), axis=-1))
    return max(1e-4, 2.0 * scale * dD * 4.0 * max(float(np.max(np.abs(K))), float(np.max(np.abs(Q)))) * O.shape[-2])


def scale_of(d):
    return 1.0 / math.sqrt(d)


ROW_REL = 1.5e-2  # per-row relative L2 error of a gradient row (global bar 5e-3)


def check_rows(got, ref, label="", bar=ROW_REL):
    """Per-row relative error of each gradient (rows of dQ, dK, dV: the last
    axis is the head dim).  Every row must satisfy
        ||got_row - ref_row|| <= bar * max(||ref_row||, median row norm / 4)
    so a single wrong row fails even where the global rel-L2 (dominated by
    millions of correct elements) would not; the floor keeps rows whose exact
    gradient is nearly zero from failing on rounding alone.  Returns the worst
    ratio per tensor."""
    worst = {}
    for k in ("dQ", "dK", "dV"):
        g = got[k].reshape(-1, got[k].shape[-1])
        r = ref[k].reshape(-1, ref[k].shape[-1])
        err = np.linalg.norm(g - r, axis=1)
        nrm = np.linalg.norm(r, axis=1)
        floor = max(float(np.median(nrm)) / 4.0, 1e-30)
        ratio = err / np.maximum(nrm, floor)
        worst[k] = float(np.max(ratio))
        worst[k + "_row"] = int(np.argmax(ratio))
    say("    per-row", label, " ".join("%s=%.3g" % (k, v) for k, v in worst.items() if not k.endswith("_row")))
    for k in ("dQ", "dK", "dV"):
        assert worst[k] <= bar, (label, k, worst)
    return worst
