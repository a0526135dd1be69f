"""Backward parity on the GPU: libfa's fa_fwd + fa_bwd (through the C ABI)
against the fp64 oracle's analytic gradients on identical seeded inputs."""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
import tiled_online_softmax_03_amd as fa
from gpu_util import check_grads, check_rows, oracle_view, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.lib()


def _run(inp, scale, causal):
    O, LSE = fa.forward(inp["Q"], inp["K"], inp["V"], scale, causal)
    dQ, dK, dV = fa.backward(inp["Q"], inp["K"], inp["V"], O, inp["dO"], LSE, scale, causal)
    torch.cuda.synchronize()
    return O, LSE, dQ, dK, dV


def _ref(inp, scale, causal, heads=None):
    """Oracle gradients, for all heads or for a list of flattened (b, h) heads."""
    t = {k: inp[k] for k in ("Q", "K", "V", "dO")}
    if heads is not None:
        t = {k: v.reshape(-1, 1, v.shape[2], v.shape[3])[heads] for k, v in t.items()}
    dQ, dK, dV, _, _ = oracle.bwd(oracle_view(t["Q"]), oracle_view(t["K"]), oracle_view(t["V"]),
                                  oracle_view(t["dO"]), scale, causal)
    return {"dQ": dQ, "dK": dK, "dV": dV}


def _got(dQ, dK, dV, heads=None):
    g = {"dQ": dQ, "dK": dK, "dV": dV}
    if heads is not None:
        g = {k: v.reshape(-1, 1, v.shape[2], v.shape[3])[heads] for k, v in g.items()}
    return {k: to_np(v) for k, v in g.items()}


SHAPES = [
    (1, 1, 1, 1, 64),
    (1, 2, 1, 300, 128),
    (1, 1, 77, 5, 64),
    (2, 1, 130, 130, 128),
    (1, 3, 129, 257, 64),
    (1, 2, 200, 333, 128),
    (1, 1, 383, 129, 64),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_ragged(shape, causal, dtype):
    B, H, Nq, Nk, d = shape
    seed = zlib.crc32(repr((shape, causal, dtype, "bwd")).encode()) % 10000
    inp = synth.make_inputs(B, H, Nq, Nk, d, dtype, seed, device="cuda")
    scale = 1.0 / math.sqrt(d)
    say("bwd ragged", shape, dtype, causal)
    O, LSE, dQ, dK, dV = _run(inp, scale, causal)
    check_grads(_got(dQ, dK, dV), _ref(inp, scale, causal), "ragged")


def test_workload_tiny_f32():
    w = synth.WORKLOADS["tiny_f32"]
    inp = synth.workload_inputs(w, device="cuda")
    say("bwd", w.name)
    O, LSE, dQ, dK, dV = _run(inp, w.scale, w.causal)
    check_grads(_got(dQ, dK, dV), _ref(inp, w.scale, w.causal), w.name)


def test_workload_cross_f16():
    w = synth.WORKLOADS["cross_1024x8192_f16"]
    inp = synth.workload_inputs(w, device="cuda")
    say("bwd", w.name, "full size; oracle on sampled heads")
    O, LSE, dQ, dK, dV = _run(inp, w.scale, w.causal)
    heads = [0, 37, 63]
    check_grads(_got(dQ, dK, dV, heads), _ref(inp, w.scale, w.causal, heads), w.name)


# Heads of the training shape checked against the oracle: four on each of the
# eight XCDs.  The non-causal grids give each XCD a contiguous range of 32 heads
# (xcd_remap), so head h runs on XCD h // 32; the picks include the first and
# last head of every range and two heads inside it (32 heads, 1/8 of the 256).
TRAIN_HEADS = sorted(32 * x + o for x in range(8) for o in (0, 31, 10 + x, 21 + x))


def test_workload_train():
    w = synth.WORKLOADS["train_b8h32n4096d128"]
    inp = synth.workload_inputs(w, device="cuda")
    say("bwd", w.name, "full size; oracle on %d heads over the 8 XCD placements" % len(TRAIN_HEADS))
    O, LSE, dQ, dK, dV = _run(inp, w.scale, w.causal)
    got, ref = _got(dQ, dK, dV, TRAIN_HEADS), _ref(inp, w.scale, w.causal, TRAIN_HEADS)
    check_grads(got, ref, w.name)
    check_rows(got, ref, w.name)
    _all_head_invariants(inp, O, dK, dV, w.scale)


def _all_head_invariants(inp, O, dK, dV, scale):
    """Two identities of exact attention over every head, with bounds that
    follow the kernels' rounding steps (research-attention section 01's
    softmax rows sum to 1; the softmax gradient of a row sums to 0):

      sum_j dV_j = sum_i dO_i: P is rounded to bf16 before the product (2^-9
      relative each, and each row of P sums to 1) and every dV element is
      stored in bf16 (2^-9 relative), so per column
        |sum_j dV_jc - sum_i dO_ic| <= 2^-9 (sum_i |dO_ic| + sum_j |dV_jc|).

      sum_j dK_j = 0: sum_j dK_jc = scale sum_i Q_ic sum_j dS_ij, and
      sum_j dS_ij (as the kernel uses it) deviates from 0 by D's error (D is
      formed from the bf16-stored O: |D - D*| <= sum_c |dO_ic| |O_ic - O*_ic|,
      with |O - O*| <= 2^-7 |O| for the stored output) plus the bf16 rounding
      of dS (2^-9 sum_j |dS_ij|, and sum_j |dS_ij| <= ||dO_i|| max_j ||V_j||
      + |D_i| since the P_ij sum to 1); the bf16 stores add 2^-9 sum_j |dK_jc|.
    Everything is float64 on the GPU; a factor 1.25 covers the fp32
    accumulation and exponential."""
    f = lambda t: t.double()
    Q, V, dO, Od = f(inp["Q"]), f(inp["V"]), f(inp["dO"]), f(O)
    dVd, dKd = f(dV), f(dK)
    u = 2.0 ** -9
    lhs_v = (dVd.sum(2) - dO.sum(2)).abs()
    bound_v = 1.25 * u * (dO.abs().sum(2) + dVd.abs().sum(2))
    D = (dO * Od).sum(-1)
    dD = (dO.abs() * (2.0 ** -7) * Od.abs()).sum(-1)
    vmax = V.norm(dim=-1).amax(dim=-1, keepdim=True)
    row = dD + u * (dO.norm(dim=-1) * vmax + D.abs())
    bound_k = 1.25 * (scale * (Q.abs() * row.unsqueeze(-1)).sum(2) + u * dKd.abs().sum(2))
    lhs_k = dKd.sum(2).abs()
    rv = (lhs_v / bound_v).max().item()
    rk = (lhs_k / bound_k).max().item()
    say("    all heads: sum dV = sum dO within %.3g of its bound, sum dK = 0 within %.3g of its bound" % (rv, rk))
    assert rv <= 1.0 and rk <= 1.0, (rv, rk)


def test_bwd_deterministic():
    inp = synth.make_inputs(2, 2, 300, 260, 128, "bf16", 9, device="cuda")
    _, _, dQ1, dK1, dV1 = _run(inp, 0.1, False)
    for _ in range(3):
        _, _, dQ2, dK2, dV2 = _run(inp, 0.1, False)
        assert torch.equal(dK1, dK2) and torch.equal(dV1, dV2) and torch.equal(dQ1, dQ2)


@pytest.mark.parametrize("d,dtype,causal", [(64, "f16", True), (128, "bf16", False), (128, "f16", True)])
def test_stages_equal_fa_bwd(d, dtype, causal):
    """fa_bwd_stage(0..n-1) in order is exactly fa_bwd.  At d = 128 on 16-bit
    data stage 0 is the dQ pass (which forms D) and stage 1 the dK/dV pass, so
    those two alone already give fa_bwd's bits and stage 2 changes nothing."""
    inp = synth.make_inputs(1, 3, 333, 200, d, dtype, 11, device="cuda")
    say("bwd stages", (1, 3, 333, 200, d, dtype, causal))
    O, LSE, dQ, dK, dV = _run(inp, 0.125, causal)
    ws = fa.alloc_workspace(inp["Q"], inp["K"])
    sQ, sK, sV = (torch.full_like(t, float("nan")) for t in (dQ, dK, dV))
    for st in range(fa.fa_bwd_num_stages()):
        fa.fa_bwd_stage(st, inp["Q"], inp["K"], inp["V"], O, inp["dO"], LSE, sQ, sK, sV, ws, 0.125, causal)
        torch.cuda.synchronize()
        if d == 128 and st == 0:
            assert torch.equal(sQ, dQ), "stage 0 writes dQ on this path"
            assert torch.isnan(sK).all() and torch.isnan(sV).all()
        if d == 128 and st == 1:
            assert torch.equal(sK, dK) and torch.equal(sV, dV), "stage 1 writes dK, dV on this path"
    assert torch.equal(sQ, dQ) and torch.equal(sK, dK) and torch.equal(sV, dV)
