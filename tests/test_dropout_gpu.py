"""Dropout parity on the GPU: fa_fwd_dropout and fa_bwd_dropout (through the
C ABI) against the fp64 oracle run under the oracle's own keep mask -- the
oracle's Philox4x32-10 and the kernels' are separate implementations of the
generator's published definition, so matching results also show the masks
agree.  Two tests compare the masks themselves, bit for bit: one-hot V makes
O equal to the dropped probabilities (forward mask), one-hot dO makes dV
equal to their transpose (the mask the dK/dV pass draws again)."""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
import tiled_online_softmax_03_amd as fa
from gpu_util import check_forward, check_grads, oracle_view, say, to_np, zero_grad_bound

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.lib()


def _rate(p):
    t = fa.fa_dropout_threshold(p)
    assert t >= 0
    return t, (256.0 / (256 - t) if t else 1.0)


def _fwd(inp, p, seed, scale, causal):
    Q, K, V = inp["Q"], inp["K"], inp["V"]
    O = torch.empty_like(Q)
    LSE = torch.empty(Q.shape[:3], device=Q.device, dtype=torch.float32)
    fa.fa_fwd_dropout(Q, K, V, O, LSE, p, seed, scale, causal)
    return O, LSE


def _bwd(inp, O, LSE, p, seed, scale, causal):
    Q, K, V, dO = inp["Q"], inp["K"], inp["V"], inp["dO"]
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    fa.fa_bwd_dropout(Q, K, V, O, dO, LSE, dQ, dK, dV, fa.alloc_workspace(Q, K), p, seed, scale, causal)
    torch.cuda.synchronize()
    return dQ, dK, dV


def _check_head_set(inp, O, LSE, grads, p, seed, scale, causal, label, heads=None):
    """Oracle forward and backward under its own mask, for all heads or the
    listed flattened heads, against the GPU results."""
    t, ks = _rate(p)
    B, H, Nq, d = inp["Q"].shape
    Nk = inp["K"].shape[2]
    BH = B * H
    heads = list(range(BH)) if heads is None else heads
    flat = lambda x: x.reshape(BH, 1, x.shape[2], x.shape[3])
    Og, Lg, Or, Lr, Ar = [], [], [], [], []
    got = {"dQ": [], "dK": [], "dV": []}
    ref = {"dQ": [], "dK": [], "dV": []}
    vmax = 0.0
    for h in heads:
        q, k, v = (oracle_view(flat(inp[n])[h:h + 1]) for n in ("Q", "K", "V"))
        keep = oracle.dropout_keep(1, 1, Nq, Nk, t, seed, bh0=h)
        o_ref, l_ref = oracle.fwd_dropout(q, k, v, keep, ks, scale, causal)
        a_ref, _ = oracle.fwd_dropout(q, k, np.abs(v), keep, ks, scale, causal)
        vmax = max(vmax, float(np.abs(v).max()))
        Og.append(to_np(flat(O)[h:h + 1]))
        Lg.append(to_np(LSE.reshape(BH, 1, Nq)[h:h + 1]))
        Or.append(o_ref)
        Lr.append(l_ref)
        Ar.append(a_ref)
        if grads is not None:
            do = oracle_view(flat(inp["dO"])[h:h + 1])
            dq, dk, dv, _, _ = oracle.bwd_dropout(q, k, v, do, keep, ks, scale, causal)
            for n, r in (("dQ", dq), ("dK", dk), ("dV", dv)):
                ref[n].append(r)
                got[n].append(to_np(flat(grads[n])[h:h + 1]))
    # the elementwise bound: P~ = P / (1 - rate) multiplies the fp16 rounding terms
    check_forward(np.concatenate(Og), np.concatenate(Lg), np.concatenate(Or), np.concatenate(Lr),
                  inp["Q"].dtype, label, np.concatenate(Ar), Nk, vmax * ks, max_abs_bar="auto")
    if grads is not None:
        zero = zero_grad_bound(to_np(O), to_np(inp["dO"]), to_np(inp["K"]), to_np(inp["Q"]), scale, inp["Q"].dtype)
        check_grads({n: np.concatenate(v) for n, v in got.items()}, {n: np.concatenate(v) for n, v in ref.items()},
                    label, zero_abs=zero)


SHAPES = [
    (1, 1, 1, 1, 64),
    (1, 2, 1, 300, 128),
    (1, 1, 77, 5, 64),
    (2, 1, 130, 130, 128),
    (1, 3, 129, 257, 64),
    (1, 2, 200, 333, 128),
]


@pytest.mark.parametrize("p", [0.1, 0.5])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_ragged(shape, causal, dtype, p):
    B, H, Nq, Nk, d = shape
    seed = zlib.crc32(repr(("dropout", shape, causal, dtype, p)).encode())
    inp = synth.make_inputs(B, H, Nq, Nk, d, dtype, seed % 10000, device="cuda")
    scale = 1.0 / math.sqrt(d)
    say("dropout", shape, dtype, "causal" if causal else "", "p", p, "seed", seed)
    O, LSE = _fwd(inp, p, seed, scale, causal)
    dQ, dK, dV = _bwd(inp, O, LSE, p, seed, scale, causal)
    _check_head_set(inp, O, LSE, {"dQ": dQ, "dK": dK, "dV": dV}, p, seed, scale, causal, "ragged")


@pytest.mark.parametrize("causal", [False, True])
def test_forward_mask_exact(causal):
    """V_j = e_j (one-hot value rows): O_ij = P_ij Z_ij / (1 - rate) is zero
    exactly where the element was dropped (or masked); every P_ij is far from
    underflow for N(0,1) logits, so the nonzero pattern is Z itself."""
    B, H, Nq, Nk, d = 2, 3, 300, 128, 128
    p, seed = 0.3, 0x5eed_0001_0203
    inp = synth.make_inputs(B, H, Nq, Nk, d, "bf16", 11, device="cuda", with_dO=False)
    inp["V"] = torch.eye(Nk, d, dtype=torch.bfloat16, device="cuda").expand(B, H, Nk, d).contiguous()
    O, _ = _fwd(inp, p, seed, 1.0 / math.sqrt(d), causal)
    torch.cuda.synchronize()
    keep = oracle.dropout_keep(B, H, Nq, Nk, _rate(p)[0], seed).astype(bool)
    if causal:
        keep &= np.tril(np.ones((Nq, Nk), dtype=bool))
    assert np.array_equal(to_np(O)[..., :Nk] != 0, keep)


def test_backward_mask_exact():
    """dO_i = e_i (one-hot gradient rows, Nq <= d): dV_jc = P~_cj, so the
    nonzero pattern of dV is the transposed keep mask the dK/dV pass drew."""
    B, H, Nq, Nk, d = 1, 2, 128, 300, 128
    p, seed = 0.25, 987654321
    inp = synth.make_inputs(B, H, Nq, Nk, d, "bf16", 12, device="cuda")
    inp["dO"] = torch.eye(Nq, d, dtype=torch.bfloat16, device="cuda").expand(B, H, Nq, d).contiguous()
    scale = 1.0 / math.sqrt(d)
    O, LSE = _fwd(inp, p, seed, scale, False)
    dQ, dK, dV = _bwd(inp, O, LSE, p, seed, scale, False)
    keep = oracle.dropout_keep(B, H, Nq, Nk, _rate(p)[0], seed).astype(bool)
    assert np.array_equal(to_np(dV)[..., :Nq] != 0, np.swapaxes(keep, 2, 3))


def test_zero_rate_is_plain():
    """A rate below 1/512 rounds to t = 0: exactly fa_fwd / fa_bwd."""
    inp = synth.make_inputs(1, 2, 200, 333, 128, "bf16", 13, device="cuda")
    O, LSE = _fwd(inp, 0.001, 5, 0.1, False)
    dQ, dK, dV = _bwd(inp, O, LSE, 0.001, 5, 0.1, False)
    O2, L2 = fa.forward(inp["Q"], inp["K"], inp["V"], 0.1)
    g2 = fa.backward(inp["Q"], inp["K"], inp["V"], O2, inp["dO"], L2, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(LSE, L2)
    for a, b in zip((dQ, dK, dV), g2):
        assert torch.equal(a, b)


def test_seed_determinism():
    inp = synth.make_inputs(1, 2, 300, 400, 64, "f16", 14, device="cuda")
    O1, L1 = _fwd(inp, 0.2, 42, 0.125, False)
    g1 = _bwd(inp, O1, L1, 0.2, 42, 0.125, False)
    O2, L2 = _fwd(inp, 0.2, 42, 0.125, False)
    g2 = _bwd(inp, O2, L2, 0.2, 42, 0.125, False)
    O3, _ = _fwd(inp, 0.2, 43, 0.125, False)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and all(torch.equal(a, b) for a, b in zip(g1, g2))
    assert not torch.equal(O1, O3)
    assert torch.equal(L1, _fwd(inp, 0.2, 43, 0.125, False)[1])  # LSE does not see the mask


def test_workload_train_dropout():
    """The training shape (B8 H32 N4096 d128 bf16) with rate 0.1: full-size
    launches, two whole heads checked against the oracle."""
    w = synth.WORKLOADS["train_b8h32n4096d128"]
    inp = synth.workload_inputs(w, device="cuda")
    p, seed = 0.1, 20260101
    say("dropout", w.name, "full size, p", p)
    O, LSE = _fwd(inp, p, seed, w.scale, w.causal)
    dQ, dK, dV = _bwd(inp, O, LSE, p, seed, w.scale, w.causal)
    _check_head_set(inp, O, LSE, {"dQ": dQ, "dK": dK, "dV": dV}, p, seed, w.scale, w.causal, w.name,
                    heads=[0, w.B * w.H - 1])


def test_workload_cross_dropout():
    w = synth.WORKLOADS["cross_1024x8192_f16"]
    inp = synth.workload_inputs(w, device="cuda")
    p, seed = 0.2, 77
    say("dropout", w.name, "full size, p", p)
    O, LSE = _fwd(inp, p, seed, w.scale, w.causal)
    dQ, dK, dV = _bwd(inp, O, LSE, p, seed, w.scale, w.causal)
    _check_head_set(inp, O, LSE, {"dQ": dQ, "dK": dK, "dV": dV}, p, seed, w.scale, w.causal, w.name,
                    heads=[0, 37, 63])
