"""Forward parity on the GPU: libfa's fa_fwd (through the C ABI) against the
fp64 oracle on identical seeded inputs."""
import json
import math
import os
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
import tiled_online_softmax_03_amd as fa
from gpu_util import check_forward, oracle_view, say, to_np

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.lib()  # loud failure if the library is missing


def _run_fwd(inp, scale, causal):
    O, LSE = fa.forward(inp["Q"], inp["K"], inp["V"], scale, causal)
    torch.cuda.synchronize()
    return O, LSE


def _full_check(B, H, Nq, Nk, d, dtype, causal, seed, sigma=1.0, label="", max_abs_bar=True):
    inp = synth.make_inputs(B, H, Nq, Nk, d, dtype, seed, sigma, device="cuda", with_dO=False)
    scale = 1.0 / math.sqrt(d)
    say("fwd", label, (B, H, Nq, Nk, d, dtype, causal))
    O, LSE = _run_fwd(inp, scale, causal)
    q, k, v = oracle_view(inp["Q"]), oracle_view(inp["K"]), oracle_view(inp["V"])
    O_ref, LSE_ref = oracle.fwd(q, k, v, scale, causal)
    A_ref, _ = oracle.fwd(q, k, np.abs(v), scale, causal)
    return check_forward(to_np(O), to_np(LSE), O_ref, LSE_ref, DT[dtype], label, A_ref, Nk, float(np.abs(v).max()),
                         max_abs_bar)


# ---------------------------------------------------------------- the pages' worked examples

def _pad(x, d):
    out = np.zeros(x.shape[:-1] + (d,))
    out[..., : x.shape[-1]] = x
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_worked_row(dtype, d):
    g = json.load(open(os.path.join(GOLDEN, "online_row_example.json")))
    s, v = np.array(g["scores"]), np.array(g["values"])
    Q = _pad(np.array([[1.0, 0.0]]), d)[None, None]
    K = _pad(np.stack([s, np.zeros(4)], 1), d)[None, None]
    V = _pad(v, d)[None, None]
    t = lambda x: torch.from_numpy(x).to(DT[dtype]).cuda().contiguous()
    O, LSE = _run_fwd({"Q": t(Q), "K": t(K), "V": t(V)}, 1.0, False)
    O_ref, LSE_ref = oracle.fwd(Q, K, V, 1.0)
    A_ref, _ = oracle.fwd(Q, K, np.abs(V), 1.0)
    check_forward(to_np(O), to_np(LSE), O_ref, LSE_ref, DT[dtype], "worked row", A_ref, 4, 2.0)
    # the page's printed result (6 decimals), to the output dtype's resolution
    assert np.max(np.abs(to_np(O)[0, 0, 0, :2] - g["result"])) <= 1e-2


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_four_token_example(dtype, causal):
    g = json.load(open(os.path.join(GOLDEN, "four_token_example.json")))
    X = _pad(np.array(g["X"]), 64)[None, None]
    t = torch.from_numpy(X).to(DT[dtype]).cuda().contiguous()
    scale = 1.0 / math.sqrt(2.0)
    O, LSE = _run_fwd({"Q": t, "K": t, "V": t}, scale, causal)
    O_ref, LSE_ref = oracle.fwd(X, X, X, scale, causal)
    A_ref, _ = oracle.fwd(X, X, np.abs(X), scale, causal)
    check_forward(to_np(O), to_np(LSE), O_ref, LSE_ref, DT[dtype], "4-token", A_ref, 4, 1.0)
    if not causal:
        Og = to_np(O)[0, 0]
        assert np.max(np.abs(Og[0, :2] - g["token0"])) <= 1e-2
        assert np.max(np.abs(Og[1, :2] - g["token1"])) <= 1e-2
        assert np.all(Og[:, 2:] == 0.0)  # zero padding stays zero


# ---------------------------------------------------------------- ragged and degenerate shapes

SHAPES = [
    # B, H, Nq, Nk, d
    (1, 1, 1, 1, 64),
    (1, 2, 1, 300, 64),
    (1, 1, 77, 5, 128),
    (2, 1, 130, 130, 128),
    (1, 3, 129, 257, 64),
    (1, 2, 200, 333, 128),
    (2, 2, 64, 64, 64),
    (1, 1, 383, 129, 64),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_ragged(shape, causal, dtype):
    B, H, Nq, Nk, d = shape
    _full_check(B, H, Nq, Nk, d, dtype, causal, seed=zlib.crc32(repr((shape, causal, dtype)).encode()) % 10000, label="ragged")


def test_large_logits_rescale():
    """Wide logits (sigma 4 on Q and K) force many running-max updates and
    near-one-hot rows, whose outputs are single value rows of magnitude up to
    ~4.5: checked against the elementwise arithmetic bound and rel-L2."""
    _full_check(1, 2, 256, 700, 64, "f16", False, seed=77, sigma=4.0, label="wide logits", max_abs_bar=False)
    _full_check(1, 2, 256, 256, 128, "bf16", True, seed=78, sigma=4.0, label="wide logits causal",
                max_abs_bar=False)


# ---------------------------------------------------------------- the evaluation workloads

def test_workload_tiny_f32():
    w = synth.WORKLOADS["tiny_f32"]
    _full_check(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.causal, w.seed, w.sigma_qk, w.name)


def test_workload_single_head_fwd():
    w = synth.WORKLOADS["single_head_fwd"]
    _full_check(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.causal, w.seed, w.sigma_qk, w.name)


def _run_fwd_ws(inp, scale, causal):
    """fa_fwd_ws (V packed once into the workspace), the forward bench.py times for Nq >= 2048."""
    Q, K = inp["Q"], inp["K"]
    B, H, Nq, d = Q.shape
    ws = torch.empty(fa.fa_fwd_workspace_size(B, H, Nq, K.shape[2], d), device="cuda", dtype=torch.uint8)
    O = torch.empty_like(Q)
    LSE = torch.empty((B, H, Nq), device="cuda", dtype=torch.float32)
    fa.fa_fwd_ws(Q, K, inp["V"], O, LSE, ws, scale, causal)
    torch.cuda.synchronize()
    return O, LSE


def _sampled_check(w, rows_per_head, heads=None, label="", run=_run_fwd):
    """Full-size launch; the oracle evaluates sampled query rows one by one."""
    inp = synth.workload_inputs(w, device="cuda", with_dO=False)
    say("fwd", label or w.name, "full size", (w.B, w.H, w.Nq, w.Nk, w.d))
    O, LSE = run(inp, w.scale, w.causal)
    BH = w.B * w.H
    heads = list(range(BH)) if heads is None else heads
    rows = synth.sample_rows(w.Nq, BH, rows_per_head)
    Qf = inp["Q"].reshape(BH, w.Nq, w.d)
    Kf = inp["K"].reshape(BH, w.Nk, w.d)
    Vf = inp["V"].reshape(BH, w.Nk, w.d)
    Og, Lg, Or, Lr, Ar = [], [], [], [], []
    vmax = 0.0
    for h in heads:
        r = torch.tensor(rows[h], device="cuda")
        q = oracle_view(Qf[h])[None, None]
        k = oracle_view(Kf[h])[None, None]
        v = oracle_view(Vf[h])[None, None]
        rr = np.array(rows[h])[None]
        o_ref, l_ref = oracle.fwd_rows(q, k, v, rr, w.scale, w.causal)
        a_ref, _ = oracle.fwd_rows(q, k, np.abs(v), rr, w.scale, w.causal)
        vmax = max(vmax, float(np.abs(v).max()))
        Og.append(to_np(O.reshape(BH, w.Nq, w.d)[h][r]))
        Lg.append(to_np(LSE.reshape(BH, w.Nq)[h][r]))
        Or.append(o_ref.reshape(len(rows[h]), w.d))
        Lr.append(l_ref.reshape(len(rows[h])))
        Ar.append(a_ref.reshape(len(rows[h]), w.d))
    return check_forward(np.concatenate(Og), np.concatenate(Lg), np.concatenate(Or), np.concatenate(Lr),
                         w.torch_dtype, label or w.name, np.concatenate(Ar), w.Nk, vmax)


def test_workload_cross_f16_fwd():
    _sampled_check(synth.WORKLOADS["cross_1024x8192_f16"], rows_per_head=64)


def test_workload_train_fwd():
    w = synth.WORKLOADS["train_b8h32n4096d128"]
    _sampled_check(w, rows_per_head=16, heads=list(range(0, w.B * w.H, 3)))


def test_workload_long_causal():
    """B1 H32 N65536 d128 causal at full size: 256 seeded query rows of every
    head against the oracle (rows 0, 1 and N-1 always among them)."""
    w = synth.WORKLOADS["long_causal_n65536"]
    _sampled_check(w, rows_per_head=256)


@pytest.mark.parametrize("name,rows,step", [("long_causal_n65536", 256, 1), ("train_b8h32n4096d128", 16, 3),
                                            ("single_head_fwd", 256, 1)])
def test_workload_fwd_ws(name, rows, step):
    """The same full-size checks through fa_fwd_ws, the launch bench.py times for these workloads."""
    w = synth.WORKLOADS[name]
    _sampled_check(w, rows_per_head=rows, heads=list(range(0, w.B * w.H, step)), label=w.name + " fa_fwd_ws",
                   run=_run_fwd_ws)


def test_deterministic():
    inp = synth.make_inputs(2, 4, 500, 700, 128, "bf16", 5, device="cuda", with_dO=False)
    O1, L1 = _run_fwd(inp, 0.1, False)
    for _ in range(3):
        O2, L2 = _run_fwd(inp, 0.1, False)
        assert torch.equal(O1, O2) and torch.equal(L1, L2)


def test_o_rel_l2_headroom():
    """The O rel-L2 bar (1e-3 against the oracle rounded to bf16) at the
    training shape, with its headroom tracked.  P feeds the P V product as
    fp16, 2^-12 relative rounding per element; the rows' O is a random-walk
    average of V (|O| ~ |V| / sqrt(effective keys)), so that rounding moves
    O by about 2^-12 of itself, some 6 % of a bf16 output ulp, and about that
    share of outputs lands on the neighbouring bf16 value: rel-L2 8.5e-4 on
    this config.  A change that adds error anywhere in the forward shows up
    here before it reaches the bar."""
    w = synth.WORKLOADS["train_b8h32n4096d128"]
    e = _sampled_check(w, rows_per_head=32, heads=list(range(0, w.B * w.H, 2)), label="headroom")
    assert e["O_rel_l2_vs_rounded"] <= 9.5e-4, e
