"""Split-KV forward parity on the GPU: fa_fwd_splitkv (through the C ABI)
against the fp64 oracle on identical seeded inputs.  The result must be the
same attention as fa_fwd's, so the oracle is the plain definition; the cases
stress what the split adds -- key ranges that are empty, ranges whose keys
are all masked for some rows (causal), ranges ending at a ragged key tail --
and the merge of the partial states."""
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
    fa.lib()


def _run(inp, scale, causal, G):
    O, LSE = fa.forward_splitkv(inp["Q"], inp["K"], inp["V"], scale, causal, num_splits=G)
    torch.cuda.synchronize()
    return O, LSE


def _full_check(B, H, Nq, Nk, d, dtype, causal, G, seed, sigma=1.0, label="", max_abs_bar=True):
    inp = synth.make_inputs(B, H, Nq, Nk, d, dtype, seed, sigma, device="cuda", with_dO=False)
    scale = 1.0 / math.sqrt(d)
    say("splitkv", label, (B, H, Nq, Nk, d, dtype, causal), "splits", G)
    O, LSE = _run(inp, scale, causal, G)
    q, k, v = oracle_view(inp["Q"]), oracle_view(inp["K"]), oracle_view(inp["V"])
    O_ref, LSE_ref = oracle.fwd(q, k, v, scale, causal)
    A_ref, _ = oracle.fwd(q, k, np.abs(v), scale, causal)
    return check_forward(to_np(O), to_np(LSE), O_ref, LSE_ref, DT[dtype], label, A_ref, Nk, float(np.abs(v).max()),
                         max_abs_bar)


CASES = [
    # B, H, Nq, Nk, d, splits
    (1, 1, 1, 1, 64, 2),        # one key: every range but the first is empty
    (1, 2, 1, 300, 64, 3),      # ragged tail inside the last range
    (1, 1, 77, 5, 128, 4),
    (2, 1, 130, 130, 128, 2),
    (1, 3, 129, 257, 64, 5),    # more ranges than whole tiles allow: empty ranges
    (1, 2, 200, 333, 128, 7),
    (1, 1, 383, 129, 64, 16),
    (2, 2, 64, 700, 64, 11),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES, ids=lambda s: "x".join(map(str, s)))
def test_ragged(case, causal, dtype):
    B, H, Nq, Nk, d, G = case
    seed = zlib.crc32(repr(("splitkv", case, causal, dtype)).encode()) % 10000
    _full_check(B, H, Nq, Nk, d, dtype, causal, G, seed, label="ragged")


@pytest.mark.parametrize("G", [1, 2, 4])
def test_worked_row(G):
    g = json.load(open(os.path.join(GOLDEN, "online_row_example.json")))
    s, v = np.array(g["scores"]), np.array(g["values"])
    pad = lambda x: np.concatenate([x, np.zeros(x.shape[:-1] + (64 - x.shape[-1],))], -1)
    Q = pad(np.array([[1.0, 0.0]]))[None, None]
    K = pad(np.stack([s, np.zeros(4)], 1))[None, None]
    V = pad(v)[None, None]
    t = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda().contiguous()
    O, LSE = _run({"Q": t(Q), "K": t(K), "V": t(V)}, 1.0, False, G)
    assert np.max(np.abs(to_np(O)[0, 0, 0, :2] - g["result"])) <= 1e-2


def test_wide_logits():
    """sigma 4 logits: the running maximum differs strongly between ranges,
    so the merge's rescaling factors span many orders of magnitude."""
    _full_check(1, 2, 256, 1500, 64, "f16", False, 6, seed=91, sigma=4.0, label="wide logits", max_abs_bar=False)
    _full_check(1, 2, 300, 300, 128, "bf16", True, 3, seed=92, sigma=4.0, label="wide logits causal",
                max_abs_bar=False)


@pytest.mark.parametrize("G", [None, 8, 64])
def test_workload_single_head_fwd(G):
    """The single-head 4096 x 4096 d64 forward: 16 query tiles, the shape
    split-KV exists for.  None = the library's own split choice."""
    w = synth.WORKLOADS["single_head_fwd"]
    if G is None:
        G = fa.fa_fwd_num_splits(w.B, w.H, w.Nq, w.Nk, w.d, w.causal)
        assert G > 1
    _full_check(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.causal, G, w.seed, w.sigma_qk, w.name)


def _sampled(w, G, rows_per_head, heads):
    inp = synth.workload_inputs(w, device="cuda", with_dO=False)
    say("splitkv", w.name, "full size", (w.B, w.H, w.Nq, w.Nk, w.d), "splits", G)
    O, LSE = _run(inp, w.scale, w.causal, G)
    BH = w.B * w.H
    rows = synth.sample_rows(w.Nq, BH, rows_per_head)
    Og, Lg, Or, Lr, Ar = [], [], [], [], []
    vmax = 0.0
    for h in heads:
        r = torch.tensor(rows[h], device="cuda")
        q = oracle_view(inp["Q"].reshape(BH, w.Nq, w.d)[h])[None, None]
        k = oracle_view(inp["K"].reshape(BH, w.Nk, w.d)[h])[None, None]
        v = oracle_view(inp["V"].reshape(BH, w.Nk, w.d)[h])[None, None]
        rr = np.array(rows[h])[None]
        o_ref, l_ref = oracle.fwd_rows(q, k, v, rr, w.scale, w.causal)
        a_ref, _ = oracle.fwd_rows(q, k, np.abs(v), rr, w.scale, w.causal)
        vmax = max(vmax, float(np.abs(v).max()))
        Og.append(to_np(O.reshape(BH, w.Nq, w.d)[h][r]))
        Lg.append(to_np(LSE.reshape(BH, w.Nq)[h][r]))
        Or.append(o_ref.reshape(len(rows[h]), w.d))
        Lr.append(l_ref.reshape(len(rows[h])))
        Ar.append(a_ref.reshape(len(rows[h]), w.d))
    check_forward(np.concatenate(Og), np.concatenate(Lg), np.concatenate(Or), np.concatenate(Lr), w.torch_dtype,
                  w.name, np.concatenate(Ar), w.Nk, vmax)


def test_workload_cross_f16():
    """The cross-attention stress shape (1024 queries against 8192 keys, wide
    fp16 logits), split four ways."""
    w = synth.WORKLOADS["cross_1024x8192_f16"]
    _sampled(w, 4, rows_per_head=64, heads=[0, 17, 63])


def test_causal_long():
    """Causal 4096 x 4096 d128 in 8 ranges: early query tiles have whole
    ranges above the diagonal, rows inside a range may see no allowed key."""
    w = synth.Workload("causal_4096_d128", 1, 2, 4096, 4096, 128, "bf16", True, False, 4321)
    _sampled(w, 8, rows_per_head=128, heads=[0, 1])


def test_deterministic():
    inp = synth.make_inputs(1, 2, 300, 2000, 128, "bf16", 6, device="cuda", with_dO=False)
    O1, L1 = _run(inp, 0.1, False, 5)
    for _ in range(3):
        O2, L2 = _run(inp, 0.1, False, 5)
        assert torch.equal(O1, O2) and torch.equal(L1, L2)
