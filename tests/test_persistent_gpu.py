"""The persistent passes.  On non-causal launches at d = 128 on 16-bit data
the forward key loop (fwd_r64_kernel), the dQ pass and the dK/dV pass run one
workgroup per compute unit, each walking the work items it * grid + w and
copying the next item's operands while the current one computes.  These
shapes put the item counts just above and at about twice the compute-unit
count (so some workgroups run one item, others two or three), with odd step
counts (the LDS stage of an item's first tile alternates) and ragged query and
key edges.  Every item's result must not depend on which workgroup ran it or
what that workgroup ran before: sampled heads, among them heads whose items
ran second on their workgroup, must equal bit for bit the same head run alone
(one item per workgroup); the whole batch is checked against the fp64 oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
import tiled_online_softmax_03_amd as fa
from gpu_util import check_forward, check_grads, oracle_view, say, to_np

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.lib()


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _cases():
    cu = _cus() if torch.cuda.is_available() else 256
    return [
        # forward and dQ: H query tiles (one each); dK/dV: 2 H key blocks of 3 steps
        (1, cu + 1, 130, 131, "bf16", 301),
        # forward and dQ: 2 B H query tiles of 5 key tiles; dK/dV: B H key blocks of 5 steps
        (2, cu // 2 + 3, 300, 320, "f16", 302),
    ]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "B%dH%d-%dx%d-%s" % c[:5])
def test_persistent_items(case):
    B, H, Nq, Nk, dtype, seed = case
    d = 128
    inp = synth.make_inputs(B, H, Nq, Nk, d, dtype, seed, device="cuda")
    Q, K, V, dO = inp["Q"], inp["K"], inp["V"], inp["dO"]
    scale = 1.0 / math.sqrt(d)
    say("persistent items", case, "compute units", _cus())
    O, LSE = fa.forward(Q, K, V, scale, False)
    ws = torch.empty(fa.fa_fwd_workspace_size(B, H, Nq, Nk, d), device="cuda", dtype=torch.uint8)
    O2, L2 = torch.empty_like(O), torch.empty_like(LSE)
    fa.fa_fwd_ws(Q, K, V, O2, L2, ws, scale, False)
    dQ, dK, dV = fa.backward(Q, K, V, O, dO, LSE, scale, False)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(LSE, L2), "fa_fwd_ws differs from fa_fwd"

    q, k, v, do = oracle_view(Q), oracle_view(K), oracle_view(V), oracle_view(dO)
    dQr, dKr, dVr, Or, Lr = oracle.bwd(q, k, v, do, scale, False)
    Ar, _ = oracle.fwd(q, k, np.abs(v), scale, False)
    check_forward(to_np(O2), to_np(L2), Or, Lr, DT[dtype], "persistent", Ar, Nk, float(np.abs(v).max()),
                  max_abs_bar="auto")
    check_grads({"dQ": to_np(dQ), "dK": to_np(dK), "dV": to_np(dV)}, {"dQ": dQr, "dK": dKr, "dV": dVr},
                "persistent")

    # the same heads alone: with B H = 1 every workgroup runs one item
    BH = B * H
    cu = _cus()
    heads = sorted({0, 1, BH // 3, cu // 2 + 1, BH - 2, BH - 1})
    flat = lambda t: t.reshape(BH, *t.shape[2:])
    for h in heads:
        one = lambda t: flat(t)[h][None, None].contiguous()
        q1, k1, v1, do1 = one(Q), one(K), one(V), one(dO)
        O1, L1 = fa.forward(q1, k1, v1, scale, False)
        ws1 = torch.empty(fa.fa_fwd_workspace_size(1, 1, Nq, Nk, d), device="cuda", dtype=torch.uint8)
        O1w, L1w = torch.empty_like(O1), torch.empty_like(L1)
        fa.fa_fwd_ws(q1, k1, v1, O1w, L1w, ws1, scale, False)
        dQ1, dK1, dV1 = fa.backward(q1, k1, v1, O1, do1, L1, scale, False)
        torch.cuda.synchronize()
        for name, big, alone in (("O", O2, O1w), ("LSE", L2, L1w), ("dQ", dQ, dQ1), ("dK", dK, dK1), ("dV", dV, dV1)):
            assert torch.equal(flat(big)[h], alone[0, 0]), "head %d: %s differs from the head run alone" % (h, name)
    say("    heads", heads, "equal bit for bit to the same heads run alone")
