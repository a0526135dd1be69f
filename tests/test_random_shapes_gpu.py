"""Seeded random shapes through the whole path: fa_fwd_ws against fa_fwd bit
for bit (at d = 128 on 16-bit data the former runs the 64-row key loop, the
latter the eight-wave one), the forward against the fp64 oracle, and fa_bwd's
gradients (the one-wave-per-SIMD dK/dV and dQ passes at d = 128) against the
oracle's.  The sizes are drawn to land off every tile boundary: query rows
that leave a wave's 64 rows or a workgroup's 256 partly empty, key counts
below, at and past one or several 64-key tiles, causal with Nq above and
below Nk."""
import math
import random

import numpy as np
import pytest
import torch

import oracle
import synth
import tiled_online_softmax_03_amd as fa
from gpu_util import check_forward, check_grads, oracle_view, say, to_np

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "f16": torch.float16}


def _cases(n=24, seed=20261203):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        d = rng.choice([64, 128, 128])
        dtype = rng.choice(["bf16", "f16"])
        causal = rng.random() < 0.5
        B, H = rng.choice([1, 2]), rng.choice([1, 2, 3])
        Nq = rng.choice([rng.randint(1, 70), rng.randint(60, 300), rng.randint(250, 700)])
        Nk = rng.choice([rng.randint(1, 70), rng.randint(60, 400), rng.randint(350, 1300)])
        out.append((B, H, Nq, Nk, d, dtype, causal, 5000 + i))
    return out


CASES = _cases()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.lib()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%dx%dx%dx%dx%d-%s-%s" % (c[:6] + ("causal" if c[6] else "full",)))
def test_random_shape(case):
    B, H, Nq, Nk, d, dtype, causal, seed = case
    inp = synth.make_inputs(B, H, Nq, Nk, d, dtype, seed, device="cuda")
    Q, K, V, dO = inp["Q"], inp["K"], inp["V"], inp["dO"]
    scale = 1.0 / math.sqrt(d)
    say("random shape", case)
    O, LSE = fa.forward(Q, K, V, scale, causal)
    ws = torch.empty(fa.fa_fwd_workspace_size(B, H, Nq, Nk, d), device="cuda", dtype=torch.uint8)
    O2, L2 = torch.empty_like(O), torch.empty_like(LSE)
    fa.fa_fwd_ws(Q, K, V, O2, L2, ws, scale, causal)
    dQ, dK, dV = fa.backward(Q, K, V, O, dO, LSE, scale, causal)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(LSE, L2), "fa_fwd_ws differs from fa_fwd"

    q, k, v, do = oracle_view(Q), oracle_view(K), oracle_view(V), oracle_view(dO)
    dQr, dKr, dVr, Or, Lr = oracle.bwd(q, k, v, do, scale, causal)
    Ar, _ = oracle.fwd(q, k, np.abs(v), scale, causal)
    check_forward(to_np(O), to_np(LSE), Or, Lr, DT[dtype], "random", Ar, Nk, float(np.abs(v).max()),
                  max_abs_bar="auto")
    check_grads({"dQ": to_np(dQ), "dK": to_np(dK), "dV": to_np(dV)}, {"dQ": dQr, "dK": dKr, "dV": dVr}, "random")
