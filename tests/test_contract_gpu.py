"""Documented limits of the input contract (include/fa.h), pinned on the GPU.

The forward forms P V on the fp16 matrix core: V is converted to fp16 there.
Every bf16 value from 2^-14 up to 65280 (the largest bf16 number below
65504, the largest fp16) has an exact fp16 image, so inside that range the
result is the oracle's; 65536 and beyond turn into infinity and the rows that
weight that key come out non-finite.  The contract says |V| <= 65504, and this
test holds the library to both halves of that statement.  The backward forms dV, dP with bf16
operands and is not limited by it."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
import tiled_online_softmax_03_amd as fa
from gpu_util import check_forward, oracle_view, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.lib()


def _inputs(vfill, seed):
    B, H, N, d = 1, 2, 200, 128
    inp = synth.make_inputs(B, H, N, N, d, "bf16", seed, device="cuda", with_dO=False)
    V = inp["V"].clone()
    V[:, :, 7, :5] = torch.tensor(vfill, dtype=torch.float32).to(torch.bfloat16)
    V[:, :, 150, 3] = -torch.tensor(vfill[0], dtype=torch.float32).to(torch.bfloat16)
    inp["V"] = V
    return inp


@pytest.mark.parametrize("ws", [False, True], ids=["fa_fwd", "fa_fwd_ws"])
def test_v_at_the_fp16_limit_is_exact(ws):
    # the largest bf16 numbers inside fp16's range (bf16 has 8 significant bits: 65504
    # itself is not one, it rounds to 65536); each is an fp16 number as well
    inp = _inputs([65280.0, 65024.0, 61440.0, 49152.0, 32768.0], seed=31)
    scale = 1.0 / math.sqrt(128)
    Q, K, V = inp["Q"], inp["K"], inp["V"]
    assert float(V.float().abs().max()) <= 65504.0
    O = torch.empty_like(Q)
    LSE = torch.empty(Q.shape[:3], device=Q.device, dtype=torch.float32)
    if ws:
        w = torch.empty(fa.fa_fwd_workspace_size(*Q.shape[:3], K.shape[2], 128), device=Q.device, dtype=torch.uint8)
        fa.fa_fwd_ws(Q, K, V, O, LSE, w, scale)
    else:
        fa.fa_fwd(Q, K, V, O, LSE, scale)
    torch.cuda.synchronize()
    q, k, v = oracle_view(Q), oracle_view(K), oracle_view(V)
    O_ref, LSE_ref = oracle.fwd(q, k, v, scale, False)
    A_ref, _ = oracle.fwd(q, k, np.abs(v), scale, False)
    say("V up to 65504", "ws" if ws else "plain")
    # outputs reach thousands here: the max-abs bar is for O of order 1 (half a bf16
    # ulp of 2^12 alone is 8); rel-L2 and the elementwise arithmetic bound hold
    check_forward(to_np(O), to_np(LSE), O_ref, LSE_ref, torch.bfloat16, "V at the fp16 limit", A_ref, 200,
                  float(np.abs(v).max()), max_abs_bar=False)


def test_v_beyond_the_fp16_limit_is_not_finite():
    # 65536 is a bf16 number above the largest fp16: the documented limit
    inp = _inputs([65536.0, 1.0, 1.0, 1.0, 1.0], seed=32)
    O, LSE = fa.forward(inp["Q"], inp["K"], inp["V"], 1.0 / math.sqrt(128))
    torch.cuda.synchronize()
    O = to_np(O)
    say("V beyond 65504: column 0 finite?", bool(np.all(np.isfinite(O[..., 0]))))
    assert not np.all(np.isfinite(O[..., 0]))  # the key's weight reaches every row
    assert np.all(np.isfinite(O[..., 1:3]))      # columns without such a value are unaffected
    assert np.all(np.isfinite(to_np(LSE)))       # the softmax statistics do not involve V
