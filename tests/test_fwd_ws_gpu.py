"""fa_fwd_ws (V packed once into fp16 V^T tiles, then copied as is by the key
loop) against fa_fwd and the fp64 oracle.  Both paths feed the matrix cores
the same fp16 V values in the same order, so their O and LSE must agree bit
for bit; the oracle checks one shape per dtype directly."""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
import tiled_online_softmax_03_amd as fa
from gpu_util import check_forward, oracle_view, say, to_np

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.lib()


def _ws_fwd(inp, scale, causal, ws=None):
    Q, K, V = inp["Q"], inp["K"], inp["V"]
    B, H, Nq, d = Q.shape
    if ws is None:
        ws = torch.empty(fa.fa_fwd_workspace_size(B, H, Nq, K.shape[2], d), device="cuda", dtype=torch.uint8)
    O = torch.empty_like(Q)
    LSE = torch.empty((B, H, Nq), device="cuda", dtype=torch.float32)
    fa.fa_fwd_ws(Q, K, V, O, LSE, ws, scale, causal)
    torch.cuda.synchronize()
    return O, LSE


SHAPES = [
    (1, 1, 1, 1, 64),
    (1, 2, 1, 300, 128),
    (1, 1, 77, 5, 64),
    (2, 1, 130, 130, 128),
    (1, 3, 129, 257, 64),
    (1, 2, 200, 333, 128),
    (1, 1, 383, 1029, 64),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_equals_fa_fwd(shape, causal, dtype):
    B, H, Nq, Nk, d = shape
    seed = zlib.crc32(repr((shape, causal, dtype, "fwd_ws")).encode()) % 10000
    inp = synth.make_inputs(B, H, Nq, Nk, d, dtype, seed, device="cuda", with_dO=False)
    scale = 1.0 / math.sqrt(d)
    say("fwd_ws", shape, dtype, causal)
    O, LSE = _ws_fwd(inp, scale, causal)
    O2, L2 = fa.forward(inp["Q"], inp["K"], inp["V"], scale, causal)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(LSE, L2)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_oracle_parity(dtype):
    B, H, Nq, Nk, d = 1, 2, 300, 700, 128
    inp = synth.make_inputs(B, H, Nq, Nk, d, dtype, 321, device="cuda", with_dO=False)
    scale = 1.0 / math.sqrt(d)
    say("fwd_ws oracle", dtype)
    O, LSE = _ws_fwd(inp, scale, False)
    q, k, v = oracle_view(inp["Q"]), oracle_view(inp["K"]), oracle_view(inp["V"])
    O_ref, LSE_ref = oracle.fwd(q, k, v, scale, False)
    A_ref, _ = oracle.fwd(q, k, np.abs(v), scale, False)
    check_forward(to_np(O), to_np(LSE), O_ref, LSE_ref, DT[dtype], "fwd_ws", A_ref, Nk, float(np.abs(v).max()))


def test_workspace_reuse():
    """One workspace, a large call and then a smaller one: the second sees none
    of the first's tiles."""
    big = synth.make_inputs(2, 4, 512, 2048, 128, "bf16", 5, device="cuda", with_dO=False)
    small = synth.make_inputs(1, 3, 200, 333, 128, "bf16", 6, device="cuda", with_dO=False)
    ws = torch.empty(fa.fa_fwd_workspace_size(2, 4, 512, 2048, 128), device="cuda", dtype=torch.uint8)
    for inp in (big, small):
        O, LSE = _ws_fwd(inp, 0.09, False, ws)
        O2, L2 = fa.forward(inp["Q"], inp["K"], inp["V"], 0.09, False)
        torch.cuda.synchronize()
        assert torch.equal(O, O2) and torch.equal(LSE, L2)


@pytest.mark.parametrize("name", ["train_b8h32n4096d128", "cross_1024x8192_f16", "single_head_fwd"])
def test_workloads_equal_fa_fwd(name):
    w = synth.WORKLOADS[name]
    inp = synth.workload_inputs(w, device="cuda", with_dO=False)
    say("fwd_ws", w.name, "full size")
    O, LSE = _ws_fwd(inp, w.scale, w.causal)
    O2, L2 = fa.forward(inp["Q"], inp["K"], inp["V"], w.scale, w.causal)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(LSE, L2)


def test_long_causal_equal_fa_fwd():
    w = synth.WORKLOADS["long_causal_n65536"]
    inp = synth.make_inputs(1, 4, 16384, 16384, 128, "bf16", w.seed, device="cuda", with_dO=False)
    say("fwd_ws causal 16384")
    O, LSE = _ws_fwd(inp, w.scale, True)
    O2, L2 = fa.forward(inp["Q"], inp["K"], inp["V"], w.scale, True)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(LSE, L2)


def _rising(B, H, Nq, Nk, d, dtype, step_log2, seed):
    """Q rows of ones (times a per-row factor in [0.5, 1.36]), key j a multiple
    a_j of ones with a_j rising along the keys, so that the scaled score of key
    j, in log2 units, grows by about `step_log2` per key (times the row
    factor): every 64-key tile raises each row's maximum well past the
    rescale threshold of 8, and the reference maximum moves on every tile."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    td = DT[dtype]
    scale = 1.0 / math.sqrt(d)
    unit = d * scale * math.log2(math.e)  # log2-scaled score of ones . ones
    rows = 0.5 + (torch.arange(Nq, device="cuda", dtype=torch.float32) % 7) / 7.0
    a = step_log2 * torch.arange(Nk, device="cuda", dtype=torch.float32) / unit
    Q = (rows[:, None] * torch.ones(d, device="cuda")).expand(B, H, Nq, d).to(td).contiguous()
    K = (a[:, None] * torch.ones(d, device="cuda")).expand(B, H, Nk, d).to(td).contiguous()
    V = torch.randn((B, H, Nk, d), generator=g, device="cuda").to(td).contiguous()
    return {"Q": Q, "K": K, "V": V}, scale


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_rescale_every_tile(causal, dtype):
    """The maximum rises on every key tile, so the d = 128 key loop's rescale
    branch (which recomputes the first 32 keys' exponentials after the vote)
    runs on every step: still fa_fwd's bits, and the oracle's values."""
    Nq, Nk = (700, 700) if causal else (300, 1000)
    inp, scale = _rising(1, 2, Nq, Nk, 128, dtype, 0.2, 77)
    say("fwd_ws rescale every tile", dtype, causal)
    O, LSE = _ws_fwd(inp, scale, causal)
    O2, L2 = fa.forward(inp["Q"], inp["K"], inp["V"], scale, causal)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(LSE, L2)
    q, k, v = oracle_view(inp["Q"]), oracle_view(inp["K"]), oracle_view(inp["V"])
    O_ref, LSE_ref = oracle.fwd(q, k, v, scale, causal)
    A_ref, _ = oracle.fwd(q, k, np.abs(v), scale, causal)
    check_forward(to_np(O), to_np(LSE), O_ref, LSE_ref, DT[dtype], "fwd_ws rising", A_ref, Nk,
                  float(np.abs(v).max()), max_abs_bar="auto")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_wide_logits(dtype):
    """Q, K ~ N(0, 4^2) at d = 128: scores spread over hundreds of log2 units,
    so the vote fires on irregular tiles and row blocks."""
    inp = synth.make_inputs(1, 2, 260, 900, 128, dtype, 91, sigma_qk=4.0, device="cuda", with_dO=False)
    scale = 1.0 / math.sqrt(128)
    say("fwd_ws wide logits", dtype)
    O, LSE = _ws_fwd(inp, scale, False)
    O2, L2 = fa.forward(inp["Q"], inp["K"], inp["V"], scale, False)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(LSE, L2)
    q, k, v = oracle_view(inp["Q"]), oracle_view(inp["K"]), oracle_view(inp["V"])
    O_ref, LSE_ref = oracle.fwd(q, k, v, scale, False)
    A_ref, _ = oracle.fwd(q, k, np.abs(v), scale, False)
    check_forward(to_np(O), to_np(LSE), O_ref, LSE_ref, DT[dtype], "fwd_ws wide", A_ref, 900,
                  float(np.abs(v).max()), max_abs_bar=False)
