"""Memory is O(N) in the sequence length (page 1 "Flash Attention 原理与实现",
section "性能对比", and research-attention section 06: report peak memory on
its own): the library never allocates device memory -- every byte a call
touches is a caller tensor or a caller workspace -- and each workspace grows
linearly in N, while one materialised score matrix would grow as N^2."""
import math

import pytest
import torch

import synth
import tiled_online_softmax_03_amd as fa
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.lib()


def _free():
    torch.cuda.synchronize()
    return torch.cuda.mem_get_info()[0]


def test_calls_allocate_nothing():
    B, H, N, d = 1, 8, 16384, 128
    inp = synth.make_inputs(B, H, N, N, d, "bf16", 77, device="cuda")
    Q, K, V, dO = inp["Q"], inp["K"], inp["V"], inp["dO"]
    s = 1.0 / math.sqrt(d)
    O, LSE = torch.empty_like(Q), torch.empty((B, H, N), device="cuda", dtype=torch.float32)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    ws_f = torch.empty(fa.fa_fwd_workspace_size(B, H, N, N, d), device="cuda", dtype=torch.uint8)
    G = 4
    ws_s = torch.empty(fa.fa_fwd_splitkv_workspace_size(B, H, N, N, d, G), device="cuda", dtype=torch.uint8)
    ws_b = fa.alloc_workspace(Q, K)
    calls = {
        "fa_fwd": lambda: fa.fa_fwd(Q, K, V, O, LSE, s),
        "fa_fwd_ws": lambda: fa.fa_fwd_ws(Q, K, V, O, LSE, ws_f, s),
        "fa_fwd_splitkv": lambda: fa.fa_fwd_splitkv(Q, K, V, O, LSE, G, ws_s, s),
        "fa_fwd_dropout": lambda: fa.fa_fwd_dropout(Q, K, V, O, LSE, 0.1, 5, s),
        "fa_bwd": lambda: fa.fa_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, ws_b, s),
        "fa_bwd_dropout": lambda: fa.fa_bwd_dropout(Q, K, V, O, dO, LSE, dQ, dK, dV, ws_b, 0.1, 5, s),
        "fa_bwd_noalloc": lambda: fa.fa_bwd_noalloc(Q, K, V, O, dO, LSE, dQ, dK, dV, s),
    }
    for name, call in calls.items():  # first calls: code objects and the runtime's own set-up
        call()
    torch.cuda.synchronize()
    for name, call in calls.items():
        torch.cuda.reset_peak_memory_stats()
        before, alloc = _free(), torch.cuda.memory_allocated()
        for _ in range(3):
            call()
        after = _free()
        say("   ", name, "free device bytes before/after", before, after)
        assert after == before, (name, before, after)
        assert torch.cuda.max_memory_allocated() == alloc, name  # the binding allocates no tensor either


@pytest.mark.parametrize("d", [64, 128])
def test_workspaces_linear_in_n(d):
    # every caller-owned buffer of a fwd + bwd step, per head, at N = 4096 .. 65536
    rows = []
    for N in (4096, 8192, 16384, 32768, 65536):
        io = 4 * N * d * 2 + 4 * N * d * 2 + 2 * N * 4  # Q,K,V,O + dO,dQ,dK,dV (bf16), LSE
        ws = fa.fa_fwd_workspace_size(1, 1, N, N, d) + fa.fa_bwd_workspace_size(1, 1, N, N, d)
        rows.append((N, io + ws, N * N * 2))
        say("    N=%6d  step bytes per head %12d   one bf16 score matrix %14d" % rows[-1])
    per_n = [b / n for n, b, _ in rows]
    assert max(per_n) / min(per_n) < 1.01, per_n           # linear in N
    assert rows[-1][2] / rows[-1][1] > 30                   # far below N^2 at 64K
