"""fa_fwd and fa_bwd captured in a HIP graph: the library only enqueues
kernels on the caller's stream (no allocation, memset or synchronisation),
so a captured forward + backward replays to the eager results.  Each replay
is compared with the eager run, with the program's own eager work and
synchronisations between replays."""
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


@pytest.mark.parametrize("packed_v", [False, True], ids=["fa_fwd", "fa_fwd_ws"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape,dtype", [((1, 1, 256, 256, 64), "f32"), ((2, 3, 300, 520, 128), "bf16"),
                                         ((1, 2, 129, 257, 64), "f16")], ids=["tiny_f32", "bf16_d128", "f16_d64"])
def test_graph_replay(shape, dtype, causal, packed_v):
    B, H, Nq, Nk, d = shape
    inp = synth.make_inputs(B, H, Nq, Nk, d, dtype, 77, device="cuda")
    Q, K, V, dO = inp["Q"], inp["K"], inp["V"], inp["dO"]
    scale = 1.0 / math.sqrt(d)
    say("graph", shape, dtype, causal)
    # eager reference
    O_e, L_e = fa.forward(Q, K, V, scale, causal)
    g_e = fa.backward(Q, K, V, O_e, dO, L_e, scale, causal)
    torch.cuda.synchronize()
    # static buffers for the captured step
    O, L = torch.empty_like(O_e), torch.empty_like(L_e)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    ws = fa.alloc_workspace(Q, K)
    fws = torch.empty(fa.fa_fwd_workspace_size(B, H, Nq, Nk, d), device="cuda", dtype=torch.uint8)

    def fwd(s):
        if packed_v:
            fa.fa_fwd_ws(Q, K, V, O, L, fws, scale, causal, s)
        else:
            fa.fa_fwd(Q, K, V, O, L, scale, causal, s)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside capture
        fwd(side)
        fa.fa_bwd(Q, K, V, O, dO, L, dQ, dK, dV, ws, scale, causal, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        s = torch.cuda.current_stream()
        fwd(s)
        fa.fa_bwd(Q, K, V, O, dO, L, dQ, dK, dV, ws, scale, causal, s)
    for rep in range(3):
        for t in (O, L, dQ, dK, dV):
            t.fill_(float("nan"))  # stale results cannot pass
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(O, O_e) and torch.equal(L, L_e), rep
        for a, b in zip((dQ, dK, dV), g_e):
            assert torch.equal(a, b), rep
        # eager work of the program between replays
        fa.forward(Q, K, V, scale, causal)
        torch.cuda.synchronize()
