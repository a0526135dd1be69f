"""fa_bwd_noalloc, the backward that takes no workspace (its D rows live in
the library's fixed device array), against fa_bwd through the C ABI: the same
kernels, so the same bits, on two calls in a row with the second smaller than
the first (the array keeps the first call's rows, which must not leak into the
second).  Also its size limit and argument checks."""
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


def _both(B, H, Nq, Nk, d, dtype, causal, seed):
    inp = synth.make_inputs(B, H, Nq, Nk, d, dtype, seed, device="cuda")
    scale = 1.0 / math.sqrt(d)
    Q, K, V, dO = inp["Q"], inp["K"], inp["V"], inp["dO"]
    O, LSE = fa.forward(Q, K, V, scale, causal)
    ref = fa.backward(Q, K, V, O, dO, LSE, scale, causal)
    got = [torch.full_like(t, float("nan")) for t in ref]
    fa.fa_bwd_noalloc(Q, K, V, O, dO, LSE, *got, scale, causal)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("dtype,causal", [("bf16", False), ("f16", True), ("f32", False)])
def test_noalloc_equals_fa_bwd_twice_second_smaller(dtype, causal):
    for k, shape in enumerate([(2, 4, 1000, 700, 128), (1, 3, 333, 517, 64)]):
        say("noalloc call", k + 1, shape, dtype, causal)
        ref, got = _both(*shape, dtype, causal, seed=500 + k)
        for name, r, g in zip(("dQ", "dK", "dV"), ref, got):
            assert torch.equal(r, g), (shape, name)


def test_noalloc_full_training_shape():
    # B8 H32 N4096 d128: 1M rows of D, well inside the array
    say("noalloc training shape")
    ref, got = _both(8, 32, 4096, 4096, 128, "bf16", False, seed=1003)
    for r, g in zip(ref, got):
        assert torch.equal(r, g)


def test_noalloc_limits():
    lib = fa.lib()
    P = torch.empty(16, device="cuda").data_ptr()
    args = lambda B, H, Nq, d=64: (P, P, P, P, P, P, P, P, P, B, H, Nq, 8, d, 0.125, 0, 0, None)
    # one row more than the array holds: refused before any launch
    assert lib.fa_bwd_noalloc(*args(1, 1, fa.FA_NOALLOC_MAX_ROWS + 1)) == fa.FA_ERR_UNSUPPORTED
    assert lib.fa_bwd_noalloc(*args(0, 1, 8)) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_bwd_noalloc(*args(1, 1, 8, d=96)) == fa.FA_ERR_UNSUPPORTED
    null = (P, P, P, P, P, P, None, P, P, 1, 1, 8, 8, 64, 0.125, 0, 0, None)
    assert lib.fa_bwd_noalloc(*null) == fa.FA_ERR_INVALID_ARG
