"""Properties of exact attention checked on the GPU path itself, at sizes and
shapes beyond what the oracle comparison covers, without the oracle.

Each follows from the definition of softmax attention (O = softmax(s Q K^T) V,
rows of P summing to one, LSE = log of the row normaliser):
  * one key: P = [1], so O = V_0 and LSE = the single scaled score;
  * Q = 0: every allowed score is 0, so O is the mean of the allowed V rows
    and LSE = ln(number of allowed keys);
  * V + c (same c for every key): O + c, since the rows of P sum to one;
  * K + c: every score of row i moves by s (q_i . c), which softmax ignores:
    O unchanged, LSE moves by s (q_i . c);
  * permuting K and V rows together (no mask): O unchanged;
  * backward: sum_j dV_j = sum_i dO_i, and sum_j dK_j = 0 (each row of dS
    sums to zero).
Where rounding would blur a property, inputs sit on a grid of multiples of
1/8 (exact in bf16 and fp16, and their products and sums exact in fp32)."""
import math

import pytest
import torch

import tiled_online_softmax_03_amd as fa
from gpu_util import say

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.lib()  # loud failure if the library is missing


def _randn(shape, seed, dtype, grid=False):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g)
    if grid:  # multiples of 1/8 in [-4, 4]
        x = torch.clamp(torch.round(x * 8.0) / 8.0, -4.0, 4.0)
    return x.to(dtype).contiguous().cuda()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_single_key(dtype, d, causal):
    B, H, Nq = 2, 3, 131
    say("invariant single key", dtype, d, causal)
    Q = _randn((B, H, Nq, d), 11, DT[dtype], grid=True)
    K = _randn((B, H, 1, d), 12, DT[dtype], grid=True)
    V = _randn((B, H, 1, d), 13, DT[dtype])
    scale = 1.0 / math.sqrt(d)
    O, LSE = fa.forward(Q, K, V, scale=scale, causal=causal)
    torch.cuda.synchronize()
    # P = [1] exactly; V passes through fp16 unchanged but for bf16 values below
    # fp16's subnormal step (2^-24)
    assert (O.double() - V.double().expand(B, H, Nq, d)).abs().max().item() <= 2.0 ** -24
    s = scale * (Q.double() * K.double()).sum(-1)  # exact on the grid
    assert (LSE.double() - s).abs().max().item() <= 1e-5 * (1.0 + s.abs().max().item())


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries(dtype, causal):
    B, H, Nq, Nk, d = 1, 2, 200, 333, 128
    say("invariant Q = 0", dtype, causal)
    Q = torch.zeros((B, H, Nq, d), dtype=DT[dtype], device="cuda")
    K = _randn((B, H, Nk, d), 21, DT[dtype])
    V = _randn((B, H, Nk, d), 22, DT[dtype])
    O, LSE = fa.forward(Q, K, V, scale=0.125, causal=causal)
    torch.cuda.synchronize()
    Vd = V.double()
    if causal:  # row i sees keys 0..min(i, Nk-1)
        cnt = torch.clamp(torch.arange(Nq, device="cuda") + 1, max=Nk).double()
        ref = torch.cumsum(Vd, dim=2)[:, :, (cnt - 1).long()] / cnt[None, None, :, None]
    else:
        cnt = torch.full((Nq,), float(Nk), device="cuda", dtype=torch.float64)
        ref = Vd.mean(dim=2, keepdim=True).expand(B, H, Nq, d)
    rel = 2.0 ** -7 if dtype == "bf16" else 2.0 ** -10  # twice the output half-ulp
    assert ((O.double() - ref).abs() - rel * ref.abs()).max().item() <= 1e-5
    assert (LSE.double() - torch.log(cnt)[None, None, :]).abs().max().item() <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_value_shift(dtype, causal):
    B, H, Nq, Nk, d = 2, 2, 150, 270, 64
    say("invariant V + c", dtype, causal)
    Q = _randn((B, H, Nq, d), 31, DT[dtype])
    K = _randn((B, H, Nk, d), 32, DT[dtype])
    V = _randn((B, H, Nk, d), 33, DT[dtype], grid=True)
    c = torch.linspace(-0.75, 0.75, d).mul(8).round().div(8)  # multiples of 1/8
    Vc = (V.double() + c.double().cuda()).to(DT[dtype]).contiguous()  # exact on the grid
    O, LSE = fa.forward(Q, K, V, scale=0.125, causal=causal)
    Oc, LSEc = fa.forward(Q, K, Vc, scale=0.125, causal=causal)
    torch.cuda.synchronize()
    rel = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11  # one output half-ulp each
    err = (Oc.double() - O.double() - c.double().cuda()).abs() - rel * (O.double().abs() + Oc.double().abs())
    assert err.max().item() <= 1e-5
    assert torch.equal(LSE, LSEc), "V does not enter the softmax"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_key_shift(dtype, causal):
    B, H, Nq, Nk, d = 2, 2, 129, 257, 128
    say("invariant K + c", dtype, causal)
    Q = _randn((B, H, Nq, d), 41, DT[dtype], grid=True)
    K = _randn((B, H, Nk, d), 42, DT[dtype], grid=True)
    V = _randn((B, H, Nk, d), 43, DT[dtype])
    c = torch.linspace(-0.5, 0.5, d).mul(8).round().div(8)
    Kc = (K.double() + c.double().cuda()).to(DT[dtype]).contiguous()  # exact on the grid
    scale = 1.0 / math.sqrt(d)
    O, LSE = fa.forward(Q, K, V, scale=scale, causal=causal)
    Oc, LSEc = fa.forward(Q, Kc, V, scale=scale, causal=causal)
    torch.cuda.synchronize()
    # scores are exact in fp32 on the grid; what moves is where the reference
    # maximum sits, i.e. which fp16 values P rounds to: a few ulps of O
    rel, flo = (2.0 ** -7, 1e-3) if dtype == "bf16" else (2.0 ** -10, 2e-4)
    assert ((Oc.double() - O.double()).abs() - rel * O.double().abs()).max().item() <= flo
    shift = scale * (Q.double() * c.double().cuda()).sum(-1)
    assert (LSEc.double() - LSE.double() - shift).abs().max().item() <= 1e-4 * (1.0 + LSE.abs().max().item())


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
def test_key_permutation(dtype, d):
    B, H, Nq, Nk = 1, 3, 256, 515
    say("invariant permuted keys", dtype, d)
    Q = _randn((B, H, Nq, d), 51, DT[dtype])
    K = _randn((B, H, Nk, d), 52, DT[dtype])
    V = _randn((B, H, Nk, d), 53, DT[dtype])
    perm = torch.randperm(Nk, generator=torch.Generator().manual_seed(54)).cuda()
    O, LSE = fa.forward(Q, K, V, scale=1.0 / math.sqrt(d))
    Op, LSEp = fa.forward(Q, K[:, :, perm].contiguous(), V[:, :, perm].contiguous(), scale=1.0 / math.sqrt(d))
    torch.cuda.synchronize()
    diff = (Op.double() - O.double())
    assert diff.abs().max().item() <= 1e-2
    assert diff.norm().item() <= 2e-3 * O.double().norm().item()
    assert (LSEp - LSE).abs().max().item() <= 1e-4


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 200, 333, 128), (2, 1, 383, 129, 64), (1, 1, 1, 77, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_gradient_sums(shape, causal, dtype):
    B, H, Nq, Nk, d = shape
    say("invariant gradient sums", shape, causal, dtype)
    Q = _randn((B, H, Nq, d), 61, DT[dtype])
    K = _randn((B, H, Nk, d), 62, DT[dtype])
    V = _randn((B, H, Nk, d), 63, DT[dtype])
    dO = _randn((B, H, Nq, d), 64, DT[dtype])
    O, LSE = fa.forward(Q, K, V, scale=1.0 / math.sqrt(d), causal=causal)
    dQ, dK, dV = fa.backward(Q, K, V, O, dO, LSE, scale=1.0 / math.sqrt(d), causal=causal)
    torch.cuda.synchronize()
    dV_sum, dO_sum = dV.double().sum(2), dO.double().sum(2)
    assert (dV_sum - dO_sum).abs().max().item() <= 2e-2 * (1.0 + dO_sum.abs().max().item())
    dK_sum = dK.double().sum(2)
    assert dK_sum.abs().max().item() <= 2e-2 * (1e-3 + dK.double().abs().sum(2).max().item())
