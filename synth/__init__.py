"""Seeded synthetic inputs for attention workloads.

This module only draws random numbers and casts them; it holds none of the
attention arithmetic.  Both the HIP path (tests, bench) and the fp64 oracle
receive tensors made here, so the oracle sees exactly the bits the kernels
read.

Recipe (every workload): a ``torch.Generator`` on the requested device seeded
with the workload's seed draws fp32 N(0, 1) tensors in the order Q, K, V, dO;
Q and K are multiplied by ``sigma_qk``; each tensor is then cast to the
workload dtype with round-to-nearest-even (``Tensor.to``).  Layout is
contiguous [B, H, N, d].
"""
from __future__ import annotations

from dataclasses import dataclass, replace
import math

import torch

DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str  # "bf16" | "f16" | "f32"
    causal: bool
    backward: bool
    seed: int
    sigma_qk: float = 1.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    def fwd_flops(self) -> float:
        """4*B*H*Nq*Nk*d, halved under the causal mask."""
        f = 4.0 * self.B * self.H * self.Nq * self.Nk * self.d
        return f / 2 if self.causal else f

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads the method is evaluated on.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 1, 256, 256, 64, "f32", False, True, 1001),
    "single_head_fwd": Workload("single_head_fwd", 1, 1, 4096, 4096, 64, "bf16", False, False, 1002),
    "train_b8h32n4096d128": Workload("train_b8h32n4096d128", 8, 32, 4096, 4096, 128, "bf16", False, True, 1003),
    "long_causal_n65536": Workload("long_causal_n65536", 1, 32, 65536, 65536, 128, "bf16", True, False, 1004),
    "cross_1024x8192_f16": Workload("cross_1024x8192_f16", 4, 16, 1024, 8192, 64, "f16", False, True, 1005,
                                    sigma_qk=2.0),
}


def make_inputs(B: int, H: int, Nq: int, Nk: int, d: int, dtype: str, seed: int,
                sigma_qk: float = 1.0, device="cpu", with_dO: bool = True):
    """Return dict(Q, K, V[, dO]) of contiguous [B, H, N, d] tensors."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    td = DTYPES[dtype]

    def draw(n, s=1.0):
        x = torch.randn((B, H, n, d), generator=g, device=dev, dtype=torch.float32)
        if s != 1.0:
            x.mul_(s)
        return x.to(td).contiguous()

    out = {"Q": draw(Nq, sigma_qk), "K": draw(Nk, sigma_qk), "V": draw(Nk)}
    if with_dO:
        out["dO"] = draw(Nq)
    return out


def workload_inputs(w: Workload, device="cpu", with_dO=None):
    if with_dO is None:
        with_dO = w.backward
    return make_inputs(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.seed, w.sigma_qk, device, with_dO)


def sample_rows(N: int, H: int, count: int = 256, base_seed: int = 4000):
    """Per-head query rows to check on long sequences: rows 0, 1 and N-1 plus
    distinct rows drawn from torch.Generator seeded with base_seed + h.
    Returns a list of H sorted int lists."""
    out = []
    for h in range(H):
        fixed = sorted({0, min(1, N - 1), N - 1})
        g = torch.Generator().manual_seed(base_seed + h)
        need = max(0, min(count, N) - len(fixed))
        pool = torch.randperm(N, generator=g).tolist()
        extra = [r for r in pool if r not in fixed][:need]
        out.append(sorted(fixed + extra))
    return out
