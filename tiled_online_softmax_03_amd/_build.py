"""Build libfa.so (gfx950) in-tree with hipcc.

Every source is compiled for gfx950 only, with packed-fp32 VALU ops disabled
(they are emitted by the compiler on its own otherwise) and hardware fp32
atomics for the dQ accumulator.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfa.so")
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip"]
# Per-source extra flags.  fa_bwd.hip: matrix products write VGPRs unless a
# kernel pins an accumulator to AGPRs itself (bwd_dkdv_kv_kernel keeps dV/dK in
# AGPRs and needs S/dP in VGPRs, where its softmax reads them; the other
# kernels of the file use no AGPRs and compile to the same code either way).
EXTRA = {"fa_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def device_flags(src: str) -> list:
    """The flags every device compile of `src` uses (the build and the resource check)."""
    return [*DEVICE, *EXTRA.get(src, [])]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
DEVICE = ["-x", "hip", "--offload-arch=" + ARCH, "-munsafe-fp-atomics",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD_DIR, src + ".o")
    cmd = [HIPCC, *COMMON, *device_flags(src), "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(jobs: int = 4, out: str = LIB) -> str:
    """Compile every HIP source and link libfa.so (or `out`); returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
