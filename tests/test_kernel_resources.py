"""Register use of the gfx950 kernels, from the compiler's own resource report
(CPU only: hipcc cross-compiles the sources with
-Rpass-analysis=kernel-resource-usage and nothing runs).

Every instantiation on the 16-bit path without dropout (what fa_fwd,
fa_fwd_ws, fa_fwd_splitkv and fa_bwd launch for bf16 and fp16 inputs, d = 64
and 128, causal or not) must keep all its values in registers: a ScratchSize
above 0 means spilled registers going through memory on every step.  The
float32 and dropout variants are reported, not held to it (their spills are
stated with the kernel notes of the library's design record).  The dK/dV
and dQ passes that run one wave per SIMD may use the whole register file."""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tiled_online_softmax_03_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _report(src):
    # the library's own device flags for this source
    sys.path.insert(0, ROOT)
    from tiled_online_softmax_03_amd import _build
    cmd = [HIPCC, "-O3", "-std=c++17", *_build.device_flags(src), "--cuda-device-only", "-S", "-o", os.devnull,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, src),
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    out = {}
    for block in re.split(r"remark: Function Name: ", r.stderr)[1:]:
        name = block.split()[0]
        get = lambda key: int(re.search(key + r": (\d+)", block).group(1))
        out[name] = {"vgpr": get(r"VGPRs"), "agpr": get(r"AGPRs"), "scratch": get(r"ScratchSize \[bytes/lane\]")}
    return out


def _demangled_args(name):
    """Template arguments of a mangled fa:: kernel name: the list of integers
    (Li<n>E) and booleans (Lb<0|1>E) in order."""
    return [int(v) for v in re.findall(r"L[ib](\d+)E", name)]


def _hot(name):
    a = _demangled_args(name)
    if "fwd_kernel" in name and "merge" not in name:
        # fwd_kernel<D, BC, NW, E, CAUSAL, SPLIT, DROP, PREV>
        return a[3] != 2 and a[6] == 0
    if "bwd_dkdv_kernel" in name:  # <D, E, CAUSAL, DROP>
        return a[1] != 2 and a[3] == 0
    if "bwd_dkdv_kv_kernel" in name or "bwd_dq_kv_kernel" in name or "fwd_r64_kernel" in name:
        # <E, CAUSAL>: d = 128, 16-bit, no dropout only
        return True
    if "bwd_dq_kernel" in name:  # <D, BC, E, CAUSAL, DROP>
        return a[2] != 2 and a[4] == 0
    if "v_pack_kernel" in name:  # <D, BC, E>
        return a[2] != 2
    return True  # bwd_pre_kernel, fwd_merge_kernel


@pytest.fixture(scope="module")
def reports():
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    rep = {}
    for src in ("fa_fwd.hip", "fa_bwd.hip"):
        rep.update(_report(src))
    return rep


def test_every_kernel_reported(reports):
    names = ("fwd_kernel", "fwd_r64_kernel", "fwd_merge_kernel", "v_pack_kernel", "bwd_pre_kernel", "bwd_dkdv_kernel",
             "bwd_dkdv_kv_kernel", "bwd_dq_kernel", "bwd_dq_kv_kernel")
    kinds = {k for n in reports for k in names if "_ZN2fa%d%s" % (len(k), k) in n}
    assert kinds == set(names), sorted(reports)


def test_hot_path_does_not_spill(reports):
    hot = {n: r for n, r in reports.items() if _hot(n)}
    assert len(hot) >= 20, len(hot)
    spilling = {n: r for n, r in hot.items() if r["scratch"] > 0}
    for n, r in sorted(reports.items()):
        print("%-90s vgpr %3d agpr %3d scratch %4d%s" % (n[:90], r["vgpr"], r["agpr"], r["scratch"],
                                                        "" if _hot(n) else "  (not held)"))
    assert not spilling, spilling
    for n, r in hot.items():
        if "bwd_dkdv_kv_kernel" in n or "bwd_dq_kv_kernel" in n or "fwd_r64_kernel" in n:
            # one wave per SIMD: the whole register file, 256 of each kind; the
            # dK/dV pass's AGPRs hold exactly its 128 accumulators (no VGPR
            # spilled into them)
            assert r["vgpr"] <= 256 and r["agpr"] <= 256, (n, r)
            if "bwd_dkdv_kv_kernel" in n:
                assert r["agpr"] == 128, (n, r)
        else:
            assert r["vgpr"] + r["agpr"] <= 256, (n, r)  # two waves per SIMD
