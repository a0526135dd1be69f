"""Wait states around the matrix products the kernels write as inline
assembly (CPU only: hipcc cross-compiles the sources to gfx950 assembly and
nothing runs).

Products that pin an accumulator or an operand to AGPRs are inline assembly
(fa_common.hpp: mfma_acc, mfma_bagpr), so the compiler's hazard recognizer,
which inserts the wait states around the products it emits itself, does not
see them.  The kernels' schedules keep the distances; this test reads the
generated code and holds every such product to the two rules the compiler
applies to its own 32x32x16 products on this target (its output for a
product followed by a dependent read, and for a vector write followed by a
product, shows them):
 * a vector instruction writing a register that the product reads must be at
   least 2 wait states before it;
 * nothing but another product's accumulator input may read or write the
   product's result registers within 12 wait states after it.
Each instruction counts one wait state and s_nop n counts n + 1; a product in
between counts one, however long it stalls issue, so the check is
conservative."""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tiled_online_softmax_03_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

VALU_WRITE_BEFORE_PRODUCT = 2
PRODUCT_RESULT_LATENCY = 12


def _regs(op):
    m = re.fullmatch(r"([va])(\d+)", op)
    if m:
        return {(m.group(1), int(m.group(2)))}
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", op)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return set()


def _split(ins):
    parts = ins.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    return parts[0], [o.strip() for o in re.split(r",(?![^\[]*\])", parts[1])]


def _instructions(lines):
    """(text, from_inline_asm, wait_states) per instruction; labels break a window."""
    out, in_asm = [], False
    for ln in lines:
        t = ln.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        t = t.split(";")[0].strip()
        if not t:
            continue
        if t.endswith(":"):
            out.append(("<label>", False, 0))
            continue
        if t.startswith("."):
            continue
        m = re.match(r"s_nop\s+(\d+)", t)
        out.append((t, in_asm, int(m.group(1)) + 1 if m else 1))
    return out


def findings(lines):
    ins = _instructions(lines)
    bad = []
    for k, (t, in_asm, _) in enumerate(ins):
        if t == "<label>":
            continue
        op, ops = _split(t)
        if not (in_asm and op.startswith("v_mfma") and len(ops) >= 4):
            continue
        srcs = _regs(ops[1]) | _regs(ops[2]) | _regs(ops[3])
        ws, j = 0, k - 1
        while j >= 0 and ws < VALU_WRITE_BEFORE_PRODUCT:
            u, _, w = ins[j]
            if u == "<label>":
                break
            uop, uops = _split(u)
            if uop.startswith("v_") and not uop.startswith("v_mfma") and uops and _regs(uops[0]) & srcs:
                bad.append(("vector write %d wait states before" % ws, u, t))
            ws += w
            j -= 1
        dst = _regs(ops[0])
        ws, j = 0, k + 1
        while j < len(ins) and ws < PRODUCT_RESULT_LATENCY:
            u, _, w = ins[j]
            if u == "<label>":
                break
            uop, uops = _split(u)
            if uop.startswith("v_mfma"):
                if len(uops) >= 3 and (_regs(uops[1]) | _regs(uops[2])) & dst:
                    bad.append(("result used as an A/B operand %d wait states after" % ws, t, u))
            elif uops and not uop.startswith("s_"):
                touched = set().union(*[_regs(o) for o in uops])
                if touched & dst:
                    bad.append(("result touched %d wait states after" % ws, t, u))
            ws += w
            j += 1
    return bad


def _functions(asm_text):
    funcs, cur = {}, None
    for ln in asm_text.split("\n"):
        m = re.match(r"^(_Z\w+):", ln)
        if m:
            cur = funcs.setdefault(m.group(1), [])
            continue
        if cur is not None:
            cur.append(ln)
            if "s_endpgm" in ln:
                cur = None
    return funcs


@pytest.fixture(scope="module")
def assembly():
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    sys.path.insert(0, ROOT)
    from tiled_online_softmax_03_amd import _build
    out = {}
    for src in ("fa_fwd.hip", "fa_bwd.hip"):
        cmd = [HIPCC, "-O3", "-std=c++17", *_build.device_flags(src), "--cuda-device-only", "-S", "-o", "-",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, src)]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
        assert r.returncode == 0, r.stderr[-2000:]
        out.update(_functions(r.stdout))
    return out


def test_checker_catches_the_patterns():
    """The scanner flags a vector write right before a product and a read of
    the result right after it, and passes the same code with the distances."""
    bad = ["v_mov_b32 v5, v9", ";;#ASMSTART", "v_mfma_f32_32x32x16_bf16 v[0:15], v[2:5], a[0:3], v[0:15]",
           ";;#ASMEND", "v_add_f32 v20, v3, v3", "v_fma_f32 v21, v7, s0, v1"]
    kinds = {b[0].split()[0] for b in findings(bad)}
    assert kinds == {"vector", "result"}, findings(bad)
    good = ["v_mov_b32 v5, v9", "s_nop 1", ";;#ASMSTART", "v_mfma_f32_32x32x16_bf16 v[0:15], v[2:5], a[0:3], v[0:15]",
            ";;#ASMEND", "s_nop 7", "s_nop 3", "v_fma_f32 v21, v7, s0, v1"]
    assert findings(good) == []


def test_inline_products_keep_their_wait_states(assembly):
    checked = {n: f for n, f in assembly.items() if any("v_mfma" in ln and "ASMSTART" in prev
                                                        for prev, ln in zip(f, f[1:]))}
    names = {re.search(r"_ZN2fa\d+(\w+?_kernel)", n).group(1) for n in checked}
    assert {"bwd_dkdv_kv_kernel", "bwd_dq_kv_kernel", "fwd_r64_kernel"} <= names, names
    bad = {n: findings(f) for n, f in checked.items()}
    bad = {n: b for n, b in bad.items() if b}
    for n, b in bad.items():
        for x in b[:5]:
            print(n[:60], x)
    assert not bad, {n: len(b) for n, b in bad.items()}


# Exponentials per matrix product in each one-wave-per-SIMD kernel's step
# program: the forward issues one per product (64 keys x 64 rows per wave per
# 64 products), dK/dV one per two (32 per 64), dQ two per three (64 per 96).
EXP_PER_PRODUCT = {"fwd_r64_kernel": 1.0, "bwd_dkdv_kv_kernel": 0.5, "bwd_dq_kv_kernel": 2.0 / 3.0}


def _blocks(lines):
    """Straight-line blocks of a function: (label, instructions)."""
    out, cur, lab = [], [], "entry"
    for ln in lines:
        t = ln.split(";")[0].strip()
        if re.match(r"^\.?LBB\w*:", t):
            out.append((lab, cur))
            cur, lab = [], t
            continue
        if t and not t.startswith("."):
            cur.append(t)
    out.append((lab, cur))
    return out


def interleaving_gaps(lines, per_product):
    """Blocks that hold a step's products (16 or more) but fewer of its
    exponentials than the step program puts beside them: the compiler moved
    vector work away from the products that were to hide it."""
    bad = []
    for lab, b in _blocks(lines):
        n_mfma = sum(1 for t in b if t.startswith("v_mfma"))
        n_exp = sum(1 for t in b if t.startswith("v_exp_f32"))
        if n_mfma >= 16 and n_exp < per_product * n_mfma:
            bad.append((lab, n_mfma, n_exp))
    return bad


def test_interleaving_checker_catches_a_moved_exponential():
    prods = ["v_mfma_f32_32x32x16_bf16 v[0:15], v[2:5], a[0:3], v[0:15]"] * 16
    assert interleaving_gaps([".LBB0_1:", *prods, *["v_exp_f32_e32 v1, v1"] * 16], 1.0) == []
    moved = [".LBB0_1:", *prods, *["v_exp_f32_e32 v1, v1"] * 8, ".LBB0_2:", *["v_exp_f32_e32 v1, v1"] * 8]
    assert interleaving_gaps(moved, 1.0) == [(".LBB0_1:", 16, 8)]


def test_step_exponentials_stay_beside_the_products(assembly):
    """Each step of the one-wave-per-SIMD kernels interleaves its softmax
    exponentials with its matrix products, and only that hides them.  A
    change that lets the compiler sink them into a rarely taken branch's
    join (it did once: the forward's rescale branch) keeps every result and
    loses the overlap; this fails on it."""
    seen = set()
    bad = {}
    for n, f in assembly.items():
        m = re.search(r"_ZN2fa\d+(\w+?_kernel)", n)
        if not m or m.group(1) not in EXP_PER_PRODUCT:
            continue
        seen.add(m.group(1))
        gaps = interleaving_gaps(f, EXP_PER_PRODUCT[m.group(1)])
        if gaps:
            bad[n] = gaps
    assert seen == set(EXP_PER_PRODUCT), seen
    assert not bad, bad
