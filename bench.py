"""Benchmark of the attention hot path on one MI355X.

One step = fa_fwd followed by fa_bwd (its three stages, launched one by one
so each kernel can be timed with HIP events on the stream it runs on) over
one batch of seeded synthetic inputs already resident in HBM.  The default
workload is B=8, H=32, Nq=Nk=4096, d=128, bf16, non-causal.

Prints ONE JSON line: whole-step throughput in TFLOP/s (forward counted as
4*B*H*Nq*Nk*d, backward as 2.5x that), the forward alone, the per-kernel
times, a roofline entry for the dominant kernel and a CPU baseline (the fp64
oracle timed on a bounded sample of the same workload on this host).

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--workload NAME]
                    [--no-cpu-baseline] [--cpu-heads 48] [--copy-probe-mib 0]
                    [--no-sclk]
    python bench.py --memory-sweep     (peak memory of a whole step against N, one JSON line)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd & fwd+bwd TFLOP/s, % bf16 MFMA peak, at B8·H32·N4096·d128"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak (published)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="train_b8h32n4096d128")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=48, help="heads in the oracle's timed sample")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a known-size reference "
                         "for hardware byte counters)")
    ap.add_argument("--no-sclk", action="store_true", help="skip sampling the graphics clock under load")
    ap.add_argument("--no-gemm-reference", action="store_true",
                    help="skip timing the vendor bf16 GEMM (torch.matmul) used as this box's attainable-rate reference")
    ap.add_argument("--fwd-only", action="store_true",
                    help="time the forward alone (implied for workloads that have no backward)")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="dropout rate on P (fa_fwd_dropout / fa_bwd_dropout; the backward is then timed as one "
                         "call)")
    ap.add_argument("--seed", type=int, default=1234, help="dropout seed")
    ap.add_argument("--fwd-plain", action="store_true",
                    help="time fa_fwd (V converted in the key loop) even where fa_fwd_ws (V packed once) is used")
    ap.add_argument("--splits", default=None,
                    help="forward through fa_fwd_splitkv with this many key ranges ('auto' = "
                         "fa_fwd_num_splits); implies --fwd-only")
    ap.add_argument("--memory-sweep", action="store_true",
                    help="instead of the step benchmark: peak memory and time of a whole step at B1 H32 "
                         "d128 for N = 4096 .. 65536")
    return ap.parse_args()


FWD_WS_MIN_NQ = 2048


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the attention path here runs on a single MI355X "
              "(--gpus %d is not supported)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import tiled_online_softmax_03_amd as fa

    if args.memory_sweep:
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(2)
        memory_sweep()
        return
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    fa.lib()
    w = synth.WORKLOADS[args.workload]
    fwd_only = args.fwd_only or args.splits is not None or not w.backward
    dev = torch.device("cuda:0")
    inp = synth.workload_inputs(w, device=dev, with_dO=not fwd_only)
    Q, K, V, dO = inp["Q"], inp["K"], inp["V"], inp.get("dO")
    O = torch.empty_like(Q)
    LSE = torch.empty((w.B, w.H, w.Nq), device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream()
    splits = None
    if args.splits is None and fwd_only and not args.fwd_plain and args.dropout <= 0:
        # forward-only shapes with too few query tiles for 256 CUs (one head of 4096 rows)
        # take the split-KV forward, the library's path for them
        auto = fa.fa_fwd_num_splits(w.B, w.H, w.Nq, w.Nk, w.d, w.causal)
        if auto > 1:
            args.splits = "auto"
    if args.splits is not None:
        splits = (fa.fa_fwd_num_splits(w.B, w.H, w.Nq, w.Nk, w.d, w.causal) if args.splits == "auto"
                  else int(args.splits))
        nws = fa.fa_fwd_splitkv_workspace_size(w.B, w.H, w.Nq, w.Nk, w.d, splits)
        split_ws = torch.empty(max(nws, 1), device=dev, dtype=torch.uint8) if nws > 0 else None
    drop = args.dropout > 0
    # fa_fwd_ws packs V once per call; that pays off when every V tile would otherwise be
    # staged by many query tiles (measured: +3-9 % from 16 query tiles per head up,
    # -7 % at 4), so it serves the workloads with Nq >= 2048.
    use_ws = not args.fwd_plain and splits is None and not drop and w.Nq >= FWD_WS_MIN_NQ
    if use_ws:
        fwd_ws = torch.empty(fa.fa_fwd_workspace_size(w.B, w.H, w.Nq, w.Nk, w.d), device=dev, dtype=torch.uint8)
    if drop and splits is not None:
        print("split-KV has no dropout variant", file=sys.stderr)
        sys.exit(2)
    if fwd_only:
        nst = 0
    else:
        dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
        ws = fa.alloc_workspace(Q, K)
        nst = 1 if drop else fa.fa_bwd_num_stages()
        if not drop and bwd_dq_first(w):
            nst = 2  # dQ (forming D), dK/dV; the library's stage 2 launches nothing on this path

    def launch_step(events=None):
        if events is not None:
            events[0].record(stream)
        if drop:
            fa.fa_fwd_dropout(Q, K, V, O, LSE, args.dropout, args.seed, w.scale, w.causal, stream)
        elif use_ws:
            fa.fa_fwd_ws(Q, K, V, O, LSE, fwd_ws, w.scale, w.causal, stream)
        elif splits is None:
            fa.fa_fwd(Q, K, V, O, LSE, w.scale, w.causal, stream)
        else:
            fa.fa_fwd_splitkv(Q, K, V, O, LSE, splits, split_ws, w.scale, w.causal, stream)
        if events is not None:
            events[1].record(stream)
        for s in range(nst):
            if drop:
                fa.fa_bwd_dropout(Q, K, V, O, dO, LSE, dQ, dK, dV, ws, args.dropout, args.seed, w.scale, w.causal,
                                  stream)
            else:
                fa.fa_bwd_stage(s, Q, K, V, O, dO, LSE, dQ, dK, dV, ws, w.scale, w.causal, stream)
            if events is not None:
                events[2 + s].record(stream)

    for _ in range(args.warmup):
        launch_step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 + nst)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        launch_step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    peak_mem = torch.cuda.max_memory_allocated()

    # the forward slot: fa_fwd_ws launches the V^T packing kernel and then the key loop
    fwd_name = "v_pack_kernel + fwd_kernel" if use_ws else "fwd_kernel"
    stage_names = ["bwd_dq_kernel", "bwd_dkdv_kernel"] if bwd_dq_first(w) else \
        ["bwd_pre_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"]
    names = [fwd_name] + (["fa_bwd_dropout (3 kernels)"] if drop else stage_names[:nst])
    per = {n: [] for n in names}
    for e in evs:
        for k, n in enumerate(names):
            per[n].append(e[k].elapsed_time(e[k + 1]))
    kern_ms = {n: sum(v) / len(v) for n, v in per.items()}
    step_ms = (t1 - t0) * 1e3 / args.steps
    step_events = [e[0].elapsed_time(e[-1]) for e in evs]  # fa_fwd start .. last backward stage end

    sclk = None if args.no_sclk else sample_sclk(launch_step)
    gemm_ref = None if args.no_gemm_reference else vendor_gemm_reference()

    F = w.fwd_flops()
    total_flops = (1.0 if fwd_only else 3.5) * F
    value = total_flops / (step_ms * 1e-3) / 1e12
    fwd_tflops = F / (kern_ms[fwd_name] * 1e-3) / 1e12
    bwd_ms = sum(kern_ms[n] for n in names[1:])
    bwd_tflops = 2.5 * F / (bwd_ms * 1e-3) / 1e12 if bwd_ms > 0 else None

    # algorithmic work per launch of each kernel
    elt = {"bf16": 2, "f16": 2, "f32": 4}[w.dtype]
    rows = w.B * w.H * w.Nq
    # (one matrix product of a head is 2*Nq*Nk*d flops = F/2 per head summed)
    work = {
        fwd_name: ("mfma", F),                        # S, P V
        "bwd_pre_kernel": ("hbm", 2 * rows * w.d * elt + rows * 4),  # read O, dO; write D
        "bwd_dkdv_kernel": ("mfma", 2.0 * F),         # S, dP, dV, dK
        "bwd_dq_kernel": ("mfma", 1.5 * F),           # S, dP, dQ
        "fa_bwd_dropout (3 kernels)": ("mfma", 2.5 * F),  # the whole backward, 2.5 F by the metric's convention
    }
    dom = max(names, key=lambda n: kern_ms[n])
    launched = {n: k for n, k in launched_kernels(w, use_ws, drop, splits).items() if n in names}
    bound, units = work[dom]
    traffic = measured_traffic(w.name, dom) if splits is None and not drop else None
    if bound == "mfma":
        achieved = units / (kern_ms[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma",
                "kernel": dom if splits is None else "fwd_kernel (split ranges) + fwd_merge_kernel",
                "launched": launched.get(dom),
                "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                "flops_per_launch": units, "avg_launch_ms": kern_ms[dom]}
    else:
        achieved = units / (kern_ms[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": traffic, "bytes_per_launch": units,
                "avg_launch_ms": kern_ms[dom]}

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inp, args.cpu_heads, fwd_only)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q, K, V, dO)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal,
                   "step": ("fa_fwd_dropout(p=%g)" % args.dropout if drop else
                            "fa_fwd_ws" if use_ws else
                            "fa_fwd" if splits is None else "fa_fwd_splitkv(%d ranges)" % splits)
                   + ("" if fwd_only else " + fa_bwd_dropout" if drop else " + fa_bwd")},
        "fwd_tflops": fwd_tflops,
        "fwd_pct_peak": 100.0 * fwd_tflops / PEAK_BF16_TFLOPS,
        "bwd_tflops": bwd_tflops,
        "fwd_bwd_pct_peak": None if fwd_only else 100.0 * value / PEAK_BF16_TFLOPS,
        "kernel_ms": kern_ms,
        "kernels_launched": launched,
        "step_ms_events": spread(step_events),
        "kernel_ms_spread": {n: spread(v) for n, v in per.items()},
        "peak_mem_bytes": peak_mem,
        "sclk_mhz_under_load": sclk,
        "vendor_gemm_bf16": gemm_ref,
        "versions": versions(torch),
        "describe": fa.fa_describe(w.d, fa.dtype_code(w.torch_dtype), w.causal),
        "device": torch.cuda.get_device_properties(0).gcnArchName,
        "torch": torch.__version__,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def spread(v):
    """Median, min, max and interquartile range of a list of times (ms)."""
    import statistics
    v = sorted(v)
    q = statistics.quantiles(v, n=4) if len(v) >= 2 else [v[0]] * 3
    return {"median": statistics.median(v), "min": v[0], "max": v[-1], "iqr": q[2] - q[0], "n": len(v)}


def sample_sclk(launch_step, seconds=4.0):
    """Graphics clock (MHz, mean over the XCDs) and socket power (W) read with
    amd-smi while the step runs back to back; None when the tool is missing or
    says nothing."""
    import re
    import subprocess
    import threading

    import torch

    out = {}

    def query():
        time.sleep(seconds / 3)
        try:
            r = subprocess.run(["amd-smi", "metric", "--clock", "--power", "--json"], capture_output=True,
                               text=True, timeout=seconds)
            out["text"] = r.stdout
        except Exception as e:  # tool absent or hung: no reading
            out["error"] = repr(e)

    th = threading.Thread(target=query)
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end or th.is_alive():
        for _ in range(10):
            launch_step()
        torch.cuda.synchronize()
    th.join()
    text = out.get("text", "")
    # "gfx_<i>": {"clk": {"value": V, "unit": "MHz"}, ...}
    vals = [float(m) for m in re.findall(r'"gfx_\d+":\s*\{\s*"clk":\s*\{\s*"value":\s*([0-9.]+)', text)]
    if not vals:
        return None
    # "socket_power": {"value": W, "unit": "W"}: the board's draw, against its power cap
    pw = re.findall(r'"socket_power":\s*\{\s*"value":\s*([0-9.]+)', text)
    return {"mean": sum(vals) / len(vals), "min": min(vals), "max": max(vals), "xcds": len(vals),
            "socket_power_w": float(pw[0]) if pw else None, "source": "amd-smi metric --clock --power"}


def bwd_dq_first(w):
    """The library's backward order for this workload without dropout: at
    d = 128 on 16-bit data the dQ pass runs first and forms D = rowsum(dO * O)
    itself (stage 0), the dK/dV pass follows (stage 1); elsewhere D, dK/dV,
    dQ (stages 0, 1, 2)."""
    return w.d == 128 and w.dtype in ("bf16", "f16")


def launched_kernels(w, use_ws, drop, splits):
    """The kernel each timed stage launches for this workload, as the library
    routes it (d = 128 on 16-bit data without dropout takes the
    one-wave-per-SIMD kernels; fa_fwd_ws packs V first)."""
    kv = w.d == 128 and w.dtype in ("bf16", "f16") and not drop
    if splits is not None:
        fwd = "fwd_kernel (split ranges) + fwd_merge_kernel"
    elif use_ws:
        fwd = "v_pack_kernel + " + ("fwd_r64_kernel" if kv else "fwd_kernel")
    else:
        fwd = "fwd_kernel"
    fwd_name = "v_pack_kernel + fwd_kernel" if use_ws else "fwd_kernel"
    out = {fwd_name: fwd}
    if drop:
        out["fa_bwd_dropout (3 kernels)"] = "bwd_pre_kernel + bwd_dkdv_kernel + bwd_dq_kernel"
    else:
        if not kv:
            out["bwd_pre_kernel"] = "bwd_pre_kernel"
        out.update({"bwd_dkdv_kernel": "bwd_dkdv_kv_kernel" if kv else "bwd_dkdv_kernel",
                    "bwd_dq_kernel": "bwd_dq_kv_kernel (forms D first)" if kv else "bwd_dq_kernel"})
    return out


def vendor_gemm_reference(m=8192, n=8192, k=8192, iters=40):
    """A calibration beside the step, not part of it: the sustained rate of the
    vendor's bf16 GEMM (torch.matmul, i.e. hipBLASLt) on this machine, on N(0, 1)
    operands and on an all-zero A.  Under sustained load the graphics clock
    settles where the board's power allows, and that depends on the data the
    matrix cores switch on, so this is the dense-MFMA rate the box actually
    delivers, beside the published peak the roofline uses."""
    import torch

    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    a = torch.randn((m, k), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    b = torch.randn((k, n), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    out = {"shape_mnk": [m, n, k], "iters": iters}
    for name, A in (("tflops", a), ("tflops_zero_a", torch.zeros_like(a))):
        for _ in range(5):
            c = A @ b
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            c = A @ b
        e1.record()
        torch.cuda.synchronize()
        out[name] = 2.0 * m * n * k / (e0.elapsed_time(e1) / iters * 1e-3) / 1e12
    del a, b, c
    out["frac_of_peak"] = out["tflops"] / PEAK_BF16_TFLOPS
    return out


def versions(torch):
    import platform

    import tiled_online_softmax_03_amd as fa
    v = {"torch": torch.__version__, "hip_runtime": torch.version.hip, "python": platform.python_version()}
    # the compiler that built libfa, from the library itself (no child process: under a
    # profiler a child would initialise the GPU before it could exec anything)
    v["libfa_build"] = fa.fa_build_info()
    try:
        with open("/opt/rocm/.info/version") as f:
            v["rocm"] = f.read().strip()
    except OSError:
        v["rocm"] = None
    p = torch.cuda.get_device_properties(0)
    v["device"] = {"name": p.name, "arch": p.gcnArchName, "compute_units": p.multi_processor_count,
                   "memory_bytes": p.total_memory}
    return v


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def memory_sweep():
    """Peak device memory and time of one whole step (fa_fwd_ws + fa_bwd, every
    buffer caller-owned: inputs, outputs, both workspaces) at B1 H32 d128, bf16,
    non-causal, for N = 4096 .. 65536, against the size one materialised bf16
    score matrix would take.  The library allocates nothing itself, so torch's
    peak-allocated counter sees every byte."""
    import torch

    import synth
    import tiled_online_softmax_03_amd as fa

    fa.lib()
    dev = torch.device("cuda:0")
    rows = []
    B, H, d = 1, 32, 128
    for n in (4096, 8192, 16384, 32768, 65536):
        torch.cuda.empty_cache()
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        inp = synth.make_inputs(B, H, n, n, d, "bf16", seed=7000 + n, device=dev)
        Q, K, V, dO = inp["Q"], inp["K"], inp["V"], inp["dO"]
        O = torch.empty_like(Q)
        LSE = torch.empty((B, H, n), device=dev, dtype=torch.float32)
        dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
        ws_f = torch.empty(fa.fa_fwd_workspace_size(B, H, n, n, d), device=dev, dtype=torch.uint8)
        ws_b = fa.alloc_workspace(Q, K)
        scale = d ** -0.5
        stream = torch.cuda.current_stream()

        def step():
            fa.fa_fwd_ws(Q, K, V, O, LSE, ws_f, scale, False, stream)
            fa.fa_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, ws_b, scale, False, stream)

        step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        reps = 2
        for _ in range(reps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        ms = e0.elapsed_time(e1) / reps
        flops = 3.5 * 4.0 * B * H * n * n * d
        rows.append({"N": n, "peak_bytes": peak,
                     "workspace_bytes": ws_f.numel() + ws_b.numel(),
                     "materialised_S_bf16_bytes": B * H * n * n * 2, "step_ms": ms, "step_tflops": flops / ms / 1e9})
        print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
        del inp, Q, K, V, dO, O, LSE, dQ, dK, dV, ws_f, ws_b
    print(json.dumps({"memory_sweep": "fa_fwd_ws + fa_bwd, B1 H32 d128 bf16, non-causal", "rows": rows,
                      "device": torch.cuda.get_device_properties(0).gcnArchName}), flush=True)


def cpu_baseline_fwd(w, inp, heads):
    import numpy as np
    import torch

    import oracle
    import synth

    BH = w.B * w.H
    o = oracle.load()
    long = w.Nq * w.Nk > (1 << 26)  # a full head would take minutes: sampled rows
    views = {}
    for k in ("Q", "K", "V"):
        t = inp[k].reshape(BH, 1, inp[k].shape[2], w.d)[:heads].to("cpu")
        if t.dtype == torch.float32:
            t = t.to(torch.bfloat16)
        views[k] = t.double().numpy()
    if long:
        rows = synth.sample_rows(w.Nq, BH, 256)[:heads]
        rr = np.array(rows)
        t0 = time.perf_counter()
        for h in range(heads):
            o.fwd_rows(views["Q"][h:h + 1], views["K"][h:h + 1], views["V"][h:h + 1], rr[h:h + 1], w.scale, w.causal)
        dt = time.perf_counter() - t0
        # flops of the sampled rows: 4*d per allowed key
        keys = sum((r + 1 if w.causal else w.Nk) for h in range(heads) for r in rows[h])
        flops = 4.0 * w.d * keys
        sample = "256 sampled query rows in each of %d of %d heads of %s, forward, fp64, %.2f s" % (
            heads, BH, w.name, dt)
    else:
        t0 = time.perf_counter()
        o.fwd(views["Q"], views["K"], views["V"], w.scale, w.causal)
        dt = time.perf_counter() - t0
        flops = heads * w.fwd_flops() / BH
        sample = "%d of %d heads of %s, forward, fp64, %.2f s" % (heads, BH, w.name, dt)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": o.num_threads(), "kind": "oracle",
            "sample": sample, "seconds": dt, "gflops_fp64_effective": flops / dt / 1e9,
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def kernel_source_sha256() -> str:
    import glob
    import hashlib
    h = hashlib.sha256()
    # the kernels' sources only (the host-side ABI code does not change what a kernel moves)
    csrc = os.path.join(ROOT, "tiled_online_softmax_03_amd", "csrc")
    for f in sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.hpp"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` (read + written) from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE record of this workload, scaled by the
    same counters' reading of a known-size copy -- or None when there is no
    record or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    k = rec.get("kernels", {}).get(kernel)
    if k is None or rec.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    return k["read_bytes"] + k["write_bytes"]


def cpu_baseline(w, inp, heads, fwd_only=False):
    """The fp64 oracle (fwd + analytic bwd, untiled; or the forward alone) on
    the first `heads` heads of the same inputs -- for the long causal
    workload, on 256 sampled rows of each of those heads -- timed on this
    host's cores."""
    import oracle

    BH = w.B * w.H
    heads = max(1, min(heads, BH))
    if fwd_only:
        return cpu_baseline_fwd(w, inp, heads)
    views = {}
    for k in ("Q", "K", "V", "dO"):
        t = inp[k].reshape(BH, 1, inp[k].shape[2], w.d)[:heads]
        t = t.to("cpu")
        if t.dtype == __import__("torch").float32:
            t = t.to(__import__("torch").bfloat16)
        views[k] = t.double().numpy()
    o = oracle.load()
    t0 = time.perf_counter()
    o.bwd(views["Q"], views["K"], views["V"], views["dO"], w.scale, w.causal)
    dt = time.perf_counter() - t0
    flops = heads * 3.5 * w.fwd_flops() / BH
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": o.num_threads(), "kind": "oracle",
            "sample": "%d of %d heads of %s, forward + backward, fp64, %.2f s" % (heads, BH, w.name, dt),
            "seconds": dt, "gflops_fp64_effective": flops / dt / 1e9, "host_cpus": os.cpu_count(),
            "cpu_model": cpu_model()}


if __name__ == "__main__":
    main()
