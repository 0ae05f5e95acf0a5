#!/usr/bin/env python3
"""Benchmark of the block-sparse matmul training step on one MI355X.

A step is one pass of the whole per-batch path over one batch of synthetic input:
fprop (y = x.W), bprop (dx = dy.W^T) and updat (dW over the present blocks), each
one launch of libbsmm through its C ABI on the current HIP stream.  The layout
compile and the one-time table upload happen before timing; identity_init is timed
once on its own and reported beside the step.

Workload (default): hidden 4096, block 32, minibatch 64, a Bernoulli(0.5) 128x128
block layout (the usage example of the kiteco/blocksparse README, whose placeholders
and weight are float32), float32 storage and arithmetic, feature_axis 1, seed 1001;
bf16 storage with fp32 accumulation is timed beside it (other_dtypes).  Inputs are
seeded synthetic data (synth.workload_problem); there is no dataset.

Timing: R copies of the step's buffers are made, R chosen so that every pass cycles
through at least --rotate-mib MiB of its own operands (the timed launches then read
HBM rather than the 256 MiB Infinity Cache).  After W untimed warm-up steps, exactly
K steps run from HIP graphs (one captured over min(R, K) buffer sets, replayed, and
one for the remainder), bracketed by torch.cuda.synchronize(): that is ms_per_step
and value.  (--overlap runs bprop and updat, the independent halves of the backward
pass, on two streams joined at the end of each step.)  Then each pass is launched
eagerly K times on its own over the rotating sets, with each kernel's dispatch
timestamps recorded (hipExtLaunchKernelGGL start/stop events via
bsmm_profile_begin/end, on the launch stream): the per-pass kernel durations, the
roofline fractions, and a "warm" duration on a single buffer set.

Prints one JSON line (rank 0, N = 1).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0                       # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}   # dense, per dtype
DT_BYTES = {"f32": 4, "bf16": 2, "f16": 2}
PASSES = ("fprop", "bprop", "updat")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="hidden4096_b32_n64")
    ap.add_argument("--dtype", default=None, help="storage dtype (default: the workload's first, f32 for the "
                                                  "usage-example workload)")
    ap.add_argument("--extra-dtypes", default="bf16", help="comma list of further dtypes to time (reported aside)")
    ap.add_argument("--rotate-mib", type=float, default=1024.0)
    ap.add_argument("--overlap", action="store_true",
                    help="run bprop and updat concurrently on two streams in the timed graph "
                         "(measured slower on MI355X: the two kernels compete rather than overlap)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-layer-norm", action="store_true",
                    help="skip the layer_norm, l2_normalize, SparseProj and BlocksparseConv timing")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (for scaling rocprofv3 byte counters)")
    ap.add_argument("--pass-only", choices=PASSES, default=None,
                    help="only launch this pass, --steps times over the rotating buffer sets after --warmup "
                         "launches, and print its kernel time (for per-pass rocprofv3 counter runs)")
    ap.add_argument("--floor", action="store_true",
                    help="only time plain device reads, writes and copies of the benchmark's byte counts "
                         "(torch kernels over rotating buffers): the practical HBM floor at these sizes")
    return ap.parse_args()


def pass_cost(P, dtype):
    """FLOPs and algorithmic HBM bytes of one launch of each pass."""
    b, N, G, nnz = P.block, P.N, len(P.xs), P.nnz
    s = DT_BYTES[dtype]
    C, K = P.R * b, P.S * b
    flops = 2.0 * N * b * b * nnz
    x, y, w = N * C * s, N * K * s, nnz * b * b * s
    dw = nnz * b * b * 4
    return {
        "fprop": (flops, x + y + w),
        "bprop": (flops, y + x + w),
        "updat": (flops * G, G * (x + y) + dw),
    }


def roof(flops, nbytes, dtype):
    t_mfma = flops / (MFMA_PEAK_TFLOPS[dtype] * 1e12)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    return ("mfma", t_mfma) if t_mfma >= t_hbm else ("hbm", t_hbm)


# Sources that decide what a pass's kernels do (kernel code, shared device headers,
# argument set-up and layout tables).  A stored counter reading is used only while the
# hash of these files matches the one recorded with it.
KERNEL_SOURCES = {
    "fprop": ["mm.hip", "mmt.hip", "rows.hip", "common.h", "kernels.h", "lut_format.h", "api.hip", "layout.cpp"],
    "bprop": ["mm.hip", "mmt.hip", "rows.hip", "common.h", "kernels.h", "lut_format.h", "api.hip", "layout.cpp"],
    "updat": ["updat.hip", "common.h", "kernels.h", "lut_format.h", "api.hip", "layout.cpp"],
}


def kernel_sources_sha256(kernel_key):
    """Hash of the sources behind one pass's kernels (KERNEL_SOURCES)."""
    d = os.path.join(ROOT, "block_sparse_matrix_amd", "csrc")
    h = hashlib.sha256()
    for fn in KERNEL_SOURCES[kernel_key]:
        h.update(fn.encode())
        h.update(open(os.path.join(d, fn), "rb").read())
    return h.hexdigest()


def traffic_record(kernel_key, workload, dtype):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if its kernel
    source still matches; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_key}_{workload}_{dtype}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256") != kernel_sources_sha256(kernel_key):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    import torch
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))


def cpu_baseline(P, dtype, target_s):
    """The oracle, untouched, on the host cores: whole passes of the same workload,
    repeated until about target_s seconds have elapsed."""
    import oracle
    import synth
    bits = synth.to_bits
    L, b, fa, N = P.layout, P.block, P.fa, P.N
    x, dy, w = bits(P.xs[0]), bits(P.dys[0]), bits(P.w)
    flops_step = 3 * 2.0 * N * b * b * P.nnz
    done, flops = 0, 0.0
    t0 = time.perf_counter()
    while True:
        oracle.fprop(L, b, fa, x, w, N, dtype)
        oracle.bprop(L, b, fa, dy, w, N, dtype)
        oracle.updat(L, b, fa, [x], [dy], N, dtype)
        done += 1
        flops += flops_step
        if time.perf_counter() - t0 >= target_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{done} full steps (fprop+bprop+updat) of the same workload and seed, "
                      f"{dt:.1f} s on the host, fp64 accumulation",
            "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
            "threads_note": "cores = the oracle's OpenMP threads (OMP_NUM_THREADS, else every CPU in the "
                            "affinity set)"}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def rotation_sets(P, dtype, rotate_mib, set_bytes, cap_bytes=16 << 30):
    """Buffer sets so that each pass cycles through at least rotate_mib MiB of its own
    operands (at most 64 sets, and at most cap_bytes in all)."""
    cost = pass_cost(P, dtype)
    need = max(int(np.ceil(rotate_mib * 2**20 / cost[p][1])) for p in PASSES)
    return max(1, min(64, need, cap_bytes // max(set_bytes, 1)))


def run_dtype(args, name, dtype, rotate_mib, steps, warmup):
    import torch
    import block_sparse_matrix_amd as bs
    import synth

    t0 = time.perf_counter()
    P = synth.workload_problem(name, dtype)
    m = bs.BlocksparseMatMul(P.layout, block_size=P.block, feature_axis=P.fa)
    t_prep = time.perf_counter() - t0   # input generation and layout compile
    t0 = time.perf_counter()
    bs.BlocksparseMatMul(P.layout, block_size=P.block, feature_axis=P.fa)
    t_layout = time.perf_counter() - t0   # layout compile alone
    h, N, G = m.handle, P.N, len(P.xs)
    dev = torch.device("cuda", 0)
    xs0 = [t.to(dev) for t in P.xs]
    dys0 = [t.to(dev) for t in P.dys]
    w0 = P.w.to(dev)
    es = xs0[0].element_size()
    set_bytes = (sum(t.numel() for t in xs0 + dys0) + w0.numel()) * es + (xs0[0].numel() + dys0[0].numel()) * es \
        + w0.numel() * 4
    R = rotation_sets(P, dtype, rotate_mib, set_bytes)
    sets = []
    for _ in range(R):
        sets.append(dict(xs=[t.clone() for t in xs0], dys=[t.clone() for t in dys0], w=w0.clone(),
                         y=torch.empty(m.o_shape(N), dtype=w0.dtype, device=dev),
                         dx=torch.empty(m.i_shape(N), dtype=w0.dtype, device=dev),
                         dw=torch.empty(m.w_shape, dtype=torch.float32, device=dev)))
    ws = {}   # workspaces, allocated once (the graphs replay them)
    for p, code in (("fprop", 0), ("bprop", 1), ("updat", 2)):
        nb = bs.bsmm_workspace_size(h, code, N, w0.dtype)
        ws[p] = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev) if nb else None

    def fprop(s):
        bs.bsmm_fprop(h, s["xs"][0], s["w"], s["y"], N, ws=ws["fprop"])

    def bprop(s):
        bs.bsmm_bprop(h, s["dys"][0], s["w"], s["dx"], N, ws=ws["bprop"])

    def updat(s, accumulate=False):
        bs.bsmm_updat(h, s["xs"], s["dys"], s["dw"], N, accumulate=accumulate, ws=ws["updat"])

    def step(s):
        fprop(s)
        bprop(s)
        updat(s)

    side = torch.cuda.Stream(device=dev)   # default priority

    def step_overlap(s):
        # dx and dW of a backward pass are independent: the weight-read-bound bprop and
        # the gradient-write-bound updat run concurrently on two streams, joined per step
        cur = torch.cuda.current_stream(dev)
        fprop(s)
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            updat(s)
        bprop(s)
        cur.wait_stream(side)

    # identity_init, timed once on its own (after a warm-up launch)
    wi = torch.empty(m.w_shape, dtype=w0.dtype, device=dev)
    bs.bsmm_identity_init(h, wi)
    torch.cuda.synchronize()
    bs.bsmm_profile_begin()
    bs.bsmm_identity_init(h, wi)
    ident = bs.bsmm_profile_end()["identity"]

    # Graphs: exactly `steps` steps, the i-th on buffer set i % R.
    def capture(nsets):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in sets[:nsets]:
                (step_overlap if args.overlap else step)(s)
        return g

    for i in range(max(warmup, 1)):
        step(sets[i % R])
    torch.cuda.synchronize()
    full = capture(min(R, steps))
    reps, rem = (steps // R, steps % R) if steps > R else (1, 0)
    tail = capture(rem) if rem else None
    for i in range(warmup):   # untimed warm-up steps
        step(sets[i % R])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        full.replay()
    if tail is not None:
        tail.replay()
    torch.cuda.synchronize()
    ms_graph = (time.perf_counter() - t0) * 1e3 / steps

    # Eager launches with each kernel's dispatch timestamps recorded (HIP events on the
    # launch stream): the per-kernel durations behind the roofline figures.  Each pass
    # is timed on its own over the rotating sets, so every launch starts from cold
    # buffers (within a step, bprop would find W still cached by fprop).
    one = {"fprop": fprop, "bprop": bprop, "updat": updat}

    def eager(nsets):
        prof = {}
        for p in PASSES:
            for i in range(warmup):
                one[p](sets[i % nsets])
            torch.cuda.synchronize()
            bs.bsmm_profile_begin()
            for i in range(steps):
                one[p](sets[i % nsets])
            torch.cuda.synchronize()
            prof[p] = bs.bsmm_profile_end()[p]
        return prof

    for i in range(warmup):
        step(sets[i % R])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(sets[i % R])
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1e3 / steps
    prof_cold = eager(R)
    prof_warm = eager(1)
    # the accumulating weight gradient (dW += sum), cold over the rotating sets; it reads
    # the stored dW as well, so its algorithmic bytes are G*(|x|+|dy|) + 2*|dW|
    for i in range(warmup):
        updat(sets[i % R], accumulate=True)
    torch.cuda.synchronize()
    bs.bsmm_profile_begin()
    for i in range(steps):
        updat(sets[i % R], accumulate=True)
    torch.cuda.synchronize()
    acc_tot, acc_cnt = bs.bsmm_profile_end()["updat"]
    cost = pass_cost(P, dtype)
    per = {}
    for p in PASSES:
        flops, nbytes = cost[p]
        tot, cnt = prof_cold[p]
        us = tot / cnt * 1e3
        bound, tstar = roof(flops, nbytes, dtype)
        wt, wc = prof_warm[p]
        per[p] = {"kernel": m.kernel_name(p, N, w0.dtype, G if p == "updat" else 1),
                  "kernel_us": round(us, 3), "tflops": round(flops / (us * 1e-6) / 1e12, 3),
                  "alg_GBs": round(nbytes / (us * 1e-6) / 1e9, 1), "alg_bytes": int(nbytes), "flops": int(flops),
                  "bound": bound, "roofline_us": round(tstar * 1e6, 3), "frac": round(tstar / (us * 1e-6), 4),
                  "warm_kernel_us": round(wt / wc * 1e3, 3)}
    aflops, abytes = cost["updat"][0], cost["updat"][1] + P.nnz * P.block * P.block * 4
    aus = acc_tot / acc_cnt * 1e3
    abound, atstar = roof(aflops, abytes, dtype)
    acc = {"kernel_us": round(aus, 3), "alg_bytes": int(abytes), "alg_GBs": round(abytes / (aus * 1e-6) / 1e9, 1),
           "bound": abound, "roofline_us": round(atstar * 1e6, 3), "frac": round(atstar / (aus * 1e-6), 4)}
    flops_step = sum(cost[p][0] for p in PASSES)
    return dict(P=P, ms=ms_graph, ms_eager=ms_eager, per=per, acc=acc, flops_step=flops_step, R=R, steps=steps,
                identity_us=ident[0] / max(ident[1], 1) * 1e3, layout_ms=t_layout * 1e3, prep_s=t_prep)


def roofline_of(per, workload, dtype):
    """The roofline object of the slowest pass (the dominant kernel of a step)."""
    dom = max(PASSES, key=lambda p: per[p]["kernel_us"])
    d = per[dom]
    if d["bound"] == "hbm":
        achieved, peak, unit = d["alg_bytes"] / (d["kernel_us"] * 1e-6) / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = d["flops"] / (d["kernel_us"] * 1e-6) / 1e12, MFMA_PEAK_TFLOPS[dtype], "TFLOP/s"
    return {"bound": d["bound"], "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic_record(dom, workload, dtype),
            "pass": dom, "kernel": d["kernel"], "kernel_us": d["kernel_us"],
            "alg_bytes_per_launch": d["alg_bytes"], "flops_per_launch": d["flops"]}


def run_pass_only(args, name, dtype):
    """One pass of the workload, args.steps launches over rotating buffer sets (cold), after
    args.warmup: the per-pass kernel time, and a clean dispatch list for counter runs."""
    import torch
    import block_sparse_matrix_amd as bs
    import synth
    P = synth.workload_problem(name, dtype)
    m = bs.BlocksparseMatMul(P.layout, block_size=P.block, feature_axis=P.fa)
    h, N, G = m.handle, P.N, len(P.xs)
    dev = torch.device("cuda", 0)
    p = args.pass_only
    code = {"fprop": 0, "bprop": 1, "updat": 2}[p]
    cost = pass_cost(P, dtype)
    w0 = P.w.to(dev)
    if p == "fprop":
        ins, outs = [P.xs[0].to(dev)], torch.empty(m.o_shape(N), dtype=w0.dtype, device=dev)
    elif p == "bprop":
        ins, outs = [P.dys[0].to(dev)], torch.empty(m.i_shape(N), dtype=w0.dtype, device=dev)
    else:
        ins = [t.to(dev) for t in P.xs] + [t.to(dev) for t in P.dys]
        outs = torch.empty(m.w_shape, dtype=torch.float32, device=dev)
    set_bytes = sum(t.numel() * t.element_size() for t in ins) + outs.numel() * outs.element_size() \
        + (w0.numel() * w0.element_size() if p != "updat" else 0)
    R = max(1, min(64, int(np.ceil(args.rotate_mib * 2**20 / cost[p][1])), (16 << 30) // set_bytes))
    sets = [([t.clone() for t in ins], w0.clone() if p != "updat" else None, torch.empty_like(outs)) for _ in range(R)]
    nb = bs.bsmm_workspace_size(h, code, N, w0.dtype)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None

    def launch(s):
        i, w, o = s
        if p == "fprop":
            bs.bsmm_fprop(h, i[0], w, o, N, ws=ws)
        elif p == "bprop":
            bs.bsmm_bprop(h, i[0], w, o, N, ws=ws)
        else:
            bs.bsmm_updat(h, i[:G], i[G:], o, N, ws=ws)

    for i in range(args.warmup):
        launch(sets[i % R])
    torch.cuda.synchronize()
    bs.bsmm_profile_begin()
    for i in range(args.steps):
        launch(sets[i % R])
    torch.cuda.synchronize()
    tot, cnt = bs.bsmm_profile_end()[p]
    us = tot / cnt * 1e3
    flops, nbytes = cost[p]
    bound, tstar = roof(flops, nbytes, dtype)
    print(json.dumps({"workload": name, "dtype": dtype, "pass": p, "kernel": m.kernel_name(p, N, w0.dtype, G if p == "updat" else 1),
                      "launches": args.steps, "warmup": args.warmup, "buffer_sets_rotated": R, "kernel_us": round(us, 3),
                      "alg_bytes": int(nbytes), "flops": int(flops), "bound": bound,
                      "roofline_us": round(tstar * 1e6, 3), "frac": round(tstar / (us * 1e-6), 4)}))


def run_floor(args):
    """Plain streaming kernels (torch) at the benchmark's sizes, cold over rotating buffers:
    read (sum) of |W| bf16 and fp32, write (fill) of |dW| fp32, copy of |W| bf16."""
    import torch
    out = {}
    for label, nbytes, op in (("read_17.8MB", 17807360, "sum"), ("read_35.6MB", 35614720, "sum"),
                              ("write_33.5MB", 33554432, "fill"), ("copy_17.8MB", 17807360, "copy")):
        n = nbytes // 4
        R = max(2, (1 << 30) // nbytes)
        bufs = [torch.ones(n, device="cuda") for _ in range(R)]
        dst = [torch.empty(n, device="cuda") for _ in range(R)] if op == "copy" else None
        acc = torch.empty((), device="cuda")
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

        def go(i):
            if op == "sum":
                torch.sum(bufs[i % R], 0, out=acc)
            elif op == "fill":
                bufs[i % R].fill_(2.0)
            else:
                dst[i % R].copy_(bufs[i % R])

        for i in range(args.warmup):
            go(i)
        torch.cuda.synchronize()
        for i in range(args.steps):
            ev[i][0].record()
            go(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)[len(ev) // 2]
        out[label] = {"bytes": nbytes, "median_us_events": round(us, 3), "op": op}
    print(json.dumps({"floor": out, "note": "torch kernels; the rocprofv3 kernel trace of this command gives "
                                            "their GPU durations"}))


def run_layer_norm(reps=20):
    """Kernel time of layer_norm and its gradient on the band workload's activation
    (N = 4096 vectors of C = 8192 bf16 features), both feature axes, over rotating buffer
    sets; HBM-bound: algorithmic bytes = |x| + |y| forward, |x| + |dy| + |dx| gradient."""
    import numpy as np
    import torch
    import block_sparse_matrix_amd as bs
    import synth
    N, C, dt = 4096, 8192, "bf16"
    out = {"workload": "layer_norm, N=4096 x C=8192 bf16 (hidden8192_b32_n4096_g8 activation)", "epsilon": 1e-6}
    for axis in (1, 0):
        P = synth.norm_problem(np.random.default_rng(7 + axis), N, C, axis, dt)
        R = 4   # 4 sets x 4 tensors x 64 MiB: timed launches read HBM, not the 256 MiB cache
        xs = [P.x.cuda() for _ in range(R)]
        dys = [P.dy.cuda() for _ in range(R)]
        ys = [torch.empty_like(xs[0]) for _ in range(R)]
        dxs = [torch.empty_like(xs[0]) for _ in range(R)]
        g, b = P.g.cuda(), P.b.cuda()
        mean, rstd = torch.empty(N, device="cuda"), torch.empty(N, device="cuda")
        dg, db = torch.empty_like(g), torch.empty_like(b)
        for i in range(4):
            bs.bsmm_layer_norm(xs[i % R], g, b, ys[i % R], mean, rstd, axis, 1e-6, False)
            bs.bsmm_layer_norm_grad(dys[i % R], xs[i % R], g, b, mean, rstd, dxs[i % R], dg, db, axis, False)
        torch.cuda.synchronize()
        bs.bsmm_profile_begin()
        for i in range(reps):
            bs.bsmm_layer_norm(xs[i % R], g, b, ys[i % R], mean, rstd, axis, 1e-6, False)
            bs.bsmm_layer_norm_grad(dys[i % R], xs[i % R], g, b, mean, rstd, dxs[i % R], dg, db, axis, False)
        torch.cuda.synchronize()
        pr = bs.bsmm_profile_end()
        act = N * C * 2
        for key, nb in (("layer_norm", 2 * act + 2 * C * 4), ("layer_norm_grad", 3 * act + 4 * C * 4)):
            us = pr[key][0] / pr[key][1] * 1e3
            gbs = nb / (us * 1e-6) / 1e9
            out[f"{key}_axis{axis}"] = {"kernel_us": round(us, 3), "alg_bytes": nb, "achieved_GBps": round(gbs, 1),
                                        "peak_GBps": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4),
                                        "bound": "hbm"}
    return out


def run_sparse_proj(reps=20):
    """Kernel time of the SparseProj ops on the band workload's activation: nhidden 8192
    dense features projected to 4096 (every other block of 32, proj_stride 64), N = 4096,
    bf16, features last, over rotating buffer sets; HBM-bound, algorithmic bytes: gather
    2*N*P, scatter N*P + N*H, scatter_add / scatter_mul 2*N*H + N*P, gather_mul 3*N*P
    (elements of 2 bytes; P = 4096, H = 8192)."""
    import numpy as np
    import torch
    import block_sparse_matrix_amd as bs
    import synth
    N, H, Pn, dt = 4096, 8192, 4096, "bf16"
    P = synth.proj_problem(np.random.default_rng(17), N, H, Pn, 1, dt, False)
    proj = bs.SparseProj(H, Pn, 64, 32)
    R = 4   # 4 sets x ~224 MiB: timed launches read HBM, not the 256 MiB cache
    xs = [P.x.cuda() for _ in range(R)]
    ss = [P.s.cuda() for _ in range(R)]
    gs = [torch.empty(N, Pn, dtype=xs[0].dtype, device="cuda") for _ in range(R)]
    zs = [torch.empty_like(xs[0]) for _ in range(R)]
    h = proj.handle

    def launch(i):
        x, s, g, z = xs[i % R], ss[i % R], gs[i % R], zs[i % R]
        bs.bsmm_proj_gather(h, x, g, N)
        bs.bsmm_proj_scatter(h, s, z, N)
        bs.bsmm_proj_scatter_add(h, x, s, z, N)
        bs.bsmm_proj_scatter_mul(h, x, s, z, N)
        bs.bsmm_proj_gather_mul(h, x, zs[(i + 1) % R], g, N)

    for i in range(4):
        launch(i)
    torch.cuda.synchronize()
    bs.bsmm_profile_begin()
    for i in range(reps):
        launch(i)
    torch.cuda.synchronize()
    pr = bs.bsmm_profile_end()
    e = 2
    nbytes = {"proj_gather": 2 * N * Pn * e, "proj_scatter": (N * Pn + N * H) * e,
              "proj_scatter_add": (2 * N * H + N * Pn) * e, "proj_scatter_mul": (2 * N * H + N * Pn) * e,
              "proj_gather_mul": 3 * N * Pn * e}
    out = {"workload": "SparseProj nhidden 8192 -> nproj 4096 (blocks of 32, proj_stride 64), N=4096, bf16, "
                       "features last"}
    for key, nb in nbytes.items():
        us = pr[key][0] / pr[key][1] * 1e3
        gbs = nb / (us * 1e-6) / 1e9
        out[key[5:]] = {"kernel_us": round(us, 3), "alg_bytes": nb, "achieved_GBps": round(gbs, 1),
                        "peak_GBps": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4), "bound": "hbm"}
    return out


def run_conv(reps=3, dt="bf16", strides=(1, 1)):
    """Kernel time of BlocksparseConv (fprop, input gradient, filter gradient) on a 2-D
    workload: 256 input and output channels in blocks of 32 x 32 channels (half of the
    8 x 8 block grid present, consecutive channels), 3 x 3 filter, 32 x 32 images,
    N = 32, SAME, stride 1 and bf16 unless given.  FLOPs per pass 2 * N * M*P*Q *
    nblocks * Bc * Bk * T*R*S; algorithmic bytes |I| + |O| + |F| (fprop, bprop), |I| +
    |dO| + |dF| (float32 dF)."""
    import numpy as np
    import torch
    import block_sparse_matrix_amd as bs
    import synth
    N, C, B, TRS, DHW = 32, 256, 32, (3, 3), (32, 32)
    nb = (C // B) * (C // B) // 2
    MPQ = tuple((d + s - 1) // s for d, s in zip(DHW, strides))   # SAME
    P = synth.conv_problem(np.random.default_rng(23), N, C, C, B, B, nb, TRS, DHW, MPQ, dt,
                           contiguous_blocks=True)
    conv = bs.BlocksparseConv(P.BCK, TRS, DHW, strides=strides)
    F, I, dO = P.F.cuda(), P.I.cuda(), P.dO.cuda()
    O, dI = torch.empty_like(dO), torch.empty_like(I)
    dF = torch.empty(conv.f_shape(), dtype=torch.float32, device="cuda")
    h = conv.handle
    tdt = synth.DTYPES[dt]

    def launch():
        bs.bsmm_conv_fprop(h, F, I, O, N)
        bs.bsmm_conv_bprop(h, F, dO, dI, N)
        bs.bsmm_conv_updat(h, I, dO, dF, N)

    launch()
    torch.cuda.synchronize()
    bs.bsmm_profile_begin()
    for _ in range(reps):
        launch()
    torch.cuda.synchronize()
    pr = bs.bsmm_profile_end()
    es = 4 if dt == "f32" else 2
    flops = 2.0 * N * MPQ[0] * MPQ[1] * nb * B * B * TRS[0] * TRS[1]
    iact, oact, fb = N * C * DHW[0] * DHW[1] * es, N * C * MPQ[0] * MPQ[1] * es, nb * B * B * TRS[0] * TRS[1]
    nbytes = {"conv_fprop": iact + oact + es * fb, "conv_bprop": iact + oact + es * fb,
              "conv_updat": iact + oact + 4 * fb}
    out = {"workload": f"BlocksparseConv 2-D, C = K = {C} in {B}x{B}-channel blocks ({nb} of 64), 3x3 filter, "
                       f"32x32 images, N = {N}, SAME, strides {tuple(strides)}, {dt}"}
    for key, nbt in nbytes.items():
        us = pr[key][0] / pr[key][1] * 1e3
        bound, tstar = roof(flops, nbt, dt)
        out[key[5:]] = {"kernel_us": round(us, 3), "tflops": round(flops / (us * 1e-6) / 1e12, 3),
                        "alg_bytes": int(nbt), "flops": int(flops), "bound": bound,
                        "roofline_us": round(tstar * 1e6, 3), "frac": round(tstar / (us * 1e-6), 5),
                        "kernels": conv.kernel_name(key[5:], tdt)}
    return out


def run_l2_normalize(P, reps=40):
    """Kernel time of BlocksparseMatMul.l2_normalize (weight normalisation per output
    feature, bf16 weights -> bf16) and its gradient (bf16 upstream -> fp32 dW) on this
    workload's layout, over rotating weight sets; HBM-bound: algorithmic bytes = |W| read
    + |W| written forward, |dOut| + |W| read + |dW| (fp32) written for the gradient."""
    import torch
    import block_sparse_matrix_amd as bs
    m = bs.BlocksparseMatMul(P.layout, block_size=P.block, feature_axis=P.fa)
    w0 = P.w.to(torch.bfloat16)
    R = 16
    ws = [w0.cuda() for _ in range(R)]
    outs = [torch.empty_like(ws[0]) for _ in range(R)]
    dys = [torch.ones_like(ws[0]) for _ in range(R)]
    dws = [torch.empty(ws[0].shape, device="cuda") for _ in range(R)]
    g = torch.ones(m.K, device="cuda")
    dg = torch.empty_like(g)
    for i in range(3):
        bs.bsmm_l2_normalize(m.handle, ws[i], g, outs[i], None)
        bs.bsmm_l2_normalize_grad(m.handle, dys[i], ws[i], g, dws[i], dg)
    torch.cuda.synchronize()
    bs.bsmm_profile_begin()
    for i in range(reps):
        bs.bsmm_l2_normalize(m.handle, ws[i % R], g, outs[i % R], None)
        bs.bsmm_l2_normalize_grad(m.handle, dys[i % R], ws[i % R], g, dws[i % R], dg)
    torch.cuda.synchronize()
    pr = bs.bsmm_profile_end()
    W = w0.numel() * 2
    out = {"workload": f"l2_normalize on the {P.nnz}-block layout, bf16 weights"}
    for key, nb in (("l2_normalize", 2 * W + 8 * m.K), ("l2_normalize_grad", 2 * W + 2 * W + 8 * m.K)):
        us = pr[key][0] / pr[key][1] * 1e3
        gbs = nb / (us * 1e-6) / 1e9
        out[key] = {"kernel_us": round(us, 3), "alg_bytes": nb, "achieved_GBps": round(gbs, 1),
                    "peak_GBps": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4), "bound": "hbm"}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the passes are single-device kernels; multi-GPU sharding is not implemented).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.floor:
        run_floor(args)
        return
    if args.pass_only:
        import synth
        wl = synth.WORKLOADS[args.workload]
        run_pass_only(args, args.workload, args.dtype or wl.dtypes[0])
        return
    import torch
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    wl = synth.WORKLOADS[args.workload]
    dtype = args.dtype or wl.dtypes[0]
    res = run_dtype(args, args.workload, dtype, args.rotate_mib, args.steps, args.warmup)
    P, per = res["P"], res["per"]
    roofline = roofline_of(per, args.workload, dtype)
    value = res["flops_step"] / (res["ms"] * 1e-3) / 1e12
    out = {
        "metric": "effective TFLOP/s (nonzero blocks) fprop/bprop/updat; % MFMA or HBM roofline",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": res["steps"], "warmup": args.warmup,
        "ms_per_step": round(res["ms"], 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype, "data": "synthetic",
        "config": {"workload": args.workload, "hidden": wl.hidden, "block": wl.block, "minibatch": P.N,
                   "feature_axis": wl.fa, "layout": wl.layout_kind, "seed": wl.seed, "nnz": P.nnz,
                   "passes": "fprop+bprop+updat", "buffer_sets_rotated": res["R"]},
        "roofline": roofline,
        "per_pass": per,
        "updat_accumulate": res["acc"],
        "timing": "ms_per_step: HIP-graph replay of the three launches per step over rotating buffer sets"
                  + (" (bprop and updat on two streams, joined each step)" if args.overlap else "")
                  + "; per_pass.kernel_us: dispatch timestamps of eager launches, one stream",
        "eager_ms_per_step": round(res["ms_eager"], 5),
        "identity_init_us": round(res["identity_us"], 3),
        "layout_compile_ms": round(res["layout_ms"], 3),
    }
    extras = {}
    for xd in [t for t in args.extra_dtypes.split(",") if t and t in wl.dtypes and t != dtype]:
        r = run_dtype(args, args.workload, xd, args.rotate_mib, args.steps, args.warmup)
        extras[xd] = {"value": round(r["flops_step"] / (r["ms"] * 1e-3) / 1e12, 3), "ms_per_step": round(r["ms"], 5),
                      "eager_ms_per_step": round(r["ms_eager"], 5),
                      "roofline": roofline_of(r["per"], args.workload, xd), "per_pass": r["per"],
                      "updat_accumulate": r["acc"], "buffer_sets_rotated": r["R"]}
    if extras:
        out["other_dtypes"] = extras
    if not args.no_layer_norm:
        out["layer_norm"] = run_layer_norm()
        out["l2_normalize"] = run_l2_normalize(P)
        out["sparse_proj"] = run_sparse_proj()
        out["conv"] = run_conv()
        out["conv_f32"] = run_conv(dt="f32")
        out["conv_strided"] = run_conv(strides=(2, 2))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(P, dtype, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
