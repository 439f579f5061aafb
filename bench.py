#!/usr/bin/env python3
"""Benchmark of the low-bit weight-only quantized linear path on one MI355X.

Headline workload (the dense decode stack at M = 1): LAYERS layers, each four
2-bit group-128 linears (qkv 4096->6144, o 4096->4096, gate|up 4096->28672,
down 14336->4096) run at M = 1 token through lbq_linear_forward. A step is one
pass over every layer. Each layer has its own copy of the packed weights in
HBM (same bytes, distinct addresses), 1.96 GB per step at 32 layers, so the
256 MB last-level cache cannot serve repeats: every step streams the packed
weights from HBM.

  value = packed-weight bytes per step * steps / wall time of the timed steps

The steps are replayed from a HIP graph captured once (no Python launch
overhead in the timed region), inputs resident in HBM. The dominant kernel is
the matrix-core GEMV with the fused rotation (gemv_mfma_kernel; it serves all
four linears, one launch each); its launch durations are measured live with
HIP events on the stream it is launched on, for each of its launches
in an eager pass over the same steps (lbq_linear_forward_timed: the kernel's
launch itself carries the events, so they hold its own begin / end times, the
same quantity rocprofv3 reports); roofline.achieved = its algorithmic
bytes (packed planes + scale/zero words) summed over those launches / their
summed durations. roofline.traffic (HBM bytes per launch, from rocprofv3
FETCH_SIZE + WRITE_SIZE scaled by a copy kernel of known size) is read from
the committed counter summary and reported only while the kernel sources are
the ones the counters were taken on.

extra: every other part of the hot path, each against its own roofline: the
single 4096x4096 linear, the stack at M = 4 and 16, the 5120/17408 FFN pair at
M = 1, 8, 64, 256 (the TFLOP/s at M = 64 is the metric's second half), the
product-VQ 4096->14336 linear at M = 1, 16, 64, the 256-expert MoE block at
M = 32, the router and the rotation alone.

Prints one JSON line. With --summarize it instead turns rocprofv3 outputs of
this script into the text summary kept under profiles/.
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "packed-weight HBM GB/s (% of peak) for 2-bit dequant-GEMV at M=1; TFLOP/s at M=64"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA
DOMINANT = "gemv_mfma_kernel"
# sources the dominant kernel is built from (traffic from counters is stale once they change)
DOMINANT_SOURCES = ["bit_weight_only_amd/csrc/gemv_mfma.hip", "bit_weight_only_amd/csrc/mx_core.h",
                    "bit_weight_only_amd/csrc/gemm_common.h", "bit_weight_only_amd/csrc/device.h"]
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "gemv_mfma_dense_stack_m1.txt")
CALIB_BYTES = 512 << 20        # the copy kernel reads and writes this many bytes


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for p in DOMINANT_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def roofline(nbytes, flops, seconds):
    """Lower bound and binding unit for algorithmic bytes / flops over a duration."""
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_F16_PEAK_TFLOPS * 1e12)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    return {"bound": bound, "frac": round(max(t_hbm, t_mfma) / seconds, 4),
            "GBps": round(nbytes / seconds / 1e9, 1), "TFLOPs": round(flops / seconds / 1e12, 2)}


# ---------------------------------------------------------------- timing helpers

def time_graph(torch, fn, steps, warmup):
    """Capture fn(stream_ptr) once into a HIP graph, replay warmup + steps times;
    return wall seconds of the timed replays."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(ctypes.c_void_p(s.cuda_stream))        # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    t = time.perf_counter() - t0
    del g
    return t


def check(st, what):
    if st != 0:
        raise RuntimeError(f"{what} failed with status {st}")


class Linears:
    """COPIES device copies of one packed linear plus per-M buffers."""

    def __init__(self, L, torch, K, N, bits, fmt, planes, meta, signs, codebook, copies):
        dev = torch.device("cuda:0")
        self.L, self.torch, self.K, self.N, self.bits = L, torch, K, N, bits
        s_dev = torch.from_numpy(signs).to(dev)
        cb = None if codebook is None else torch.from_numpy(codebook).to(dev)
        self.copies = [L.PackedLinear(K, N, bits, fmt, torch.from_numpy(planes).to(dev), torch.from_numpy(meta).to(dev),
                                      s_dev, cb) for _ in range(copies)]
        self.bytes = planes.nbytes + meta.nbytes + (0 if codebook is None else codebook.nbytes)

    def calls(self, M, x):
        torch = self.torch
        y = torch.empty((M, self.N), dtype=torch.float16, device=x.device)
        ws = torch.empty(max(1, self.copies[0].workspace_bytes(M)), dtype=torch.uint8, device=x.device)
        self._keep = (x, y, ws)
        return [(ctypes.byref(c.struct), ctypes.c_void_p(x.data_ptr()), M, ctypes.c_void_p(y.data_ptr()),
                 ctypes.c_void_p(ws.data_ptr()), ws.numel()) for c in self.copies]


def run_calls(lib, calls):
    fwd = lib.lbq_linear_forward

    def fn(sp):
        for (w, x, M, y, ws, n) in calls:
            check(fwd(w, x, M, y, ws, n, sp), "lbq_linear_forward")
    return fn


# ---------------------------------------------------------------- headline

class Stack:
    """Packed dense-stack weights, LAYERS device copies, and per-shape buffers."""

    def __init__(self, L, torch, layers: int, M: int):
        self.L, self.torch, self.layers, self.M = L, torch, layers, M
        dev = torch.device("cuda:0")
        self.shapes = []
        for idx, (name, k, n) in enumerate(synth.DENSE_STACK_SHAPES):
            w = synth.weights(n, k, workload=synth.W_STACK, item=idx)
            s = synth.signs(k, workload=synth.W_STACK, item=idx)
            planes, meta = L.pack(w, 2, s)
            del w
            lin = Linears(L, torch, k, n, 2, L.FMT_RTN_PLANES, planes, meta, s, None, layers)
            x = torch.from_numpy(synth.activations(M, k, workload=synth.W_STACK, item=idx)).to(dev)
            self.shapes.append(dict(name=name, K=k, N=n, lin=lin, calls=lin.calls(M, x), bytes=lin.bytes))
        self.bytes_per_step = sum(sh["bytes"] for sh in self.shapes) * layers
        self.flops_per_step = sum(2.0 * M * sh["K"] * sh["N"] for sh in self.shapes) * layers
        self.lib = L.lib()
        self.order = [(sh, sh["calls"][layer]) for layer in range(layers) for sh in self.shapes]

    def step(self, sp):
        fwd = self.lib.lbq_linear_forward
        for sh, (w, x, M, y, ws, n) in self.order:
            check(fwd(w, x, M, y, ws, n, sp), "lbq_linear_forward")


def event_pass(torch, stack, reps=2):
    """Eager steps on one stream through lbq_linear_forward_timed: HIP events
    created on this process's runtime take the main kernel's own begin / end
    times (for the single-token GEMV, the kernel launch itself carries them).
    {shape: [seconds]}."""
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    fwd = stack.lib.lbq_linear_forward_timed
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(len(stack.order) * reps)]
    for e0, e1 in pairs:          # create the underlying events
        e0.record(stream)
        e1.record(stream)
    torch.cuda.synchronize()
    torch.cuda._sleep(300_000_000)
    done = []
    i = 0
    for _ in range(reps):
        for sh, (w, x, M, y, ws, n) in stack.order:
            e0, e1 = pairs[i]
            i += 1
            check(fwd(w, x, M, y, ws, n, sp, ctypes.c_void_p(e0.cuda_event), ctypes.c_void_p(e1.cuda_event)),
                  "lbq_linear_forward_timed")
            done.append((sh["name"], e0, e1))
    torch.cuda.synchronize()
    per = {}
    for name, e0, e1 in done:
        per.setdefault(name, []).append(e0.elapsed_time(e1) * 1e-3)
    return per


def calibration_copy(torch):
    """A plain elementwise copy of CALIB_BYTES (read and write; torch's unary
    multiply-by-one kernel): the reference dispatch the counter summary scales
    FETCH_SIZE / WRITE_SIZE by."""
    n = CALIB_BYTES // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    del a, b


def traffic_from_summary():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when absent or taken on other kernel sources."""
    try:
        with open(PROFILE_SUMMARY) as f:
            text = f.read()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines() if line.startswith("@") and ":" in line)
    try:
        if fields["@source_hash"].strip() != source_hash():
            return None
        return float(fields["@traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline(L, budget_s=12.0):
    """The oracle on this host: y = x W_hat^T for the dense-stack matrices at
    M = 1, whole matrices, repeated over the four shapes until ~budget_s."""
    from oracle import lbq_oracle as O   # test infrastructure: the oracle is the reported baseline

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    prepared = []
    for idx, (name, k, n) in enumerate(synth.DENSE_STACK_SHAPES):
        w = synth.weights(n, k, workload=synth.W_STACK, item=idx)
        s = synth.signs(k, workload=synth.W_STACK, item=idx)
        planes, meta = L.pack(w, 2, s)
        del w
        x = synth.activations(1, k, workload=synth.W_STACK, item=idx)
        prepared.append((name, k, n, planes, meta, s, x))
    total_bytes, total_t, calls = 0, 0.0, []
    while total_t < budget_s:
        for (name, k, n, planes, meta, s, x) in prepared:
            t0 = time.perf_counter()
            O.linear_rtn(x, planes, meta, s, 2, n, k)
            total_t += time.perf_counter() - t0
            total_bytes += planes.nbytes + meta.nbytes
            calls.append(name)
        if len(calls) >= 16:
            break
    return {"value": round(total_bytes / total_t / 1e9, 6), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"the oracle (numpy fp64: unpack, dequantize, inverse-rotate, matmul) on whole dense-stack "
                      f"matrices at M=1, 2-bit ({len(calls)} calls: {', '.join(calls)}), {total_bytes} packed bytes "
                      f"in {total_t:.1f} s; elementwise numpy work single-threaded, BLAS on {threads} threads"}


# ---------------------------------------------------------------- extra measurements

def measure_linears(torch, L, lin, M, steps, x=None, workload=0):
    dev = torch.device("cuda:0")
    if x is None:
        x = torch.from_numpy(synth.activations(M, lin.K, workload=workload, item=M)).to(dev)
    calls = lin.calls(M, x)
    t = time_graph(torch, run_calls(L.lib(), calls), steps, 2)
    per = t / steps / len(calls)
    out = {"M": M, "us_per_call": round(per * 1e6, 3)}
    out.update(roofline(lin.bytes, 2.0 * M * lin.K * lin.N, per))
    return out


def extra_single(torch, L, steps):
    cfg = synth.SINGLE_LINEAR
    w = synth.weights(cfg["N"], cfg["K"], workload=synth.W_SINGLE)
    s = synth.signs(cfg["K"], workload=synth.W_SINGLE)
    planes, meta = L.pack(w, 2, s)
    lin = Linears(L, torch, cfg["K"], cfg["N"], 2, 0, planes, meta, s, None, 64)
    r = measure_linears(torch, L, lin, 1, steps, workload=synth.W_SINGLE)
    del lin
    return r


def extra_stack(torch, L, M, steps, layers=8):
    st = Stack(L, torch, layers, M)
    t = time_graph(torch, st.step, steps, 2)
    per = t / steps
    out = {"M": M, "layers": layers, "us_per_layer": round(per / layers * 1e6, 2)}
    out.update(roofline(st.bytes_per_step, st.flops_per_step, per))
    del st
    torch.cuda.empty_cache()
    return out


def extra_ffn(torch, L, steps):
    cfg = synth.FFN_SWEEP
    mats = []
    for (k, n, bits, item) in [(cfg["K_gu"], cfg["N_gu"], cfg["bits_gu"], 1), (cfg["N_gu"], cfg["K_gu"], cfg["bits_dn"], 2)]:
        w = synth.weights(n, k, workload=synth.W_FFN, item=item)
        s = synth.signs(k, workload=synth.W_FFN, item=item)
        planes, meta = L.pack(w, bits, s)
        del w
        mats.append(Linears(L, torch, k, n, bits, 0, planes, meta, s, None, 6))
    dev = torch.device("cuda:0")
    res = {}
    for M in cfg["M"]:
        calls = []
        for lin in mats:
            x = torch.from_numpy(synth.activations(M, lin.K, workload=synth.W_FFN, item=M)).to(dev)
            calls += lin.calls(M, x)
            lin._keep_m = lin._keep
        t = time_graph(torch, run_calls(L.lib(), calls), steps, 2)
        per = t / steps / 6           # one gate|up + one down
        nbytes = sum(m.bytes for m in mats)
        flops = sum(2.0 * M * m.K * m.N for m in mats)
        r = {"M": M, "us_per_ffn": round(per * 1e6, 2)}
        r.update(roofline(nbytes, flops, per))
        res[f"M{M}"] = r
    del mats
    torch.cuda.empty_cache()
    return res


def extra_pvq(torch, L, steps):
    cfg = synth.PVQ_LINEAR
    cb = synth.codebook(workload=synth.W_PVQ)
    w = synth.weights(cfg["N"], cfg["K"], workload=synth.W_PVQ)
    s = synth.signs(cfg["K"], workload=synth.W_PVQ)
    idx, sc = L.pack(w, 2, s, L.FMT_PVQ_4x8, cb)
    del w
    lin = Linears(L, torch, cfg["K"], cfg["N"], 2, L.FMT_PVQ_4x8, idx, sc, s, cb, 24)
    res = {f"M{M}": measure_linears(torch, L, lin, M, steps, workload=synth.W_PVQ) for M in cfg["M"]}
    del lin
    torch.cuda.empty_cache()
    return res


def extra_moe(torch, L, steps):
    cfg = synth.MOE_BLOCK
    E, H, F, k, M = cfg["E"], cfg["hidden"], cfg["ffn"], cfg["top_k"], cfg["M"]
    dev = torch.device("cuda:0")
    bits = synth.expert_bits(E, workload=synth.W_MOE)
    sh = synth.signs(H, workload=synth.W_MOE, item=1)
    sf = synth.signs(F, workload=synth.W_MOE, item=2)
    packed = L.pack_moe_host(lambda e: synth.weights(2 * F, H, workload=synth.W_MOE, item=1000 + e),
                             lambda e: synth.weights(H, F, workload=synth.W_MOE, item=5000 + e), bits, sh, sf)
    moe = L.moe_from_host(packed, bits, sh, sf, H, F, k)
    per_expert = [0] * E
    for e in range(E):
        b = int(bits[e])
        per_expert[e] = (2 * F * H + H * F) * b // 8 + (2 * F * H + H * F) // 128 * 4
    # a few token batches with their own logits: different expert subsets per call
    batches = []
    touched = []
    for item in range(4):
        x = torch.from_numpy(synth.activations(M, H, workload=synth.W_MOE, item=item)).to(dev)
        lg_np = synth.logits(M, E, workload=synth.W_MOE, item=item)
        ids = np.argsort(-lg_np, axis=1, kind="stable")[:, :k]
        touched.append(sum(per_expert[e] for e in np.unique(ids)))
        lg = torch.from_numpy(lg_np).to(dev)
        y = torch.empty((M, H), dtype=torch.float16, device=dev)
        ws = torch.empty(moe.workspace_bytes(M), dtype=torch.uint8, device=dev)
        batches.append((x, lg, y, ws))
    lib = L.lib()

    def fn(sp):
        for (x, lg, y, ws) in batches:
            check(lib.lbq_moe_forward(ctypes.byref(moe.struct), ctypes.c_void_p(x.data_ptr()),
                                      ctypes.c_void_p(lg.data_ptr()), M, ctypes.c_void_p(y.data_ptr()),
                                      ctypes.c_void_p(ws.data_ptr()), ws.numel(), sp), "lbq_moe_forward")
    t = time_graph(torch, fn, steps, 2)
    per = t / steps / len(batches)
    nbytes = float(np.mean(touched))
    flops = 2.0 * M * k * (2 * F * H + H * F)
    out = {"M": M, "us_per_block": round(per * 1e6, 2), "touched_bytes_avg": int(nbytes)}
    out.update(roofline(nbytes, flops, per))

    # the router alone and the rotation alone (latency-bound launches)
    lg = batches[0][1]
    ids = torch.empty((M, k), dtype=torch.int32, device=dev)
    wts = torch.empty((M, k), dtype=torch.float32, device=dev)
    cnt = torch.empty(E, dtype=torch.int32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(M * k, dtype=torch.int32, device=dev)

    def route(sp):
        for _ in range(20):
            check(lib.lbq_moe_route(ctypes.c_void_p(lg.data_ptr()), M, E, k, ctypes.c_void_p(ids.data_ptr()),
                                    ctypes.c_void_p(wts.data_ptr()), ctypes.c_void_p(cnt.data_ptr()),
                                    ctypes.c_void_p(off.data_ptr()), ctypes.c_void_p(perm.data_ptr()), sp),
                  "lbq_moe_route")
    out["router_us"] = round(time_graph(torch, route, steps, 2) / steps / 20 * 1e6, 3)
    xr = torch.empty((M, H), dtype=torch.float16, device=dev)
    x0, s_dev = batches[0][0], torch.from_numpy(sh).to(dev)

    def rot(sp):
        for _ in range(20):
            check(lib.lbq_rotate(ctypes.c_void_p(x0.data_ptr()), M, H, ctypes.c_void_p(s_dev.data_ptr()),
                                 ctypes.c_void_p(xr.data_ptr()), sp), "lbq_rotate")
    out["rotate_us"] = round(time_graph(torch, rot, steps, 2) / steps / 20 * 1e6, 3)
    del moe, packed, batches
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- counter summary

def summarize(fetch_dir, write_dir, trace_dir, command, out_path):
    """Turn rocprofv3 outputs of this script into the profiles/ text summary:
    kernel-trace statistics, and FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of
    the dominant kernel scaled by what the same counters read for the copy of
    CALIB_BYTES."""
    import csv

    def counters(d, name):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            rows += [r for r in csv.DictReader(open(f)) if r["Counter_Name"] == name]
        per_dispatch = {}
        for r in rows:
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
        return per_dispatch

    fetch, write = counters(fetch_dir, "FETCH_SIZE"), counters(write_dir, "WRITE_SIZE")

    def pick(d, sub):
        v = [x for (i, kname), x in d.items() if sub in kname]
        return (float(np.mean(v)) if v else float("nan")), len(v)

    k_fetch, n1 = pick(fetch, DOMINANT)
    k_write, n2 = pick(write, DOMINANT)
    c_fetch, n3 = pick(fetch, "AUnaryFunctor")   # the multiply-by-one copy of calibration_copy()
    c_write, n4 = pick(write, "AUnaryFunctor")
    f_fetch = CALIB_BYTES / (c_fetch * 1024.0)
    f_write = CALIB_BYTES / (c_write * 1024.0)
    traffic = k_fetch * 1024.0 * f_fetch + k_write * 1024.0 * f_write
    stats = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True):
        stats += list(csv.DictReader(open(f)))
    trace = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        trace += list(csv.DictReader(open(f)))
    # the event pass starts behind the one spin kernel (torch.cuda._sleep) of the command
    spin = [int(r["Start_Timestamp"]) for r in trace if "spin_kernel" in r["Kernel_Name"]]
    t_spin = max(spin) if spin else 0
    dom = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace
           if DOMINANT in r["Kernel_Name"] and int(r["Start_Timestamp"]) > t_spin]
    dom_all = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace if DOMINANT in r["Kernel_Name"]]
    # the dominant kernel's launches in the stack: its algorithmic bytes per launch on average
    stack_bytes = [planes_meta_bytes(k, n, 2) for (_, k, n) in synth.DENSE_STACK_SHAPES]
    lines = [
        "rocprofv3 summary: matrix-core dequant-GEMV with fused rotation (gemv_mfma_kernel),",
        "dense decode stack at M=1 (qkv 4096->6144, o 4096->4096, gate|up 4096->28672, down 14336->4096;",
        "2-bit group-128).",
        "",
        f"commands (run from the repository root, cd /tmp && export TMPDIR=/tmp first):",
        f"  rocprofv3 --kernel-trace --stats -d <dir> -o k --output-format csv -- {command}",
        f"  rocprofv3 --pmc FETCH_SIZE -d <dir> -o f --output-format csv -- {command}",
        f"  rocprofv3 --pmc WRITE_SIZE -d <dir> -o w --output-format csv -- {command}",
        f"  python3 bench.py --summarize <fetch dir> <write dir> <trace dir>",
        "",
        "kernel-trace statistics (per kernel name, all launches of the command):",
        f"  {'kernel':90s} {'calls':>7s} {'avg us':>10s} {'total us':>12s}",
    ]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"]))[:12]:
        lines.append(f"  {r['Name'][:90]:90s} {int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.3f} "
                     f"{float(r['TotalDurationNs']) / 1e3:12.1f}")
    lines += [
        "",
        f"{DOMINANT} launch durations from the trace: all {len(dom_all)} launches (graph replays and the",
        f"event pass) {float(np.mean(dom_all)) if dom_all else float('nan'):.3f} us on average; the {len(dom)} "
        f"launches of the event pass (after the spin",
        f"kernel; the launches bench.py times with HIP events) {float(np.mean(dom)) if dom else float('nan'):.3f} us "
        f"on average.",
        "",
        f"counters (KiB per dispatch, mean): {DOMINANT}: FETCH_SIZE {k_fetch:.1f} (n={n1}), "
        f"WRITE_SIZE {k_write:.1f} (n={n2})",
        f"copy of {CALIB_BYTES} bytes (read and write): FETCH_SIZE {c_fetch:.1f} (n={n3}), WRITE_SIZE {c_write:.1f} "
        f"(n={n4})",
        f"scale factors (bytes per counter KiB / 1024): fetch {f_fetch:.4f}, write {f_write:.4f}",
        f"algorithmic bytes per launch of {DOMINANT} in the stack (mean over qkv, o, gate|up, down): "
        f"{float(np.mean(stack_bytes)):.0f}",
        "",
        f"@source_hash: {source_hash()}",
        f"@traffic_bytes_per_launch: {traffic:.0f}",
    ]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def trace_table(trace_dir, out_path):
    """Per-kernel durations of every part of the hot path, from a rocprofv3
    kernel trace of the default bench command."""
    import csv

    stats = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True):
        stats += list(csv.DictReader(open(f)))
    lines = [
        "rocprofv3 kernel-trace statistics of the default bench command (all parts of the hot path:",
        "dense stack at M=1, 4, 16; FFN pair at M=1, 8, 64, 256; product-VQ at M=1, 16, 64; MoE block at M=32;",
        "oracle timing on the host runs no GPU kernels).",
        "",
        "command (run from the repository root, cd /tmp && export TMPDIR=/tmp first):",
        "  rocprofv3 --kernel-trace --stats -d <dir> -o k --output-format csv -- python3 bench.py",
        "  python3 bench.py --trace-summary <dir> <this file>",
        "",
        f"  {'kernel':100s} {'calls':>7s} {'avg us':>10s} {'min us':>9s} {'total us':>12s}",
    ]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"  {r['Name'][:100]:100s} {int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.3f} "
                     f"{float(r['MinNs']) / 1e3:9.3f} {float(r['TotalDurationNs']) / 1e3:12.1f}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def planes_meta_bytes(k, n, bits):
    return n * k * bits // 8 + n * (k // 128) * 4


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--no-extra", action="store_true", help="skip the measurements of the other configurations")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing on the host")
    ap.add_argument("--summarize", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "TRACE_DIR"),
                    help="write the counter summary under profiles/ from rocprofv3 outputs, then exit")
    ap.add_argument("--summary-command", default="python3 bench.py --steps 5 --warmup 1 --no-extra --no-cpu")
    ap.add_argument("--trace-summary", nargs=2, metavar=("TRACE_DIR", "OUT"),
                    help="write a per-kernel table of a rocprofv3 --kernel-trace --stats run of the default "
                         "command (python3 bench.py) to OUT, then exit")
    args = ap.parse_args()
    if args.summarize:
        summarize(*args.summarize, args.summary_command, PROFILE_SUMMARY)
        return
    if args.trace_summary:
        trace_table(*args.trace_summary)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this implementation runs on one GPU; the multi-GPU sharding is a design note, "
                                   "so --gpus must be 1"}), flush=True)
        sys.exit(2)

    import torch
    from bit_weight_only_amd import lbq as L

    L.lib()
    log(f"[bench] packing dense stack ({args.layers} layers)")
    stack = Stack(L, torch, args.layers, 1)
    log(f"[bench] {stack.bytes_per_step / 1e9:.3f} GB packed weights per step")
    calibration_copy(torch)

    # timed region: graph replay of `steps` steps (barrier + synchronize on both sides)
    t = time_graph(torch, stack.step, args.steps, args.warmup)
    per_step = t / args.steps
    value = stack.bytes_per_step / per_step / 1e9
    log(f"[bench] timed: {per_step * 1e3:.3f} ms/step, {value:.1f} GB/s")

    # dominant kernel: HIP events around each of its launches on their stream
    per = event_pass(torch, stack)
    shape_stats = {}
    dom_b = dom_t = 0.0
    dom_n = 0
    for sh in stack.shapes:
        d = np.array(per[sh["name"]])
        avg = float(d.mean())
        shape_stats[sh["name"]] = {"K": sh["K"], "N": sh["N"], "bytes": sh["bytes"], "avg_us": round(avg * 1e6, 3),
                                   "GBps": round(sh["bytes"] / avg / 1e9, 1), "kernels": "gemv_mfma"}
        dom_b += sh["bytes"] * len(d)
        dom_t += float(d.sum())
        dom_n += len(d)
    achieved = dom_b / dom_t / 1e9
    log(f"[bench] per-launch: {json.dumps(shape_stats)}")

    extra = {"per_shape_M1": shape_stats,
             "dominant_kernel": {"name": DOMINANT, "launches": dom_n, "avg_us": round(dom_t / dom_n * 1e6, 3),
                                 "bytes_per_launch_avg": round(dom_b / dom_n)}}
    del stack
    torch.cuda.empty_cache()
    if not args.no_extra:
        steps = max(5, args.steps // 2)
        log("[bench] extra: single 4096x4096 linear, M=1")
        extra["single_linear_M1"] = extra_single(torch, L, steps)
        for M in (4, 16):
            log(f"[bench] extra: dense stack M={M}")
            extra[f"stack_M{M}"] = extra_stack(torch, L, M, steps)
        log("[bench] extra: FFN pair 5120/17408, M=1,8,64,256")
        extra["ffn_pair"] = extra_ffn(torch, L, steps)
        log("[bench] extra: product-VQ 4096->14336")
        extra["pvq"] = extra_pvq(torch, L, steps)
        log("[bench] extra: MoE block")
        extra["moe_block"] = extra_moe(torch, L, steps)
        m64 = extra["ffn_pair"]["M64"]
        extra["TFLOPs_at_M64"] = {"value": m64["TFLOPs"], "frac_of_mfma_peak": round(m64["TFLOPs"] / MFMA_F16_PEAK_TFLOPS, 4),
                                  "workload": "FFN pair 5120->17408 (2-bit) + 17408->5120 (3-bit), M=64"}

    cpu = None
    if not args.no_cpu:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline(L)

    traffic = traffic_from_summary()
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(per_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": f"dense decode stack, {args.layers} layers x (qkv 4096->6144, o 4096->4096, "
                               f"gate|up 4096->28672, down 14336->4096), 2-bit group-128 bit-planes, M=1",
                   "layers": args.layers, "M": 1, "bits": 2, "packed_bytes_per_step": stack_bytes(args.layers),
                   "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic)},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


def stack_bytes(layers):
    return sum(planes_meta_bytes(k, n, 2) for (_, k, n) in synth.DENSE_STACK_SHAPES) * layers


if __name__ == "__main__":
    main()
