#!/usr/bin/env python3
"""Benchmark of the low-bit weight-only quantized linear path on one MI355X.

Headline workload: a dense decode stack of LAYERS layers, each four 2-bit
group-128 linears (qkv 4096->6144, o 4096->4096, gate|up 4096->28672,
down 14336->4096) run at M = 1 token through lbq_linear_forward. A step is one
pass over every layer. Each layer has its own copy of the packed weights in
HBM (same bytes, distinct addresses), 1.96 GB per step at 32 layers, so the
256 MB last-level cache cannot serve repeats: every step streams the packed
weights from HBM.

value = packed-weight bytes per step * steps / wall time of the timed steps
(the steps are replayed from a HIP graph captured once, so Python launch
overhead is not in the timed region). The dominant kernel's duration is
measured live with HIP events around each of its launches on the stream the
library launches on, in a second pass over the same work; roofline.achieved =
algorithmic bytes per launch / that duration.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "packed-weight HBM GB/s (% of peak) for 2-bit dequant-GEMV at M=1; TFLOP/s at M=64"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


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
            s_dev = torch.from_numpy(s).to(dev)
            copies = []
            for _ in range(layers):
                pl = torch.from_numpy(planes).to(dev)
                mt = torch.from_numpy(meta).to(dev)
                copies.append(L.PackedLinear(k, n, 2, L.FMT_RTN_PLANES, pl, mt, s_dev))
            x = torch.from_numpy(synth.activations(M, k, workload=synth.W_STACK, item=idx)).to(dev)
            y = torch.empty((M, n), dtype=torch.float16, device=dev)
            ws = torch.empty(copies[0].workspace_bytes(M), dtype=torch.uint8, device=dev)
            self.shapes.append(dict(name=name, K=k, N=n, copies=copies, x=x, y=y, ws=ws,
                                    bytes=planes.size + meta.size))
        self.bytes_per_step = sum(sh["bytes"] for sh in self.shapes) * layers
        self.flops_per_step = sum(2.0 * M * sh["K"] * sh["N"] for sh in self.shapes) * layers
        lib = L.lib()
        self._fwd = lib.lbq_linear_forward
        self._calls = []
        for layer in range(layers):
            for sh in self.shapes:
                w = sh["copies"][layer]
                self._calls.append((sh, ctypes.byref(w.struct), ctypes.c_void_p(sh["x"].data_ptr()),
                                    ctypes.c_void_p(sh["y"].data_ptr()), ctypes.c_void_p(sh["ws"].data_ptr()),
                                    sh["ws"].numel()))

    def step(self, stream_ptr, events=None):
        M = self.M
        for (sh, wref, x, y, ws, nws) in self._calls:
            if events is not None:
                e0, e1 = events.pop()
                e0.record()
            st = self._fwd(wref, x, M, y, ws, nws, stream_ptr)
            if st != 0:
                raise RuntimeError(f"lbq_linear_forward failed: {st}")
            if events is not None:
                e1.record()
                events.append_done(sh, e0, e1)


class EventPool:
    def __init__(self, torch, n):
        self.free = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        self.done = []

    def pop(self):
        return self.free.pop()

    def append_done(self, sh, e0, e1):
        self.done.append((sh, e0, e1))


def time_graph(torch, fn, steps, warmup):
    """Capture fn() once into a HIP graph, replay warmup + steps times; return wall seconds of the timed steps."""
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
    return time.perf_counter() - t0, g


def kernel_event_pass(torch, stack, reps=2):
    """Per-launch HIP events around every lbq_linear_forward of the stack,
    enqueued behind a sleep so the host runs ahead and the GPU executes the
    launches back to back. Returns {shape: [durations_s]}."""
    n = len(stack._calls) * reps
    pool = EventPool(torch, n)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    torch.cuda.synchronize()
    torch.cuda._sleep(200_000_000)
    for _ in range(reps):
        stack.step(sp, pool)
    torch.cuda.synchronize()
    per = {}
    for sh, e0, e1 in pool.done:
        per.setdefault(sh["name"], []).append(e0.elapsed_time(e1) * 1e-3)
    return per


def cpu_baseline(L, budget_s=15.0):
    """The oracle on this host: y = x W_hat^T for a row sample of each stack matrix at M = 1."""
    from oracle import lbq_oracle as O

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    frac = 1.0 / 16.0
    total_bytes = 0
    total_t = 0.0
    rows_used = {}
    for idx, (name, k, n) in enumerate(synth.DENSE_STACK_SHAPES):
        rows = max(1, int(n * frac))
        w = synth.weights(n, k, workload=synth.W_STACK, item=idx)[:rows]
        s = synth.signs(k, workload=synth.W_STACK, item=idx)
        planes, meta = L.pack(w, 2, s)
        x = synth.activations(1, k, workload=synth.W_STACK, item=idx)
        t0 = time.perf_counter()
        O.linear_rtn(x, planes, meta, s, 2, rows, k)
        total_t += time.perf_counter() - t0
        total_bytes += planes.size + meta.size
        rows_used[name] = rows
        if total_t > budget_s:
            break
    return {"value": round(total_bytes / total_t / 1e9, 6), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle (numpy fp64: unpack, dequantize, inverse-rotate, matmul) on the first 1/16 of the rows "
                      f"of each dense-stack matrix at M=1, 2-bit: rows {rows_used}, {total_bytes} packed bytes in "
                      f"{total_t:.2f} s; elementwise numpy work is single-threaded, BLAS uses {threads} threads"}


def extra_m(torch, L, layers, M, steps):
    st = Stack(L, torch, layers, M)
    t, _ = time_graph(torch, st.step, steps, 2)
    per_step = t / steps
    out = {"M": M, "layers": layers, "ms_per_step": round(per_step * 1e3, 4),
           "packed_GBps": round(st.bytes_per_step / per_step / 1e9, 1),
           "TFLOPs": round(st.flops_per_step / per_step / 1e12, 3)}
    del st
    torch.cuda.empty_cache()
    return out


def extra_ffn_gemm(torch, L, steps):
    """The 5120/17408 FFN pair (gate|up 2-bit, down 3-bit) through the MFMA GEMM at M = 64 and 256."""
    dev = torch.device("cuda:0")
    cfg = synth.FFN_SWEEP
    mats = []
    for (k, n, bits, item) in [(cfg["K_gu"], cfg["N_gu"], cfg["bits_gu"], 1),
                               (cfg["N_gu"], cfg["K_gu"], cfg["bits_dn"], 2)]:
        w = synth.weights(n, k, workload=synth.W_FFN, item=item)
        s = synth.signs(k, workload=synth.W_FFN, item=item)
        planes, meta = L.pack(w, bits, s)
        del w
        copies = [L.PackedLinear(k, n, bits, 0, torch.from_numpy(planes).to(dev), torch.from_numpy(meta).to(dev),
                                 torch.from_numpy(s).to(dev)) for _ in range(6)]
        mats.append((k, n, copies, planes.size + meta.size))
    res = {}
    for M in (64, 256):
        bufs = []
        for (k, n, copies, nb) in mats:
            x = torch.from_numpy(synth.activations(M, k, workload=synth.W_FFN, item=M)).to(dev)
            y = torch.empty((M, n), dtype=torch.float16, device=dev)
            ws = torch.empty(copies[0].workspace_bytes(M), dtype=torch.uint8, device=dev)
            bufs.append((k, n, copies, x, y, ws))
        lib = L.lib()

        def fn(sp, bufs=bufs, M=M):
            for c in range(6):
                for (k, n, copies, x, y, ws) in bufs:
                    st = lib.lbq_linear_forward(ctypes.byref(copies[c].struct), ctypes.c_void_p(x.data_ptr()), M,
                                                ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                                                ws.numel(), sp)
                    assert st == 0
        t, _ = time_graph(torch, fn, steps, 2)
        flops = 6 * sum(2.0 * M * k * n for (k, n, *_r) in mats)
        nbytes = 6 * sum(m[3] for m in mats)
        per = t / steps
        res[f"M{M}"] = {"TFLOPs": round(flops / per / 1e12, 2),
                        "frac_of_mfma_peak": round(flops / per / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                        "packed_GBps": round(nbytes / per / 1e9, 1), "us_per_ffn": round(per / 6 * 1e6, 2)}
    del mats
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--no-extra", action="store_true", help="skip the M=4/16, M=64/256 and other secondary figures")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing on the host")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; the multi-GPU sharding is a design note, "
                                   "so --gpus must be 1"}), flush=True)
        sys.exit(2)

    import torch
    from bit_weight_only_amd import lbq as L

    L.lib()
    log(f"[bench] packing dense stack ({args.layers} layers)")
    stack = Stack(L, torch, args.layers, 1)
    log(f"[bench] {stack.bytes_per_step / 1e9:.3f} GB packed weights per step")

    # timed region: graph replay of `steps` steps
    t, graph = time_graph(torch, stack.step, args.steps, args.warmup)
    per_step = t / args.steps
    value = stack.bytes_per_step / per_step / 1e9
    log(f"[bench] timed: {per_step * 1e3:.3f} ms/step, {value:.1f} GB/s")
    del graph

    # dominant kernel timing: per-launch HIP events on the launch stream
    per = kernel_event_pass(torch, stack)
    shape_stats = {}
    tot_b = tot_t = 0.0
    for sh in stack.shapes:
        d = np.array(per[sh["name"]])
        avg = float(d.mean())
        shape_stats[sh["name"]] = {"K": sh["K"], "N": sh["N"], "bytes": sh["bytes"], "avg_us": round(avg * 1e6, 3),
                                   "GBps": round(sh["bytes"] / avg / 1e9, 1)}
        tot_b += sh["bytes"] * len(d)
        tot_t += float(d.sum())
    achieved = tot_b / tot_t / 1e9
    log(f"[bench] per-launch: {json.dumps(shape_stats)}")

    extra = {"per_shape_M1": shape_stats}
    if not args.no_extra:
        for M in (4, 16):
            log(f"[bench] extra: dense stack M={M}")
            extra[f"stack_M{M}"] = extra_m(torch, L, 8, M, max(5, args.steps // 2))
        log("[bench] extra: FFN pair through the MFMA GEMM")
        extra["ffn_gemm"] = extra_ffn_gemm(torch, L, max(5, args.steps // 2))

    cpu = None
    if not args.no_cpu:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline(L)

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
                   "layers": args.layers, "M": 1, "bits": 2, "packed_bytes_per_step": stack.bytes_per_step,
                   "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
