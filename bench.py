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
product-VQ 4096->14336 linear at M = 1, 16, 64 (2 and 6 bits per weight),
the 256-expert MoE block at
M = 32 (and its prefill at 256 and 2048 tokens), the router and the rotation
alone, and the screened readout of an 8-bit 2048 -> 131072 vocabulary weight
against its plain 8-bit readout.

Every extra cycles over device copies of its weights totalling at least
1 GiB (four times the 256 MB last-level cache), so repeats stream from HBM, and
reports the median, p10 and p90 of per-step times (HIP events between graph
replays). extra.stream_floor times a plain streaming read of each GEMV
launch's byte count (lbq_stream_read, the kernel's own begin / end events, a
sweep of launch shapes) and reports each GEMV shape against it and against the
HBM peak. The GPU clocks are read before and after the timed region.

cpu_baseline: the oracle on this host's cores, a bounded sample (two of the
stack's matrices at M = 1), the one-time preparation (unpack, dequantize,
inverse-rotate) timed apart from the per-call fp64 product, the product also
with one BLAS thread. --cpu-configs runs the per-configuration version.

Prints one JSON line. With --summarize it instead turns rocprofv3 outputs of
this script into the text summary kept under profiles/.
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import io
import json
import os
import subprocess
import sys
import time
from contextlib import redirect_stdout

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
POOL_BYTES = 1 << 30           # every measurement cycles over at least this many bytes of weights


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# sources each profiled kernel is built from (a counter summary is stale once they change)
KERNEL_SOURCES = {
    "gemv_mfma_kernel": DOMINANT_SOURCES,
    "gemm_rtn_kernel": ["bit_weight_only_amd/csrc/gemm_rtn.hip", "bit_weight_only_amd/csrc/gemm_common.h",
                        "bit_weight_only_amd/csrc/device.h"],
    "gemm_pvq_kernel": ["bit_weight_only_amd/csrc/gemm.hip", "bit_weight_only_amd/csrc/gemm_common.h",
                        "bit_weight_only_amd/csrc/device.h"],
    "gemm_mx_kernel": ["bit_weight_only_amd/csrc/gemm_mx.hip", "bit_weight_only_amd/csrc/mx_core.h",
                       "bit_weight_only_amd/csrc/gemm_common.h", "bit_weight_only_amd/csrc/device.h"],
    "moe_mx_kernel": ["bit_weight_only_amd/csrc/moe_mx.hip", "bit_weight_only_amd/csrc/mx_core.h",
                      "bit_weight_only_amd/csrc/gemm_common.h", "bit_weight_only_amd/csrc/device.h"],
    "gemm_rtn_grouped_kernel": ["bit_weight_only_amd/csrc/gemm_rtn.hip", "bit_weight_only_amd/csrc/gemm_common.h",
                                "bit_weight_only_amd/csrc/device.h"],
    "select_kernel": ["bit_weight_only_amd/csrc/readout.hip", "bit_weight_only_amd/csrc/device.h"],
    "gemv_pvq_mx_kernel": ["bit_weight_only_amd/csrc/pvq_mx.hip", "bit_weight_only_amd/csrc/mx_core.h",
                           "bit_weight_only_amd/csrc/gemm_common.h", "bit_weight_only_amd/csrc/device.h"],
}


def source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for p in (sources or DOMINANT_SOURCES):
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

def stats(vals, scale=1.0, nd=3):
    """median / p10 / p90 of vals * scale."""
    a = np.asarray(vals, dtype=np.float64) * scale
    return {"median": round(float(np.median(a)), nd), "p10": round(float(np.percentile(a, 10)), nd),
            "p90": round(float(np.percentile(a, 90)), nd)}


def gpu_clocks():
    """Current shader / memory clock levels of the first GPU as the amdgpu
    kernel module reports them (sysfs dpm tables; the line marked '*' is
    current)."""
    out = {}
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))[:1]:
        d = os.path.dirname(f)
        for name in ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk"):
            try:
                with open(os.path.join(d, name)) as fh:
                    cur = [l.split(":", 1)[1].strip().rstrip("*").strip() for l in fh if l.strip().endswith("*")]
                out[name[7:]] = cur[0] if cur else None
            except OSError:
                pass
    if not out:
        try:
            r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
            js = json.loads(r.stdout)
            card = js[sorted(js)[0]]
            out = {k.split(" ")[0]: v for k, v in card.items() if "clock" in k}
        except Exception as e:  # pragma: no cover
            out = {"error": str(e)[:80]}
    return out


def time_graph(torch, fn, steps, warmup, per_step=None):
    """Capture fn(stream_ptr) once into a HIP graph, replay warmup + steps times;
    return wall seconds of the timed replays. With per_step a list, HIP events
    recorded between the replays append each step's seconds to it."""
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
    evs = None
    if per_step is not None:
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if evs:
            evs[i].record()
        g.replay()
    if evs:
        evs[steps].record()
    torch.cuda.synchronize()
    t = time.perf_counter() - t0
    if evs:
        per_step += [evs[i].elapsed_time(evs[i + 1]) * 1e-3 for i in range(steps)]
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

    def __init__(self, L, torch, layers: int, M: int, path: int = 0):
        self.L, self.torch, self.layers, self.M, self.path = L, torch, layers, M, path
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
        if self.path:   # an explicit kernel path (lbq_linear_forward_path)
            fwd = self.lib.lbq_linear_forward_path
            for sh, (w, x, M, y, ws, n) in self.order:
                check(fwd(w, x, M, y, ws, n, self.path, sp), "lbq_linear_forward_path")
            return
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


def trace_avgs_from_summary():
    """rocprofv3's mean duration of the dominant kernel in the committed
    summary: over the eager event-pass launches (the ones timed live here) and
    over the graph-replayed launches of the timed steps; None when the summary
    is absent or was taken on other kernel sources."""
    try:
        with open(PROFILE_SUMMARY) as f:
            text = f.read()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines() if line.startswith("@") and ":" in line)
    if fields.get("@source_hash", "").strip() != source_hash():
        return None
    out = {}
    for key in ("event_pass", "graph_replay"):
        try:
            out[key] = float(fields[f"@trace_avg_us_{key}"])
        except (KeyError, ValueError):
            out[key] = None
    return out


# ---------------------------------------------------------------- CPU baseline

def host_info():
    """CPU model, usable cores and the BLAS NumPy is built with."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    buf = io.StringIO()
    with redirect_stdout(buf):
        np.show_config()
    cfg = buf.getvalue()
    blas = [l.strip() for l in cfg.splitlines() if "name:" in l or "openblas configuration" in l.lower()]
    return {"cpu_model": model, "cores_usable": len(os.sched_getaffinity(0)), "numpy_blas": blas[:4]}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def oracle_times(O, x, planes, meta, s, bits, n, k, runs=5):
    """One-time preparation (unpack, dequantize, inverse-rotate) and the
    per-call fp64 product y = x W_hat^T of the oracle: (prep s, [product s], w_hat)."""
    t0 = time.perf_counter()
    w_hat = O.dequant_weight_rtn(planes, meta, s, bits, n, k)
    prep = time.perf_counter() - t0
    O.linear(x, w_hat)   # warm-up
    prod = []
    for _ in range(runs):
        t0 = time.perf_counter()
        O.linear(x, w_hat)
        prod.append(time.perf_counter() - t0)
    return prep, prod, w_hat


def cpu_baseline(L):
    """The oracle on this host for the headline workload, a bounded sample:
    the o (4096x4096) and down (14336x4096) matrices of the dense stack, 2-bit,
    M = 1. value = packed bytes / (preparation + product), the oracle's cost
    per call as it stands (linear_rtn does both); the parts are reported apart,
    and the product again with one BLAS thread."""
    from oracle import lbq_oracle as O   # test infrastructure: the oracle is the reported baseline

    threads = blas_threads()
    prep_t = prod_med = prod1_med = 0.0
    nbytes, names = 0, []
    for idx, (name, k, n) in enumerate(synth.DENSE_STACK_SHAPES):
        if name not in ("o", "down"):
            continue
        w = synth.weights(n, k, workload=synth.W_STACK, item=idx)
        s = synth.signs(k, workload=synth.W_STACK, item=idx)
        planes, meta = L.pack(w, 2, s)
        del w
        x = synth.activations(1, k, workload=synth.W_STACK, item=idx)
        prep, prod, w_hat = oracle_times(O, x, planes, meta, s, 2, n, k)
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                prod1 = [0.0] * 3
                for i in range(3):
                    t0 = time.perf_counter()
                    O.linear(x, w_hat)
                    prod1[i] = time.perf_counter() - t0
        except Exception:  # pragma: no cover
            prod1 = [float("nan")]
        del w_hat
        prep_t += prep
        prod_med += float(np.median(prod))
        prod1_med += float(np.median(prod1))
        nbytes += planes.nbytes + meta.nbytes
        names.append(name)
    info = host_info()
    return {"value": round(nbytes / (prep_t + prod_med) / 1e9, 6), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"the oracle (numpy fp64) on the dense stack's {' and '.join(names)} matrices, 2-bit, M=1: "
                      f"{nbytes} packed bytes; one-time preparation (unpack, dequantize, inverse-rotate) "
                      f"{prep_t:.2f} s, then the fp64 product y = x W_hat^T {prod_med * 1e3:.1f} ms per call "
                      f"(median of 5 after a warm-up) on {threads} BLAS threads, {prod1_med * 1e3:.1f} ms on one; "
                      f"elementwise numpy work single-threaded",
            "prep_s": round(prep_t, 3), "product_ms": round(prod_med * 1e3, 3),
            "product_ms_1thread": round(prod1_med * 1e3, 3),
            "product_only_GBps": round(nbytes / prod_med / 1e9, 4), **info}


def cpu_configs(L, rows=1024, runs=5):
    """Per-configuration oracle timings on this host (the preparation and the
    per-call product, each the median of `runs` after a warm-up, on all BLAS
    threads and on one), on `rows` output rows of each matrix scaled to the
    full row count (rows are independent, the costs linear in them); the MoE
    block on 8 of its routed experts scaled to the touched ones. Prints one
    JSON object."""
    from oracle import lbq_oracle as O   # test infrastructure: the oracle is the reported baseline
    from threadpoolctl import threadpool_limits

    def one(x, w, s, bits, n_full, fmt="rtn", cb=None):
        n, k = w.shape
        res = {}
        for label, lim in (("all", None), ("1thread", 1)):
            with threadpool_limits(limits=lim):
                preps, prods = [], []
                for r in range(runs + 1):
                    t0 = time.perf_counter()
                    if fmt == "rtn":
                        planes, meta = L.pack(w, bits, s)
                        w_hat = O.dequant_weight_rtn(planes, meta, s, bits, n, k)
                    else:
                        idx, sc = L.pack(w, 2, s, L.FMT_PVQ_4x8, cb)
                        w_hat = O.dequant_weight_pvq(idx.reshape(n, -1), sc.view(np.uint16), cb, s)
                    t1 = time.perf_counter()
                    O.linear(x, w_hat)
                    t2 = time.perf_counter()
                    if r:
                        preps.append(t1 - t0)
                        prods.append(t2 - t1)
                # the host packer's own time is not the oracle's: time it alone and take it out
                t0 = time.perf_counter()
                if fmt == "rtn":
                    L.pack(w, bits, s)
                else:
                    L.pack(w, 2, s, L.FMT_PVQ_4x8, cb)
                tpack = time.perf_counter() - t0
                scale = n_full / n
                res[label] = {"prep_s": round(max(0.0, float(np.median(preps)) - tpack) * scale, 4),
                              "product_s": round(float(np.median(prods)) * scale, 5)}
        return res

    out = {"host": host_info(), "blas_threads": blas_threads(), "rows_sampled": rows, "runs": runs, "configs": {}}
    C = out["configs"]
    cfg = synth.SINGLE_LINEAR
    w = synth.weights(cfg["N"], cfg["K"], workload=synth.W_SINGLE)[:rows]
    s = synth.signs(cfg["K"], workload=synth.W_SINGLE)
    C["single_linear_M1"] = {"bytes": planes_meta_bytes(cfg["K"], cfg["N"], 2),
                             **one(synth.activations(1, cfg["K"], workload=synth.W_SINGLE), w, s, 2, cfg["N"])}
    for idx, (name, k, n) in enumerate(synth.DENSE_STACK_SHAPES):
        w = synth.weights(n, k, workload=synth.W_STACK, item=idx)[:rows]
        s = synth.signs(k, workload=synth.W_STACK, item=idx)
        for M in synth.DENSE_STACK_M:
            C[f"stack_{name}_M{M}"] = {"bytes": planes_meta_bytes(k, n, 2),
                                       **one(synth.activations(M, k, workload=synth.W_STACK, item=M), w, s, 2, n)}
    f = synth.FFN_SWEEP
    for (k, n, bits, item) in [(f["K_gu"], f["N_gu"], f["bits_gu"], 1), (f["N_gu"], f["K_gu"], f["bits_dn"], 2)]:
        w = synth.weights(n, k, workload=synth.W_FFN, item=item)[:rows]
        s = synth.signs(k, workload=synth.W_FFN, item=item)
        for M in f["M"]:
            C[f"ffn_{k}x{n}_b{bits}_M{M}"] = {"bytes": planes_meta_bytes(k, n, bits),
                                             **one(synth.activations(M, k, workload=synth.W_FFN, item=M), w, s, bits, n)}
    p = synth.PVQ_LINEAR
    cb = synth.codebook(workload=synth.W_PVQ)
    w = synth.weights(p["N"], p["K"], workload=synth.W_PVQ)[:rows]
    s = synth.signs(p["K"], workload=synth.W_PVQ)
    for M in p["M"]:
        C[f"pvq_M{M}"] = {"bytes": p["N"] * p["K"] // 4 + 2 * p["N"] + 1024,
                          **one(synth.activations(M, p["K"], workload=synth.W_PVQ, item=M), w, s, 2, p["N"], "pvq", cb)}
    # MoE block: the oracle's expert-by-expert FFN on 8 routed experts, scaled to all routed ones
    m = synth.MOE_BLOCK
    E, H, F, k, M = m["E"], m["hidden"], m["ffn"], m["top_k"], m["M"]
    bits = synth.expert_bits(E, workload=synth.W_MOE)
    sh = synth.signs(H, workload=synth.W_MOE, item=1)
    sf = synth.signs(F, workload=synth.W_MOE, item=2)
    x = synth.activations(M, H, workload=synth.W_MOE)
    lg = synth.logits(M, E, workload=synth.W_MOE)
    ids, _ = O.route(lg, k)
    touched = np.unique(ids)
    sample = touched[:8]
    res = {}
    for label, lim in (("all", None), ("1thread", 1)):
        with threadpool_limits(limits=lim):
            prep = prod = 0.0
            for e in sample:
                b = int(bits[e])
                t0 = time.perf_counter()
                pg, mg = L.pack(synth.weights(2 * F, H, workload=synth.W_MOE, item=1000 + int(e)), b, sh)
                pd, md = L.pack(synth.weights(H, F, workload=synth.W_MOE, item=5000 + int(e)), b, sf)
                t1 = time.perf_counter()
                wg = O.dequant_weight_rtn(pg, mg, sh, b, 2 * F, H)
                wd = O.dequant_weight_rtn(pd, md, sf, b, H, F)
                t2 = time.perf_counter()
                rows_e, _ = np.nonzero(ids == e)
                O.expert_ffn(x[rows_e], wg, wd)
                t3 = time.perf_counter()
                prep += t2 - t1
                prod += t3 - t2
            scale = len(touched) / len(sample)
            res[label] = {"prep_s": round(prep * scale, 4), "product_s": round(prod * scale, 5)}
    C["moe_block_M32"] = {"experts_touched": int(len(touched)), "experts_sampled": int(len(sample)), **res}
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------- extra measurements

def copies_for(nbytes):
    """Device copies of an nbytes weight that together reach POOL_BYTES."""
    return max(1, -(-POOL_BYTES // int(nbytes)))


def measure_linears(torch, L, lin, M, steps, x=None, workload=0):
    dev = torch.device("cuda:0")
    if x is None:
        x = torch.from_numpy(synth.activations(M, lin.K, workload=workload, item=M)).to(dev)
    calls = lin.calls(M, x)
    per_step = []
    t = time_graph(torch, run_calls(L.lib(), calls), steps, 2, per_step)
    per = t / steps / len(calls)
    out = {"M": M, "us_per_call": round(per * 1e6, 3), "copies": len(calls),
           "us_per_call_stats": stats(per_step, 1e6 / len(calls))}
    out.update(roofline(lin.bytes, 2.0 * M * lin.K * lin.N, per))
    return out


def extra_single(torch, L, steps):
    cfg = synth.SINGLE_LINEAR
    w = synth.weights(cfg["N"], cfg["K"], workload=synth.W_SINGLE)
    s = synth.signs(cfg["K"], workload=synth.W_SINGLE)
    planes, meta = L.pack(w, 2, s)
    lin = Linears(L, torch, cfg["K"], cfg["N"], 2, 0, planes, meta, s, None, copies_for(planes.nbytes + meta.nbytes))
    r = measure_linears(torch, L, lin, 1, steps, workload=synth.W_SINGLE)
    del lin
    return r


def extra_stack(torch, L, M, steps, layers=None, path=0):
    layers = layers or copies_for(stack_bytes(1))
    st = Stack(L, torch, layers, M, path)
    per_step = []
    t = time_graph(torch, st.step, steps, 2, per_step)
    per = t / steps
    out = {"M": M, "layers": layers, "us_per_layer": round(per / layers * 1e6, 2),
           "us_per_layer_stats": stats(per_step, 1e6 / layers, 2)}
    out.update(roofline(st.bytes_per_step, st.flops_per_step, per))
    del st
    torch.cuda.empty_cache()
    return out


def extra_ffn(torch, L, steps, Ms=None):
    cfg = synth.FFN_SWEEP
    mats = []
    pair_bytes = planes_meta_bytes(cfg["K_gu"], cfg["N_gu"], cfg["bits_gu"]) + \
        planes_meta_bytes(cfg["N_gu"], cfg["K_gu"], cfg["bits_dn"])
    copies = copies_for(pair_bytes)
    for (k, n, bits, item) in [(cfg["K_gu"], cfg["N_gu"], cfg["bits_gu"], 1), (cfg["N_gu"], cfg["K_gu"], cfg["bits_dn"], 2)]:
        w = synth.weights(n, k, workload=synth.W_FFN, item=item)
        s = synth.signs(k, workload=synth.W_FFN, item=item)
        planes, meta = L.pack(w, bits, s)
        del w
        mats.append(Linears(L, torch, k, n, bits, 0, planes, meta, s, None, copies))
    dev = torch.device("cuda:0")
    res = {}
    for M in (Ms or cfg["M"]):
        calls = []
        for lin in mats:
            x = torch.from_numpy(synth.activations(M, lin.K, workload=synth.W_FFN, item=M)).to(dev)
            calls += lin.calls(M, x)
            lin._keep_m = lin._keep
        per_step = []
        t = time_graph(torch, run_calls(L.lib(), calls), steps, 2, per_step)
        per = t / steps / copies           # one gate|up + one down
        nbytes = sum(m.bytes for m in mats)
        flops = sum(2.0 * M * m.K * m.N for m in mats)
        r = {"M": M, "us_per_ffn": round(per * 1e6, 2), "copies": copies,
             "us_per_ffn_stats": stats(per_step, 1e6 / copies, 2)}
        r.update(roofline(nbytes, flops, per))
        res[f"M{M}"] = r
    del mats
    torch.cuda.empty_cache()
    return res


def extra_pvq(torch, L, steps, Ms=None, bits=2):
    """The product-VQ linear 4096 -> 14336; bits 4 and 6 are two and three
    residual stages (idx and row scales per stage)."""
    cfg = synth.PVQ_LINEAR
    cb = synth.codebook(workload=synth.W_PVQ)
    w = synth.weights(cfg["N"], cfg["K"], workload=synth.W_PVQ)
    s = synth.signs(cfg["K"], workload=synth.W_PVQ)
    idx, sc = L.pack(w, bits, s, L.FMT_PVQ_4x8, cb)
    del w
    lin = Linears(L, torch, cfg["K"], cfg["N"], bits, L.FMT_PVQ_4x8, idx, sc, s, cb,
                  copies_for(idx.nbytes + sc.nbytes + cb.nbytes))
    res = {f"M{M}": measure_linears(torch, L, lin, M, steps, workload=synth.W_PVQ) for M in (Ms or cfg["M"])}
    del lin
    torch.cuda.empty_cache()
    return res


def extra_readout(torch, L, steps, Ms=None):
    """Screened readout over the nibble-split planes of an 8-bit vocabulary
    weight against the plain 8-bit readout (lbq_linear_forward at 8 bits) of
    the same weight; each call on its own device copy (pool of 1 GiB or more).
    Bytes: the screen reads the high-nibble planes and their scale/zero words
    of every row (half the 8-bit planes), plus both nibble planes of the
    survivors; the plain readout reads all 8-bit planes and meta."""
    cfg = synth.READOUT
    K, N, cand = cfg["K"], cfg["N"], cfg["cand"]
    dev = torch.device("cuda:0")
    w = synth.weights(N, K, workload=synth.W_READOUT)
    s = synth.signs(K, workload=synth.W_READOUT)
    planes, meta = L.pack(w, 8, s)
    del w
    hi, lo, hm = L.split_nibbles(planes, meta, K, N)
    s_dev = torch.from_numpy(s).to(dev)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1)).to(dev)

    n_copies = copies_for(hi.nbytes + lo.nbytes + hm.nbytes + meta.nbytes)
    ros = [L.PackedReadout(K, N, up(hi), up(lo), up(hm), up(meta), s_dev) for _ in range(n_copies)]
    screen_bytes = hi.nbytes + hm.nbytes
    lin8 = Linears(L, torch, K, N, 8, L.FMT_RTN_PLANES, planes, meta, s, None,
                   copies_for(planes.nbytes + meta.nbytes))
    del hi, lo, hm, planes
    lib = L.lib()
    res = {}
    for M in (Ms or cfg["M"]):
        x = torch.from_numpy(synth.activations(M, K, workload=synth.W_READOUT, item=M)).to(dev)
        coarse = torch.empty((M, N), dtype=torch.float16, device=dev)
        ids = torch.empty((M, cand), dtype=torch.int32, device=dev)
        lg = torch.empty((M, cand), dtype=torch.float32, device=dev)
        ws = torch.empty(ros[0].workspace_bytes(M, cand), dtype=torch.uint8, device=dev)

        def fn(sp):
            for r in ros:
                check(lib.lbq_readout_screened(ctypes.byref(r.struct), ctypes.c_void_p(x.data_ptr()), M, cand,
                                               ctypes.c_void_p(coarse.data_ptr()), ctypes.c_void_p(ids.data_ptr()),
                                               ctypes.c_void_p(lg.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                                               ws.numel(), sp), "lbq_readout_screened")
        per_step = []
        t = time_graph(torch, fn, steps, 2, per_step) / steps / len(ros)
        surv = M * cand * (K // 128) * 128   # both nibble planes of every survivor
        full = measure_linears(torch, L, lin8, M, steps, x=x)
        res[f"M{M}"] = {"M": M, "cand": cand, "us_per_call": round(t * 1e6, 3),
                        "us_per_call_stats": stats(per_step, 1e6 / len(ros)),
                        "screen_bytes": screen_bytes, "GBps": round((screen_bytes + surv) / t / 1e9, 1),
                        "frac": round((screen_bytes + surv) / t / 1e9 / HBM_PEAK_GBS, 4),
                        "full_8bit_us": full["us_per_call"], "speedup_vs_full_8bit": round(full["us_per_call"] / (t * 1e6), 3)}
        del coarse, ids, lg, ws
    del ros, lin8
    torch.cuda.empty_cache()
    return res


def extra_moe(torch, L, steps, extras=True, M=None):
    cfg = synth.MOE_BLOCK
    E, H, F, k = cfg["E"], cfg["hidden"], cfg["ffn"], cfg["top_k"]
    M = M or cfg["M"]
    dev = torch.device("cuda:0")
    bits = synth.expert_bits(E, workload=synth.W_MOE)
    sh = synth.signs(H, workload=synth.W_MOE, item=1)
    sf = synth.signs(F, workload=synth.W_MOE, item=2)
    packed = L.pack_moe_host(lambda e: synth.weights(2 * F, H, workload=synth.W_MOE, item=1000 + e),
                             lambda e: synth.weights(H, F, workload=synth.W_MOE, item=5000 + e), bits, sh, sf)
    # device copies of the whole block (every expert) reaching the pool size
    n_copies = copies_for(packed["planes"].nbytes + packed["meta"].nbytes)
    moes = [L.moe_from_host(packed, bits, sh, sf, H, F, k) for _ in range(n_copies)]
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
        ws = torch.empty(moes[0].workspace_bytes(M), dtype=torch.uint8, device=dev)
        batches.append((x, lg, y, ws))
    lib = L.lib()
    order = [(moes[c], batches[b]) for c in range(n_copies) for b in range(len(batches))]

    def fn(sp):
        for moe, (x, lg, y, ws) in order:
            check(lib.lbq_moe_forward(ctypes.byref(moe.struct), ctypes.c_void_p(x.data_ptr()),
                                      ctypes.c_void_p(lg.data_ptr()), M, ctypes.c_void_p(y.data_ptr()),
                                      ctypes.c_void_p(ws.data_ptr()), ws.numel(), sp), "lbq_moe_forward")
    per_step = []
    t = time_graph(torch, fn, steps, 2, per_step)
    per = t / steps / len(order)
    nbytes = float(np.mean(touched))
    flops = 2.0 * M * k * (2 * F * H + H * F)
    out = {"M": M, "us_per_block": round(per * 1e6, 2), "touched_bytes_avg": int(nbytes), "block_copies": n_copies,
           "us_per_block_stats": stats(per_step, 1e6 / len(order), 2),
           "expert_path": "grouped MFMA GEMM" if M * k >= 4 * E else "matrix-core expert GEMV"}
    out.update(roofline(nbytes, flops, per))
    if not extras:
        del moes, packed, batches
        torch.cuda.empty_cache()
        return out

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
    del moes, packed, batches
    torch.cuda.empty_cache()
    return out


# launch shapes the streaming-read floor is swept over (workgroups, threads)
FLOOR_SHAPES = [(256, 1024), (512, 512), (512, 1024), (1024, 256), (1024, 512), (2048, 256)]


def stream_floor(torch, L, sizes, reps=40):
    """Per byte count: the fastest median duration of a plain streaming read
    over FLOOR_SHAPES (each launch on its own window of a 1.5 GiB buffer, cold
    in the last-level cache; events on the kernel's own begin / end), and the
    empty launch."""
    lib = L.lib()
    dev = torch.device("cuda:0")
    pool_n = 3 << 29
    pool = torch.empty(pool_n, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def run(nbytes, grid, block):
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in pairs:
            e0.record(stream)
            e1.record(stream)
        torch.cuda.synchronize()
        windows = max(1, pool_n // max(nbytes, 1))
        for r, (e0, e1) in enumerate(pairs):
            off = (r % windows) * nbytes
            check(lib.lbq_stream_read(ctypes.c_void_p(pool.data_ptr() + off), nbytes, grid, block,
                                      ctypes.c_void_p(sink.data_ptr()), sp, ctypes.c_void_p(e0.cuda_event),
                                      ctypes.c_void_p(e1.cuda_event)), "lbq_stream_read")
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) * 1e-3 for e0, e1 in pairs[2:]]

    out = {}
    for name, nbytes in sizes.items():
        nb = (int(nbytes) + 15) // 16 * 16
        best = None
        for grid, block in FLOOR_SHAPES:
            d = run(nb, grid, block)
            med = float(np.median(d))
            if best is None or med < best[0]:
                best = (med, grid, block, d)
        out[name] = {"bytes": nb, "floor_us": stats(best[3], 1e6), "GBps_at_floor": round(nb / best[0] / 1e9, 1),
                     "shape": [best[1], best[2]]}
    out["empty_launch_us"] = {f"{g}x{b}": stats(run(0, g, b), 1e6)["median"]
                              for g, b in [(1, 64), (256, 256), (256, 1024), (2048, 256)]}
    del pool
    torch.cuda.empty_cache()
    return out


def stack_floor(torch, L, layers, shapes, steps):
    """The headline step with every GEMV launch replaced by a plain streaming
    read of the same bytes (at that size's fastest launch shape from
    stream_floor), layer copies at distinct addresses, replayed from a HIP graph
    like the headline: the floor of any one-launch-per-linear design. Also the
    same graph of empty launches. Returns per-layer microseconds."""
    lib = L.lib()
    dev = torch.device("cuda:0")
    sizes = [((int(planes_meta_bytes(k, n, 2)) + 255) // 256 * 256, tuple(shapes[name])) for (name, k, n) in
             synth.DENSE_STACK_SHAPES]
    per_layer = sum(b for b, _ in sizes)
    pool = torch.empty(per_layer * layers, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    calls = []
    off = 0
    for _ in range(layers):
        for nb, (g, b) in sizes:
            calls.append((pool.data_ptr() + off, nb, g, b))
            off += nb

    def reads(sp):
        for (p, nb, g, b) in calls:
            check(lib.lbq_stream_read(ctypes.c_void_p(p), nb, g, b, ctypes.c_void_p(sink.data_ptr()), sp, None, None),
                  "lbq_stream_read")

    def empties(sp):
        for (p, nb, g, b) in calls:
            check(lib.lbq_stream_read(ctypes.c_void_p(p), 0, 256, 1024, ctypes.c_void_p(sink.data_ptr()), sp, None,
                                      None), "lbq_stream_read")
    st_r, st_e = [], []
    time_graph(torch, reads, steps, 2, st_r)
    time_graph(torch, empties, steps, 2, st_e)
    del pool
    torch.cuda.empty_cache()
    return {"layers": layers, "read_us_per_layer": stats(st_r, 1e6 / layers, 2),
            "GBps_at_floor": round(per_layer * layers / float(np.median(st_r)) / 1e9, 1),
            "frac_of_hbm_peak": round(per_layer * layers / float(np.median(st_r)) / 1e9 / HBM_PEAK_GBS, 4),
            "empty_us_per_layer": stats(st_e, 1e6 / layers, 2)}


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
    dom_graph = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace
                 if DOMINANT in r["Kernel_Name"] and int(r["Start_Timestamp"]) < t_spin]
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
        f"@trace_avg_us_event_pass: {float(np.mean(dom)) if dom else float('nan'):.3f}",
        f"@trace_avg_us_graph_replay: {float(np.mean(dom_graph)) if dom_graph else float('nan'):.3f}",
    ]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# counters per pass of the --pmc runs (each pass within one run's hardware limits)
PMC_PASSES = [
    "SQ_WAVES SQ_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE "
    "GRBM_GUI_ACTIVE",
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU_MFMA_MOPS_F8 SQ_INSTS_VALU_MFMA_MOPS_F6F4 "
    "SQ_INSTS_VMEM_RD SQ_INST_CYCLES_VMEM_RD GRBM_GUI_ACTIVE",
    "FETCH_SIZE",
    "WRITE_SIZE",
]
N_CU, N_SIMD, N_XCC = 256, 4, 8


def pmc_summary(case, kernel, out_path, dirs):
    """Per-dispatch counter means of one kernel (name containing `kernel`)
    over rocprofv3 --pmc runs of 'bench.py --case CASE', one directory per pass,
    written as a text summary with the derived figures: matrix-core busy
    fraction, VALU instructions per MFMA instruction, LDS bank conflicts per
    LDS instruction, and HBM bytes against the algorithmic bytes."""
    import csv

    vals = {}
    names = set()
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                names.add(r["Kernel_Name"])
                if kernel not in r["Kernel_Name"]:
                    continue
                key = (f, r["Dispatch_Id"], r["Counter_Name"])
                vals.setdefault(key, []).append(float(r["Counter_Value"]))
    per = {}
    durs = {}
    for (_, disp, cname), v in vals.items():
        # one row per dispatch and counter, summed over the counter's instances
        # (shader engines, XCDs): GRBM_GUI_ACTIVE is then the sum of the 8
        # XCDs' busy cycles
        per.setdefault(cname, []).append(sum(v))
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if kernel in r["Kernel_Name"]:
                    durs[(f, r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
    mean = {c: float(np.mean(v)) for c, v in per.items()}
    n = {c: len(v) for c, v in per.items()}
    lines = [f"rocprofv3 counters of {kernel} in 'python3 bench.py --case {case}' (per-dispatch means)", "",
             "commands (from the repository root, cd /tmp && export TMPDIR=/tmp first), one run per pass:"]
    for p in PMC_PASSES:
        lines.append(f"  rocprofv3 --pmc {p} -d <dir> -o p --output-format csv -- python3 bench.py --case {case} --steps 2")
    lines.append(f"  python3 bench.py --pmc-summary {case} {kernel} <this file> <dir>...")
    lines.append("")
    for c in sorted(mean):
        lines.append(f"  {c:28s} {mean[c]:18.1f}  (n={n[c]})")
    lines.append("")
    if durs:
        lines.append(f"dispatch duration under counter collection: {float(np.mean(list(durs.values()))):.2f} us "
                     f"(mean over {len(durs)} dispatches of all passes)")
    gui = mean.get("GRBM_GUI_ACTIVE")
    if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
        lines.append(f"matrix-core busy: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {N_XCC} XCDs x {N_CU} CUs x "
                     f"{N_SIMD} SIMDs) = {mean['SQ_VALU_MFMA_BUSY_CYCLES'] / (gui / N_XCC * N_CU * N_SIMD):.4f}")
    if mean.get("SQ_INSTS_MFMA"):
        lines.append(f"VALU instructions per MFMA instruction: {mean.get('SQ_INSTS_VALU', 0) / mean['SQ_INSTS_MFMA']:.2f}")
    if mean.get("SQ_INSTS_LDS"):
        lines.append(f"LDS bank conflict cycles per LDS instruction: "
                     f"{mean.get('SQ_LDS_BANK_CONFLICT', 0) / mean['SQ_INSTS_LDS']:.3f}")
    if mean.get("SQ_LDS_IDX_ACTIVE"):
        c = mean.get("SQ_LDS_BANK_CONFLICT", 0.0)
        lines.append(f"LDS bank conflicts per conflict-free LDS cycle: {c / max(1.0, mean['SQ_LDS_IDX_ACTIVE'] - c):.3f}")
    mops = sum(mean.get(f"SQ_INSTS_VALU_MFMA_MOPS_{t}", 0.0) for t in ("F16", "F8", "F6F4"))
    if mops:
        lines.append(f"MFMA work: {mops * 512:.4g} flops per dispatch (MOPS x 512, F16 + F8 + F6F4)")
    if "FETCH_SIZE" in mean:
        lines.append(f"FETCH_SIZE {mean['FETCH_SIZE']:.1f} KiB, WRITE_SIZE {mean.get('WRITE_SIZE', float('nan')):.1f} KiB "
                     f"per dispatch (scale by the copy-kernel factors of the headline summary: fetch x2.0, write x1.0)")
        lines.append(f"HBM bytes per dispatch (scaled): "
                     f"{mean['FETCH_SIZE'] * 1024 * 2.0 + mean.get('WRITE_SIZE', 0.0) * 1024:.0f}")
    lines.append("")
    srcs = next((v for k, v in KERNEL_SOURCES.items() if k in kernel), None)
    if srcs:
        lines.append(f"@source_hash: {source_hash(srcs)}  ({', '.join(os.path.basename(p) for p in srcs)})")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def trace_table(trace_dir, out_path, case=None):
    """Per-kernel durations from a rocprofv3 kernel trace of the default bench
    command (every part of the hot path), or of 'bench.py --case CASE'."""
    import csv

    stats = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True):
        stats += list(csv.DictReader(open(f)))
    if case:
        lines = [f"rocprofv3 kernel-trace statistics of 'python3 bench.py --case {case} --steps 10' (the case's",
                 "graph-replayed launches and its untimed warm-up and capture).",
                 "",
                 "command (run from the repository root, cd /tmp && export TMPDIR=/tmp first):",
                 f"  rocprofv3 --kernel-trace --stats -d <dir> -o k --output-format csv -- python3 bench.py --case {case} --steps 10",
                 f"  python3 bench.py --trace-summary <dir> <this file> {case}",
                 ""]
    else:
        lines = [
            "rocprofv3 kernel-trace statistics of the default bench command (all parts of the hot path:",
            "dense stack at M=1, 4, 16; FFN pair at M=1, 8, 64, 256; product-VQ at M=1, 16, 64 at 2 and 6 bits",
            "per weight; MoE block at M=32, 256, 2048; the screened 8-bit readout at M=1, 4; the streaming-read",
            "floor; oracle timing on the host runs no GPU kernels).",
            "",
            "command (run from the repository root, cd /tmp && export TMPDIR=/tmp first):",
            "  rocprofv3 --kernel-trace --stats -d <dir> -o k --output-format csv -- python3 bench.py",
            "  python3 bench.py --trace-summary <dir> <this file>",
            ""]
    lines += [
        f"  {'kernel':130s} {'calls':>7s} {'avg us':>10s} {'min us':>9s} {'total us':>12s}",
    ]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"  {r['Name'][:130]:130s} {int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.3f} "
                     f"{float(r['MinNs']) / 1e3:9.3f} {float(r['TotalDurationNs']) / 1e3:12.1f}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def planes_meta_bytes(k, n, bits):
    return n * k * bits // 8 + n * (k // 128) * 4


# ---------------------------------------------------------------- main

CASES = ("stack1", "stack4", "stack16", "stack16mx", "single", "ffn1", "ffn8", "ffn64", "ffn256", "pvq1", "pvq16", "pvq64", "moe",
         "moe256", "moe2048", "readout1", "readout4", "pvq6bpw1", "pvq6bpw16", "pvq6bpw64")


def run_case(torch, L, case, steps):
    """One measurement alone (for rocprofv3 counter runs): prints its result."""
    if case == "stack16mx":   # the dense stack at 16 tokens on the matrix-core GEMM (LBQ_PATH_GEMM_MX)
        r = extra_stack(torch, L, 16, steps, path=L.PATH_GEMM_MX)
    elif case.startswith("stack"):
        M = int(case[5:])
        r = extra_stack(torch, L, M, steps) if M > 1 else extra_stack(torch, L, 1, steps)
    elif case == "single":
        r = extra_single(torch, L, steps)
    elif case.startswith("ffn"):
        r = extra_ffn(torch, L, steps, Ms=(int(case[3:]),))
    elif case.startswith("pvq6bpw"):
        r = extra_pvq(torch, L, steps, Ms=(int(case[7:]),), bits=6)
    elif case.startswith("pvq"):
        r = extra_pvq(torch, L, steps, Ms=(int(case[3:]),))
    elif case.startswith("readout"):
        r = extra_readout(torch, L, steps, Ms=(int(case[7:]),))
    else:
        r = extra_moe(torch, L, steps, extras=False, M=int(case[3:]) if len(case) > 3 else None)
    print(json.dumps({"case": case, "result": r}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--no-extra", action="store_true", help="skip the measurements of the other configurations")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing on the host")
    ap.add_argument("--case", choices=CASES, help="run one measurement alone (for counter runs), then exit")
    ap.add_argument("--cpu-configs", action="store_true",
                    help="time the oracle per configuration on this host (no GPU), print JSON, then exit")
    ap.add_argument("--summarize", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "TRACE_DIR"),
                    help="write the counter summary under profiles/ from rocprofv3 outputs, then exit")
    ap.add_argument("--summary-command", default="python3 bench.py --steps 5 --warmup 1 --no-extra --no-cpu")
    ap.add_argument("--trace-summary", nargs="+", metavar="ARG",
                    help="TRACE_DIR OUT [CASE]: write a per-kernel table of a rocprofv3 --kernel-trace --stats "
                         "run of the default command (python3 bench.py), or of 'bench.py --case CASE', to OUT, "
                         "then exit")
    ap.add_argument("--pmc-summary", nargs="+", metavar="ARG",
                    help="CASE KERNEL OUT DIR...: counters of one kernel from rocprofv3 --pmc runs of "
                         "'bench.py --case CASE' (one directory per pass), written to OUT, then exit")
    args = ap.parse_args()
    if args.summarize:
        summarize(*args.summarize, args.summary_command, PROFILE_SUMMARY)
        return
    if args.trace_summary:
        trace_table(*args.trace_summary)
        return
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary[:3], args.pmc_summary[3:])
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this implementation runs on one GPU; the multi-GPU sharding is a design note, "
                                   "so --gpus must be 1"}), flush=True)
        sys.exit(2)
    if args.cpu_configs:
        from bit_weight_only_amd import lbq as L
        cpu_configs(L)
        return

    import torch
    from bit_weight_only_amd import lbq as L

    L.lib()
    if args.case:
        run_case(torch, L, args.case, args.steps)
        return
    log(f"[bench] packing dense stack ({args.layers} layers)")
    stack = Stack(L, torch, args.layers, 1)
    log(f"[bench] {stack.bytes_per_step / 1e9:.3f} GB packed weights per step")
    calibration_copy(torch)

    # timed region: graph replay of `steps` steps (synchronize on both sides;
    # events between the replays give the per-step spread)
    clocks_before = gpu_clocks()
    step_times = []
    t = time_graph(torch, stack.step, args.steps, args.warmup, step_times)
    clocks_after = gpu_clocks()
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
                                   "us": stats(d, 1e6), "GBps": round(sh["bytes"] / avg / 1e9, 1),
                                   "frac_of_hbm_peak": round(sh["bytes"] / avg / 1e9 / HBM_PEAK_GBS, 4),
                                   "kernels": "gemv_mfma"}
        dom_b += sh["bytes"] * len(d)
        dom_t += float(d.sum())
        dom_n += len(d)
    achieved = dom_b / dom_t / 1e9
    log(f"[bench] per-launch: {json.dumps(shape_stats)}")

    extra = {"per_shape_M1": shape_stats,
             "dominant_kernel": {"name": DOMINANT, "launches": dom_n, "avg_us": round(dom_t / dom_n * 1e6, 3),
                                 "bytes_per_launch_avg": round(dom_b / dom_n),
                                 "trace_avg_us": trace_avgs_from_summary()},
             "step_ms": stats(step_times, 1e3, 4),
             "gpu_clocks": {"before": clocks_before, "after": clocks_after}}
    del stack
    torch.cuda.empty_cache()

    # the streaming-read floor of each GEMV launch's byte count (and the layer)
    log("[bench] extra: streaming-read floor per launch size")
    sizes = {name: planes_meta_bytes(k, n, 2) for (name, k, n) in synth.DENSE_STACK_SHAPES}
    sizes["single_linear"] = planes_meta_bytes(4096, 4096, 2)
    fl = stream_floor(torch, L, sizes)
    layer_floor = 0.0
    for name, st in shape_stats.items():
        f = fl[name]["floor_us"]["median"]
        layer_floor += f
        st["floor_us"] = f
        st["frac_of_floor"] = round(f / st["us"]["median"], 4)
    fl["layer_floor_us"] = round(layer_floor, 3)
    fl["layer_floor_frac_of_hbm_peak"] = round(stack_bytes(1) / (layer_floor * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    log("[bench] extra: the headline step with streaming reads in place of the GEMVs")
    sf = stack_floor(torch, L, args.layers, {name: fl[name]["shape"] for (name, _, _) in synth.DENSE_STACK_SHAPES},
                     args.steps)
    sf["headline_frac_of_floor"] = round(sf["read_us_per_layer"]["median"] /
                                         (extra["step_ms"]["median"] * 1e3 / args.layers), 4)
    fl["stack"] = sf
    extra["stream_floor"] = fl

    if not args.no_extra:
        steps = max(5, args.steps // 2)
        log("[bench] extra: single 4096x4096 linear, M=1")
        extra["single_linear_M1"] = extra_single(torch, L, steps)
        sl = extra["single_linear_M1"]
        sl["floor_us"] = fl["single_linear"]["floor_us"]["median"]
        sl["frac_of_floor"] = round(sl["floor_us"] / sl["us_per_call_stats"]["median"], 4)
        for M in (4, 16):
            log(f"[bench] extra: dense stack M={M}")
            extra[f"stack_M{M}"] = extra_stack(torch, L, M, steps)
        log("[bench] extra: FFN pair 5120/17408, M=1,8,64,256")
        extra["ffn_pair"] = extra_ffn(torch, L, steps)
        log("[bench] extra: product-VQ 4096->14336")
        extra["pvq"] = extra_pvq(torch, L, steps)
        log("[bench] extra: product-VQ 4096->14336 at 6 bits per weight (three residual stages)")
        extra["pvq_6bpw"] = extra_pvq(torch, L, steps, bits=6)
        log("[bench] extra: MoE block")
        extra["moe_block"] = extra_moe(torch, L, steps)
        for M in (256, 2048):
            log(f"[bench] extra: MoE block, {M} tokens (prefill)")
            extra[f"moe_block_M{M}"] = extra_moe(torch, L, max(3, steps // 2), extras=False, M=M)
        log("[bench] extra: screened readout 2048 -> 131072 (8-bit, nibble-split)")
        extra["readout"] = extra_readout(torch, L, steps)
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
