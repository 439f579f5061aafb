"""Shared helpers for the GPU parity tests: pack with the library, upload,
and compute the oracle's answer on the same inputs (sampled rows for large
weights: rows of a linear are independent, so the oracle packs and decodes
only those)."""
import os
import sys

import numpy as np

import synth
from oracle import lbq_oracle as O

TOL = 2e-3       # relative L2 bound on fp16 outputs (fp16 activations, fp32 accumulation)


def say(*a):
    """Print a progress / result line; with LBQ_PARITY_LOG set, also append it
    to that file (the measured errors of a GPU run, kept for the results table)."""
    print(*a, flush=True)
    sys.stdout.flush()
    path = os.environ.get("LBQ_PARITY_LOG")
    if path:
        test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
        with open(path, "a") as f:
            f.write(f"{test}\t{' '.join(str(x) for x in a)}\n")


def cuda():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def make_rtn(n, k, bits, workload, item):
    from bit_weight_only_amd import lbq

    w = synth.weights(n, k, workload=workload, item=item)
    s = synth.signs(k, workload=workload, item=item)
    planes, meta = lbq.pack(w, bits, s)
    pl = lbq.PackedLinear.from_host(planes, meta, s, k, n, bits)
    return w, s, planes, meta, pl


def make_pvq(n, k, workload, item, cb=None):
    from bit_weight_only_amd import lbq

    cb = synth.codebook(workload=workload) if cb is None else cb
    w = synth.weights(n, k, workload=workload, item=item)
    s = synth.signs(k, workload=workload, item=item)
    idx, sc = lbq.pack(w, 2, s, lbq.FMT_PVQ_4x8, cb)
    pl = lbq.PackedLinear.from_host(idx, sc, s, k, n, 2, lbq.FMT_PVQ_4x8, cb)
    return w, s, cb, idx, sc, pl


def oracle_rtn_rows(w, s, bits, x16, rows=None):
    """Oracle y[:, rows] from the oracle's own packing of W[rows]."""
    sub = w if rows is None else w[rows]
    planes, meta, _ = O.pack_rtn(sub, bits, s)
    return O.linear_rtn(x16, planes, meta, s, bits, sub.shape[0], sub.shape[1])


def oracle_pvq_rows(w, s, cb, x16, rows=None):
    sub = w if rows is None else w[rows]
    idx, sc = O.pack_pvq(sub, s, cb)
    return O.linear_pvq(x16, idx, sc, cb, s)


def sample_rows(n, count=96, seed=0):
    if n <= count:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    r = rng.choice(n, count, replace=False)
    r[:2] = [0, n - 1]                      # always include both ends
    return np.sort(r)


def to_dev(a, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
