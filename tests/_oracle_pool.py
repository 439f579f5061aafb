"""Oracle work for the full-size parity tests, spread over host processes.

Rows of a linear and experts of a MoE block are independent, so the oracle
(unchanged, single-threaded NumPy per job) runs on chunks of rows or on single
experts in a pool of spawned processes. Each job regenerates its seeded inputs
from the same generators the test uses, so only small arrays cross processes.
Nothing here computes anything the oracle does not: the jobs call oracle
functions and slice their results.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np

import synth
from oracle import lbq_oracle as O

_POOL = None


def pool() -> cf.ProcessPoolExecutor:
    """One pool per test session; spawned workers (the parent may hold a GPU context)."""
    global _POOL
    if _POOL is None:
        n = max(1, min(8, len(os.sched_getaffinity(0))))
        _POOL = cf.ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"))
    return _POOL


def chunks(n: int, size: int):
    return [(r0, min(n, r0 + size)) for r0 in range(0, n, size)]


# ---------------------------------------------------------------- jobs (run in workers)

def rtn_rows_job(n, k, bits, workload, item, r0, r1, x16):
    """Oracle y[:, r0:r1] and codes of rows r0:r1 from the oracle's own packing."""
    w = synth.weights(n, k, workload=workload, item=item)[r0:r1]
    s = synth.signs(k, workload=workload, item=item)
    planes, meta, q = O.pack_rtn(w, bits, s)
    y = None if x16 is None else O.linear_rtn(x16, planes, meta, s, bits, r1 - r0, k)
    return y, q


def moe_expert_job(e, hidden, ffn, bits_e, workload, x16_rows):
    """FFN of expert e (oracle packing, dequantization, SwiGLU) on its tokens."""
    sh = synth.signs(hidden, workload=workload, item=1)
    sf = synth.signs(ffn, workload=workload, item=2)
    pg, mg, _ = O.pack_rtn(synth.weights(2 * ffn, hidden, workload=workload, item=1000 + e), bits_e, sh)
    pd, md, _ = O.pack_rtn(synth.weights(hidden, ffn, workload=workload, item=5000 + e), bits_e, sf)
    w_gu = O.dequant_weight_rtn(pg, mg, sh, bits_e, 2 * ffn, hidden)
    w_dn = O.dequant_weight_rtn(pd, md, sf, bits_e, hidden, ffn)
    return O.expert_ffn(x16_rows, w_gu, w_dn)


# ---------------------------------------------------------------- parent-side helpers

def rtn_all_rows(n, k, bits, workload, item, x16=None, chunk=2048):
    """(y [M][n] or None, codes uint8 [n][k]) over every row, by row chunks."""
    futs = [pool().submit(rtn_rows_job, n, k, bits, workload, item, r0, r1, x16) for r0, r1 in chunks(n, chunk)]
    res = [f.result() for f in futs]
    y = None if x16 is None else np.concatenate([r[0] for r in res], axis=1)
    q = np.concatenate([r[1] for r in res], axis=0)
    return y, q


def moe_all_tokens(x16, logits, top_k, bits, hidden, ffn, workload):
    """The oracle's MoE block over every token, each routed expert's FFN in its own job."""
    ids, _ = O.route(logits, top_k)
    futs = {}
    for e in np.unique(ids):
        rows, _ = np.nonzero(ids == e)
        futs[int(e)] = pool().submit(moe_expert_job, int(e), hidden, ffn, int(bits[e]), workload, x16[rows])
    outs = {e: f.result() for e, f in futs.items()}
    return O.moe_forward(x16, logits, top_k, expert_outputs=lambda e, rows: outs[e])
