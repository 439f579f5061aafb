"""The no-allocation entry point lbq_linear_forward_noalloc (static device
scratch instead of a caller workspace) against lbq_linear_forward on the same
inputs: two calls in a row, the second smaller, each bit-identical to the
workspace entry point (the same kernels and plans) and within the oracle's
tolerance. Runs last: it shares one device array across calls."""
import numpy as np
import pytest

import synth
from oracle import lbq_oracle as O
from _helpers import TOL, cuda, make_rtn, make_pvq, oracle_rtn_rows, oracle_pvq_rows, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return cuda()


@pytest.fixture(scope="module")
def L():
    from bit_weight_only_amd import lbq
    lbq.lib()
    return lbq


def _both(L, pl, x):
    a = L.linear_forward(pl, x).cpu().numpy()
    b = L.linear_forward_noalloc(pl, x).cpu().numpy()
    return a, b


@pytest.mark.parametrize("bits", [2, 3, 8])
def test_noalloc_matches_workspace_entry_point(L, dev, bits):
    """GEMM with split-K (partials and arrival counters in the scratch) at 64
    tokens, then a smaller call at 9 tokens (fewer tiles, the counters cleared
    again), then one token (the matrix-core GEMV, no scratch)."""
    n, k = 1024, 4096
    w, s, planes, meta, pl = make_rtn(n, k, bits, 30, bits)
    for m in (64, 9, 1):
        say(f"noalloc rtn bits={bits} m={m} ws={pl.workspace_bytes(m)}")
        x16 = synth.activations(m, k, workload=30, item=m)
        a, b = _both(L, pl, to_dev(x16, dev))
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), m
        assert O.rel_l2(b.astype(np.float64), oracle_rtn_rows(w, s, bits, x16)) < TOL


def test_noalloc_pvq_gemm(L, dev):
    n, k = 512, 2048
    w, s, cb, idx, sc, pl = make_pvq(n, k, 30, 7)
    for m in (40, 17):
        say(f"noalloc pvq m={m}")
        x16 = synth.activations(m, k, workload=30, item=100 + m)
        a, b = _both(L, pl, to_dev(x16, dev))
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), m
        assert O.rel_l2(b.astype(np.float64), oracle_pvq_rows(w, s, cb, x16)) < TOL


def test_noalloc_pvq_three_stages(L, dev):
    """6 bits per weight (three residual stages): the GEMM at 40 then 17
    tokens and the matrix-core GEMV at 3, identical bits to the workspace call."""
    n, k = 384, 1024
    cb = synth.codebook(workload=30)
    w = synth.weights(n, k, workload=30, item=8)
    s = synth.signs(k, workload=30, item=8)
    idx, sc = L.pack(w, 6, s, L.FMT_PVQ_4x8, cb)
    pl = L.PackedLinear.from_host(idx, sc, s, k, n, 6, L.FMT_PVQ_4x8, cb)
    for m in (40, 17, 3):
        say(f"noalloc pvq 6 bpw m={m}")
        x16 = synth.activations(m, k, workload=30, item=200 + m)
        a, b = _both(L, pl, to_dev(x16, dev))
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), m
        oi, os_ = O.pack_pvq_stages(w, s, cb, 3)
        assert O.rel_l2(b.astype(np.float64), O.linear_pvq_stages(x16, oi, os_, cb, s)) < TOL


def test_noalloc_rejects_oversized_calls(L, dev):
    """A call whose workspace exceeds the scratch array is refused before any
    launch (LBQ_ERR_WORKSPACE), and the next call still works."""
    import torch

    n, k = 64, 17408
    w, s, planes, meta, pl = make_rtn(n, k, 2, 31, 0)
    m = 4000   # rotated activations alone: 4000 * 17408 * 2 bytes > 64 MiB
    assert pl.workspace_bytes(m) > 64 << 20
    x = torch.zeros((m, k), dtype=torch.float16, device=dev)
    with pytest.raises(L.LbqError) as e:
        L.linear_forward_noalloc(pl, x)
    assert e.value.status == -5
    x16 = synth.activations(5, k, workload=31)
    a, b = _both(L, pl, to_dev(x16, dev))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
