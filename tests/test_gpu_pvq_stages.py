"""Residual product-VQ stages (2, 4 and 6 bits per weight; three stages carry
the 48 index bits per 8-weight vector of the gridbook card's 6.0-bpw rung) on
the GPU, through the C ABI, against the oracle on the same seeded inputs:
indices read back bit-exact, and every decoder (the matrix-core GEMV with one
accumulator per stage, the MFMA GEMM with the stages folded into one fp16 B
value per weight) within the linear layers' tolerance."""
import numpy as np
import pytest

import synth
from oracle import lbq_oracle as O
from _helpers import TOL, cuda, sample_rows, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return cuda()


@pytest.fixture(scope="module")
def L():
    from bit_weight_only_amd import lbq
    lbq.lib()
    return lbq


def make(L, n, k, bits, item, cb=None):
    cb = synth.codebook(workload=80) if cb is None else cb
    w = synth.weights(n, k, workload=80, item=item)
    s = synth.signs(k, workload=80, item=item)
    idx, sc = L.pack(w, bits, s, L.FMT_PVQ_4x8, cb)
    pl = L.PackedLinear.from_host(idx, sc, s, k, n, bits, L.FMT_PVQ_4x8, cb)
    return w, s, cb, idx, sc, pl


def oracle_rows(w, s, cb, stages, x, rows=None):
    sub = w if rows is None else w[rows]
    oi, os_ = O.pack_pvq_stages(sub, s, cb, stages)
    return O.linear_pvq_stages(x, oi, os_, cb, s)


@pytest.mark.parametrize("bits", [4, 6])
@pytest.mark.parametrize("n,k", [(17, 512), (130, 1024), (257, 640)])
@pytest.mark.parametrize("m,path", [(1, 0), (3, 0), (4, 1), (1, 2), (5, 0), (16, 0), (64, 0)])
def test_pvq_stages_small(L, dev, bits, n, k, m, path):
    w, s, cb, idx, sc, pl = make(L, n, k, bits, n + k)
    x = synth.activations(m, k, workload=80, item=m)
    if path == 1 and k % 512:
        # residual stages run on the matrix-core GEMV (K a multiple of 512) or
        # the GEMM only: a forced GEMV elsewhere is refused before any launch
        with pytest.raises(L.LbqError) as err:
            L.linear_forward(pl, to_dev(x, dev), path=path)
        assert err.value.status == -2
        return
    y = L.linear_forward(pl, to_dev(x, dev), path=path).cpu().numpy().astype(np.float64)
    e = O.rel_l2(y, oracle_rows(w, s, cb, bits // 2, x))
    say(f"pvq stages bits={bits} n={n} k={k} m={m} path={path}: rel_l2 {e:.3e}")
    assert e < TOL


@pytest.mark.parametrize("bits", [4, 6])
def test_pvq_stages_indices_read_back(L, dev, bits):
    n, k = 300, 1024
    w, s, cb, idx, sc, pl = make(L, n, k, bits, 7)
    got = L.unpack_codes(pl).cpu().numpy()
    oi, _ = O.pack_pvq_stages(w, s, cb, bits // 2)
    assert np.array_equal(got, oi.reshape(-1, k // 4))


def test_pvq_stages_forced_gemv_refused_when_unsupported(L, dev):
    w, s, cb, idx, sc, pl = make(L, 9, 640, 6, 3)
    x = to_dev(synth.activations(2, 640, workload=80, item=2), dev)
    with pytest.raises(L.LbqError) as e:
        L.linear_forward(pl, x, path=L.PATH_GEMV)
    assert e.value.status == -2


@pytest.mark.parametrize("m", [1, 4, 16, 64])
def test_pvq_6bpw_full_shape_sampled(L, dev, m):
    """The product-VQ linear 4096 -> 14336 at 6 bits per weight (three stages),
    at the bench's launch configuration; sampled rows (both ends) against the
    oracle, which packs those rows itself; error below the 2-bit format's at
    the same shape (the stages lower the weight error)."""
    cfg = synth.PVQ_LINEAR
    k, n = cfg["K"], cfg["N"]
    cb = synth.codebook(workload=synth.W_PVQ)
    w = synth.weights(n, k, workload=synth.W_PVQ)
    s = synth.signs(k, workload=synth.W_PVQ)
    idx, sc = L.pack(w, 6, s, L.FMT_PVQ_4x8, cb)
    pl = L.PackedLinear.from_host(idx, sc, s, k, n, 6, L.FMT_PVQ_4x8, cb)
    x = synth.activations(m, k, workload=synth.W_PVQ, item=m)
    y = L.linear_forward(pl, to_dev(x, dev)).cpu().numpy().astype(np.float64)
    rows = sample_rows(n, 64, seed=m)
    want = oracle_rows(w, s, cb, 3, x, rows)
    e = O.rel_l2(y[:, rows], want)
    exact = x.astype(np.float64) @ w[rows].astype(np.float64).T
    say(f"pvq 6 bpw 4096x14336 m={m}: rel_l2 {e:.3e}, output error vs unquantized {O.rel_l2(want, exact):.3f}")
    assert e < TOL
