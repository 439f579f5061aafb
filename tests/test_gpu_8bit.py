"""8-bit group codes (the non-expert path's width) on the GPU: codes read
back bit-exact, the matrix-core GEMV (four 2-bit digits of each code on the
fp4 operand, scales 1, 4, 16, 64), the MFMA GEMM (codes inserted into the fp16
mantissa), against the oracle on the same seeded inputs."""
import numpy as np
import pytest

import synth
from oracle import lbq_oracle as O
from _helpers import TOL, cuda, make_rtn, oracle_rtn_rows, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return cuda()


@pytest.fixture(scope="module")
def L():
    from bit_weight_only_amd import lbq
    lbq.lib()
    return lbq


@pytest.mark.parametrize("n,k", [(1, 128), (3, 256), (130, 512), (257, 1152), (4096, 4096)])
def test_8bit_codes_bit_exact(L, dev, n, k):
    w, s, planes, meta, pl = make_rtn(n, k, 8, 60, n + k)
    got = L.unpack_codes(pl).cpu().numpy()
    assert np.array_equal(got, O.unpack_planes(planes.view(np.uint32), 8, k))
    rows = np.arange(n) if n <= 300 else np.sort(np.random.default_rng(1).choice(n, 64, replace=False))
    _, _, q = O.pack_rtn(w[rows], 8, s)
    assert np.array_equal(got[rows], q)


@pytest.mark.parametrize("n,k", [(17, 512), (300, 1536), (1030, 2048), (33, 16384), (4096, 4096)])
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_8bit_matrix_core_gemv(L, dev, n, k, m):
    say(f"8-bit gemv n={n} k={k} m={m}")
    w, s, planes, meta, pl = make_rtn(n, k, 8, 61, n + k)
    x = synth.activations(m, k, workload=61, item=m)
    y = L.linear_forward(pl, to_dev(x, dev), path=L.PATH_GEMV).cpu().numpy().astype(np.float64)
    want = O.linear_rtn(x, planes.view(np.uint32), meta.view(np.uint16), s, 8, n, k)
    e = O.rel_l2(y, want)
    say(f"  rel_l2 {e:.3e}")
    assert e < TOL


@pytest.mark.parametrize("n,k", [(1, 128), (70, 384), (130, 1152), (200, 2176), (4096, 4096)])
@pytest.mark.parametrize("m", [1, 5, 17, 64, 129])
def test_8bit_gemm_and_auto(L, dev, n, k, m):
    """The MFMA GEMM at 8 bits (and the AUTO path: K not a multiple of 512 at
    one token has no staged VALU GEMV at 8 bits and takes the GEMM)."""
    say(f"8-bit gemm n={n} k={k} m={m}")
    w, s, planes, meta, pl = make_rtn(n, k, 8, 62, n + k)
    x = synth.activations(m, k, workload=62, item=m)
    xd = to_dev(x, dev)
    y = L.linear_forward(pl, xd, path=L.PATH_GEMM).cpu().numpy().astype(np.float64)
    want = O.linear_rtn(x, planes.view(np.uint32), meta.view(np.uint16), s, 8, n, k)
    assert O.rel_l2(y, want) < TOL
    if m == 1:
        ya = L.linear_forward(pl, xd).cpu().numpy().astype(np.float64)
        assert O.rel_l2(ya, want) < TOL


def test_8bit_forced_staged_gemv_is_refused(L, dev):
    w, s, planes, meta, pl = make_rtn(64, 384, 8, 63, 0)
    x = to_dev(synth.activations(2, 384, workload=63), dev)
    with pytest.raises(L.LbqError) as e:
        L.linear_forward(pl, x, path=L.PATH_GEMV)
    assert e.value.status == -2


@pytest.mark.parametrize("m", [3, 40])
def test_8bit_large_scales(L, dev, m):
    """Weights 2000 times the usual size: 8-bit scales near 0.6 and zero
    terms of s z up to about 75; both paths stay within the tolerance."""
    n, k = 96, 1024
    w = synth.weights(n, k, workload=64, item=m) * 2000.0
    s = synth.signs(k, workload=64, item=m)
    planes, meta = L.pack(w, 8, s)
    pl = L.PackedLinear.from_host(planes, meta, s, k, n, 8)
    x = synth.activations(m, k, workload=64, item=m)
    y = L.linear_forward(pl, to_dev(x, dev)).cpu().numpy().astype(np.float64)
    assert np.isfinite(y).all()
    assert O.rel_l2(y, oracle_rtn_rows(w, s, 8, x)) < TOL


def test_8bit_gptq_weights(L, dev):
    """GPTQ at 8 bits through the GPU path."""
    k, n = 1024, 512
    xc = synth.calibration(2048, k, workload=65, item=0).astype(np.float64)
    h = xc.T @ xc / xc.shape[0]
    s = synth.signs(k, workload=65)
    w = synth.weights(n, k, workload=65)
    planes, meta = L.pack_gptq(w, 8, s, L.gptq_factor(h, s))
    pl = L.PackedLinear.from_host(planes, meta, s, k, n, 8)
    for m in (1, 33):
        x = synth.activations(m, k, workload=65, item=m)
        y = L.linear_forward(pl, to_dev(x, dev)).cpu().numpy().astype(np.float64)
        want = O.linear_rtn(x, planes.view(np.uint32), meta.view(np.uint16), s, 8, n, k)
        assert O.rel_l2(y, want) < TOL
