"""GPTQ-packed weights (lbq_gptq_factor + lbq_pack_gptq: group-128 GPTQ in
the rotated basis) through the GPU path: the packed format is the RTN one, so
the matrix-core GEMV and the MFMA GEMM decode them unchanged. Outputs against
the oracle's decode of the packed buffer, codes against the oracle's own GPTQ
on sampled rows, and the method's point on the GPU: a smaller layer-output
error than RTN on inputs from the calibration distribution."""
import numpy as np
import pytest

import synth
from oracle import lbq_oracle as O
from _helpers import TOL, cuda, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return cuda()


@pytest.fixture(scope="module")
def L():
    from bit_weight_only_amd import lbq
    lbq.lib()
    return lbq


@pytest.fixture(scope="module")
def packed(L):
    """The 4096 x 4096 single linear packed by GPTQ (2 bits) and by RTN, with
    a Hessian from 8192 calibration rows."""
    k = n = 4096
    x = synth.calibration(2 * k, k, workload=42, item=0).astype(np.float64)
    h = x.T @ x / x.shape[0]
    s = synth.signs(k, workload=synth.W_SINGLE)
    w = synth.weights(n, k, workload=synth.W_SINGLE)
    u = L.gptq_factor(h, s)
    g_planes, g_meta = L.pack_gptq(w, 2, s, u)
    r_planes, r_meta = L.pack(w, 2, s)
    return dict(k=k, n=n, h=h, s=s, w=w, g=(g_planes, g_meta), r=(r_planes, r_meta))


@pytest.mark.parametrize("m", [1, 4, 64])
def test_gptq_weights_on_the_gpu_match_the_oracle(L, dev, packed, m):
    k, n, s = packed["k"], packed["n"], packed["s"]
    planes, meta = packed["g"]
    pl = L.PackedLinear.from_host(planes, meta, s, k, n, 2)
    x = synth.activations(m, k, workload=42, item=m)
    y = L.linear_forward(pl, to_dev(x, dev)).cpu().numpy().astype(np.float64)
    want = O.linear_rtn(x, planes.view(np.uint32), meta.view(np.uint16), s, 2, n, k)
    e = O.rel_l2(y, want)
    say(f"gptq m={m} rel_l2 {e:.3e}")
    assert e < TOL


def test_gptq_codes_read_back_match_the_oracles_gptq(L, dev, packed):
    k, n, s, w = packed["k"], packed["n"], packed["s"], packed["w"]
    planes, meta = packed["g"]
    pl = L.PackedLinear.from_host(planes, meta, s, k, n, 2)
    codes = L.unpack_codes(pl).cpu().numpy()
    rows = np.sort(np.random.default_rng(9).choice(n, 16, replace=False))
    _, _, q = O.pack_gptq(w[rows], 2, s, O.gptq_factor(packed["h"], s))
    assert np.array_equal(codes[rows], q)
    say("gptq codes of 16 sampled rows: mismatches 0")


def test_gptq_lowers_the_output_error_on_the_gpu(L, dev, packed):
    """y = x W^T on calibration-distributed tokens: the GPU output of the GPTQ
    weight is closer to the unquantized product than that of the RTN weight."""
    k, n, s, w = packed["k"], packed["n"], packed["s"], packed["w"]
    x = synth.calibration(64, k, workload=42, item=0, sample=1)   # held-out rows, same distribution
    x = (x / np.abs(x).max()).astype(np.float16)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    errs = {}
    for name in ("g", "r"):
        planes, meta = packed[name]
        pl = L.PackedLinear.from_host(planes, meta, s, k, n, 2)
        y = L.linear_forward(pl, to_dev(x, dev)).cpu().numpy().astype(np.float64)
        errs[name] = O.rel_l2(y, exact)
    say(f"output error vs unquantized: gptq {errs['g']:.4f}  rtn {errs['r']:.4f}")
    assert errs["g"] < 0.8 * errs["r"]
