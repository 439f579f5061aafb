"""GPU parity of the matrix-core GEMM for five to sixteen tokens of 2-bit RTN
codes (fp4 codes x three e4m3 activation pieces, per-(token, group) E8M0
scale, zero-point term on an fp16 MFMA) through the C ABI, against the CPU
oracle on the same seeded inputs."""
import numpy as np
import pytest

import synth
from oracle import lbq_oracle as O
from _helpers import TOL, cuda, make_rtn, oracle_rtn_rows, sample_rows, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return cuda()


@pytest.fixture(scope="module")
def L():
    from bit_weight_only_amd import lbq
    lbq.lib()
    return lbq


@pytest.mark.parametrize("n,k", [(17, 512), (200, 2048), (1000, 4608), (4100, 1024), (90, 14336)])
@pytest.mark.parametrize("m", [1, 5, 8, 13, 16])
def test_gemm_mx_small_shapes(L, dev, n, k, m):
    """Every output row: ragged N (17, 200, 1000, 90 rows: partial 16-row blocks
    and 64-row tiles), one to many K slices (K = 512: one slice of four groups;
    4608 and 14336: uneven slices of whole 4-group words), one row block per
    wave (N < 8192), every token count of a tile (tokens past M are zeros)."""
    say(f"gemm mx n={n} k={k} m={m}")
    w, s, planes, meta, pl = make_rtn(n, k, 2, 31, n + k + m)
    x = synth.activations(m, k, workload=31, item=m)
    y = L.linear_forward(pl, to_dev(x, dev), path=L.PATH_GEMM_MX).cpu().numpy().astype(np.float64)
    want = oracle_rtn_rows(w, s, 2, x)
    e = O.rel_l2(y, want)
    say(f"  rel_l2 {e:.3e}")
    assert e < TOL


@pytest.mark.parametrize("n,k,m", [(8200, 4096, 16), (8192, 512, 7), (12000, 14336, 9)])
def test_gemm_mx_two_row_blocks(L, dev, n, k, m):
    """Tall matrices take two row blocks per wave (128-row tiles; 8200 rows
    leave a ragged last tile): sampled rows, both ends included."""
    say(f"gemm mx nb=2 n={n} k={k} m={m}")
    w, s, planes, meta, pl = make_rtn(n, k, 2, 32, m)
    x = synth.activations(m, k, workload=32, item=m)
    y = L.linear_forward(pl, to_dev(x, dev), path=L.PATH_GEMM_MX).cpu().numpy().astype(np.float64)
    rows = sample_rows(n, 96, seed=m)
    want = oracle_rtn_rows(w, s, 2, x, rows)
    e = O.rel_l2(y[:, rows], want)
    say(f"  rel_l2 {e:.3e}")
    assert e < TOL


@pytest.mark.parametrize("n,k", [(4096, 4096), (4096, 14336)])
@pytest.mark.parametrize("m", [5, 16])
def test_gemm_mx_error_against_fp16_gemm(L, dev, n, k, m):
    """The pieces carry about twelve significant bits of each rotated
    activation and the codes enter exactly; the error against the oracle stays
    within that of the fp16 GEMM (fp16 activations, fp16-rounded decoded
    weights) on the same inputs."""
    say(f"gemm mx vs fp16 gemm n={n} k={k} m={m}")
    w, s, planes, meta, pl = make_rtn(n, k, 2, 33, n + k)
    x = synth.activations(m, k, workload=33, item=m)
    xd = to_dev(x, dev)
    a = L.linear_forward(pl, xd, path=L.PATH_GEMM_MX).cpu().numpy().astype(np.float64)
    b = L.linear_forward(pl, xd, path=L.PATH_GEMM).cpu().numpy().astype(np.float64)
    rows = sample_rows(n, 256, seed=m)
    want = oracle_rtn_rows(w, s, 2, x, rows)
    ea, eb = O.rel_l2(a[:, rows], want), O.rel_l2(b[:, rows], want)
    say(f"  gemm mx {ea:.3e}  fp16 gemm {eb:.3e}")
    assert ea < TOL and eb < TOL
    assert ea <= 1.5 * eb


def test_gemm_mx_tokens_of_very_different_size(L, dev):
    """Each (token, group) carries its own E8M0 scale on the A rows and its own
    zero-point sum; tokens 10^6 apart in size would expose one applied to the
    wrong token."""
    n, k, m = 300, 2048, 8
    w, s, planes, meta, pl = make_rtn(n, k, 2, 34, m)
    x = synth.activations(m, k, workload=34, item=m).astype(np.float64)
    x *= (10.0 ** np.array([3, -3, 1, -1, 2, -2, 0, 3]))[:, None]
    x = x.astype(np.float16)
    y = L.linear_forward(pl, to_dev(x, dev), path=L.PATH_GEMM_MX).cpu().numpy().astype(np.float64)
    want = oracle_rtn_rows(w, s, 2, x)
    for t in range(m):
        assert O.rel_l2(y[t], want[t]) < TOL, t


def test_gemm_mx_only_on_request(L, dev):
    """AUTO keeps the fp16 GEMM from five tokens on (the matrix-core GEMM
    measured no faster end to end): AUTO gives the forced fp16 GEMM's bits."""
    n, k = 256, 4096
    w, s, planes, meta, pl = make_rtn(n, k, 2, 35, 1)
    for m in (5, 16):
        x = to_dev(synth.activations(m, k, workload=35, item=m), dev)
        a = L.linear_forward(pl, x).cpu().numpy()
        b = L.linear_forward(pl, x, path=L.PATH_GEMM).cpu().numpy()
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), m


def test_gemm_mx_repeat_calls_bit_identical(L, dev):
    """Split-K partial tiles are summed by the last slice to arrive, in slice
    order: repeat calls give identical bits (the workspace keeps the previous
    call's partials and counters)."""
    n, k, m = 1024, 14336, 12
    w, s, planes, meta, pl = make_rtn(n, k, 2, 36, m)
    x = to_dev(synth.activations(m, k, workload=36, item=m), dev)
    import torch
    ws = torch.empty(pl.workspace_bytes(m), dtype=torch.uint8, device=dev)
    a = L.linear_forward(pl, x, ws=ws, path=L.PATH_GEMM_MX).cpu().numpy()
    for _ in range(3):
        b = L.linear_forward(pl, x, ws=ws, path=L.PATH_GEMM_MX).cpu().numpy()
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_gemm_mx_zero_activations_and_zero_tokens(L, dev):
    """All-zero activations give exact zeros (every piece, sum and term is
    zero); M = 0 is a no-op."""
    n, k, m = 130, 1024, 6
    w, s, planes, meta, pl = make_rtn(n, k, 2, 37, m)
    x = np.zeros((m, k), np.float16)
    y = L.linear_forward(pl, to_dev(x, dev), path=L.PATH_GEMM_MX).cpu().numpy()
    assert not np.any(y.view(np.uint16) & 0x7FFF)
    y0 = L.linear_forward(pl, to_dev(np.zeros((0, k), np.float16), dev), path=L.PATH_GEMM_MX)
    assert y0.shape == (0, n)


def test_gemm_mx_refused_where_unsupported(L, dev):
    """Forcing the matrix-core GEMM on 3-bit codes, K not a multiple of 512,
    or more than sixteen tokens returns LBQ_ERR_SHAPE before any launch."""
    cases = [(3, 1024, 8), (2, 640, 8), (2, 1024, 17)]
    for bits, k, m in cases:
        w, s, planes, meta, pl = make_rtn(64, k, bits, 38, k + m)
        x = to_dev(synth.activations(m, k, workload=38, item=m), dev)
        with pytest.raises(L.LbqError) as e:
            L.linear_forward(pl, x, path=L.PATH_GEMM_MX)
        assert e.value.status == -2, (bits, k, m)
