"""GPU parity of the dense path through the C ABI: rotation, decoded codes,
dequant-GEMV (M <= 16) and MFMA dequant-GEMM, RTN and product-VQ, against the
CPU oracle on the same seeded inputs."""
import numpy as np
import pytest

import synth
from oracle import lbq_oracle as O
from _helpers import (TOL, cuda, make_pvq, make_rtn, oracle_pvq_rows, oracle_rtn_rows, sample_rows, say, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return cuda()


@pytest.fixture(scope="module")
def L():
    from bit_weight_only_amd import lbq
    lbq.lib()
    return lbq


# ---------------------------------------------------------------- rotation

@pytest.mark.parametrize("m,k", [(1, 128), (3, 4096), (16, 14336), (5, 17408), (64, 5120)])
def test_rotate_matches_oracle(L, dev, m, k):
    say(f"rotate m={m} k={k}")
    x = synth.activations(m, k, workload=10, item=k)
    s = synth.signs(k, workload=10, item=k)
    got = L.rotate(to_dev(x, dev), to_dev(s, dev)).cpu().numpy().astype(np.float64)
    want = O.rotate(x.astype(np.float64), s)
    err = np.abs(got - want)
    assert np.all(err <= 2.0 ** -10 * np.abs(want) + 2.0 ** -20), float(err.max())
    assert O.rel_l2(got, want) < 5e-4


# ---------------------------------------------------------------- codes

@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("n,k", [(1, 128), (3, 256), (130, 512), (257, 1152)])
def test_unpacked_codes_bit_exact(L, dev, bits, n, k):
    say(f"codes bits={bits} n={n} k={k}")
    w, s, planes, meta, pl = make_rtn(n, k, bits, 11, n * 10 + bits)
    got = L.unpack_codes(pl).cpu().numpy()
    _, _, q = O.pack_rtn(w, bits, s)
    assert np.array_equal(got, q)
    assert np.array_equal(got, O.unpack_planes(planes.view(np.uint32), bits, k))


def test_unpacked_codes_full_dense_down(L, dev):
    k, n = 14336, 4096
    say("codes full 14336x4096 2-bit")
    w, s, planes, meta, pl = make_rtn(n, k, 2, synth.W_STACK, 3)
    got = L.unpack_codes(pl).cpu().numpy()
    assert np.array_equal(got, O.unpack_planes(planes.view(np.uint32), 2, k))
    rows = sample_rows(n, 32, seed=3)
    _, _, q = O.pack_rtn(w[rows], 2, s)
    assert np.array_equal(got[rows], q)


def test_pvq_codes_roundtrip(L, dev):
    w, s, cb, idx, sc, pl = make_pvq(64, 512, 12, 1)
    got = L.unpack_codes(pl).cpu().numpy()
    oi, _ = O.pack_pvq(w, s, cb)
    assert np.array_equal(got, oi)


# ---------------------------------------------------------------- GEMV (M <= 16)

@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("n,k", [(1, 128), (3, 256), (130, 512), (257, 1024), (64, 4096)])
@pytest.mark.parametrize("m", [1, 2, 3, 5, 8, 13, 16])
def test_gemv_small_shapes(L, dev, bits, n, k, m):
    say(f"gemv bits={bits} n={n} k={k} m={m}")
    w, s, planes, meta, pl = make_rtn(n, k, bits, 13, n + k + bits)
    x = synth.activations(m, k, workload=13, item=m)
    y = L.linear_forward(pl, to_dev(x, dev), path=L.PATH_GEMV).cpu().numpy().astype(np.float64)
    want = oracle_rtn_rows(w, s, bits, x)
    assert O.rel_l2(y, want) < TOL


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("n,k", [(17, 512), (300, 1536), (1030, 2048), (4100, 512), (33, 16384)])
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_gemv_matrix_core_tokens(L, dev, bits, n, k, m):
    """One to four tokens with K a multiple of 512 run the matrix-core GEMV
    (fp8 activation pieces x fp4 codes, rotation in the prologue): ragged N,
    fewer tiles than workgroups (n = 17, 300), more (n = 4100, 257 tiles),
    long rows (K = 16384, 128 groups: three and four tokens go in two passes),
    every token count it serves. Forced GEMV path: AUTO sends the two-pass
    cases to the GEMM."""
    say(f"gemv mfma bits={bits} n={n} k={k} m={m}")
    w, s, planes, meta, pl = make_rtn(n, k, bits, 17, n + k + bits)
    x = synth.activations(m, k, workload=17, item=m)
    y = L.linear_forward(pl, to_dev(x, dev), path=L.PATH_GEMV).cpu().numpy().astype(np.float64)
    rows = np.arange(n) if n <= 1100 else sample_rows(n, 48, seed=m)
    want = oracle_rtn_rows(w, s, bits, x, rows)
    assert O.rel_l2(y[:, rows], want) < TOL


@pytest.mark.parametrize("m", [1, 2])
def test_gemv_matrix_core_tall_4bit(L, dev, m):
    """Tall 4-bit matrices with small rotations launch two 512-thread
    workgroups per compute unit (1025 row tiles here, the last one ragged: 16393 = 1024 * 16 + 9);
    sampled rows against the oracle, both ends included."""
    n, k, bits = 16393, 1024, 4
    say(f"gemv mfma tall 4-bit n={n} k={k} m={m}")
    w, s, planes, meta, pl = make_rtn(n, k, bits, 18, m)
    x = synth.activations(m, k, workload=18, item=m)
    y = L.linear_forward(pl, to_dev(x, dev)).cpu().numpy().astype(np.float64)
    rows = sample_rows(n, 64, seed=m)
    want = oracle_rtn_rows(w, s, bits, x, rows)
    assert O.rel_l2(y[:, rows], want) < TOL


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("n,k", [(257, 4096), (130, 5120), (67, 8192)])
@pytest.mark.parametrize("m", [1, 2])
def test_gemv_fused_and_staged_rotation_agree(L, dev, bits, n, k, m):
    """One or two tokens normally rotate inside the GEMV prologue; signs that
    are not 16-byte aligned send the same call through the separate rotation
    launch and the staged GEMV. Both must match the oracle and each other."""
    import torch

    say(f"gemv fused/staged bits={bits} n={n} k={k} m={m}")
    w, s, planes, meta, pl = make_rtn(n, k, bits, 16, n + k + bits)
    x = to_dev(synth.activations(m, k, workload=16, item=m), dev)
    a = L.linear_forward(pl, x).cpu().numpy().astype(np.float64)
    buf = torch.zeros(k + 16, dtype=torch.int8, device=dev)
    buf[1:1 + k].copy_(pl.signs)
    pl_odd = L.PackedLinear(k, n, bits, L.FMT_RTN_PLANES, pl.planes, pl.meta, buf[1:1 + k])
    assert pl_odd.signs.data_ptr() % 16 == 1
    b = L.linear_forward(pl_odd, x).cpu().numpy().astype(np.float64)
    want = oracle_rtn_rows(w, s, bits, x.cpu().numpy())
    assert O.rel_l2(a, want) < TOL
    assert O.rel_l2(b, want) < TOL
    assert O.rel_l2(a, b) < 1e-3


def test_gemv_single_linear_full(L, dev):
    """The 4096x4096 2-bit single linear at M=1, every output."""
    say("gemv single linear 4096x4096 M=1")
    w, s, planes, meta, pl = make_rtn(4096, 4096, 2, synth.W_SINGLE, 0)
    x = synth.activations(1, 4096, workload=synth.W_SINGLE)
    y = L.linear_forward(pl, to_dev(x, dev)).cpu().numpy().astype(np.float64)
    want = oracle_rtn_rows(w, s, 2, x)
    e = O.rel_l2(y, want)
    say(f"  rel_l2={e:.3e}")
    assert e < TOL


@pytest.mark.parametrize("shape", synth.DENSE_STACK_SHAPES, ids=[s[0] for s in synth.DENSE_STACK_SHAPES])
@pytest.mark.parametrize("m", synth.DENSE_STACK_M)
def test_gemv_dense_stack_sampled(L, dev, shape, m):
    name, k, n = shape
    say(f"gemv dense stack {name} k={k} n={n} m={m}")
    w, s, planes, meta, pl = make_rtn(n, k, 2, synth.W_STACK, synth.DENSE_STACK_SHAPES.index(shape))
    x = synth.activations(m, k, workload=synth.W_STACK, item=m)
    y = L.linear_forward(pl, to_dev(x, dev)).cpu().numpy().astype(np.float64)
    rows = sample_rows(n, 64, seed=m)
    want = oracle_rtn_rows(w, s, 2, x, rows)
    e = O.rel_l2(y[:, rows], want)
    say(f"  rel_l2={e:.3e}")
    assert e < TOL


# ---------------------------------------------------------------- MFMA GEMM

@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("n,k", [(1, 128), (70, 256), (130, 512), (64, 1024), (130, 4096), (200, 2176)])
@pytest.mark.parametrize("m", [1, 17, 33, 64, 100, 129])
def test_gemm_small_shapes(L, dev, bits, n, k, m):
    """Few output rows and long rows make the GEMM split K over workgroups
    (4096 and 2176 inputs here; 2176 = 17 groups splits unevenly)."""
    say(f"gemm bits={bits} n={n} k={k} m={m}")
    w, s, planes, meta, pl = make_rtn(n, k, bits, 14, n + k + bits)
    x = synth.activations(m, k, workload=14, item=m)
    y = L.linear_forward(pl, to_dev(x, dev), path=L.PATH_GEMM).cpu().numpy().astype(np.float64)
    want = oracle_rtn_rows(w, s, bits, x)
    assert O.rel_l2(y, want) < TOL


@pytest.mark.parametrize("swap", [False, True], ids=["gu2_dn3", "gu3_dn2"])
@pytest.mark.parametrize("m", synth.FFN_SWEEP["M"])
def test_ffn_sweep_sampled(L, dev, swap, m):
    """5120 -> 17408 gate|up and 17408 -> 5120 down at mixed 2/3-bit widths;
    M = 1 runs the GEMV, M = 8, 64, 256 the MFMA GEMM."""
    cfg = synth.FFN_SWEEP
    b_gu, b_dn = (cfg["bits_gu"], cfg["bits_dn"]) if not swap else (cfg["bits_dn"], cfg["bits_gu"])
    for (k, n, bits, item) in [(cfg["K_gu"], cfg["N_gu"], b_gu, 1), (cfg["N_gu"], cfg["K_gu"], b_dn, 2)]:
        say(f"ffn sweep k={k} n={n} bits={bits} m={m}")
        w, s, planes, meta, pl = make_rtn(n, k, bits, synth.W_FFN, item)
        x = synth.activations(m, k, workload=synth.W_FFN, item=m)
        y = L.linear_forward(pl, to_dev(x, dev)).cpu().numpy().astype(np.float64)
        rows = sample_rows(n, 48, seed=m + item)
        want = oracle_rtn_rows(w, s, bits, x, rows)
        e = O.rel_l2(y[:, rows], want)
        say(f"  rel_l2={e:.3e}")
        assert e < TOL


def test_gemv_and_gemm_agree(L, dev):
    w, s, planes, meta, pl = make_rtn(512, 2048, 2, 15, 1)
    x = to_dev(synth.activations(16, 2048, workload=15), dev)
    a = L.linear_forward(pl, x, path=L.PATH_GEMV).cpu().numpy().astype(np.float64)
    b = L.linear_forward(pl, x, path=L.PATH_GEMM).cpu().numpy().astype(np.float64)
    assert O.rel_l2(a, b) < 1e-3


def test_repeat_calls_bit_identical(L, dev):
    w, s, planes, meta, pl = make_rtn(1024, 4096, 3, 15, 2)
    for m in (1, 64):
        x = to_dev(synth.activations(m, 4096, workload=15, item=m), dev)
        a = L.linear_forward(pl, x).cpu().numpy()
        b = L.linear_forward(pl, x).cpu().numpy()
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_zero_tokens_is_noop(L, dev):
    import torch

    w, s, planes, meta, pl = make_rtn(64, 256, 2, 15, 3)
    x = torch.empty((0, 256), dtype=torch.float16, device=dev)
    y = L.linear_forward(pl, x)
    assert y.shape == (0, 64)


def test_zero_weights_give_zero_output(L, dev):
    """All-zero weights pack to codes 0 with the degenerate scale 1. The GEMM
    decodes round(s q) = 0 and a zero-point term of 0, so it returns exact
    zeros. The GEMV inserts codes into fp16 1.0 and removes the offsets with
    per-class activation sums, which leaves an fp32 cancellation residue of a
    few ulps of those sums; a wrong offset or zero point would leave residues
    of order 1 or more."""
    from bit_weight_only_amd import lbq

    k, n = 256, 32
    s = synth.signs(k, workload=15)
    planes, meta = lbq.pack(np.zeros((n, k), np.float32), 2, s)
    pl = lbq.PackedLinear.from_host(planes, meta, s, k, n, 2)
    x = to_dev(synth.activations(5, k, workload=15), dev)
    y = L.linear_forward(pl, x, path=L.PATH_GEMM).cpu().numpy().astype(np.float64)
    assert np.abs(y).max() == 0.0
    y = L.linear_forward(pl, x[:3], path=L.PATH_GEMV).cpu().numpy().astype(np.float64)
    assert np.abs(y).max() < 2e-3


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("m", [3, 40])
def test_large_scales_stay_finite(L, dev, bits, m):
    """Weights 2000 times the usual size give group scales near the packer's
    limit of 128 (2-bit) and code-weighted zero terms near the top of the fp16
    constants the GEMM decodes with; both paths stay within tolerance."""
    n, k = 96, 1024
    w = synth.weights(n, k, workload=15, item=40 + bits) * 2000.0
    s = synth.signs(k, workload=15, item=40 + bits)
    planes, meta = L.pack(w, bits, s)
    pl = L.PackedLinear.from_host(planes, meta, s, k, n, bits)
    x = synth.activations(m, k, workload=15, item=m)
    y = L.linear_forward(pl, to_dev(x, dev)).cpu().numpy().astype(np.float64)
    assert np.isfinite(y).all()
    assert O.rel_l2(y, oracle_rtn_rows(w, s, bits, x)) < TOL


# ---------------------------------------------------------------- product-VQ

# GEMV path: one to four tokens at K a multiple of 512 run on the matrix cores,
# the rest on the VALU lookup GEMV
@pytest.mark.parametrize("n,k", [(1, 128), (17, 512), (130, 512), (257, 1024), (257, 4096)])
@pytest.mark.parametrize("m,path", [(1, 1), (2, 1), (3, 1), (4, 1), (16, 1), (1, 2), (40, 2), (64, 2), (129, 2)])
def test_pvq_small_shapes(L, dev, n, k, m, path):
    say(f"pvq n={n} k={k} m={m} path={path}")
    w, s, cb, idx, sc, pl = make_pvq(n, k, 16, n + k)
    x = synth.activations(m, k, workload=16, item=m)
    y = L.linear_forward(pl, to_dev(x, dev), path=path).cpu().numpy().astype(np.float64)
    want = oracle_pvq_rows(w, s, cb, x)
    assert O.rel_l2(y, want) < TOL


@pytest.mark.parametrize("m", [2, 4])
def test_pvq_tokens_of_very_different_size(L, dev, m):
    """Each token's groups carry their own power-of-two scale into the matrix
    cores (one A row per token piece); tokens 10^6 apart in size would expose
    a scale applied to the wrong rows."""
    n, k = 96, 1024
    w, s, cb, idx, sc, pl = make_pvq(n, k, 16, 77)
    x = synth.activations(m, k, workload=16, item=90 + m).astype(np.float64)
    x *= (10.0 ** np.array([3, -3, 1, -1][:m]))[:, None]
    x = x.astype(np.float16)
    y = L.linear_forward(pl, to_dev(x, dev)).cpu().numpy().astype(np.float64)
    want = oracle_pvq_rows(w, s, cb, x)
    for t in range(m):   # each token against its own size
        assert O.rel_l2(y[t], want[t]) < TOL


@pytest.mark.parametrize("m", synth.PVQ_LINEAR["M"])
def test_pvq_linear_sampled(L, dev, m):
    cfg = synth.PVQ_LINEAR
    say(f"pvq 4096x14336 m={m}")
    w, s, cb, idx, sc, pl = make_pvq(cfg["N"], cfg["K"], synth.W_PVQ, 0)
    x = synth.activations(m, cfg["K"], workload=synth.W_PVQ, item=m)
    y = L.linear_forward(pl, to_dev(x, dev)).cpu().numpy().astype(np.float64)
    rows = sample_rows(cfg["N"], 48, seed=m)
    want = oracle_pvq_rows(w, s, cb, x, rows)
    e = O.rel_l2(y[:, rows], want)
    say(f"  rel_l2={e:.3e}")
    assert e < TOL


# ---------------------------------------------------------------- NVFP4-valued codebook

@pytest.mark.parametrize("n,k", [(17, 512), (257, 1024), (130, 640)])
@pytest.mark.parametrize("m,path", [(1, 1), (3, 1), (16, 1), (1, 2), (64, 2)])
def test_pvq_fp4_valued_codebook(L, dev, n, k, m, path):
    """The product-VQ decoders with a codebook whose values lie on the NVFP4
    (e2m1) grid (held as e4m3 bytes): every path (the matrix-core GEMV at
    K a multiple of 512 and up to four tokens, the VALU GEMV otherwise, the
    MFMA GEMM) against the oracle."""
    cb = synth.codebook_fp4(workload=16)
    w, s, cb, idx, sc, pl = make_pvq(n, k, 16, 500 + n + k, cb=cb)
    x = synth.activations(m, k, workload=16, item=500 + m)
    y = L.linear_forward(pl, to_dev(x, dev), path=path).cpu().numpy().astype(np.float64)
    assert O.rel_l2(y, oracle_pvq_rows(w, s, cb, x)) < TOL


def test_auto_path_sends_two_pass_tokens_to_the_gemm(L, dev):
    """At four tokens on 14336-long rows the matrix-core GEMV would run two
    passes over the codes; AUTO takes the MFMA GEMM there (bit-identical to the
    forced GEMM path) and keeps the one-pass GEMV at one token (bit-identical
    to the forced GEMV path)."""
    n, k = 256, 14336
    w, s, planes, meta, pl = make_rtn(n, k, 2, 24, 0)
    for m, forced in [(4, L.PATH_GEMM), (1, L.PATH_GEMV)]:
        x = to_dev(synth.activations(m, k, workload=24, item=m), dev)
        a = L.linear_forward(pl, x).cpu().numpy()
        b = L.linear_forward(pl, x, path=forced).cpu().numpy()
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), m
        assert O.rel_l2(a.astype(np.float64), oracle_rtn_rows(w, s, 2, x.cpu().numpy())) < TOL
