"""GPU parity at the workloads' full sizes, every output and every code:
the four dense-stack linears at one and four tokens (every row), the product-VQ
linear at one token (every row), the MoE block (every token), and the codes the
GPU decoders read back at full shape for every configuration. The oracle's
rows and experts are independent, so its work is spread over host processes
(tests/_oracle_pool.py); each job runs the oracle unchanged."""
import numpy as np
import pytest

import synth
from oracle import lbq_oracle as O
from _helpers import TOL, cuda, make_pvq, make_rtn, oracle_rtn_rows, sample_rows, say, to_dev
import _oracle_pool as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return cuda()


@pytest.fixture(scope="module")
def L():
    from bit_weight_only_amd import lbq
    lbq.lib()
    return lbq


# ---------------------------------------------------------------- dense stack, every row

@pytest.mark.parametrize("shape", synth.DENSE_STACK_SHAPES, ids=[s[0] for s in synth.DENSE_STACK_SHAPES])
def test_dense_stack_every_row_m1_m4(L, dev, shape):
    """Every output of each dense-stack linear at M = 1 and M = 4 (the
    matrix-core GEMV: tiles wrap round-robin over the workgroups on the tall
    shapes; down runs its four tokens in two passes)."""
    name, k, n = shape
    item = synth.DENSE_STACK_SHAPES.index(shape)
    say(f"dense stack every row {name} k={k} n={n}")
    w, s, planes, meta, pl = make_rtn(n, k, 2, synth.W_STACK, item)
    x1 = synth.activations(1, k, workload=synth.W_STACK, item=1)
    x4 = synth.activations(4, k, workload=synth.W_STACK, item=4)
    y1 = L.linear_forward(pl, to_dev(x1, dev)).cpu().numpy().astype(np.float64)
    y4 = L.linear_forward(pl, to_dev(x4, dev)).cpu().numpy().astype(np.float64)
    codes = L.unpack_codes(pl).cpu().numpy()
    want, q = P.rtn_all_rows(n, k, 2, synth.W_STACK, item, np.concatenate([x1, x4]))
    assert np.array_equal(codes, q), f"{int((codes != q).sum())} code mismatches"
    e1, e4 = O.rel_l2(y1, want[:1]), O.rel_l2(y4, want[1:])
    say(f"  rel_l2 M=1 {e1:.3e}  M=4 {e4:.3e}  code mismatches 0 of {q.size}")
    assert e1 < TOL and e4 < TOL
    for t in range(4):   # every token on its own, not only the block
        assert O.rel_l2(y4[t], want[1 + t]) < TOL


def test_single_linear_codes_full(L, dev):
    """The 4096 x 4096 2-bit single linear: every code read back by the GPU
    decoder equals the oracle's code."""
    n = k = 4096
    w, s, planes, meta, pl = make_rtn(n, k, 2, synth.W_SINGLE, 0)
    codes = L.unpack_codes(pl).cpu().numpy()
    _, q = P.rtn_all_rows(n, k, 2, synth.W_SINGLE, 0)
    assert np.array_equal(codes, q)
    say(f"single linear codes: mismatches 0 of {q.size}")


@pytest.mark.parametrize("swap", [False, True], ids=["gu2_dn3", "gu3_dn2"])
def test_ffn_sweep_codes_full(L, dev, swap):
    """Both FFN-sweep matrices (5120 -> 17408, 17408 -> 5120) at both width
    assignments: every code."""
    cfg = synth.FFN_SWEEP
    b_gu, b_dn = (cfg["bits_gu"], cfg["bits_dn"]) if not swap else (cfg["bits_dn"], cfg["bits_gu"])
    for (k, n, bits, item) in [(cfg["K_gu"], cfg["N_gu"], b_gu, 1), (cfg["N_gu"], cfg["K_gu"], b_dn, 2)]:
        say(f"ffn codes k={k} n={n} bits={bits}")
        w, s, planes, meta, pl = make_rtn(n, k, bits, synth.W_FFN, item)
        codes = L.unpack_codes(pl).cpu().numpy()
        del w, planes, meta, pl
        _, q = P.rtn_all_rows(n, k, bits, synth.W_FFN, item)
        assert np.array_equal(codes, q), f"{int((codes != q).sum())} code mismatches"
        say(f"  codes: mismatches 0 of {q.size}")


# ---------------------------------------------------------------- product-VQ, every row

def test_pvq_linear_every_row_m1(L, dev):
    """4096 -> 14336 product-VQ at one token, every output. The oracle decodes
    the packed indices of every row; the indices themselves equal the oracle's
    own nearest-entry search on 512 sampled rows (the search is the slow part:
    256 squared distances per half) and are read back by the GPU in full."""
    cfg = synth.PVQ_LINEAR
    n, k = cfg["N"], cfg["K"]
    say(f"pvq every row n={n} k={k}")
    w, s, cb, idx, sc, pl = make_pvq(n, k, synth.W_PVQ, 0)
    x = synth.activations(1, k, workload=synth.W_PVQ, item=1)
    y = L.linear_forward(pl, to_dev(x, dev)).cpu().numpy().astype(np.float64)
    got_idx = L.unpack_codes(pl).cpu().numpy()
    assert np.array_equal(got_idx, idx.reshape(n, k // 4))
    say(f"  indices read back: mismatches 0 of {got_idx.size}")
    rows = sample_rows(n, 512, seed=5)
    oi, osc = O.pack_pvq(w[rows], s, cb)
    assert np.array_equal(idx.reshape(n, k // 4)[rows], oi)
    assert np.array_equal(sc.view(np.uint16)[rows], osc)
    want = O.linear_pvq(x, idx.reshape(n, k // 4), sc.view(np.uint16), cb, s)
    e = O.rel_l2(y, want)
    say(f"  rel_l2 {e:.3e}")
    assert e < TOL


# ---------------------------------------------------------------- MoE block, every token

def test_moe_block_every_token(L, dev):
    """256 experts, hidden 2048, ffn 1024, top-8, 32 tokens, widths drawn
    2/3/4: every token against the oracle (each routed expert's FFN from the
    oracle's own packing)."""
    cfg = synth.MOE_BLOCK
    E, hidden, ffn, top_k, m = cfg["E"], cfg["hidden"], cfg["ffn"], cfg["top_k"], cfg["M"]
    say("moe every token")
    bits = synth.expert_bits(E, workload=synth.W_MOE)
    sh = synth.signs(hidden, workload=synth.W_MOE, item=1)
    sf = synth.signs(ffn, workload=synth.W_MOE, item=2)
    w_gu = lambda e: synth.weights(2 * ffn, hidden, workload=synth.W_MOE, item=1000 + e)   # noqa: E731
    w_dn = lambda e: synth.weights(hidden, ffn, workload=synth.W_MOE, item=5000 + e)       # noqa: E731
    packed = L.pack_moe_host(w_gu, w_dn, bits, sh, sf)
    moe = L.moe_from_host(packed, bits, sh, sf, hidden, ffn, top_k)
    x = synth.activations(m, hidden, workload=synth.W_MOE)
    lg = synth.logits(m, E, workload=synth.W_MOE)
    y = L.moe_forward(moe, to_dev(x, dev), to_dev(lg, dev)).cpu().numpy().astype(np.float64)
    want = P.moe_all_tokens(x, lg, top_k, bits, hidden, ffn, synth.W_MOE)
    e = O.rel_l2(y, want)
    say(f"  rel_l2 {e:.3e} over {m} tokens")
    assert e < TOL
    for t in range(m):
        assert O.rel_l2(y[t], want[t]) < TOL, t

    # codes read back from the packed block: one expert of each width, both matrices
    for b in (2, 3, 4):
        ex = int(np.nonzero(bits == b)[0][0])
        for (kk, nn, poff, moff, signs, wfn) in [
                (hidden, 2 * ffn, packed["gu_plane_off"][ex], packed["gu_meta_off"][ex], sh, w_gu),
                (ffn, hidden, packed["dn_plane_off"][ex], packed["dn_meta_off"][ex], sf, w_dn)]:
            pb, mb = L.packed_bytes(kk, nn, b)
            planes_t, meta_t = moe.tensors[5], moe.tensors[6]
            view = L.PackedLinear(kk, nn, b, L.FMT_RTN_PLANES, planes_t[int(poff):int(poff) + pb],
                                  meta_t[int(moff):int(moff) + mb], to_dev(signs, dev))
            codes = L.unpack_codes(view).cpu().numpy()
            _, _, q = O.pack_rtn(wfn(ex), b, signs)
            assert np.array_equal(codes, q), (ex, b, kk, nn)
            say(f"  expert {ex} ({b}-bit) {kk}->{nn} codes: mismatches 0 of {q.size}")


# ---------------------------------------------------------------- matrix-core GEMV vs the fp16 GEMM

@pytest.mark.parametrize("n,k", [(4096, 4096), (4096, 14336)])
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_matrix_core_gemv_error_against_fp16_gemm(L, dev, n, k, m):
    """The matrix-core GEMV contracts each rotated activation as three e4m3
    pieces; its error against the oracle stays within that of the MFMA GEMM
    (fp16 activations, fp16-rounded decoded weights) on the same inputs. The
    GEMV is forced: at three or four tokens on 14336-long rows it runs the
    tokens in two passes, where the AUTO path takes the GEMM."""
    say(f"gemv-vs-gemm error n={n} k={k} m={m}")
    w, s, planes, meta, pl = make_rtn(n, k, 2, 21, n + k)
    x = synth.activations(m, k, workload=21, item=m)
    xd = to_dev(x, dev)
    a = L.linear_forward(pl, xd, path=L.PATH_GEMV).cpu().numpy().astype(np.float64)
    b = L.linear_forward(pl, xd, path=L.PATH_GEMM).cpu().numpy().astype(np.float64)
    rows = sample_rows(n, 256, seed=m)
    want = oracle_rtn_rows(w, s, 2, x, rows)
    ea, eb = O.rel_l2(a[:, rows], want), O.rel_l2(b[:, rows], want)
    say(f"  gemv {ea:.3e}  gemm {eb:.3e}")
    assert ea < TOL and eb < TOL
    assert ea <= 1.5 * eb


@pytest.mark.parametrize("m", [2, 4])
def test_rtn_tokens_of_very_different_size(L, dev, m):
    """Each token's groups carry their own power-of-two piece scale in the
    matrix-core GEMV; tokens 10^6 apart in size would expose a scale or a
    group sum applied to the wrong token."""
    n, k = 300, 2048
    w, s, planes, meta, pl = make_rtn(n, k, 3, 22, m)
    x = synth.activations(m, k, workload=22, item=m).astype(np.float64)
    x *= (10.0 ** np.array([3, -3, 1, -1][:m]))[:, None]
    x = x.astype(np.float16)
    y = L.linear_forward(pl, to_dev(x, dev)).cpu().numpy().astype(np.float64)
    want = oracle_rtn_rows(w, s, 3, x)
    for t in range(m):
        assert O.rel_l2(y[t], want[t]) < TOL, t


@pytest.mark.parametrize("n,k,bits,m", [(8200, 4096, 2, 1), (5000, 2048, 3, 2), (16393, 1024, 4, 1)])
def test_matrix_core_gemv_wrapped_tiles_every_row(L, dev, n, k, bits, m):
    """More row tiles than workgroups (each workgroup owns several tiles dealt
    round-robin, with a ragged last tile): every output row."""
    say(f"gemv wrapped tiles n={n} k={k} bits={bits} m={m}")
    w, s, planes, meta, pl = make_rtn(n, k, bits, 23, n)
    x = synth.activations(m, k, workload=23, item=m)
    y = L.linear_forward(pl, to_dev(x, dev)).cpu().numpy().astype(np.float64)
    want = oracle_rtn_rows(w, s, bits, x)
    e = O.rel_l2(y, want)
    say(f"  rel_l2 {e:.3e}")
    assert e < TOL


# ---------------------------------------------------------------- split rotation launches

@pytest.mark.parametrize("m", [7, 40])
def test_gemm_rotation_in_several_launches(L, dev, m):
    """The GEMM's rotation split over launches (as past 1 GiB of activations),
    forced at three tokens per launch: identical bits to the one-launch call
    (the first launch alone clears the split-K counters), and the oracle's
    result."""
    n, k = 256, 4096
    w, s, planes, meta, pl = make_rtn(n, k, 2, 24, m)
    x = to_dev(synth.activations(m, k, workload=24, item=m), dev)
    a = L.linear_forward(pl, x, path=L.PATH_GEMM).cpu().numpy()
    b = L.linear_forward(pl, x, path=L.PATH_GEMM | L.PATH_SPLIT_ROTATION).cpu().numpy()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    e = O.rel_l2(b.astype(np.float64), oracle_rtn_rows(w, s, 2, x.cpu().numpy()))
    say(f"split rotation m={m} rel_l2 {e:.3e}")
    assert e < TOL
