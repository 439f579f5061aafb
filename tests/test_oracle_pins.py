"""Pins of the CPU oracle against closed forms, textbook routines, brute force
and hand-derived fixtures. None of these checks re-types the oracle's own
formula: each compares it with something computed another way."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.special

import synth
from oracle import lbq_oracle as O


# ---------------------------------------------------------------- Hadamard / rotation

def test_hadamard_orthogonal_closed_form():
    h = O.hadamard(128)
    assert np.array_equal(h @ h.T, 128.0 * np.eye(128))


def test_hadamard_matches_scipy():
    assert np.array_equal(O.hadamard(128), scipy.linalg.hadamard(128).astype(np.float64))


def test_fwht_of_basis_vectors_gives_columns():
    h = scipy.linalg.hadamard(128).astype(np.float64)
    eye = np.eye(128)
    for i in range(128):
        assert np.array_equal(O.fwht_blocks(eye[i]), h[:, i])


def test_fwht_matches_dense_product_exactly_on_integers():
    rng = np.random.default_rng(1)
    h = scipy.linalg.hadamard(128).astype(np.float64)
    v = rng.integers(-1000, 1000, size=(5, 3 * 128)).astype(np.float64)
    got = O.fwht_blocks(v)
    want = np.concatenate([v[:, b * 128:(b + 1) * 128] @ h.T for b in range(3)], axis=1)
    assert np.array_equal(got, want)


def _dense_rotation(signs):
    """blockdiag_j(H_128 diag(s_j)) / sqrt(128) from scipy's Hadamard."""
    k = len(signs)
    h = scipy.linalg.hadamard(128).astype(np.float64) / math.sqrt(128.0)
    r = np.zeros((k, k))
    for b in range(k // 128):
        sl = slice(b * 128, (b + 1) * 128)
        r[sl, sl] = h * np.asarray(signs[sl], dtype=np.float64)[None, :]
    return r


def test_rotation_equals_dense_randomized_hadamard():
    s = synth.signs(384, workload=9)
    r = _dense_rotation(s)
    v = np.random.default_rng(2).standard_normal((4, 384))
    np.testing.assert_allclose(O.rotate(v, s), v @ r.T, rtol=0, atol=1e-13)
    np.testing.assert_allclose(O.inverse_rotate(v, s), v @ r, rtol=0, atol=1e-13)


def test_rotation_is_orthogonal():
    s = synth.signs(256, workload=9, item=1)
    r = O.rotate(np.eye(256), s).T           # columns R e_i
    np.testing.assert_allclose(r @ r.T, np.eye(256), atol=1e-14)
    v = np.random.default_rng(3).standard_normal((3, 256))
    np.testing.assert_allclose(np.linalg.norm(O.rotate(v, s), axis=1), np.linalg.norm(v, axis=1), rtol=1e-14)
    np.testing.assert_allclose(O.inverse_rotate(O.rotate(v, s), s), v, atol=1e-14)


def test_rotated_group_sum_is_scaled_first_signed_input():
    """Sylvester's H_128 has column sums 128, 0, ..., 0, so the sum of one rotated
    128-block is 128 / sqrt(128) * s_0 * x_0: the matrix-core GEMV takes its
    per-group activation sum from this identity instead of a reduction."""
    h = O.hadamard(128)
    np.testing.assert_array_equal(h.sum(axis=0), np.r_[128.0, np.zeros(127)])
    k = 1024
    s = synth.signs(k, workload=9, item=3)
    v = np.random.default_rng(4).standard_normal((3, k))
    got = O.rotate(v, s).reshape(3, k // 128, 128).sum(axis=2)
    want = math.sqrt(128.0) * (s * v).reshape(3, k // 128, 128)[:, :, 0]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_rotated_basis_product_equals_plain_product():
    k, n, m = 512, 7, 3
    s = synth.signs(k, workload=9, item=2)
    w = synth.weights(n, k, workload=9).astype(np.float64)
    x = synth.activations(m, k, workload=9).astype(np.float64)
    y_rot = O.rotate(x, s) @ O.rotate(w, s).T
    y = x @ w.T
    assert O.rel_l2(y_rot, y) < 1e-12


# ---------------------------------------------------------------- fp16 / e4m3

def _all_finite_halves():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = b.view(np.float16).astype(np.float64)
    keep = np.isfinite(v)
    return b[keep], v[keep]


def _nearest_half_bruteforce(x, bits, vals):
    d = np.abs(vals - x)
    best = d.min()
    cand = bits[d == best]
    if len(cand) > 1:           # tie: prefer the even mantissa (bit 0 clear)
        even = [c for c in cand if (int(c) & 1) == 0]
        cand = even if even else cand
        # a result of zero keeps the sign of the input (IEEE rounding preserves sign)
        cand = sorted(cand, key=lambda c: (int(c) >> 15) != (1 if x < 0 else 0))
    return int(cand[0])


def test_fp16_rounding_against_bruteforce():
    bits, vals = _all_finite_halves()
    rng = np.random.default_rng(4)
    xs = list(rng.standard_normal(300) * 0.05) + list(rng.standard_normal(100) * 1e-6)
    # exact midpoints between neighbouring halves, where round-to-even decides
    pos = np.sort(vals[vals > 0])
    mids = ((pos[:-1] + pos[1:]) / 2)[rng.integers(0, len(pos) - 1, 200)]
    xs += list(mids) + list(-mids[:50])
    for x in xs:
        got = int(O.to_fp16(x).view(np.uint16))
        assert got == _nearest_half_bruteforce(x, bits, vals), x


def test_fp16_golden(golden_dir):
    with open(os.path.join(golden_dir, "fp_formats.json")) as f:
        g = json.load(f)
    for c in g["fp16_round"]:
        assert int(O.to_fp16(c["value"]).view(np.uint16)) == c["bits"], c


def test_e4m3_golden_and_torch(golden_dir):
    import torch

    with open(os.path.join(golden_dir, "fp_formats.json")) as f:
        g = json.load(f)
    for c in g["e4m3"]:
        v = O.e4m3_to_float(np.array([c["byte"]], dtype=np.uint8))[0]
        if c["value"] == "nan":
            assert np.isnan(v)
        else:
            assert v == c["value"], c
    allb = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(allb).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_to_float(allb)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


# ---------------------------------------------------------------- RTN codes

@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_rtn_codes_are_nearest_grid_point(bits):
    lvl = 2 ** bits - 1
    s = synth.signs(256, workload=9, item=3)
    w = synth.weights(5, 256, workload=9, item=bits)
    wrot = O.rotate(w.astype(np.float64), s)
    q, s16, z16 = O.rtn_quantize(wrot, bits)
    sc = s16.astype(np.float64)
    z = z16.astype(np.float64)
    bits_h, vals_h = _all_finite_halves()
    for n in range(5):
        for g in range(2):
            blk = wrot[n, g * 128:(g + 1) * 128]
            mn, mx = min(0.0, blk.min()), max(0.0, blk.max())
            assert int(s16[n, g].view(np.uint16)) == _nearest_half_bruteforce((mx - mn) / lvl, bits_h, vals_h)
            assert 0 <= z[n, g] <= lvl and z[n, g] == round(z[n, g])
            grid = (np.arange(lvl + 1) - z[n, g]) * sc[n, g]
            for i in range(128):
                err = np.abs(blk[i] - grid)
                best = err.min()
                winners = np.nonzero(err == best)[0]
                assert q[n, g * 128 + i] in winners


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_codes_are_fixed_point_of_dequantize_then_assign(bits):
    s = synth.signs(512, workload=9, item=4)
    w = synth.weights(16, 512, workload=9, item=10 + bits)
    q, s16, z16 = O.rtn_quantize(O.rotate(w, s), bits)
    what = O.dequantize(q, s16, z16)
    # with the stored (s, z): the codes come back exactly
    sc = np.repeat(s16.astype(np.float64), 128, axis=1)
    z = np.repeat(z16.astype(np.float64), 128, axis=1)
    q2 = np.clip(np.rint(what / sc) + z, 0, 2 ** bits - 1)
    assert np.array_equal(q2, q)
    # full requantization reproduces codes, scale and zero for groups whose codes span 0..L
    q3, s3, z3 = O.rtn_quantize(what, bits)
    qg = q.reshape(16, 4, 128)
    span = (qg.min(-1) == 0) & (qg.max(-1) == 2 ** bits - 1)
    assert span.mean() > 0.5
    q3g = q3.reshape(16, 4, 128)
    assert np.array_equal(q3g[span], qg[span])
    assert np.array_equal(s3[span], s16[span]) and np.array_equal(z3[span], z16[span])


def test_rtn_degenerate_group_and_overflow():
    q, s16, z16 = O.rtn_quantize(np.zeros((1, 128)), 2)
    assert np.all(q == 0) and s16[0, 0] == 1.0 and z16[0, 0] == 0.0
    assert np.all(O.dequantize(q, s16, z16) == 0.0)
    with pytest.raises(O.RangeError):
        O.rtn_quantize(np.full((1, 128), 1e6), 2)
    with pytest.raises(O.RangeError):
        O.pack_rtn(np.full((1, 128), np.nan, dtype=np.float32), 2, np.ones(128, np.int8))


def test_rtn_code_histogram_on_gaussian_groups():
    s = synth.signs(1024, workload=9, item=5)
    w = synth.weights(64, 1024, workload=9, item=20)
    q, _, _ = O.rtn_quantize(O.rotate(w, s), 2)
    h = np.bincount(q.ravel(), minlength=4) / q.size
    assert h.min() > 0.03 and h[1] > h[0] and h[2] > h[3]


def test_rtn_spike_fixtures(golden_dir):
    with open(os.path.join(golden_dir, "rtn_spikes.json")) as f:
        g = json.load(f)
    h = scipy.linalg.hadamard(128).astype(np.float64)
    for c in g["cases"]:
        k = c["K"]
        wv = np.zeros(k)
        for i, a in c["spikes"]:
            wv += a / math.sqrt(128.0) * h[:, i]
        wv[0] += c.get("offset", 0.0) * math.sqrt(128.0)   # the same b in every rotated value
        w = wv.astype(np.float32)[None, :]
        planes, meta, q = O.pack_rtn(w, c["bits"], np.ones(k, np.int8))
        want = np.full(k, c["default_code"], dtype=np.uint8)
        for i, code in c["codes_nonzero"]:
            want[i] = code
        assert np.array_equal(q[0], want), c["name"]
        assert int(meta[0, 0, 0]) == c["scale_bits"] and int(meta[0, 0, 1]) == c["zero_bits"], c["name"]
        assert np.array_equal(planes[0, 0], np.array(c["planes"], dtype=np.uint32)), c["name"]


# ---------------------------------------------------------------- bit-plane layout

@pytest.mark.parametrize("bits,words", [
    (2, [0xAAAAAAAA, 0xCCCCCCCC]),
    (3, [0xAAAAAAAA, 0xCCCCCCCC, 0xF0F0F0F0]),
    (4, [0xAAAAAAAA, 0xCCCCCCCC, 0xF0F0F0F0, 0xFF00FF00]),
])
def test_plane_words_closed_form(bits, words):
    j = np.arange(256)
    q = (j % (2 ** bits)).astype(np.uint8)[None, :]
    if bits == 4:      # codes j mod 16 repeat every 16; word pattern over 32 codes
        pass
    pl = O.pack_planes(q, bits)
    for p in range(bits):
        assert np.all(pl[0, :, p, :] == words[p]), (bits, p)
    zeros = O.pack_planes(np.zeros((1, 128), np.uint8), bits)
    assert np.all(zeros == 0)
    full = O.pack_planes(np.full((1, 128), 2 ** bits - 1, np.uint8), bits)
    assert np.all(full == 0xFFFFFFFF)


def test_plane_words_closed_form_8bit_and_nibble_split():
    """Codes 0..255 over two groups: word w of group g holds codes 128 g + 32 w
    + i, so planes 0..4 follow the bit patterns of i, plane 5 is bit 0 of w,
    plane 6 bit 1 of w, plane 7 the group index (derived by hand). The nibble
    split keeps planes 0..3 (q mod 16) and 4..7 (q div 16)."""
    q = np.arange(256, dtype=np.uint8)[None, :]
    pl = O.pack_planes(q, 8)
    low = [0xAAAAAAAA, 0xCCCCCCCC, 0xF0F0F0F0, 0xFF00FF00, 0xFFFF0000]
    for g in range(2):
        for p in range(5):
            assert np.all(pl[0, g, p, :] == low[p]), (g, p)
        assert list(pl[0, g, 5, :]) == [0, 0xFFFFFFFF, 0, 0xFFFFFFFF]
        assert list(pl[0, g, 6, :]) == [0, 0, 0xFFFFFFFF, 0xFFFFFFFF]
        assert np.all(pl[0, g, 7, :] == (0xFFFFFFFF if g else 0))
    lo, hi = O.split_nibbles(pl)
    assert np.array_equal(O.unpack_planes(lo, 4, 256), q & 15)
    assert np.array_equal(O.unpack_planes(hi, 4, 256), q >> 4)


def test_single_code_lands_in_its_word_and_bit():
    for pos in [0, 31, 32, 77, 127, 128 + 65]:
        q = np.zeros((1, 256), np.uint8)
        q[0, pos] = 5                        # binary 101 -> planes 0 and 2
        pl = O.pack_planes(q, 3)
        g, w, j = pos // 128, (pos % 128) // 32, pos % 32
        expect = np.zeros((2, 3, 4), np.uint32)
        expect[g, 0, w] = 1 << j
        expect[g, 2, w] = 1 << j
        assert np.array_equal(pl[0], expect)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_unpack_inverts_pack(bits):
    q = np.random.default_rng(5).integers(0, 2 ** bits, size=(3, 384)).astype(np.uint8)
    assert np.array_equal(O.unpack_planes(O.pack_planes(q, bits), bits, 384), q)


# ---------------------------------------------------------------- linear

def test_linear_brute_force_loop():
    k, n, m = 128, 3, 2
    s = synth.signs(k, workload=9, item=6)
    w = synth.weights(n, k, workload=9, item=30)
    x = synth.activations(m, k, workload=9, item=30)
    planes, meta, q = O.pack_rtn(w, 2, s)
    y = O.linear_rtn(x, planes, meta, s, 2, n, k)
    # brute force: dense R from scipy, explicit dequantization, explicit loops
    r = _dense_rotation(s)
    sv, zv = O.unpack_meta(meta, n, k)
    wq = np.zeros((n, k))
    for i in range(n):
        for kk in range(k):
            wq[i, kk] = (float(q[i, kk]) - float(zv[i, kk // 128])) * float(sv[i, kk // 128])
    w_hat = wq @ r              # row form of R^T w'
    for a in range(m):
        for i in range(n):
            acc = 0.0
            for kk in range(k):
                acc += float(x[a, kk]) * w_hat[i, kk]
            assert abs(acc - y[a, i]) <= 1e-12 * max(1.0, abs(acc))


def test_quantized_linear_is_close_to_unquantized_at_4_bits():
    k, n = 1024, 64
    s = synth.signs(k, workload=9, item=7)
    w = synth.weights(n, k, workload=9, item=31)
    x = synth.activations(4, k, workload=9, item=31)
    planes, meta, _ = O.pack_rtn(w, 4, s)
    y = O.linear_rtn(x, planes, meta, s, 4, n, k)
    assert O.rel_l2(y, x.astype(np.float64) @ w.astype(np.float64).T) < 0.15


# ---------------------------------------------------------------- router / MoE

def test_quantized_linear_is_close_to_unquantized_at_8_bits():
    """8-bit group codes (the non-expert path's width): a step of about 1/255
    of each group's range leaves a relative output error near 0.006."""
    k, n = 1024, 64
    s = synth.signs(k, workload=9, item=8)
    w = synth.weights(n, k, workload=9, item=8)
    x = synth.activations(3, k, workload=9, item=8)
    planes, meta, _ = O.pack_rtn(w, 8, s)
    y = O.linear_rtn(x, planes, meta, s, 8, n, k)
    assert O.rel_l2(y, x.astype(np.float64) @ w.astype(np.float64).T) < 0.015


def test_route_against_full_sort_and_softmax():
    lg = synth.logits(16, 32, workload=9)
    lg[3, 5] = lg[3, 9] = lg[3, 20] = 3.5          # a three-way tie at the top
    ids, w = O.route(lg, 4)
    for t in range(16):
        order = np.lexsort((np.arange(32), -lg[t].astype(np.float64)))
        assert list(ids[t]) == list(order[:4])
        np.testing.assert_allclose(w[t], scipy.special.softmax(lg[t, order[:4]].astype(np.float64)), rtol=1e-14)
        assert abs(w[t].sum() - 1.0) < 1e-14
    assert list(ids[3, :3]) == [5, 9, 20]


def test_silu_against_expit():
    g = np.linspace(-20, 20, 101)
    np.testing.assert_allclose(O.silu(g), g * scipy.special.expit(g), rtol=1e-14, atol=1e-300)


def _tiny_moe(e=4, h=256, f=128, bits=(2, 3, 4, 2)):
    sh = synth.signs(h, workload=9, item=40)
    sf = synth.signs(f, workload=9, item=41)
    packed = []
    for i in range(e):
        wgu = synth.weights(2 * f, h, workload=9, item=100 + i)
        wdn = synth.weights(h, f, workload=9, item=200 + i)
        b = bits[i % len(bits)]
        pg, mg, _ = O.pack_rtn(wgu, b, sh)
        pd, md, _ = O.pack_rtn(wdn, b, sf)
        packed.append((O.dequant_weight_rtn(pg, mg, sh, b, 2 * f, h), O.dequant_weight_rtn(pd, md, sf, b, h, f)))
    return packed


def test_moe_single_expert_equals_dense_swiglu():
    packed = _tiny_moe(e=1)
    x = synth.activations(3, 256, workload=9, item=42)
    lg = np.zeros((3, 1), np.float32)
    y = O.moe_forward(x, lg, 1, lambda e: packed[e])
    wgu, wdn = packed[0]
    h = x.astype(np.float64) @ wgu.T
    a = h[:, :128] * scipy.special.expit(h[:, :128]) * h[:, 128:]
    np.testing.assert_allclose(y, a @ wdn.T, rtol=1e-12, atol=1e-15)


def test_moe_grouped_equals_per_assignment_and_is_token_equivariant():
    packed = _tiny_moe()
    x = synth.activations(6, 256, workload=9, item=43)
    lg = synth.logits(6, 4, workload=9, item=43)
    y = O.moe_forward(x, lg, 2, lambda e: packed[e])
    y2 = O.moe_forward_per_assignment(x, lg, 2, lambda e: packed[e])
    np.testing.assert_allclose(y, y2, rtol=1e-12, atol=1e-15)
    perm = np.array([4, 0, 5, 2, 1, 3])
    y3 = O.moe_forward(x[perm], lg[perm], 2, lambda e: packed[e])
    np.testing.assert_allclose(y3, y[perm], rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- product-VQ

def test_pvq_encode_brute_force_loop():
    cb = synth.codebook(workload=9)
    c = O.e4m3_to_float(cb).reshape(256, 4)
    s = synth.signs(128, workload=9, item=50)
    w = synth.weights(2, 128, workload=9, item=50)
    wrot = O.rotate(w, s)
    idx, s16 = O.pvq_encode(wrot, cb)
    for n in range(2):
        sc = float(s16[n])
        for i in range(32):
            a = wrot[n, 4 * i:4 * i + 4] / sc
            best, best_j = None, None
            for j in range(256):
                d = 0.0
                for dd in range(4):
                    d += (a[dd] - c[j, dd]) ** 2
                if best is None or d < best:
                    best, best_j = d, j
            assert idx[n, i] == best_j


def test_pvq_row_scale_matches_rms_ratio():
    cb = synth.codebook(workload=9)
    c = O.e4m3_to_float(cb).reshape(-1)
    w = np.random.default_rng(6).standard_normal((8, 512)) * 0.02
    s16 = O.pvq_row_scale(w, c)
    want = np.sqrt(np.mean(w * w, axis=1)) / np.sqrt(np.mean(c * c))
    bits_h, vals_h = _all_finite_halves()
    for n in range(8):      # rounding of the two sums may differ in the last bit: stay within one fp16 step
        near = _nearest_half_bruteforce(want[n], bits_h, vals_h)
        assert abs(int(s16[n].view(np.uint16)) - near) <= 1


def test_pvq_codebook_entries_distinct_and_decode_reencodes():
    cb = synth.codebook(workload=9)
    c = O.e4m3_to_float(cb).reshape(256, 4)
    assert len({tuple(r) for r in c}) == 256
    idx = np.random.default_rng(7).integers(0, 256, size=(3, 64)).astype(np.uint8)
    scale = O.to_fp16(np.array([0.01, 0.02, 0.005])).view(np.uint16)
    what = O.pvq_dequantize(idx, scale, cb)
    sc = scale.view(np.float16).astype(np.float64)
    a = (what / sc[:, None]).reshape(3, 64, 1, 4)
    d = (a - c[None, None]) ** 2
    dist = ((d[..., 0] + d[..., 1]) + d[..., 2]) + d[..., 3]
    assert np.array_equal(np.argmin(dist, axis=-1), idx)


def test_pvq_linear_matches_explicit_gather():
    cb = synth.codebook(workload=9)
    k, n = 256, 5
    s = synth.signs(k, workload=9, item=51)
    w = synth.weights(n, k, workload=9, item=51)
    x = synth.activations(2, k, workload=9, item=51)
    idx, sc = O.pack_pvq(w, s, cb)
    y = O.linear_pvq(x, idx, sc, cb, s)
    c = O.e4m3_to_float(cb).reshape(256, 4)
    r = _dense_rotation(s)
    wq = np.zeros((n, k))
    for i in range(n):
        for kk in range(k):
            wq[i, kk] = float(sc.view(np.float16)[i]) * c[idx[i, kk // 4], kk % 4]
    np.testing.assert_allclose(y, x.astype(np.float64) @ (wq @ r).T, rtol=1e-12, atol=1e-14)
    assert O.rel_l2(y, x.astype(np.float64) @ w.astype(np.float64).T) < 0.6


# ---------------------------------------------------------------- parity metric

def test_rel_l2_hand_values():
    """The parity gate: ||a - b||_2 / ||b||_2 over the whole array, b the
    reference (values worked out by hand; a slip such as dividing by ||b||^2,
    by ||a||, or averaging per row fails one of these)."""
    b = np.array([6.0, 8.0])                    # ||b|| = 10
    a = b + np.array([3.0, 4.0])                # ||a - b|| = 5, ||a|| = 15
    assert O.rel_l2(a, b) == 0.5
    assert O.rel_l2(b, a) == 5.0 / 15.0         # the second argument is the reference
    # whole-array norm, not a mean of per-row ratios: rows (0.1, 1.0) would average 0.55
    ref = np.array([[10.0, 0.0], [0.0, 1.0]])
    got = ref + np.array([[1.0, 0.0], [0.0, 1.0]])
    assert O.rel_l2(got, ref) == np.sqrt(2.0) / np.sqrt(101.0)
    assert O.rel_l2(ref, ref) == 0.0
    # a zero reference has no relative error: the absolute norm is returned
    assert O.rel_l2(np.array([3.0, 4.0]), np.zeros(2)) == 5.0
    assert O.rel_l2(np.zeros(3), np.zeros(3)) == 0.0
    # fp16 inputs are widened exactly before the norms
    assert O.rel_l2(np.array([1.0, 2.0], np.float16), np.array([1.0, 1.0], np.float16)) == 1.0 / np.sqrt(2.0)


# ---------------------------------------------------------------- GPTQ

def _dense_rotation(signs):
    """R = blockdiag(c H_128 diag(s)) built from scipy's Hadamard matrix."""
    k = len(signs)
    h = scipy.linalg.hadamard(128).astype(np.float64) / math.sqrt(128.0)
    r = np.zeros((k, k))
    for b in range(k // 128):
        sl = slice(128 * b, 128 * b + 128)
        r[sl, sl] = h * np.asarray(signs[sl], np.float64)[None, :]
    return r


def _hessian(n_samples, k, item):
    x = synth.calibration(n_samples, k, workload=40, item=item).astype(np.float64)
    return x.T @ x / n_samples


def test_gptq_rotated_hessian_is_r_h_rt_plus_damping():
    k = 256
    s = synth.signs(k, workload=40, item=1)
    h = _hessian(512, k, 1)
    r = _dense_rotation(s)
    want = r @ h @ r.T
    want += 0.01 * np.mean(np.diag(want)) * np.eye(k)
    got = O.gptq_hessian_rotated(h, s)
    assert np.max(np.abs(got - want)) < 1e-12 * np.max(np.abs(want))
    u = O.gptq_factor(h, s)
    assert np.allclose(np.triu(u), u)                            # upper triangular
    assert np.allclose(u.T @ u @ got, np.eye(k), atol=1e-8)      # U^T U = H'^-1


def test_gptq_without_feedback_is_rtn():
    """A Hessian that is diagonal in the rotated basis (H = R^T D R) leaves no
    error to feed forward: the codes, scales and zeros are RTN's."""
    k, n = 256, 16
    s = synth.signs(k, workload=40, item=2)
    r = _dense_rotation(s)
    d = np.exp(np.random.default_rng(3).standard_normal(k))
    h = r.T @ np.diag(d) @ r
    u = O.gptq_factor(h, s)
    w = synth.weights(n, k, workload=40, item=2)
    wrot = O.rotate(w.astype(np.float64), s)
    for bits in (2, 3, 4):
        q, s16, z16 = O.gptq_quantize(wrot, u, bits)
        q0, s0, z0 = O.rtn_quantize(wrot, bits)
        assert np.array_equal(q, q0) and np.array_equal(s16, s0) and np.array_equal(z16, z0), bits


def test_gptq_matches_textbook_obs_updates():
    """The Cholesky form against the optimal-brain-surgeon sequence it is
    derived from: keep the full inverse Hessian of the columns not yet
    quantized; after column j, w_rest -= e_j Hinv[j, rest] with
    e_j = (w_j - q_j) / Hinv[j, j], and Hinv loses row and column j by the
    Schur complement. Same codes (no rounding tie is near in this seeded case)."""
    k, n = 256, 12
    s = synth.signs(k, workload=40, item=4)
    h = _hessian(600, k, 4)
    hr = O.gptq_hessian_rotated(h, s)
    w = synth.weights(n, k, workload=40, item=4)
    wrot = O.rotate(w.astype(np.float64), s)
    for bits in (2, 4):
        q, s16, z16 = O.gptq_quantize(wrot, O.gptq_factor(h, s), bits)
        lvl = 2 ** bits - 1
        ww = wrot.copy()
        hinv = np.linalg.inv(hr)
        q_ref = np.zeros((n, k), np.uint8)
        for j in range(k):
            if j % 128 == 0:   # group range from the current columns, zero included
                grp = ww[:, j:j + 128]
                mn, mx = np.minimum(grp.min(1), 0), np.maximum(grp.max(1), 0)
                sc = ((mx - mn) / lvl).astype(np.float16).astype(np.float64)
                sc[sc == 0] = 1.0
                zz = np.rint(-mn / sc)
            qj = np.clip(np.rint(ww[:, j] / sc) + zz, 0, lvl)
            e = (ww[:, j] - (qj - zz) * sc) / hinv[j, j]
            ww[:, j + 1:] -= np.outer(e, hinv[j, j + 1:])
            hinv = hinv - np.outer(hinv[:, j], hinv[j, :]) / hinv[j, j]
            q_ref[:, j] = qj
        assert np.array_equal(q, q_ref), (bits, int((q != q_ref).sum()))


def test_gptq_lowers_the_layer_output_error():
    """GPTQ's purpose: a smaller proxy loss tr(E H' E^T), E the rotated-basis
    weight error, than RTN on correlated calibration data (the property that
    makes it worth its cost; not a pinned value)."""
    k, n = 512, 64
    s = synth.signs(k, workload=40, item=5)
    h = _hessian(1024, k, 5)
    hr = O.gptq_hessian_rotated(h, s, damp=0.0 + 1e-12)
    u = O.gptq_factor(h, s)
    w = synth.weights(n, k, workload=40, item=5)
    wrot = O.rotate(w.astype(np.float64), s)
    for bits in (2, 3):
        q, s16, z16 = O.gptq_quantize(wrot, u, bits)
        q0, s0, z0 = O.rtn_quantize(wrot, bits)
        e_g = O.dequantize(q, s16, z16) - wrot
        e_r = O.dequantize(q0, s0, z0) - wrot
        loss_g = np.trace(e_g @ hr @ e_g.T)
        loss_r = np.trace(e_r @ hr @ e_r.T)
        assert loss_g < 0.8 * loss_r, (bits, loss_g / loss_r)


def test_e2m1_grid_in_e4m3_and_fp4_codebook(golden_dir):
    """The NVFP4-valued codebook: its e4m3 bytes decode to values of the e2m1
    grid only (hand-derived encodings), its 256 entries are distinct, and the
    product-VQ encoder's brute-force definition holds for it too."""
    with open(os.path.join(golden_dir, "fp_formats.json")) as f:
        g = json.load(f)["e2m1_in_e4m3"]
    vals = O.e4m3_to_float(np.array(g["e4m3_bytes"], np.uint8))
    assert list(vals) == g["values"]
    grid = set(g["values"]) | {-v for v in g["values"]}
    cb = synth.codebook_fp4(workload=4)
    dec = O.e4m3_to_float(cb)
    assert set(np.unique(dec).tolist()) <= grid
    assert len(np.unique(cb.view(np.dtype((np.void, 4))))) == 256
    # encode against the fp4-valued codebook by brute force on a small weight
    s = synth.signs(128, workload=9, item=11)
    w = synth.weights(3, 128, workload=9, item=11)
    idx, sc = O.pack_pvq(w, s, cb)
    wrot = O.rotate(w.astype(np.float64), s)
    scale = sc.view(np.float16).astype(np.float64)
    c = dec.reshape(256, 4)
    for n in range(3):
        for i in range(32):
            a = wrot[n, 4 * i:4 * i + 4] / scale[n]
            d = [(((a[0] - e[0]) ** 2 + (a[1] - e[1]) ** 2) + (a[2] - e[2]) ** 2) + (a[3] - e[3]) ** 2 for e in c]
            assert idx[n, i] == int(np.argmin(d))


# ---------------------------------------------------------------- nibble-split screened readout

def test_nibble_hi_meta_hand_values_and_split_identity():
    """The high-nibble weight's (scale, zero): hand-derived values, and the
    identity s (16 h + 7.5 - z) + s (l - 7.5) = s (q - z) through dequantize
    of the two nibble weights against the 8-bit one (a lost midpoint or a
    wrong factor of 16 fails it)."""
    s = np.array([[0.0099945068359375, 2.0 ** -10, 15.5]], np.float16)
    z = np.array([[37.0, 0.0, 255.0]], np.float16)
    hi = O.nibble_hi_meta(O.pack_meta(s, z)).view(np.float16).astype(np.float64)
    assert hi[0, :, 0].tolist() == [0.15991210937500, 2.0 ** -6, 248.0]
    assert hi[0, :, 1].tolist() == [1.84375, -0.46875, 15.46875]
    rng = np.random.default_rng(5)
    n, k = 6, 384
    q = rng.integers(0, 256, (n, k)).astype(np.uint8)
    s8 = (rng.uniform(1e-4, 1e-2, (n, k // 128))).astype(np.float16)
    z8 = rng.integers(0, 256, (n, k // 128)).astype(np.float16)
    meta = O.pack_meta(s8, z8)
    lo, hi_pl = O.split_nibbles(O.pack_planes(q, 8))
    hs, hz = O.unpack_meta(O.nibble_hi_meta(meta), n, k)
    coarse = O.dequantize(O.unpack_planes(hi_pl, 4, k), hs, hz)
    rest = O.dequantize(O.unpack_planes(lo, 4, k), s8, np.full_like(z8, 7.5))
    assert np.array_equal(coarse + rest, O.dequantize(q, s8, z8))


def test_top_rows_against_library_sort_with_ties():
    rng = np.random.default_rng(9)
    v = rng.integers(-3, 4, (5, 40)).astype(np.float64)   # many ties
    got = O.top_rows(v, 7)
    for t in range(5):
        want = np.lexsort((np.arange(40), -v[t]))[:7]
        assert got[t].tolist() == want.tolist()


def test_screened_readout_exact_on_candidates_and_coarse_bound():
    """Exact logits of the screened rows equal the plain 8-bit readout's; every
    coarse logit is within 7.5 sum_g s_g sum_k |x'_k| of the exact one (the low
    nibble's largest deviation from its midpoint); the 8-bit argmax survives
    the screen on this seeded case."""
    n, k, m, cand = 300, 256, 3, 8
    sg = synth.signs(k, workload=9, item=21)
    w = synth.weights(n, k, workload=9, item=21)
    x = synth.activations(m, k, workload=9, item=21)
    planes, meta, _ = O.pack_rtn(w, 8, sg)
    lo, hi = O.split_nibbles(planes)
    coarse, ids, exact = O.screened_readout(x, hi, lo, meta, sg, n, k, cand)
    full = O.linear_rtn(x, planes, meta, sg, 8, n, k)
    for t in range(m):
        assert np.allclose(exact[t], full[t, ids[t]], rtol=0, atol=1e-12 * np.abs(full).max())
        assert int(np.argmax(full[t])) in ids[t].tolist()
    s8, _ = O.unpack_meta(meta, n, k)
    xr = np.abs(O.rotate(x.astype(np.float64), sg)).reshape(m, k // 128, 128).sum(-1)   # [M][G]
    bound = 7.5 * xr @ s8.astype(np.float64).T                                          # [M][N]
    assert np.all(np.abs(full - coarse) <= bound * (1 + 1e-12))


# ---------------------------------------------------------------- residual product-VQ stages

def test_pvq_one_stage_is_plain_pvq_and_stages_telescope():
    """One stage equals the plain encoder; with three stages every stage's
    indices are the brute-force nearest entries of what the earlier stages
    left (divided by that stage's RMS row scale), and the weight error falls
    stage by stage."""
    cb = synth.codebook(workload=9)
    k, n = 128, 3
    sg = synth.signs(k, workload=9, item=31)
    w = synth.weights(n, k, workload=9, item=31)
    i1, s1 = O.pack_pvq_stages(w, sg, cb, 1)
    pi, ps = O.pack_pvq(w, sg, cb)
    assert np.array_equal(i1[0], pi) and np.array_equal(s1[0], ps)
    idx, sc = O.pack_pvq_stages(w, sg, cb, 3)
    c = O.e4m3_to_float(cb).reshape(256, 4)
    wrot = O.rotate(w.astype(np.float64), sg)
    res = wrot.copy()
    errs = []
    for t in range(3):
        s_t = sc[t].view(np.float16).astype(np.float64)
        want_s = np.sqrt(np.mean(res ** 2, axis=1)) / np.sqrt(np.mean(c ** 2))
        assert np.allclose(s_t, want_s, rtol=2 ** -10)
        for r in range(n):
            for i in range(k // 4):
                a = res[r, 4 * i:4 * i + 4] / s_t[r]
                d = [(((a[0] - e[0]) ** 2 + (a[1] - e[1]) ** 2) + (a[2] - e[2]) ** 2) + (a[3] - e[3]) ** 2 for e in c]
                assert idx[t, r, i] == int(np.argmin(d))
        res = res - (c[idx[t].astype(np.int64)] * s_t[:, None, None]).reshape(n, -1)
        errs.append(np.linalg.norm(res) / np.linalg.norm(wrot))
    assert errs[0] > errs[1] > errs[2]
    assert np.allclose(O.pvq_dequantize_stages(idx, sc, cb) + res, wrot, rtol=0, atol=1e-12)
