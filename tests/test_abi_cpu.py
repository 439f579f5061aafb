"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, the host packer is byte-identical to the oracle's packing,
and every argument error is reported before anything is launched (these run
without a GPU, with fake but aligned device pointers)."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
from oracle import lbq_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from bit_weight_only_amd import lbq
    return lbq


def _header_functions():
    with open(os.path.join(ROOT, "include", "lbq.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lbq_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function(L):
    names = _header_functions()
    assert len(names) >= 11
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(L.EXPORTS) == names


def test_status_strings(L):
    for code in L.STATUS:
        s = L.status_string(code)
        assert isinstance(s, str) and s
    assert L.status_string(0) == "ok"


def test_packed_bytes(L):
    assert L.packed_bytes(4096, 4096, 2) == (4194304, 524288)
    assert L.packed_bytes(4096, 4096, 3) == (6291456, 524288)
    assert L.packed_bytes(4096, 14336, 2, L.FMT_PVQ_4x8) == (14680064, 28672)
    lib = L.lib()
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.lbq_packed_bytes(100, 4, 2, 0, ctypes.byref(a), ctypes.byref(b)) == -2
    assert lib.lbq_packed_bytes(128, 4, 5, 0, ctypes.byref(a), ctypes.byref(b)) == -3
    assert lib.lbq_packed_bytes(128, 4, 3, 1, ctypes.byref(a), ctypes.byref(b)) == -3
    assert lib.lbq_packed_bytes(128, 4, 2, 7, ctypes.byref(a), ctypes.byref(b)) == -8
    assert lib.lbq_packed_bytes(128, 4, 2, 0, None, ctypes.byref(b)) == -1


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("n,k", [(1, 128), (3, 256), (130, 512), (64, 1152)])
def test_host_pack_is_byte_identical_to_oracle(L, bits, n, k):
    w = synth.weights(n, k, workload=8, item=bits * 1000 + n)
    s = synth.signs(k, workload=8, item=k)
    planes, meta = L.pack(w, bits, s)
    op, om, _ = O.pack_rtn(w, bits, s)
    assert np.array_equal(planes, op.view(np.uint8).reshape(-1))
    assert np.array_equal(meta, om.view(np.uint8).reshape(-1))


def test_pack_rejects_rtn_scales_from_128(L):
    """The MFMA GEMM decodes with the fp16 constants -64 s and -16 s z, so the
    packer refuses RTN groups whose scale reaches 128 and keeps everything
    below (weights scaled by 2000 give scales near 80)."""
    s = synth.signs(256, workload=8, item=7)
    w = synth.weights(4, 256, workload=8, item=7)
    for bits in (2, 4):
        _, meta = L.pack(w * 2000.0, bits, s)
        sc = np.frombuffer(meta.tobytes(), dtype=np.float16)[0::2].astype(np.float64)
        assert sc.max() < 128
    _, meta = L.pack(w * 2000.0, 2, s)
    assert np.frombuffer(meta.tobytes(), dtype=np.float16)[0::2].astype(np.float64).max() > 40
    with pytest.raises(L.LbqError) as e:
        L.pack(w * 8000.0, 2, s)
    assert e.value.status == -6


def test_host_pack_full_single_linear(L):
    w = synth.weights(4096, 4096, workload=synth.W_SINGLE)
    s = synth.signs(4096, workload=synth.W_SINGLE)
    planes, meta = L.pack(w, 2, s)
    op, om, _ = O.pack_rtn(w, 2, s)
    assert np.array_equal(planes, op.view(np.uint8).reshape(-1))
    assert np.array_equal(meta, om.view(np.uint8).reshape(-1))


def test_host_pack_sampled_rows_of_large_shapes(L):
    """Full-size weights of the dense stack and the FFN sweep packed by the
    library; oracle packing of sampled rows (rows are independent)."""
    rng = np.random.default_rng(11)
    for (name, k, n), bits, wl in [(synth.DENSE_STACK_SHAPES[3], 2, synth.W_STACK),
                                   (("ffn_down", 17408, 5120), 3, synth.W_FFN)]:
        w = synth.weights(n, k, workload=wl, item=7)
        s = synth.signs(k, workload=wl, item=7)
        planes, meta = L.pack(w, bits, s)
        rows = np.sort(rng.choice(n, 24, replace=False))
        rb = k * bits // 8
        mb = (k // 128) * 4
        op, om, _ = O.pack_rtn(w[rows], bits, s)
        for i, r in enumerate(rows):
            assert np.array_equal(planes[r * rb:(r + 1) * rb], op[i].view(np.uint8).reshape(-1)), (name, r)
            assert np.array_equal(meta[r * mb:(r + 1) * mb], om[i].view(np.uint8).reshape(-1)), (name, r)


def test_host_pack_pvq_is_byte_identical_to_oracle(L):
    cb = synth.codebook(workload=synth.W_PVQ)
    for n, k in [(5, 128), (64, 1024)]:
        w = synth.weights(n, k, workload=8, item=n)
        s = synth.signs(k, workload=8, item=n)
        idx, sc = L.pack(w, 2, s, L.FMT_PVQ_4x8, cb)
        oi, os_ = O.pack_pvq(w, s, cb)
        assert np.array_equal(idx, oi.reshape(-1))
        assert np.array_equal(sc, os_.view(np.uint8).reshape(-1))


def test_host_pack_errors(L):
    s = np.ones(128, np.int8)
    with pytest.raises(L.LbqError) as e:
        L.pack(np.full((2, 128), np.nan, np.float32), 2, s)
    assert e.value.status == -6
    with pytest.raises(L.LbqError) as e:
        L.pack(np.full((2, 128), 1e9, np.float32), 2, s)
    assert e.value.status == -6
    with pytest.raises(L.LbqError) as e:
        L.pack(np.zeros((2, 128), np.float32), 2, np.zeros(128, np.int8))
    assert e.value.status == -6
    with pytest.raises(L.LbqError) as e:
        L.pack(np.zeros((2, 100), np.float32), 2, np.ones(100, np.int8))
    assert e.value.status == -2
    with pytest.raises(L.LbqError) as e:
        L.pack(np.zeros((2, 128), np.float32), 5, s)
    assert e.value.status == -3
    z, sz, _ = O.pack_rtn(np.zeros((1, 128), np.float32), 2, s)
    p, m = L.pack(np.zeros((1, 128), np.float32), 2, s)
    assert np.array_equal(p, z.view(np.uint8).reshape(-1)) and np.array_equal(m, sz.view(np.uint8).reshape(-1))


# ---------------------------------------------------------------- boundary errors, no launch

FAKE = 0x10000          # 16-byte aligned, never dereferenced: every case below fails validation first


def _w(L, K=256, N=64, bits=2, fmt=0, planes=FAKE, meta=FAKE, cb=0, signs=FAKE):
    return L.Weight(K, N, bits, fmt, planes, meta, cb, signs)


def _fwd(L, w, M=1, x=FAKE, y=FAKE, ws=FAKE, ws_bytes=1 << 20, path=0):
    return L.lib().lbq_linear_forward_path(ctypes.byref(w), x, M, y, ws, ws_bytes, path, None)


def test_linear_forward_argument_errors(L):
    assert L.lib().lbq_linear_forward(None, FAKE, 1, FAKE, FAKE, 1 << 20, None) == -1
    assert _fwd(L, _w(L, planes=0)) == -1
    assert _fwd(L, _w(L, signs=0)) == -1
    assert _fwd(L, _w(L, bits=5)) == -3
    assert _fwd(L, _w(L, bits=1)) == -3
    assert _fwd(L, _w(L, fmt=1, cb=FAKE, bits=3)) == -3
    assert _fwd(L, _w(L, fmt=1, cb=0)) == -1
    assert _fwd(L, _w(L, fmt=9)) == -8
    assert _fwd(L, _w(L, K=200)) == -2
    assert _fwd(L, _w(L, K=0)) == -2
    assert _fwd(L, _w(L, N=0)) == -2
    assert _fwd(L, _w(L, planes=FAKE + 4)) == -4
    assert _fwd(L, _w(L), M=-1) == -2
    assert _fwd(L, _w(L), x=0) == -1
    assert _fwd(L, _w(L), x=FAKE + 2) == -4
    assert _fwd(L, _w(L), y=FAKE + 8) == -4
    assert _fwd(L, _w(L), ws_bytes=511) == -5
    assert _fwd(L, _w(L), M=17, path=1) == -2
    assert _fwd(L, _w(L), path=7) == -2
    # M = 0 is a valid no-op (returns before touching any pointer)
    assert _fwd(L, _w(L), M=0, x=0, y=0, ws=0) == 0


def test_workspace_queries(L):
    lib = L.lib()
    b = ctypes.c_size_t()
    w = _w(L, K=4096)
    assert lib.lbq_linear_workspace(ctypes.byref(w), 16, ctypes.byref(b)) == 0
    assert b.value >= 16 * 4096 * 2 and b.value % 256 == 0
    assert lib.lbq_linear_workspace(ctypes.byref(w), -1, ctypes.byref(b)) == -2
    assert lib.lbq_linear_workspace(ctypes.byref(w), 1, None) == -1


def _moe(L, E=256, hidden=2048, ffn=1024, top_k=8, **kw):
    vals = dict(bits=FAKE, gu_plane_off=FAKE, gu_meta_off=FAKE, dn_plane_off=FAKE, dn_meta_off=FAKE, planes=FAKE,
                meta=FAKE, signs_hidden=FAKE, signs_ffn=FAKE)
    vals.update(kw)
    return L.Moe(E, hidden, ffn, top_k, *[vals[k] for k in ("bits", "gu_plane_off", "gu_meta_off", "dn_plane_off",
                                                           "dn_meta_off", "planes", "meta", "signs_hidden",
                                                           "signs_ffn")])


def test_moe_argument_errors(L):
    lib = L.lib()
    b = ctypes.c_size_t()
    m = _moe(L)
    assert lib.lbq_moe_workspace(ctypes.byref(m), 32, ctypes.byref(b)) == 0
    assert b.value >= 32 * 8 * (1024 * 2 + 2048 * 4)

    def fwd(mm, M=32, x=FAKE, lg=FAKE, y=FAKE, ws=FAKE, nb=1 << 26):
        return lib.lbq_moe_forward(ctypes.byref(mm), x, lg, M, y, ws, nb, None)

    assert fwd(_moe(L, bits=0)) == -1
    assert fwd(_moe(L, top_k=0)) == -2
    assert fwd(_moe(L, top_k=300, E=256)) == -2
    assert fwd(_moe(L, top_k=33, E=256)) == -2
    assert fwd(_moe(L, E=2000)) == -2
    assert fwd(_moe(L, hidden=2000)) == -2
    assert fwd(_moe(L, ffn=100)) == -2
    assert fwd(_moe(L, planes=FAKE + 1)) == -4
    assert fwd(m, M=-1) == -2
    assert fwd(m, M=2000) == -2           # 2000 * 8 assignments exceed the limit
    assert fwd(m, lg=0) == -1
    assert fwd(m, nb=1024) == -5
    assert fwd(m, M=0, x=0, lg=0, y=0, ws=0) == 0
    assert lib.lbq_moe_route(FAKE, 4, 8, 9, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -2
    assert lib.lbq_moe_route(FAKE, 4, 8, 2, 0, FAKE, FAKE, FAKE, FAKE, None) == -1


def test_rotate_and_unpack_argument_errors(L):
    lib = L.lib()
    assert lib.lbq_rotate(FAKE, 1, 100, FAKE, FAKE, None) == -2
    assert lib.lbq_rotate(FAKE, -1, 128, FAKE, FAKE, None) == -2
    assert lib.lbq_rotate(0, 1, 128, FAKE, FAKE, None) == -1
    assert lib.lbq_rotate(FAKE + 2, 1, 128, FAKE, FAKE, None) == -4
    assert lib.lbq_rotate(0, 0, 128, 0, 0, None) == 0
    w = _w(L)
    assert lib.lbq_unpack_codes(ctypes.byref(w), 0, None) == -1
    assert lib.lbq_unpack_codes(ctypes.byref(w), FAKE + 1, None) == -4
