"""ctypes binding of liblbq.so (include/lbq.h).

Argument marshalling only: torch tensors give device pointers and the current
HIP stream; every step of the computation runs in the library's kernels (or,
for ``pack``, in its host packer). There is no fallback: if the library is not
built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# LBQ_LIBRARY may name another build of the same library (the sanitizer build)
LIB_PATH = os.environ.get("LBQ_LIBRARY") or os.path.join(_HERE, "liblbq.so")

FMT_RTN_PLANES = 0
FMT_PVQ_4x8 = 1
PATH_AUTO, PATH_GEMV, PATH_GEMM, PATH_GEMM_MX = 0, 1, 2, 3
PATH_SPLIT_ROTATION = 0x100   # test flag: the GEMM's rotation in launches of <= 3 tokens

STATUS = {
    0: "LBQ_OK", -1: "LBQ_ERR_NULL", -2: "LBQ_ERR_SHAPE", -3: "LBQ_ERR_BITS", -4: "LBQ_ERR_ALIGN",
    -5: "LBQ_ERR_WORKSPACE", -6: "LBQ_ERR_RANGE", -7: "LBQ_ERR_HIP", -8: "LBQ_ERR_FORMAT",
}

# Every symbol include/lbq.h declares.
EXPORTS = [
    "lbq_status_string", "lbq_packed_bytes", "lbq_pack", "lbq_linear_workspace", "lbq_linear_forward",
    "lbq_linear_forward_path", "lbq_linear_forward_timed", "lbq_moe_workspace", "lbq_moe_forward", "lbq_moe_route", "lbq_unpack_codes",
    "lbq_rotate", "lbq_linear_forward_noalloc", "lbq_stream_read", "lbq_gptq_factor",
    "lbq_pack_gptq", "lbq_moe_forward_path", "lbq_split_nibbles", "lbq_readout_workspace", "lbq_readout_screened",
]


class LbqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


class Weight(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int32), ("N", ctypes.c_int32), ("bits", ctypes.c_int32), ("format", ctypes.c_int32),
                ("planes", ctypes.c_void_p), ("meta", ctypes.c_void_p), ("codebook", ctypes.c_void_p),
                ("signs", ctypes.c_void_p)]


class Moe(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("hidden", ctypes.c_int32), ("ffn", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("bits", ctypes.c_void_p), ("gu_plane_off", ctypes.c_void_p), ("gu_meta_off", ctypes.c_void_p),
                ("dn_plane_off", ctypes.c_void_p), ("dn_meta_off", ctypes.c_void_p), ("planes", ctypes.c_void_p),
                ("meta", ctypes.c_void_p), ("signs_hidden", ctypes.c_void_p), ("signs_ffn", ctypes.c_void_p)]


class Readout(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int32), ("N", ctypes.c_int32), ("hi_planes", ctypes.c_void_p),
                ("lo_planes", ctypes.c_void_p), ("hi_meta", ctypes.c_void_p), ("meta", ctypes.c_void_p),
                ("signs", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load liblbq.so from this package directory; raises if it is not built."""
    global _lib
    if _lib is None:
        # torch ships its own HIP runtime under the same soname as /opt/rocm's;
        # loading torch first makes the library bind to that one copy, so
        # torch's streams and allocations are valid handles for our launches.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run bit_weight_only_amd.build.build() first")
        L = ctypes.CDLL(LIB_PATH)
        c_i32, c_vp, c_sz = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
        p_sz = ctypes.POINTER(ctypes.c_size_t)
        L.lbq_status_string.argtypes = [c_i32]
        L.lbq_status_string.restype = ctypes.c_char_p
        L.lbq_packed_bytes.argtypes = [c_i32, c_i32, c_i32, c_i32, p_sz, p_sz]
        L.lbq_pack.argtypes = [c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]
        L.lbq_linear_workspace.argtypes = [ctypes.POINTER(Weight), c_i32, p_sz]
        L.lbq_linear_forward.argtypes = [ctypes.POINTER(Weight), c_vp, c_i32, c_vp, c_vp, c_sz, c_vp]
        L.lbq_linear_forward_path.argtypes = [ctypes.POINTER(Weight), c_vp, c_i32, c_vp, c_vp, c_sz, c_i32, c_vp]
        L.lbq_linear_forward_timed.argtypes = [ctypes.POINTER(Weight), c_vp, c_i32, c_vp, c_vp, c_sz, c_vp, c_vp, c_vp]
        L.lbq_moe_workspace.argtypes = [ctypes.POINTER(Moe), c_i32, p_sz]
        L.lbq_moe_forward.argtypes = [ctypes.POINTER(Moe), c_vp, c_vp, c_i32, c_vp, c_vp, c_sz, c_vp]
        L.lbq_moe_forward_path.argtypes = [ctypes.POINTER(Moe), c_vp, c_vp, c_i32, c_vp, c_vp, c_sz, c_i32, c_vp]
        L.lbq_moe_route.argtypes = [c_vp, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]
        L.lbq_unpack_codes.argtypes = [ctypes.POINTER(Weight), c_vp, c_vp]
        L.lbq_rotate.argtypes = [c_vp, c_i32, c_i32, c_vp, c_vp, c_vp]
        L.lbq_linear_forward_noalloc.argtypes = [ctypes.POINTER(Weight), c_vp, c_i32, c_vp, c_vp]
        L.lbq_stream_read.argtypes = [c_vp, c_sz, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]
        L.lbq_gptq_factor.argtypes = [c_vp, c_i32, c_vp, ctypes.c_double, c_vp]
        L.lbq_pack_gptq.argtypes = [c_vp, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]
        L.lbq_split_nibbles.argtypes = [c_vp, c_vp, c_i32, c_i32, c_vp, c_vp, c_vp]
        L.lbq_readout_workspace.argtypes = [ctypes.POINTER(Readout), c_i32, c_i32, p_sz]
        L.lbq_readout_screened.argtypes = [ctypes.POINTER(Readout), c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_sz,
                                           c_vp]
        for name in EXPORTS:
            if name != "lbq_status_string":
                getattr(L, name).restype = c_i32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().lbq_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise LbqError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


# ------------------------------------------------------------------ host packing

def packed_bytes(K: int, N: int, bits: int, fmt: int = FMT_RTN_PLANES):
    pb, mb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().lbq_packed_bytes(K, N, bits, fmt, ctypes.byref(pb), ctypes.byref(mb)), "lbq_packed_bytes")
    return pb.value, mb.value


def pack(W: np.ndarray, bits: int, signs: np.ndarray, fmt: int = FMT_RTN_PLANES, codebook: np.ndarray | None = None):
    """Pack fp32 W [N][K] on the host. Returns (planes, meta) as uint8 numpy arrays."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    signs = np.ascontiguousarray(signs, dtype=np.int8)
    pb, mb = packed_bytes(K, N, bits, fmt)
    planes = np.empty(pb, dtype=np.uint8)
    meta = np.empty(mb, dtype=np.uint8)
    cb = None if codebook is None else np.ascontiguousarray(codebook, dtype=np.uint8)
    st = lib().lbq_pack(W.ctypes.data, K, N, bits, fmt, signs.ctypes.data,
                        None if cb is None else cb.ctypes.data, planes.ctypes.data, meta.ctypes.data)
    _check(st, "lbq_pack")
    return planes, meta


def gptq_factor(H: np.ndarray, signs: np.ndarray, damp: float = 0.01) -> np.ndarray:
    """lbq_gptq_factor: U [K][K] float64 from a host Hessian H [K][K] (original basis)."""
    H = np.ascontiguousarray(H, dtype=np.float64)
    K = H.shape[0]
    signs = np.ascontiguousarray(signs, dtype=np.int8)
    U = np.empty((K, K), dtype=np.float64)
    _check(lib().lbq_gptq_factor(H.ctypes.data, K, signs.ctypes.data, float(damp), U.ctypes.data), "lbq_gptq_factor")
    return U


def pack_gptq(W: np.ndarray, bits: int, signs: np.ndarray, U: np.ndarray):
    """lbq_pack_gptq: (planes, meta) uint8 arrays in the RTN bit-plane format."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    signs = np.ascontiguousarray(signs, dtype=np.int8)
    U = np.ascontiguousarray(U, dtype=np.float64)
    pb, mb = packed_bytes(K, N, bits, FMT_RTN_PLANES)
    planes = np.empty(pb, dtype=np.uint8)
    meta = np.empty(mb, dtype=np.uint8)
    _check(lib().lbq_pack_gptq(W.ctypes.data, K, N, bits, signs.ctypes.data, U.ctypes.data, planes.ctypes.data,
                               meta.ctypes.data), "lbq_pack_gptq")
    return planes, meta


# ------------------------------------------------------------------ device side

class PackedLinear:
    """Device-resident packed weight (caller-owned torch tensors) and its lbq_weight view."""

    def __init__(self, K, N, bits, fmt, planes, meta, signs, codebook=None):
        self.K, self.N, self.bits, self.fmt = int(K), int(N), int(bits), int(fmt)
        self.planes, self.meta, self.signs, self.codebook = planes, meta, signs, codebook
        self._w = Weight(self.K, self.N, self.bits, self.fmt, planes.data_ptr(), meta.data_ptr(),
                         0 if codebook is None else codebook.data_ptr(), signs.data_ptr())

    @classmethod
    def from_host(cls, planes: np.ndarray, meta: np.ndarray, signs: np.ndarray, K: int, N: int, bits: int,
                  fmt: int = FMT_RTN_PLANES, codebook: np.ndarray | None = None, device="cuda"):
        import torch

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1)).to(device)

        return cls(K, N, bits, fmt, up(planes), up(meta), torch.from_numpy(np.ascontiguousarray(signs, np.int8)).to(device),
                   None if codebook is None else up(codebook))

    @property
    def struct(self) -> Weight:
        return self._w

    def workspace_bytes(self, M: int) -> int:
        b = ctypes.c_size_t()
        _check(lib().lbq_linear_workspace(ctypes.byref(self._w), int(M), ctypes.byref(b)), "lbq_linear_workspace")
        return b.value


def linear_forward(w: PackedLinear, x, y=None, ws=None, path: int = PATH_AUTO, stream=None):
    """y[M][N] = x[M][K] W_hat^T on the GPU (fp16 in, fp16 out)."""
    import torch

    M = int(x.shape[0])
    if y is None:
        y = torch.empty((M, w.N), dtype=torch.float16, device=x.device)
    if ws is None:
        ws = torch.empty(max(1, w.workspace_bytes(M)), dtype=torch.uint8, device=x.device)
    st = lib().lbq_linear_forward_path(ctypes.byref(w.struct), _ptr(x), M, _ptr(y), _ptr(ws), ws.numel(), int(path),
                                       _stream(stream))
    _check(st, "lbq_linear_forward")
    return y


def linear_forward_noalloc(w: PackedLinear, x, y=None, stream=None):
    """lbq_linear_forward_noalloc: y = x W_hat^T with the library's static device scratch (no workspace)."""
    import torch

    M = int(x.shape[0])
    if y is None:
        y = torch.empty((M, w.N), dtype=torch.float16, device=x.device)
    _check(lib().lbq_linear_forward_noalloc(ctypes.byref(w.struct), _ptr(x), M, _ptr(y), _stream(stream)),
           "lbq_linear_forward_noalloc")
    return y


def rotate(x, signs, out=None, stream=None):
    import torch

    M, K = int(x.shape[0]), int(x.shape[1])
    if out is None:
        out = torch.empty_like(x)
    _check(lib().lbq_rotate(_ptr(x), M, K, _ptr(signs), _ptr(out), _stream(stream)), "lbq_rotate")
    return out


def unpack_codes(w: PackedLinear, stream=None):
    import torch

    # RTN: codes [N][K]; product-VQ: indices [stages * N][K/4] (stage-major)
    n = w.N * w.K if w.fmt == FMT_RTN_PLANES else (w.bits // 2) * w.N * (w.K // 4)
    codes = torch.empty(n, dtype=torch.uint8, device=w.planes.device)
    _check(lib().lbq_unpack_codes(ctypes.byref(w.struct), _ptr(codes), _stream(stream)), "lbq_unpack_codes")
    return codes.view(w.N, -1) if w.fmt == FMT_RTN_PLANES else codes.view(-1, w.K // 4)


# ------------------------------------------------------------------ screened readout

def split_nibbles(planes8: np.ndarray, meta8: np.ndarray, K: int, N: int):
    """lbq_split_nibbles on the host: (hi_planes, lo_planes, hi_meta) as uint8 arrays."""
    planes8 = np.ascontiguousarray(planes8).view(np.uint8)
    meta8 = np.ascontiguousarray(meta8).view(np.uint8)
    G = K // 128
    hi = np.empty(N * G * 64, np.uint8)
    lo = np.empty(N * G * 64, np.uint8)
    hm = np.empty(N * G * 4, np.uint8)
    _check(lib().lbq_split_nibbles(planes8.ctypes.data, meta8.ctypes.data, K, N, hi.ctypes.data, lo.ctypes.data,
                                   hm.ctypes.data), "lbq_split_nibbles")
    return hi, lo, hm


class PackedReadout:
    """Device-resident nibble-split readout weight and its lbq_readout view."""

    def __init__(self, K, N, hi_planes, lo_planes, hi_meta, meta, signs):
        self.K, self.N = int(K), int(N)
        self.hi_planes, self.lo_planes, self.hi_meta, self.meta, self.signs = hi_planes, lo_planes, hi_meta, meta, signs
        self._r = Readout(self.K, self.N, hi_planes.data_ptr(), lo_planes.data_ptr(), hi_meta.data_ptr(),
                          meta.data_ptr(), signs.data_ptr())

    @classmethod
    def from_host(cls, planes8: np.ndarray, meta8: np.ndarray, signs: np.ndarray, K: int, N: int, device="cuda"):
        import torch

        hi, lo, hm = split_nibbles(planes8, meta8, K, N)

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1)).to(device)

        return cls(K, N, up(hi), up(lo), up(hm), up(meta8), torch.from_numpy(np.ascontiguousarray(signs, np.int8)).to(device))

    @property
    def struct(self) -> Readout:
        return self._r

    def workspace_bytes(self, M: int, cand: int) -> int:
        b = ctypes.c_size_t()
        _check(lib().lbq_readout_workspace(ctypes.byref(self._r), int(M), int(cand), ctypes.byref(b)),
               "lbq_readout_workspace")
        return b.value


def readout_screened(r: PackedReadout, x, cand: int, ws=None, stream=None):
    """lbq_readout_screened: (coarse fp16 [M][N], ids int32 [M][cand], exact logits fp32 [M][cand])."""
    import torch

    M = int(x.shape[0])
    coarse = torch.empty((M, r.N), dtype=torch.float16, device=x.device)
    ids = torch.empty((M, cand), dtype=torch.int32, device=x.device)
    logits = torch.empty((M, cand), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = torch.empty(max(1, r.workspace_bytes(M, cand)), dtype=torch.uint8, device=x.device)
    _check(lib().lbq_readout_screened(ctypes.byref(r.struct), _ptr(x), M, int(cand), _ptr(coarse), _ptr(ids),
                                      _ptr(logits), _ptr(ws), ws.numel(), _stream(stream)), "lbq_readout_screened")
    return coarse, ids, logits


# ------------------------------------------------------------------ MoE

class PackedMoe:
    """Device-resident routed-expert block: all experts' planes and meta in two
    byte buffers with per-expert offsets (see lbq_moe in include/lbq.h)."""

    def __init__(self, E, hidden, ffn, top_k, bits, gu_plane_off, gu_meta_off, dn_plane_off, dn_meta_off, planes, meta,
                 signs_hidden, signs_ffn):
        self.E, self.hidden, self.ffn, self.top_k = int(E), int(hidden), int(ffn), int(top_k)
        self.tensors = (bits, gu_plane_off, gu_meta_off, dn_plane_off, dn_meta_off, planes, meta, signs_hidden,
                        signs_ffn)
        self._m = Moe(self.E, self.hidden, self.ffn, self.top_k, *[t.data_ptr() for t in self.tensors])

    @property
    def struct(self) -> Moe:
        return self._m

    def workspace_bytes(self, M: int) -> int:
        b = ctypes.c_size_t()
        _check(lib().lbq_moe_workspace(ctypes.byref(self._m), int(M), ctypes.byref(b)), "lbq_moe_workspace")
        return b.value


def moe_forward(m: PackedMoe, x, logits, y=None, ws=None, path: int = PATH_AUTO, stream=None):
    import torch

    M = int(x.shape[0])
    if y is None:
        y = torch.empty((M, m.hidden), dtype=torch.float16, device=x.device)
    if ws is None:
        ws = torch.empty(max(1, m.workspace_bytes(M)), dtype=torch.uint8, device=x.device)
    st = lib().lbq_moe_forward_path(ctypes.byref(m.struct), _ptr(x), _ptr(logits), M, _ptr(y), _ptr(ws), ws.numel(),
                                    int(path), _stream(stream))
    _check(st, "lbq_moe_forward")
    return y


def moe_route(logits, top_k: int, stream=None):
    """Returns (ids, weights, counts, offsets, perm) device tensors."""
    import torch

    M, E = int(logits.shape[0]), int(logits.shape[1])
    dev = logits.device
    ids = torch.empty((M, top_k), dtype=torch.int32, device=dev)
    wts = torch.empty((M, top_k), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(1, M * top_k), dtype=torch.int32, device=dev)
    st = lib().lbq_moe_route(_ptr(logits), M, E, int(top_k), _ptr(ids), _ptr(wts), _ptr(counts), _ptr(offsets),
                             _ptr(perm), _stream(stream))
    _check(st, "lbq_moe_route")
    return ids, wts, counts, offsets, perm[:M * top_k]


def pack_moe_host(w_gu, w_dn, bits, signs_hidden, signs_ffn, align: int = 256):
    """Pack E experts on the host into the lbq_moe buffers.

    w_gu(e) -> fp32 [2*ffn][hidden] (gate rows first), w_dn(e) -> fp32 [hidden][ffn];
    bits: uint8 [E]. Returns a dict of numpy arrays: planes, meta (uint8),
    gu_plane_off, gu_meta_off, dn_plane_off, dn_meta_off (uint64 [E]).
    """
    E = len(bits)
    pieces_p, pieces_m = [], []
    offs = {k: np.zeros(E, dtype=np.uint64) for k in ("gu_plane_off", "gu_meta_off", "dn_plane_off", "dn_meta_off")}
    pos_p = pos_m = 0

    def put(lst, arr, pos):
        pad = (-pos) % align
        if pad:
            lst.append(np.zeros(pad, np.uint8))
        start = pos + pad
        lst.append(arr)
        return start, start + arr.size

    for e in range(E):
        b = int(bits[e])
        gp, gm = pack(w_gu(e), b, signs_hidden)
        dp, dm = pack(w_dn(e), b, signs_ffn)
        offs["gu_plane_off"][e], pos_p = put(pieces_p, gp, pos_p)
        offs["dn_plane_off"][e], pos_p = put(pieces_p, dp, pos_p)
        offs["gu_meta_off"][e], pos_m = put(pieces_m, gm, pos_m)
        offs["dn_meta_off"][e], pos_m = put(pieces_m, dm, pos_m)
    out = dict(planes=np.concatenate(pieces_p), meta=np.concatenate(pieces_m))
    out.update(offs)
    return out


def moe_from_host(packed: dict, bits, signs_hidden, signs_ffn, hidden: int, ffn: int, top_k: int, device="cuda"):
    import torch

    def up(a, dt=None):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return t.to(device)

    return PackedMoe(len(bits), hidden, ffn, top_k, up(np.asarray(bits, np.uint8)),
                     up(packed["gu_plane_off"].view(np.int64)), up(packed["gu_meta_off"].view(np.int64)),
                     up(packed["dn_plane_off"].view(np.int64)), up(packed["dn_meta_off"].view(np.int64)),
                     up(packed["planes"]), up(packed["meta"]), up(np.asarray(signs_hidden, np.int8)),
                     up(np.asarray(signs_ffn, np.int8)))
