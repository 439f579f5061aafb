"""CPU oracle for the low-bit weight-only quantized linear layer.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here. The
library under ``bit_weight_only_amd/`` never imports it, and this module
imports nothing from the library: the two share no code, constants or tables.

Everything is plain NumPy in float64 unless a step fixes another precision
(fp16 scale/zero storage, fp8 e4m3 codebook values). It is written to be read
against the pages, not to be fast.

What the pages fix, and where:

* Weights are quantized with group size 128 "in a Hadamard-rotated basis", at
  mixed 2/3/4-bit widths per routed expert, and the rotation signs are stored
  with the small tensors (LLaDA2.2-mini Orin Nano model card: property table,
  "Routed Experts" row, and the file list that names the rotation signs).
* The rotation is a random Hadamard rotation (Qwen3.8-27B Pingala-8 model
  card, "What this is").
* Low-bit weights stay packed as bit-planes in 32-bit words for the whole run
  (Qwen3-8B 2-bit BPDQ model card, opening paragraph).
* Product-VQ over 8-weight vectors whose codebook values sit on hardware fp8
  grids, decoded inside the matmul (Laguna-S-2.1 gridbook model card, opening
  paragraph).
* Routed experts chosen per token (Laguna-S-2.1 card: 256 routed experts,
  top-k, plus the LLaDA2.2-mini card's routed experts).
* Non-expert linears and the readout keep 8-bit codes, and the readout's codes
  are also stored split into high and low nibble planes for a screened
  readout (LLaDA2.2-mini card: property table, "Non-Expert Path" and
  "Readout & Embeddings" rows, and the file list).

Readings where the pages are silent (each is listed with its reason in the
design notes): Sylvester (natural) Hadamard order; signs applied before the
transform; orthonormal scale 1/sqrt(128); GPTQ-style asymmetric min/max range
that always contains 0, integer zero-point, round-half-even; fp16-rounded scale
used for code assignment; degenerate scale 0 -> 1; gate|up rows concatenated
(gate first); SwiGLU expert activation; softmax over the selected top-k logits
with ties broken toward the lower expert id; PVQ row scale by RMS matching and
nearest-entry search with ties toward the lower index; the screened readout
scores every row by its high nibbles taken at the middle of their 16-code
range, keeps a fixed number of rows per token (ties toward the lower row) and
scores those exactly from both nibbles.
"""
from __future__ import annotations

import numpy as np

GROUP = 128          # quantization group == rotation block (LLaDA2.2-mini card, "Routed Experts": group 128)
C_NORM = np.sqrt(2.0) / 16.0   # 1/sqrt(128): orthonormal Hadamard scale


class RangeError(ValueError):
    """A value cannot be stored in the format (non-finite input, fp16 overflow)."""


# ---------------------------------------------------------------------------
# Hadamard rotation (LLaDA2.2-mini card "Routed Experts"; Pingala-8 card "What this is")
# ---------------------------------------------------------------------------

def hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix: H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    assert h.shape[0] == n, "n must be a power of two"
    return h


def fwht_blocks(v: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform of every 128-block of the last axis.

    Radix-2 butterflies with half-widths 1, 2, 4, ..., 64; each butterfly maps
    (a, b) to (a + b, a - b). In natural order this is H_128 @ block.
    """
    v = np.asarray(v, dtype=np.float64)
    k = v.shape[-1]
    assert k % GROUP == 0
    a = v.reshape(-1, GROUP).copy()
    h = 1
    while h < GROUP:
        a = a.reshape(a.shape[0], GROUP // (2 * h), 2, h)
        lo = a[:, :, 0, :]
        hi = a[:, :, 1, :]
        a = np.stack([lo + hi, lo - hi], axis=2).reshape(-1, GROUP)
        h *= 2
    return a.reshape(v.shape)


def rotate(v: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """R v with R = blockdiag_j(c * H_128 * diag(s_j)), c = 1/sqrt(128).

    Signs multiply first (exact), then the butterflies, then the scale c.
    Applied along the last axis; rows of a weight matrix or tokens of x alike.
    """
    s = np.asarray(signs, dtype=np.float64)
    return fwht_blocks(np.asarray(v, dtype=np.float64) * s) * C_NORM


def inverse_rotate(v: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """R^T v = blockdiag_j(c * diag(s_j) * H_128) v (H is symmetric)."""
    s = np.asarray(signs, dtype=np.float64)
    return (fwht_blocks(np.asarray(v, dtype=np.float64)) * C_NORM) * s


# ---------------------------------------------------------------------------
# fp16 / e4m3 conversions
# ---------------------------------------------------------------------------

def to_fp16(x) -> np.ndarray:
    """Round float64 values to IEEE binary16, nearest-even (NumPy's direct cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def e4m3_to_float(b) -> np.ndarray:
    """Decode fp8 e4m3 (OCP "fn" variant) bytes by the format's definition.

    sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0; exponent 0 is
    subnormal (m/8 * 2^-6); S.1111.111 is NaN; there are no infinities.
    """
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    val = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


# ---------------------------------------------------------------------------
# Group-128 asymmetric round-to-nearest codes (LLaDA2.2-mini card: group-128
# GPTQ codes at 2/3/4 bits in the rotated basis for the routed experts, 8-bit
# codes for the non-expert path and the readout (property table, "Non-Expert
# Path" and "Readout & Embeddings" rows); RTN is the plain quantizer GPTQ's own
# rounding grid is defined by)
# ---------------------------------------------------------------------------

CODE_BITS = (2, 3, 4, 8)

def rtn_quantize(wrot: np.ndarray, bits: int):
    """Codes, fp16 scale and fp16 zero per (row, 128-group) of a rotated weight.

    For each group: mn = min(0, min w'), mx = max(0, max w');
    s = fp16((mx - mn) / L) with L = 2^bits - 1, replaced by 1 when it is 0;
    z = rint(-mn / s) (an integer in [0, L], exact in fp16);
    q = clamp(rint(w' / s) + z, 0, L). rint is round-half-even, and the
    fp16-rounded s is the one used for the codes.
    Returns q (uint8 [N][K]), s16 and z16 (float16 [N][K/128]).
    """
    if bits not in CODE_BITS:
        raise ValueError("bits must be 2, 3, 4 or 8")
    wrot = np.asarray(wrot, dtype=np.float64)
    if not np.all(np.isfinite(wrot)):
        raise RangeError("non-finite weight")
    n, k = wrot.shape
    lvl = float(2 ** bits - 1)
    g = wrot.reshape(n, k // GROUP, GROUP)
    mn = np.minimum(g.min(axis=-1), 0.0)
    mx = np.maximum(g.max(axis=-1), 0.0)
    s16 = to_fp16((mx - mn) / lvl)
    if not np.all(np.isfinite(s16)):
        raise RangeError("scale overflows fp16")
    s16 = np.where(s16 == 0, np.float16(1.0), s16)
    s = s16.astype(np.float64)
    z = np.rint(-mn / s) + 0.0           # + 0.0 turns -0.0 into +0.0
    q = np.clip(np.rint(g / s[..., None]) + z[..., None], 0.0, lvl)
    z16 = to_fp16(z)
    assert np.array_equal(z16.astype(np.float64), z), "zero-point must be exact in fp16"
    return q.reshape(n, k).astype(np.uint8), s16, z16


def group_params(wg: np.ndarray, bits: int):
    """fp16 scale and zero of one column block of groups, the rule rtn_quantize
    uses: mn = min(0, min w'), mx = max(0, max w'), s = fp16((mx - mn) / L)
    (0 -> 1), z = rint(-mn / s). wg: [N][128] float64. Returns (s16, z16)."""
    lvl = float(2 ** bits - 1)
    mn = np.minimum(wg.min(axis=-1), 0.0)
    mx = np.maximum(wg.max(axis=-1), 0.0)
    s16 = to_fp16((mx - mn) / lvl)
    if not np.all(np.isfinite(s16)):
        raise RangeError("scale overflows fp16")
    s16 = np.where(s16 == 0, np.float16(1.0), s16)
    z = np.rint(-mn / s16.astype(np.float64)) + 0.0
    return s16, to_fp16(z)


def dequantize(q: np.ndarray, s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """W'_hat[n, k] = (q[n, k] - z[n, g]) * s[n, g] in float64, g = k // 128."""
    n, k = q.shape
    qg = q.reshape(n, k // GROUP, GROUP).astype(np.float64)
    z = z16.astype(np.float64)[..., None]
    s = s16.astype(np.float64)[..., None]
    return ((qg - z) * s).reshape(n, k)


# ---------------------------------------------------------------------------
# GPTQ in the rotated basis (LLaDA2.2-mini card, property table, "Routed
# Experts" row: group-128 GPTQ in a Hadamard-rotated basis; Qwen3.8-27B
# Pingala-8 card, "What this is": LDLQ rounding behind a random Hadamard
# rotation, the same error feedback). Codes go column by column; each
# column's rounding error, scaled by the inverse Hessian's Cholesky factor, is
# pushed onto the columns not yet quantized. The stored format is the RTN one.
#
# Readings (the pages name the method, not its settings): H is the caller's
# proxy Hessian of the layer input (e.g. X^T X of calibration activations) in
# the original basis; in the rotated basis it is H' = R H R^T. Dampening adds
# 0.01 * mean(diag H') to the diagonal. Columns go in natural order (no
# reordering, so 128-groups stay the rotation blocks). A group's scale and zero
# come from its columns as they stand when its first column is reached (after
# the feedback from earlier groups), by the RTN rule. The feedback is applied
# one column at a time (the unblocked form of the algorithm).
# ---------------------------------------------------------------------------

def gptq_hessian_rotated(h: np.ndarray, signs: np.ndarray, damp: float = 0.01) -> np.ndarray:
    """H' = R H R^T plus damp * mean(diag H') on the diagonal (float64 [K][K])."""
    h = np.asarray(h, dtype=np.float64)
    a = rotate(h, signs)              # row i: R h_i, i.e. H R^T
    hr = rotate(a.T, signs).T         # R (H R^T)
    d = damp * float(np.mean(np.diag(hr)))
    if not d > 0.0:
        raise RangeError("Hessian has no positive diagonal")
    hr = hr + d * np.eye(hr.shape[0])
    return hr


def gptq_factor(h: np.ndarray, signs: np.ndarray, damp: float = 0.01) -> np.ndarray:
    """U: the upper Cholesky factor of H'^-1 (H'^-1 = U^T U), float64 [K][K]."""
    hinv = np.linalg.inv(gptq_hessian_rotated(h, signs, damp))
    hinv = (hinv + hinv.T) / 2.0
    return np.linalg.cholesky(hinv).T


def gptq_quantize(wrot: np.ndarray, u: np.ndarray, bits: int):
    """Codes, fp16 scale and zero of a rotated weight [N][K] by GPTQ with the
    factor u. For column j (group g = j // 128): at the group's first column
    its (s, z) come from the current columns; q = clamp(rint(w_j / s) + z, 0, L);
    e = (w_j - (q - z) s) / u[j, j]; then w_k -= e * u[j, k] for every k > j.
    Returns q (uint8 [N][K]), s16, z16 (float16 [N][K/128])."""
    if bits not in CODE_BITS:
        raise ValueError("bits must be 2, 3, 4 or 8")
    w = np.array(wrot, dtype=np.float64)
    if not np.all(np.isfinite(w)):
        raise RangeError("non-finite weight")
    n, k = w.shape
    lvl = float(2 ** bits - 1)
    q = np.zeros((n, k), dtype=np.uint8)
    s16 = np.zeros((n, k // GROUP), dtype=np.float16)
    z16 = np.zeros((n, k // GROUP), dtype=np.float16)
    s = z = None
    for j in range(k):
        g = j // GROUP
        if j % GROUP == 0:
            s16[:, g], z16[:, g] = group_params(w[:, j:j + GROUP], bits)
            s = s16[:, g].astype(np.float64)
            z = z16[:, g].astype(np.float64)
        qj = np.clip(np.rint(w[:, j] / s) + z, 0.0, lvl)
        err = (w[:, j] - (qj - z) * s) / u[j, j]
        w[:, j + 1:] -= np.outer(err, u[j, j + 1:])
        q[:, j] = qj.astype(np.uint8)
    return q, s16, z16


def pack_gptq(w: np.ndarray, bits: int, signs: np.ndarray, u: np.ndarray):
    """Offline GPTQ packing of one fp32 weight [N][K] with the factor u of
    gptq_factor: rotate, quantize with error feedback, bit-planes. Returns
    (planes, meta, codes) as pack_rtn."""
    w = np.asarray(w)
    if not np.all(np.isfinite(w)):
        raise RangeError("non-finite weight")
    q, s16, z16 = gptq_quantize(rotate(w.astype(np.float64), signs), u, bits)
    return pack_planes(q, bits), pack_meta(s16, z16), q


# ---------------------------------------------------------------------------
# Bit-plane layout (Qwen3-8B BPDQ card, opening paragraph: bit-planes kept
# packed in int32 words)
#
# planes: uint32 [N][K/128][bits][4]; bit j of word w of plane p holds bit p
#         of code q[n, 128*g + 32*w + j].
# meta:   uint16 [N][K/128][2]: IEEE fp16 bit patterns of (scale, zero).
# ---------------------------------------------------------------------------

def pack_planes(q: np.ndarray, bits: int) -> np.ndarray:
    q = np.asarray(q, dtype=np.uint32)
    n, k = q.shape
    qb = q.reshape(n, k // GROUP, 4, 32)
    weights = np.left_shift(np.uint32(1), np.arange(32, dtype=np.uint32))
    planes = np.zeros((n, k // GROUP, bits, 4), dtype=np.uint32)
    for p in range(bits):
        bitp = (qb >> np.uint32(p)) & np.uint32(1)
        planes[:, :, p, :] = (bitp * weights).sum(axis=-1, dtype=np.uint64).astype(np.uint32)
    return planes


def unpack_planes(planes: np.ndarray, bits: int, k: int) -> np.ndarray:
    planes = np.asarray(planes).view(np.uint32)
    n = planes.size // ((k // GROUP) * bits * 4)
    planes = planes.reshape(n, k // GROUP, bits, 4)
    j = np.arange(32, dtype=np.uint32)
    q = np.zeros((n, k // GROUP, 4, 32), dtype=np.uint32)
    for p in range(bits):
        bitp = (planes[:, :, p, :, None] >> j) & np.uint32(1)
        q |= bitp << np.uint32(p)
    return q.reshape(n, k).astype(np.uint8)


def split_nibbles(planes: np.ndarray) -> tuple:
    """The 8-bit codes' planes split into a low-nibble and a high-nibble plane
    set (LLaDA2.2-mini card, file list: the readout's codes also stored as
    high/low nibble planes). planes: uint32 [N][G][8][4]; returns (lo, hi),
    each uint32 [N][G][4][4]: planes 0..3 and 4..7, so q = lo + 16 hi."""
    p = np.asarray(planes).view(np.uint32)
    n = p.shape[0]
    p = p.reshape(n, -1, 8, 4)
    return np.ascontiguousarray(p[:, :, :4, :]), np.ascontiguousarray(p[:, :, 4:, :])


def nibble_hi_meta(meta8: np.ndarray) -> np.ndarray:
    """Scale/zero that make the high-nibble planes a 4-bit weight of their own
    (reading of the LLaDA2.2-mini card's screened readout over the nibble-split
    planes): with q = 16 h + l, the high nibble alone stands for the middle of
    the 16 codes it spans, q ~ 16 h + 7.5, so s (q - z) ~ (16 s) (h - (z - 7.5) / 16).
    meta8: uint16 [N][G][2] fp16 (s, z) of the 8-bit codes; returns the same
    layout holding (16 s, (z - 7.5) / 16), both exact in fp16 for the 8-bit
    packer's ranges (s < 16, integer z in 0..255)."""
    m = np.asarray(meta8).view(np.uint16)
    s = m[..., 0].copy().view(np.float16).astype(np.float64)
    z = m[..., 1].copy().view(np.float16).astype(np.float64)
    s_hi = 16.0 * s
    z_hi = (z - 7.5) / 16.0
    if not (np.all(to_fp16(s_hi).astype(np.float64) == s_hi) and np.all(to_fp16(z_hi).astype(np.float64) == z_hi)):
        raise RangeError("high-nibble scale or zero not exact in fp16")
    return pack_meta(to_fp16(s_hi), to_fp16(z_hi))


def top_rows(values: np.ndarray, cand: int) -> np.ndarray:
    """The `cand` largest entries of each row of values [M][N] (larger first,
    ties to the lower index): int32 [M][cand]."""
    v = np.asarray(values, dtype=np.float64)
    m, n = v.shape
    out = np.empty((m, cand), dtype=np.int32)
    for t in range(m):
        order = sorted(range(n), key=lambda i: (-v[t, i], i))
        out[t] = order[:cand]
    return out


def screened_readout(x16, hi_planes, lo_planes, meta8, signs, n: int, k: int, cand: int):
    """Screened readout over the nibble-split planes of an 8-bit weight.

    1. coarse logits of every row from the high-nibble planes alone, read as
       a 4-bit weight with nibble_hi_meta's scale and zero;
    2. per token, the `cand` rows with the largest coarse logits (top_rows);
    3. the exact logits of those rows from both nibbles, q = lo + 16 hi, with
       the 8-bit (s, z).
    Returns coarse float64 [M][N], ids int32 [M][cand], exact float64 [M][cand]."""
    x = np.asarray(x16)
    coarse = linear_rtn(x, hi_planes, nibble_hi_meta(meta8), signs, 4, n, k)
    ids = top_rows(coarse, cand)
    q = unpack_planes(lo_planes, 4, k).astype(np.uint16) + 16 * unpack_planes(hi_planes, 4, k).astype(np.uint16)
    meta_rows = np.asarray(meta8).view(np.uint16).reshape(n, k // GROUP, 2)
    exact = np.empty(ids.shape, dtype=np.float64)
    for t in range(x.shape[0]):
        rows = ids[t]
        w_hat = dequant_weight_rtn(pack_planes(q[rows], 8), meta_rows[rows], signs, 8, len(rows), k)
        exact[t] = linear(x[t:t + 1], w_hat)[0]
    return coarse, ids, exact


def pack_meta(s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    return np.stack([s16.view(np.uint16), z16.view(np.uint16)], axis=-1)


def unpack_meta(meta: np.ndarray, n: int, k: int):
    m = np.asarray(meta).view(np.uint16).reshape(n, k // GROUP, 2)
    return m[..., 0].copy().view(np.float16), m[..., 1].copy().view(np.float16)


def pack_rtn(w: np.ndarray, bits: int, signs: np.ndarray):
    """Offline packing of one fp32 weight [N][K]: rotate, RTN, bit-planes.

    Returns (planes uint32 [N][K/128][bits][4], meta uint16 [N][K/128][2],
    codes uint8 [N][K]).
    """
    w = np.asarray(w)
    if not np.all(np.isfinite(w)):
        raise RangeError("non-finite weight")
    wrot = rotate(w.astype(np.float64), signs)
    q, s16, z16 = rtn_quantize(wrot, bits)
    return pack_planes(q, bits), pack_meta(s16, z16), q


def dequant_weight_rtn(planes, meta, signs, bits: int, n: int, k: int) -> np.ndarray:
    """W_hat = R^T (dequantized rotated weight): the original-basis weight the
    packed buffers stand for, float64 [N][K]."""
    q = unpack_planes(planes, bits, k)
    s16, z16 = unpack_meta(meta, n, k)
    return inverse_rotate(dequantize(q, s16, z16), signs)


def linear(x16: np.ndarray, w_hat: np.ndarray) -> np.ndarray:
    """y = x W_hat^T in float64 (x taken exactly from fp16)."""
    return np.asarray(x16, dtype=np.float64) @ np.asarray(w_hat, dtype=np.float64).T


def linear_rtn(x16, planes, meta, signs, bits: int, n: int, k: int) -> np.ndarray:
    return linear(x16, dequant_weight_rtn(planes, meta, signs, bits, n, k))


# ---------------------------------------------------------------------------
# Product-VQ, 2 bits per weight (Laguna-S-2.1 gridbook card, opening
# paragraph: product-VQ over 8-weight vectors, codebook values on fp8 grids,
# decoded at matmul time). Each 8-weight vector is two 4-weight halves, each an
# 8-bit index into one shared 256x4 e4m3 codebook; one fp16 scale per row.
#
# idx:   uint8 [N][K/4]; byte i covers weights 4i..4i+3 (byte 2v+h is half h of vector v)
# scale: uint16 [N] fp16 bit patterns
# ---------------------------------------------------------------------------

def pvq_row_scale(wrot: np.ndarray, cb: np.ndarray) -> np.ndarray:
    """s_n = fp16(rms(w'_n) / rms(C)); sums of squares accumulate left to right."""
    wrot = np.asarray(wrot, dtype=np.float64)
    n, k = wrot.shape
    c = cb.reshape(-1)
    sum_c = np.cumsum(c * c)[-1]
    sum_w = np.cumsum(wrot * wrot, axis=1)[:, -1]
    ratio = np.sqrt(sum_w / k) / np.sqrt(sum_c / c.size)
    s16 = to_fp16(ratio)
    if not np.all(np.isfinite(s16)):
        raise RangeError("row scale overflows fp16")
    return np.where(s16 == 0, np.float16(1.0), s16)


def pvq_encode(wrot: np.ndarray, cb_bytes: np.ndarray, rows_per_chunk: int = 256):
    """Nearest codebook entry per 4-weight half, after dividing by the row scale.

    Distance = ((a0-c0)^2 + (a1-c1)^2) + (a2-c2)^2) + (a3-c3)^2 in float64,
    ties to the lower index.
    """
    cb = e4m3_to_float(cb_bytes).reshape(256, 4)
    if not np.all(np.isfinite(cb)):
        raise RangeError("codebook holds NaN")
    wrot = np.asarray(wrot, dtype=np.float64)
    if not np.all(np.isfinite(wrot)):
        raise RangeError("non-finite weight")
    n, k = wrot.shape
    s16 = pvq_row_scale(wrot, cb)
    s = s16.astype(np.float64)
    idx = np.empty((n, k // 4), dtype=np.uint8)
    for r0 in range(0, n, rows_per_chunk):
        r1 = min(n, r0 + rows_per_chunk)
        a = (wrot[r0:r1] / s[r0:r1, None]).reshape(r1 - r0, k // 4, 1, 4)
        d = (a - cb[None, None, :, :]) ** 2
        dist = ((d[..., 0] + d[..., 1]) + d[..., 2]) + d[..., 3]
        idx[r0:r1] = np.argmin(dist, axis=-1).astype(np.uint8)
    return idx, s16


def pack_pvq(w: np.ndarray, signs: np.ndarray, cb_bytes: np.ndarray):
    wrot = rotate(np.asarray(w, dtype=np.float64), signs)
    idx, s16 = pvq_encode(wrot, cb_bytes)
    return idx, s16.view(np.uint16)


def pvq_dequantize(idx: np.ndarray, scale_u16: np.ndarray, cb_bytes: np.ndarray) -> np.ndarray:
    """W'_hat[n, 4i + d] = s_n * C[idx[n, i]][d] (float64, rotated basis)."""
    cb = e4m3_to_float(cb_bytes).reshape(256, 4)
    idx = np.asarray(idx)
    n = idx.shape[0]
    s = np.asarray(scale_u16, dtype=np.uint16).view(np.float16).astype(np.float64)
    return (cb[idx.astype(np.int64)] * s[:, None, None]).reshape(n, -1)


def pack_pvq_stages(w: np.ndarray, signs: np.ndarray, cb_bytes: np.ndarray, stages: int):
    """Residual product-VQ at 2 * stages bits per weight (a reading of the
    Laguna-S-2.1 card's higher-rate FP8-CB rungs: 16 index bits per 8-weight
    vector per stage, so three stages carry the 48 bits of its 6.0-bpw rung).
    Stage 1 encodes the rotated weight as pack_pvq does; every later stage
    encodes what the stages before it left, w' minus their decode, with its own
    RMS row scale and the same codebook. Returns idx uint8 [stages][N][K/4] and
    row scales uint16 [stages][N] (fp16 bit patterns)."""
    if stages < 1:
        raise ValueError("stages must be at least 1")
    res = rotate(np.asarray(w, dtype=np.float64), signs)
    idxs, scales = [], []
    for _ in range(stages):
        idx, s16 = pvq_encode(res, cb_bytes)
        res = res - pvq_dequantize(idx, s16.view(np.uint16), cb_bytes)
        idxs.append(idx)
        scales.append(s16.view(np.uint16))
    return np.stack(idxs), np.stack(scales)


def pvq_dequantize_stages(idx: np.ndarray, scale_u16: np.ndarray, cb_bytes: np.ndarray) -> np.ndarray:
    """W'_hat = sum over stages of s_n^(t) C[idx^(t)] (float64, rotated basis)."""
    return sum(pvq_dequantize(idx[t], scale_u16[t], cb_bytes) for t in range(idx.shape[0]))


def linear_pvq_stages(x16, idx, scale_u16, cb_bytes, signs) -> np.ndarray:
    return linear(x16, inverse_rotate(pvq_dequantize_stages(idx, scale_u16, cb_bytes), signs))


def dequant_weight_pvq(idx, scale_u16, cb_bytes, signs) -> np.ndarray:
    return inverse_rotate(pvq_dequantize(idx, scale_u16, cb_bytes), signs)


def linear_pvq(x16, idx, scale_u16, cb_bytes, signs) -> np.ndarray:
    return linear(x16, dequant_weight_pvq(idx, scale_u16, cb_bytes, signs))


# ---------------------------------------------------------------------------
# Routed-expert MoE block (Laguna-S-2.1 card: routed experts, top-k; LLaDA2.2-mini
# card: per-expert code widths for routed experts)
# ---------------------------------------------------------------------------

def route(logits: np.ndarray, top_k: int):
    """Top-k experts per token (larger logit first, ties to the lower id) and
    softmax weights over the selected logits.

    Returns ids int32 [M][top_k] and weights float64 [M][top_k].
    """
    lg = np.asarray(logits, dtype=np.float32)
    m, e = lg.shape
    ids = np.empty((m, top_k), dtype=np.int32)
    wts = np.empty((m, top_k), dtype=np.float64)
    for t in range(m):
        order = sorted(range(e), key=lambda i: (-float(lg[t, i]), i))
        sel = order[:top_k]
        ids[t] = sel
        v = lg[t, sel].astype(np.float64)
        ex = np.exp(v - v.max())
        wts[t] = ex / ex.sum()
    return ids, wts


def silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def expert_ffn(x16: np.ndarray, w_gu: np.ndarray, w_dn: np.ndarray) -> np.ndarray:
    """SwiGLU expert: h = x W_gu^T, a = silu(h[:F]) * h[F:], o = a W_dn^T (float64)."""
    h = linear(x16, w_gu)
    f = w_gu.shape[0] // 2
    a = silu(h[:, :f]) * h[:, f:]
    return a @ np.asarray(w_dn, dtype=np.float64).T


def moe_forward(x16: np.ndarray, logits: np.ndarray, top_k: int, expert_weights=None,
                expert_outputs=None) -> np.ndarray:
    """y_t = sum_j w_tj * FFN_{ids[t,j]}(x_t), float64 [M][hidden].

    ``expert_weights(e)`` returns the original-basis (W_gu_hat [2F][H],
    W_dn_hat [H][F]) of expert e; experts are visited one at a time. Instead,
    ``expert_outputs(e, rows)`` may return FFN_e of the tokens ``rows`` (the
    same expert_ffn, computed elsewhere, e.g. expert by expert in parallel).
    """
    ids, wts = route(logits, top_k)
    m, h = np.asarray(x16).shape
    y = np.zeros((m, h), dtype=np.float64)
    for e in np.unique(ids):
        rows, slots = np.nonzero(ids == e)
        if expert_outputs is not None:
            o = expert_outputs(int(e), rows)
        else:
            w_gu, w_dn = expert_weights(int(e))
            o = expert_ffn(np.asarray(x16)[rows], w_gu, w_dn)
        y[rows] += wts[rows, slots][:, None] * o
    return y


def moe_forward_per_assignment(x16, logits, top_k, expert_weights) -> np.ndarray:
    """Same block computed one (token, slot) pair at a time, in slot order."""
    ids, wts = route(logits, top_k)
    m, h = np.asarray(x16).shape
    y = np.zeros((m, h), dtype=np.float64)
    for t in range(m):
        for j in range(top_k):
            w_gu, w_dn = expert_weights(int(ids[t, j]))
            y[t] += wts[t, j] * expert_ffn(np.asarray(x16)[t:t + 1], w_gu, w_dn)[0]
    return y


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))
