"""Seeded synthetic inputs shared by the oracle-side tests and the GPU-side tests.

This module only draws random numbers and names workload shapes. It holds none
of the quantization, rotation or contraction arithmetic: both the CPU oracle
(``oracle/``) and the HIP path receive what is drawn here as plain arrays.

Every draw uses ``numpy.random.default_rng([2026, workload, item, role])`` so a
(workload, item, role) triple always yields the same array on any machine.
"""
from __future__ import annotations

import numpy as np

# Role numbers of the seed triple.
ROLE_W = 0
ROLE_SIGNS = 1
ROLE_X = 2
ROLE_LOGITS = 3
ROLE_BITS = 4
ROLE_CODEBOOK = 5


def rng(workload: int, item: int, role: int) -> np.random.Generator:
    return np.random.default_rng([2026, int(workload), int(item), int(role)])


def weights(n: int, k: int, workload: int = 0, item: int = 0, std: float = 0.02) -> np.ndarray:
    """fp32 [n][k] row-major weight (PyTorch Linear order), N(0, std^2)."""
    g = rng(workload, item, ROLE_W)
    w = g.standard_normal((n, k), dtype=np.float32)
    w *= np.float32(std)
    return w


def signs(k: int, workload: int = 0, item: int = 0) -> np.ndarray:
    """Rademacher vector, int8 in {-1, +1}, length k."""
    g = rng(workload, item, ROLE_SIGNS)
    return (g.integers(0, 2, size=k, dtype=np.int8) * 2 - 1).astype(np.int8)


def activations(m: int, k: int, workload: int = 0, item: int = 0) -> np.ndarray:
    """fp16 [m][k] activations drawn N(0,1) in fp32, then cast to fp16."""
    g = rng(workload, item, ROLE_X)
    return g.standard_normal((m, k), dtype=np.float32).astype(np.float16)


def logits(m: int, e: int, workload: int = 0, item: int = 0) -> np.ndarray:
    """fp32 [m][e] router logits, N(0,1)."""
    g = rng(workload, item, ROLE_LOGITS)
    return g.standard_normal((m, e), dtype=np.float32)


def expert_bits(e: int, workload: int = 0, item: int = 0, p=(0.7, 0.2, 0.1)) -> np.ndarray:
    """Per-expert code width in {2,3,4}, drawn with probabilities p."""
    g = rng(workload, item, ROLE_BITS)
    return g.choice(np.array([2, 3, 4], dtype=np.uint8), size=e, p=list(p)).astype(np.uint8)


def codebook(workload: int = 0, item: int = 0, entries: int = 256, dim: int = 4) -> np.ndarray:
    """[entries][dim] fp8 e4m3 codebook as raw bytes (uint8).

    The entries are N(0,1) draws cast to the e4m3 grid by PyTorch's own
    float8_e4m3fn conversion. If two entries come out identical the draw is
    repeated with the next item number, so the codebook has distinct entries.
    """
    import torch

    it = item
    while True:
        g = rng(workload, it, ROLE_CODEBOOK)
        v = g.standard_normal((entries, dim), dtype=np.float32)
        b = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
        if len(np.unique(b.view(np.dtype((np.void, dim))))) == entries:
            return b
        it += 1000


# the NVFP4 (e2m1) value grid, non-negative half; as e4m3 bytes
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def codebook_fp4(workload: int = 0, item: int = 0, entries: int = 256, dim: int = 4) -> np.ndarray:
    """[entries][dim] codebook whose values lie on the NVFP4 (e2m1) grid,
    stored as fp8 e4m3 bytes (every e2m1 value is exact in e4m3). Entries are
    2 x N(0,1) draws moved to the nearest grid value (ties to the smaller
    magnitude); draws repeat with the next item until the entries are distinct."""
    import torch

    it = item
    while True:
        g = rng(workload, it, ROLE_CODEBOOK)
        v = 2.0 * g.standard_normal((entries, dim), dtype=np.float32)
        mag = np.abs(v)
        pick = np.argmin(np.abs(mag[..., None] - E2M1_VALUES), axis=-1)   # first (smaller) of equals
        q = np.sign(v) * E2M1_VALUES[pick]
        b = torch.from_numpy(q.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
        b[q == 0] = 0   # +0 for every zero
        if len(np.unique(b.view(np.dtype((np.void, dim))))) == entries:
            return b
        it += 1000


ROLE_CALIB = 6


def calibration(n: int, k: int, workload: int = 0, item: int = 0, sample: int = 0,
                rank_frac: float = 0.25) -> np.ndarray:
    """fp32 [n][k] stand-in for activations of a layer input: a low-rank
    correlated part (rank k * rank_frac) plus 0.1 isotropic noise, each channel
    scaled by a log-normal factor (a few channels much larger than the rest, as
    in transformer activations). The structure (mixing matrix, channel scales)
    is fixed by (workload, item); `sample` draws other rows of the same
    distribution (calibration rows, then held-out rows)."""
    g = rng(workload, item, ROLE_CALIB)
    r = max(1, int(k * rank_frac))
    mix = g.standard_normal((r, k), dtype=np.float32) * np.float32(1.0 / np.sqrt(r))
    scale = np.exp(np.float32(0.5) * g.standard_normal(k, dtype=np.float32))
    gs = np.random.default_rng([2026, int(workload), int(item), ROLE_CALIB, int(sample)])
    x = gs.standard_normal((n, r), dtype=np.float32) @ mix
    x += np.float32(0.1) * gs.standard_normal((n, k), dtype=np.float32)
    x *= scale[None, :]
    return x


# Workload shapes. (K, N) is (inputs, outputs) of a linear.
SINGLE_LINEAR = dict(K=4096, N=4096, M=1, bits=2)
DENSE_STACK_SHAPES = [("qkv", 4096, 6144), ("o", 4096, 4096), ("gate_up", 4096, 28672), ("down", 14336, 4096)]
DENSE_STACK_M = (1, 4, 16)
MOE_BLOCK = dict(E=256, hidden=2048, ffn=1024, top_k=8, M=32)
FFN_SWEEP = dict(K_gu=5120, N_gu=17408, bits_gu=2, bits_dn=3, M=(1, 8, 64, 256))
PVQ_LINEAR = dict(K=4096, N=14336, M=(1, 16, 64))
# 8-bit readout over a vocabulary: hidden 2048 as in the MoE block; the pages
# give no vocabulary size, 131072 rows stands in for one
READOUT = dict(K=2048, N=131072, M=(1, 4), cand=64)

# Workload numbers used as the first seed component.
W_SINGLE, W_STACK, W_MOE, W_FFN, W_PVQ = 0, 1, 2, 3, 4
W_READOUT = 5
