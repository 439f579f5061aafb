"""Low-bit weight-only quantized linear layers for AMD MI355X (gfx950).

The computation lives in liblbq.so (hand-written HIP kernels behind the C ABI
in include/lbq.h); ``bit_weight_only_amd.lbq`` is a thin ctypes binding.
"""
from . import lbq  # noqa: F401
from .lbq import (FMT_PVQ_4x8, FMT_RTN_PLANES, PATH_AUTO, PATH_GEMM, PATH_GEMV, LbqError, PackedLinear,  # noqa: F401
                  PackedMoe, linear_forward, moe_forward, moe_from_host, moe_route, pack, pack_moe_host,
                  packed_bytes, rotate, unpack_codes)
