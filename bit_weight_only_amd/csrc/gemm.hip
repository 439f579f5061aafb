// MFMA dequant-GEMM for many tokens: y = x' W'^T with W' decoded inside the
// K mainloop straight into the B operand of v_mfma_f32_16x16x32_f16 (no
// expand-to-dense round trip through memory; the gridbook card names exactly
// that round trip as its prefill gap: Laguna-S-2.1 card, "Reading it honestly").
//
// Tiling: a workgroup of 4 wavefronts owns 64 output columns (rows of W), each
// wave 16 of them, and MT*16 tokens. Per 128-wide group of K:
//   * the group's activations for the token tile are staged in LDS in the
//     folded slot order (slot c of a 32-chunk = (x[c], x[c+16])), double
//     buffered, and the next group's activations and codes are loaded while
//     the current group is contracted;
//   * lane (j, kq) of a wave decodes word column kq of row j: its 16 slots give
//     the B operands of the group's 4 k-steps (slots 4t..4t+3 for step t). The
//     A operand of lane (i, kq) is slots 4t..4t+3 of token i's chunk kq, so A
//     and B agree on which k each element is.
//   * RTN: slots hold 1 + q 2^(m-10); one packed fma with 2^(10-m) and
//     -(2^(10-m) + z) gives the exact integer q - z in fp16. The MFMA sums the
//     group exactly up to fp32 rounding; the group scale is applied once per
//     group (y += s * D_g).
//   * PVQ: the row scale is constant along K, so B holds the codebook values
//     themselves (e4m3 values are exact in fp16, staged as a 2 KB fp16 table
//     in LDS) and the scale is applied once at the end.
#include "device.h"
#include "kernels.h"

namespace lbq {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTokStride = 68;   // u32 per staged token per group (64 slots + pad)

typedef _Float16 h2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_fma(uint32_t a, uint32_t b, uint32_t c) {
  const h2v r = __builtin_elementwise_fma(__builtin_bit_cast(h2v, a), __builtin_bit_cast(h2v, b),
                                          __builtin_bit_cast(h2v, c));
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t splat_h(float v) {
  const uint32_t b = f32_to_f16_bits(v);
  return b | (b << 16);
}

// ------------------------------------------------------------------ B decoders

// RTN codes. Holds one group's worth of this lane's word column.
template <int BITS>
struct RtnB {
  const uint32_t *planes;  // uint32 [N][G][BITS][4]
  const uint32_t *meta;    // [N][G]
  int G, N;
  struct Raw {
    uint32_t w[BITS];
    uint32_t mt;
  };
  __device__ __forceinline__ Raw load(int row, int g, int kq) const {
    Raw r;
    if (row < N) {
      const uint32_t *p = planes + (static_cast<size_t>(row) * G + g) * BITS * 4 + kq;
#pragma unroll
      for (int i = 0; i < BITS; ++i) r.w[i] = p[i * 4];
      r.mt = meta[static_cast<size_t>(row) * G + g];
    } else {
#pragma unroll
      for (int i = 0; i < BITS; ++i) r.w[i] = 0;
      r.mt = 0;
    }
    return r;
  }
  // 16 slots of exact (q - z) half2 values; scale returned separately.
  __device__ __forceinline__ void decode(const Raw &r, uint32_t b[16], float &scale) const {
    uint32_t h[16];
    if constexpr (BITS == 2) decode_slots2(r.w[0], r.w[1], h);
    else decode_slots_nib<BITS>(r.w, h);
    const float z = f16_bits_to_f32(r.mt >> 16);
    scale = f16_bits_to_f32(r.mt & 0xFFFFu);
    constexpr int NC = num_classes<BITS>();
    uint32_t mul[NC], add[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      mul[c] = splat_h(class_weight<BITS>(c));
      add[c] = splat_h(-(class_weight<BITS>(c) + z));
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) b[c] = pk_fma(h[c], mul[slot_class<BITS>(c)], add[slot_class<BITS>(c)]);
  }
  static constexpr bool kGroupScale = true;
};

// Product-VQ indices: byte i of a row covers weights 4i..4i+3.
struct PvqB {
  const uint8_t *idx;      // [N][K/4]
  const uint16_t *scale;   // [N]
  const uint32_t *lut;     // LDS: 256 entries x 2 u32 (4 fp16)
  int K, N;
  struct Raw {
    uint2 w;  // 8 index bytes of word column kq: weights 32kq .. 32kq+31
  };
  __device__ __forceinline__ Raw load(int row, int g, int kq) const {
    Raw r;
    if (row < N) {
      r.w = *reinterpret_cast<const uint2 *>(idx + static_cast<size_t>(row) * (K / 4) + g * 32 + kq * 8);
    } else {
      r.w = make_uint2(0, 0);
    }
    return r;
  }
  // slot c = (w[c], w[c+16]); weights 4t..4t+3 use index byte t, weights
  // 16+4t.. use index byte t+4.
  __device__ __forceinline__ void decode(const Raw &r, uint32_t b[16], float &scale) const {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t ia = (r.w.x >> (8 * t)) & 0xFFu;
      const uint32_t ib = (r.w.y >> (8 * t)) & 0xFFu;
      const uint2 ca = *reinterpret_cast<const uint2 *>(lut + 2 * ia);
      const uint2 cb = *reinterpret_cast<const uint2 *>(lut + 2 * ib);
      b[4 * t + 0] = (ca.x & 0xFFFFu) | (cb.x << 16);
      b[4 * t + 1] = (ca.x >> 16) | (cb.x & 0xFFFF0000u);
      b[4 * t + 2] = (ca.y & 0xFFFFu) | (cb.y << 16);
      b[4 * t + 3] = (ca.y >> 16) | (cb.y & 0xFFFF0000u);
    }
    scale = 1.0f;
  }
  static constexpr bool kGroupScale = false;
};

// ------------------------------------------------------------------ mainloop

template <int MT, class Dec>
__device__ __forceinline__ void gemm_body(const Dec &dec, const uint32_t *__restrict__ xr, uint16_t *__restrict__ y,
                                          int M, int K, int N, uint32_t *lds_x, float row_scale) {
  const int G = K / kGroup;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane & 15, kq = lane >> 4;
  const int n0 = blockIdx.x * (16 * kWaves);
  const int row = n0 + wave * 16 + j;
  const int m0 = blockIdx.y * (16 * MT);
  constexpr int kChunks = 16 * MT * 4;                  // 32-element chunks per group of the token tile
  constexpr int kPerThread = (kChunks + kThreads - 1) / kThreads;
  constexpr int kBuf = 16 * MT * kTokStride;            // u32 per buffer

  float4_t acc[MT];
  float4_t yacc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};
    yacc[t] = float4_t{0.f, 0.f, 0.f, 0.f};
  }

  // prefetch registers for the staged activations
  uint4 xa[kPerThread][4];
  auto load_x = [&](int g) {
#pragma unroll
    for (int p = 0; p < kPerThread; ++p) {
      const int ch = threadIdx.x + p * kThreads;
      const int tok = ch >> 2, col = ch & 3;
      if (ch < kChunks && m0 + tok < M) {
        const uint4 *src = reinterpret_cast<const uint4 *>(xr + static_cast<size_t>(m0 + tok) * (K / 2) +
                                                           static_cast<size_t>(g) * 64 + col * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) xa[p][i] = src[i];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) xa[p][i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_x = [&](uint32_t *buf) {
#pragma unroll
    for (int p = 0; p < kPerThread; ++p) {
      const int ch = threadIdx.x + p * kThreads;
      if (ch < kChunks) {
        const int tok = ch >> 2, col = ch & 3;
        uint32_t a[16], s[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[4 * i] = xa[p][i].x;
          a[4 * i + 1] = xa[p][i].y;
          a[4 * i + 2] = xa[p][i].z;
          a[4 * i + 3] = xa[p][i].w;
        }
        fold32(a, s);
        uint4 *d = reinterpret_cast<uint4 *>(buf + tok * kTokStride + col * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] = make_uint4(s[4 * i], s[4 * i + 1], s[4 * i + 2], s[4 * i + 3]);
      }
    }
  };

  typename Dec::Raw raw = dec.load(row, 0, kq);
  load_x(0);
  for (int g = 0; g < G; ++g) {
    uint32_t *buf = lds_x + (g & 1) * kBuf;
    store_x(buf);
    __syncthreads();
    uint32_t b[16];
    float scale;
    dec.decode(raw, b, scale);
    if (g + 1 < G) {
      raw = dec.load(row, g + 1, kq);
      load_x(g + 1);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const half8_t bop = __builtin_bit_cast(half8_t, make_uint4(b[4 * t], b[4 * t + 1], b[4 * t + 2], b[4 * t + 3]));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint4 av = *reinterpret_cast<const uint4 *>(buf + (mt * 16 + j) * kTokStride + kq * 16 + 4 * t);
        const half8_t aop = __builtin_bit_cast(half8_t, av);
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, acc[mt], 0, 0, 0);
      }
    }
    if constexpr (Dec::kGroupScale) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        yacc[mt] += scale * acc[mt];
        acc[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  if constexpr (!Dec::kGroupScale) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) yacc[mt] = acc[mt];
  }
  // D layout: lane holds tokens 4*kq + r (r = 0..3) of tile mt, column j.
  if (row < N) {
    const float rs = Dec::kGroupScale ? 1.0f : row_scale;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = m0 + mt * 16 + kq * 4 + r;
        if (tok < M) y[static_cast<size_t>(tok) * N + row] = f32_to_f16_bits(yacc[mt][r] * rs);
      }
    }
  }
}

template <int BITS, int MT>
__global__ void __launch_bounds__(kThreads) gemm_rtn_kernel(const uint32_t *__restrict__ planes,
                                                            const uint32_t *__restrict__ meta,
                                                            const uint32_t *__restrict__ xr, uint16_t *__restrict__ y,
                                                            int M, int K, int N) {
  __shared__ uint32_t lds_x[2 * 16 * MT * kTokStride];
  RtnB<BITS> dec{planes, meta, K / kGroup, N};
  gemm_body<MT>(dec, xr, y, M, K, N, lds_x, 1.0f);
}

template <int MT>
__global__ void __launch_bounds__(kThreads) gemm_pvq_kernel(const uint8_t *__restrict__ idx,
                                                            const uint16_t *__restrict__ scale,
                                                            const uint8_t *__restrict__ codebook,
                                                            const uint32_t *__restrict__ xr, uint16_t *__restrict__ y,
                                                            int M, int K, int N) {
  __shared__ uint32_t lds_x[2 * 16 * MT * kTokStride];
  __shared__ uint32_t lut[512];
  // e4m3 -> fp16 table: 256 entries x 4 values, 2 u32 per entry.
  for (int e = threadIdx.x; e < 512; e += kThreads) {
    const uint32_t two = reinterpret_cast<const uint16_t *>(codebook)[e];
    uint32_t out = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) out |= static_cast<uint32_t>(e4m3_to_f16_bits((two >> (8 * h)) & 0xFFu)) << (16 * h);
    lut[e] = out;
  }
  __syncthreads();
  PvqB dec{idx, scale, lut, K, N};
  const int row = blockIdx.x * (16 * kWaves) + (threadIdx.x >> 6) * 16 + (threadIdx.x & 15);
  const float rs = row < N ? f16_bits_to_f32(scale[row]) : 0.f;
  gemm_body<MT>(dec, xr, y, M, K, N, lds_x, rs);
}

}  // namespace

hipError_t launch_gemm_rtn(const void *planes, const void *meta, const uint16_t *xr, uint16_t *y, int M, int K, int N,
                           int bits, hipStream_t s) {
  const unsigned gx = static_cast<unsigned>((N + 63) / 64);
  const bool big = M > 64;
  const unsigned gy = static_cast<unsigned>(big ? (M + 127) / 128 : (M + 63) / 64);
  const uint32_t *pl = reinterpret_cast<const uint32_t *>(planes);
  const uint32_t *mt = reinterpret_cast<const uint32_t *>(meta);
  const uint32_t *x = reinterpret_cast<const uint32_t *>(xr);
  dim3 grid(gx, gy), block(kThreads);
#define LBQ_GEMM_CASE(B)                                                                     \
  if (big) hipLaunchKernelGGL((gemm_rtn_kernel<B, 8>), grid, block, 0, s, pl, mt, x, y, M, K, N); \
  else hipLaunchKernelGGL((gemm_rtn_kernel<B, 4>), grid, block, 0, s, pl, mt, x, y, M, K, N);
  switch (bits) {
    case 2: LBQ_GEMM_CASE(2) break;
    case 3: LBQ_GEMM_CASE(3) break;
    default: LBQ_GEMM_CASE(4) break;
  }
#undef LBQ_GEMM_CASE
  return hipGetLastError();
}

hipError_t launch_gemm_pvq(const uint8_t *idx, const uint16_t *scale, const uint8_t *codebook, const uint16_t *xr,
                           uint16_t *y, int M, int K, int N, hipStream_t s) {
  const unsigned gx = static_cast<unsigned>((N + 63) / 64);
  const bool big = M > 64;
  const unsigned gy = static_cast<unsigned>(big ? (M + 127) / 128 : (M + 63) / 64);
  const uint32_t *x = reinterpret_cast<const uint32_t *>(xr);
  dim3 grid(gx, gy), block(kThreads);
  if (big) hipLaunchKernelGGL((gemm_pvq_kernel<8>), grid, block, 0, s, idx, scale, codebook, x, y, M, K, N);
  else hipLaunchKernelGGL((gemm_pvq_kernel<4>), grid, block, 0, s, idx, scale, codebook, x, y, M, K, N);
  return hipGetLastError();
}

}  // namespace lbq
