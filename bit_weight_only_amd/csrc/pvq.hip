// Product-VQ dequant-GEMV for few tokens (1 <= M <= 16). Each index byte picks
// one 4-value codebook entry (e4m3 values, held as an fp16 table in LDS) for
// four consecutive weights; the entry is contracted with four activations by
// two v_dot2_f32_f16. The row scale is constant along K and is applied once
// at the end. (Product-VQ over fp8-grid codebook values decoded at matmul
// time: Laguna-S-2.1 gridbook model card, opening paragraph.)
//
// Work split as in the RTN GEMV: L lanes per output row stride over its
// 128-weight groups (32 index bytes, two 16-byte loads per lane); the rotated
// activations of the token block are staged in LDS in natural order.
#include "device.h"
#include "kernels.h"

namespace lbq {

namespace {

constexpr int kThreads = 256;
constexpr int kGroupStride = 68;       // u32 per staged group of 128 activations (+16 B pad)
constexpr int kLdsBudget = 64 * 1024;

template <int MT, int L>
__global__ void __launch_bounds__(kThreads) gemv_pvq_kernel(const uint4 *__restrict__ idx,
                                                            const uint16_t *__restrict__ scale,
                                                            const uint8_t *__restrict__ codebook,
                                                            const uint32_t *__restrict__ xr, uint16_t *__restrict__ y,
                                                            int M, int K, int N, int Gc) {
  constexpr int R = kThreads / L;
  extern __shared__ uint32_t smem[];
  uint32_t *lut = smem;                  // 256 x 2 u32
  uint32_t *xx = smem + 512;             // [MT][Gc][kGroupStride]
  for (int e = threadIdx.x; e < 512; e += kThreads) {
    const uint32_t two = reinterpret_cast<const uint16_t *>(codebook)[e];
    lut[e] = e4m3_to_f16_bits(two & 0xFFu) | (e4m3_to_f16_bits(two >> 8) << 16);
  }
  const int G = K / kGroup;
  const int j = threadIdx.x % L;
  const int row = blockIdx.x * R + threadIdx.x / L;
  float yacc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) yacc[m] = 0.f;

  for (int g0 = 0; g0 < G; g0 += Gc) {
    const int gn = min(Gc, G - g0);
    __syncthreads();
    for (int u = threadIdx.x; u < MT * gn * 16; u += kThreads) {
      const int m = u / (gn * 16), r = u - m * gn * 16;
      const int g = r >> 4, q = r & 15;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m < M)
        v = reinterpret_cast<const uint4 *>(xr + static_cast<size_t>(m) * (K / 2) + static_cast<size_t>(g0 + g) * 64)[q];
      reinterpret_cast<uint4 *>(xx + (m * Gc + g) * kGroupStride)[q] = v;
    }
    __syncthreads();
    if (row < N) {
      const uint4 *prow = idx + (static_cast<size_t>(row) * G + g0) * 2;
      for (int g = j; g < gn; g += L) {
        const uint4 i0 = prow[2 * g], i1 = prow[2 * g + 1];
        const uint32_t iw[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
        float acc[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {      // 4 index bytes = 16 weights per q
          uint2 c[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) c[b] = *reinterpret_cast<const uint2 *>(lut + 2 * ((iw[q] >> (8 * b)) & 0xFFu));
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const uint4 *xs = reinterpret_cast<const uint4 *>(xx + (m * Gc + g) * kGroupStride + q * 8);
            const uint4 xa = xs[0], xb = xs[1];
            acc[m] = dot2(c[0].x, xa.x, acc[m]);
            acc[m] = dot2(c[0].y, xa.y, acc[m]);
            acc[m] = dot2(c[1].x, xa.z, acc[m]);
            acc[m] = dot2(c[1].y, xa.w, acc[m]);
            acc[m] = dot2(c[2].x, xb.x, acc[m]);
            acc[m] = dot2(c[2].y, xb.y, acc[m]);
            acc[m] = dot2(c[3].x, xb.z, acc[m]);
            acc[m] = dot2(c[3].y, xb.w, acc[m]);
          }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) yacc[m] += acc[m];
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int off = L / 2; off > 0; off >>= 1) yacc[m] += __shfl_xor(yacc[m], off);
  }
  if (j == 0 && row < N) {
    const float s = f16_bits_to_f32(scale[row]);
#pragma unroll
    for (int m = 0; m < MT; ++m)
      if (m < M) y[static_cast<size_t>(m) * N + row] = f32_to_f16_bits(yacc[m] * s);
  }
}

template <int MT, int L>
hipError_t launch_one(const uint8_t *idx, const uint16_t *scale, const uint8_t *codebook, const uint16_t *xr,
                      uint16_t *y, int M, int K, int N, hipStream_t s) {
  const int G = K / kGroup;
  const int per_group = MT * kGroupStride * 4;
  const int Gc = min(G, (kLdsBudget - 2048) / per_group);
  const size_t lds = 2048 + static_cast<size_t>(Gc) * per_group;
  const unsigned grid = static_cast<unsigned>((N + kThreads / L - 1) / (kThreads / L));
  hipLaunchKernelGGL((gemv_pvq_kernel<MT, L>), dim3(grid), dim3(kThreads), lds, s,
                     reinterpret_cast<const uint4 *>(idx), scale, codebook, reinterpret_cast<const uint32_t *>(xr), y,
                     M, K, N, Gc);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_mt(const uint8_t *idx, const uint16_t *scale, const uint8_t *codebook, const uint16_t *xr,
                     uint16_t *y, int M, int K, int N, hipStream_t s) {
  const int G = K / kGroup;
  if (N <= 4096 && G >= 32) return launch_one<MT, 32>(idx, scale, codebook, xr, y, M, K, N, s);
  if (N <= 8192 && G >= 16) return launch_one<MT, 16>(idx, scale, codebook, xr, y, M, K, N, s);
  return launch_one<MT, 8>(idx, scale, codebook, xr, y, M, K, N, s);
}

}  // namespace

hipError_t launch_gemv_pvq(const uint8_t *idx, const uint16_t *scale, const uint8_t *codebook, const uint16_t *xr,
                           uint16_t *y, int M, int K, int N, hipStream_t s) {
  if (M <= 1) return launch_mt<1>(idx, scale, codebook, xr, y, M, K, N, s);
  if (M <= 2) return launch_mt<2>(idx, scale, codebook, xr, y, M, K, N, s);
  if (M <= 4) return launch_mt<4>(idx, scale, codebook, xr, y, M, K, N, s);
  if (M <= 8) return launch_mt<8>(idx, scale, codebook, xr, y, M, K, N, s);
  return launch_mt<16>(idx, scale, codebook, xr, y, M, K, N, s);
}

}  // namespace lbq
