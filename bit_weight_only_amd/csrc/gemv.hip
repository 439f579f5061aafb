// Dequant-GEMV for few tokens (1 <= M <= 16): y = x' W'^T with W' decoded from
// group-128 bit-plane codes inside the contraction.
//
// Why this shape: at decode batch sizes the layer is bound by the bytes of the
// packed weight ("batching amortizes the weight read": Qwen3-8B BPDQ model
// card, Benchmarks; "decode is per-byte neutral": Laguna-S-2.1 gridbook card,
// "Reading it honestly"), so the kernel streams the planes once with 128-bit
// loads and spends as few VALU operations per weight as it can:
//   * planes of one 32-code column are merged into 2-bit (or 4-bit) fields with
//     bitfield inserts;
//   * each field pair is OR-ed into the mantissa of fp16 1.0, giving the exact
//     value 1 + q 2^(m-10), and fed to v_dot2_f32_f16 against a half2 of
//     activations: two weights per AND-OR and per dot;
//   * the constant parts (the 1.0 and the zero-point) are removed once per
//     group with per-group activation sums staged in LDS.
// Work split: L lanes share one output row and stride over its groups; lanes
// of different rows read the same activation slots, which LDS broadcasts.
// Partial sums are reduced across the L lanes in registers; the result is
// deterministic (fixed order, no atomics).
#include "gemv_core.h"
#include "kernels.h"

namespace lbq {

namespace {

constexpr int kLdsBudget = 64 * 1024;     // bytes of dynamic LDS per workgroup

template <int BITS, int MT, int L>
__global__ void __launch_bounds__(kGemvThreads) gemv_rtn_kernel(const uint4 *__restrict__ planes,
                                                                const uint32_t *__restrict__ meta,
                                                                const uint32_t *__restrict__ xr,
                                                                uint16_t *__restrict__ y, int M, int K, int N, int Gc) {
  constexpr int R = kGemvThreads / L;
  extern __shared__ uint32_t smem[];
  uint32_t *xx = smem;
  float2 *sums = reinterpret_cast<float2 *>(smem + MT * Gc * kGroupStride);

  const int G = K / kGroup;
  const int j = threadIdx.x % L;
  const int row = blockIdx.x * R + threadIdx.x / L;
  float yacc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) yacc[m] = 0.f;
  auto row_ptr = [&](int m) { return xr + static_cast<size_t>(m) * (K / 2); };

  for (int g0 = 0; g0 < G; g0 += Gc) {
    const int gn = min(Gc, G - g0);
    if (g0) __syncthreads();
    stage_groups<BITS, MT>(row_ptr, M, g0, gn, Gc, xx, sums);
    __syncthreads();
    if (row < N)
      row_partial<BITS, MT, L>(planes + (static_cast<size_t>(row) * G + g0) * BITS,
                               meta + static_cast<size_t>(row) * G + g0, xx, sums, Gc, gn, j, yacc);
  }
  reduce_cluster<MT, L>(yacc);
  if (j == 0 && row < N) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
      if (m < M) y[static_cast<size_t>(m) * N + row] = f32_to_f16_bits(yacc[m]);
  }
}

template <int BITS, int MT, int L>
hipError_t launch_one(const void *planes, const void *meta, const uint16_t *xr, uint16_t *y, int M, int K, int N,
                      hipStream_t s) {
  const int G = K / kGroup;
  const int per_group = MT * kStagedGroupBytes;
  const int Gc = min(G, kLdsBudget / per_group);
  const size_t lds = static_cast<size_t>(Gc) * per_group;
  const unsigned grid = static_cast<unsigned>((N + kGemvThreads / L - 1) / (kGemvThreads / L));
  hipLaunchKernelGGL((gemv_rtn_kernel<BITS, MT, L>), dim3(grid), dim3(kGemvThreads), lds, s,
                     reinterpret_cast<const uint4 *>(planes), reinterpret_cast<const uint32_t *>(meta),
                     reinterpret_cast<const uint32_t *>(xr), y, M, K, N, Gc);
  return hipGetLastError();
}

template <int BITS, int MT>
hipError_t launch_mt(const void *planes, const void *meta, const uint16_t *xr, uint16_t *y, int M, int K, int N,
                     hipStream_t s) {
  // Lanes per row: enough workgroups to cover the chip, at least one group per lane.
  const int G = K / kGroup;
  if (N <= 4096 && G >= 32) return launch_one<BITS, MT, 32>(planes, meta, xr, y, M, K, N, s);
  if (N <= 8192 && G >= 16) return launch_one<BITS, MT, 16>(planes, meta, xr, y, M, K, N, s);
  return launch_one<BITS, MT, 8>(planes, meta, xr, y, M, K, N, s);
}

template <int BITS>
hipError_t launch_bits(const void *planes, const void *meta, const uint16_t *xr, uint16_t *y, int M, int K, int N,
                       hipStream_t s) {
  if (M <= 1) return launch_mt<BITS, 1>(planes, meta, xr, y, M, K, N, s);
  if (M <= 2) return launch_mt<BITS, 2>(planes, meta, xr, y, M, K, N, s);
  if (M <= 4) return launch_mt<BITS, 4>(planes, meta, xr, y, M, K, N, s);
  if (M <= 8) return launch_mt<BITS, 8>(planes, meta, xr, y, M, K, N, s);
  return launch_mt<BITS, 16>(planes, meta, xr, y, M, K, N, s);
}

}  // namespace

hipError_t launch_gemv_rtn(const void *planes, const void *meta, const uint16_t *xr, uint16_t *y, int M, int K, int N,
                           int bits, hipStream_t s) {
  switch (bits) {
    case 2: return launch_bits<2>(planes, meta, xr, y, M, K, N, s);
    case 3: return launch_bits<3>(planes, meta, xr, y, M, K, N, s);
    default: return launch_bits<4>(planes, meta, xr, y, M, K, N, s);
  }
}

}  // namespace lbq
