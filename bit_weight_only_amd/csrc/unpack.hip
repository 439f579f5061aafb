// Codes as the GPU decoders see them. Each thread takes one 32-code word column
// of one (row, group), merges its bit-planes with the same routines the GEMV
// and GEMM kernels use (merge2 / merge_nibbles), and reads the codes back out
// of the merged fields. A bit-exact match of these codes with codes computed
// independently on the CPU checks the merge logic of every decoder (the
// pages' own read-back check: Pingala-8 model card, "Checks").
#include "device.h"
#include "kernels.h"

namespace lbq {

namespace {

template <int BITS>
__global__ void __launch_bounds__(256) unpack_rtn_kernel(const uint32_t *__restrict__ planes,
                                                         uint4 *__restrict__ codes, long columns) {
  const long t = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= columns) return;
  const long ng = t >> 2;
  const int w = static_cast<int>(t & 3);
  const uint32_t *pl = planes + ng * BITS * 4;
  uint32_t p[BITS];
#pragma unroll
  for (int i = 0; i < BITS; ++i) p[i] = pl[i * 4 + w];
  uint8_t out[32];
  if constexpr (BITS == 2) {
    uint32_t e, o;
    merge2(p[0], p[1], e, o);
#pragma unroll
    for (int f = 0; f < 16; ++f) {
      out[2 * f] = static_cast<uint8_t>((e >> (2 * f)) & 3u);
      out[2 * f + 1] = static_cast<uint8_t>((o >> (2 * f)) & 3u);
    }
  } else if constexpr (BITS == 8) {
    // the GEMM's route: nibble words of planes 0..3 and 4..7
    uint32_t lo[4], hi[4];
    merge_nibbles<4>(p, lo);
    merge_nibbles<4>(p + 4, hi);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        out[4 * i + r] = static_cast<uint8_t>(((lo[r] >> (4 * i)) & 15u) | (((hi[r] >> (4 * i)) & 15u) << 4));
  } else {
    uint32_t n[4];
    merge_nibbles<BITS>(p, n);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 8; ++i) out[4 * i + r] = static_cast<uint8_t>((n[r] >> (4 * i)) & 15u);
  }
  uint32_t o32[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    o32[i] = out[4 * i] | (out[4 * i + 1] << 8) | (out[4 * i + 2] << 16) | (static_cast<uint32_t>(out[4 * i + 3]) << 24);
  codes[2 * t] = make_uint4(o32[0], o32[1], o32[2], o32[3]);
  codes[2 * t + 1] = make_uint4(o32[4], o32[5], o32[6], o32[7]);
}

}  // namespace

hipError_t launch_unpack_rtn(const void *planes, int K, int N, int bits, uint8_t *codes, hipStream_t s) {
  const long columns = static_cast<long>(N) * (K / kGroup) * 4;
  if (columns == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>((columns + 255) / 256);
  const uint32_t *pl = reinterpret_cast<const uint32_t *>(planes);
  uint4 *out = reinterpret_cast<uint4 *>(codes);
  switch (bits) {
    case 2: hipLaunchKernelGGL(unpack_rtn_kernel<2>, dim3(grid), dim3(256), 0, s, pl, out, columns); break;
    case 3: hipLaunchKernelGGL(unpack_rtn_kernel<3>, dim3(grid), dim3(256), 0, s, pl, out, columns); break;
    case 4: hipLaunchKernelGGL(unpack_rtn_kernel<4>, dim3(grid), dim3(256), 0, s, pl, out, columns); break;
    default: hipLaunchKernelGGL(unpack_rtn_kernel<8>, dim3(grid), dim3(256), 0, s, pl, out, columns); break;
  }
  return hipGetLastError();
}

}  // namespace lbq
