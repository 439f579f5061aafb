// Activation rotation: x' = R x per token row, R = blockdiag(c * H_128 * diag(s)).
// One wavefront per 128-block: each lane holds two neighbouring elements; the
// first butterfly stage is in-lane, the next six exchange values with the lane
// whose index differs in one bit (a cross-lane swizzle, no LDS traffic).
// Arithmetic in fp32, result rounded to fp16 (activations are contracted in
// fp16). The rotation is the one the weights were quantized in (LLaDA2.2-mini
// Orin Nano model card: Hadamard-rotated basis with stored signs; Pingala-8
// model card, "What this is": random Hadamard rotation).
#include "gemv_core.h"
#include "kernels.h"

namespace lbq {

__global__ void __launch_bounds__(256) rotate_kernel(const uint32_t *__restrict__ x, const int8_t *__restrict__ signs,
                                                     uint32_t *__restrict__ out, int M, int K) {
  const int lane = threadIdx.x & 63;
  const int blocks_per_row = K / kGroup;
  const long blk = static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (blk >= static_cast<long>(M) * blocks_per_row) return;
  const int m = static_cast<int>(blk / blocks_per_row);
  const int b = static_cast<int>(blk % blocks_per_row);
  const long base = static_cast<long>(m) * K + b * kGroup;  // element index
  const uint32_t xv = x[(base >> 1) + lane];
  const int k0 = b * kGroup + 2 * lane;
  float v0 = half_lo(xv) * static_cast<float>(signs[k0]);
  float v1 = half_hi(xv) * static_cast<float>(signs[k0 + 1]);
  fwht128_wave(v0, v1, lane);
  const float c = kInvSqrt128;
  out[(base >> 1) + lane] = static_cast<uint32_t>(f32_to_f16_bits(v0 * c)) |
                            (static_cast<uint32_t>(f32_to_f16_bits(v1 * c)) << 16);
}

hipError_t launch_rotate(const uint16_t *x, int M, int K, const int8_t *signs, uint16_t *out, hipStream_t s) {
  const long nblk = static_cast<long>(M) * (K / kGroup);
  if (nblk == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>((nblk + 3) / 4);
  hipLaunchKernelGGL(rotate_kernel, dim3(grid), dim3(256), 0, s, reinterpret_cast<const uint32_t *>(x), signs,
                     reinterpret_cast<uint32_t *>(out), M, K);
  return hipGetLastError();
}

}  // namespace lbq
