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

#include <algorithm>

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

// Same rotation, written in the folded slot order the MFMA GEMMs stage: in
// each 32-element chunk, u32 slot c holds (x'[c], x'[c + 16]). Lane l and lane
// l ^ 8 hold the two halves of the same slots and swap one value, so every lane
// writes one whole slot. With tz non-null it also writes, per (token m, group
// g), the group sum T = sum_k x'_k of the fp16-rounded x' as the fp16 pair
// (T/16 rounded, the rounding of what is left) at tz[m * Gp + g], Gp = K/128
// rounded up to a multiple of 16, and zero pairs for g in [K/128, Gp): the RTN
// GEMM's zero-point term. It clears n_counters u32 counters (the GEMM's
// split-K arrival counters) before the GEMM launch that uses them.
__global__ void __launch_bounds__(256) rotate_folded_kernel(const uint32_t *__restrict__ x,
                                                            const int8_t *__restrict__ signs,
                                                            uint32_t *__restrict__ out, uint32_t *__restrict__ tz,
                                                            int M, int K, int Gp, uint32_t *__restrict__ counters,
                                                            int n_counters) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n_counters; i += gridDim.x * 256) counters[i] = 0;
  const int lane = threadIdx.x & 63;
  const int blocks_per_row = K / kGroup;
  const long blk = static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (blk >= static_cast<long>(M) * blocks_per_row) return;
  const int m = static_cast<int>(blk / blocks_per_row);
  const int b = static_cast<int>(blk % blocks_per_row);
  const long base = static_cast<long>(m) * K + b * kGroup;
  const uint32_t xv = x[(base >> 1) + lane];
  const int k0 = b * kGroup + 2 * lane;
  float v0 = half_lo(xv) * static_cast<float>(signs[k0]);
  float v1 = half_hi(xv) * static_cast<float>(signs[k0 + 1]);
  fwht128_wave(v0, v1, lane);
  const uint32_t r0 = f32_to_f16_bits(v0 * kInvSqrt128), r1 = f32_to_f16_bits(v1 * kInvSqrt128);
  // element 2l (+1) is slot (2l & 15) (+1) of chunk l >> 4, half (l >> 3) & 1
  const bool hi = (lane >> 3) & 1;
  const uint32_t give = hi ? r0 : r1;
  const uint32_t got = static_cast<uint32_t>(__shfl_xor(static_cast<int>(give), 8));
  const uint32_t word = hi ? (got | (r1 << 16)) : (r0 | (got << 16));
  const int slot = ((2 * lane) & 15) + (hi ? 1 : 0);
  out[(base >> 1) + (lane >> 4) * 16 + slot] = word;
  if (!tz) return;
  float T = f16_bits_to_f32(r0) + f16_bits_to_f32(r1);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) T += __shfl_xor(T, off);
  uint32_t *row = tz + static_cast<long>(m) * Gp;
  if (lane == 0) {
    const float t16 = T * 0.0625f;
    const uint32_t th = f32_to_f16_bits(t16);
    const uint32_t tl = f32_to_f16_bits(t16 - f16_bits_to_f32(th));
    row[b] = th | (tl << 16);
  }
  if (b == blocks_per_row - 1)
    for (int g = blocks_per_row + lane; g < Gp; g += 64) row[g] = 0;
}

hipError_t launch_rotate_folded(const uint16_t *x, int M, int K, const int8_t *signs, uint16_t *out, uint32_t *tz,
                                uint32_t *counters, int n_counters, hipStream_t s) {
  const long nblk = static_cast<long>(M) * (K / kGroup);
  const long need = std::max<long>((nblk + 3) / 4, (n_counters + 255) / 256);
  if (need == 0) return hipSuccess;
  hipLaunchKernelGGL(rotate_folded_kernel, dim3(static_cast<unsigned>(need)), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t *>(x), signs, reinterpret_cast<uint32_t *>(out), tz, M, K,
                     gemm_tz_stride(K), counters, n_counters);
  return hipGetLastError();
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
