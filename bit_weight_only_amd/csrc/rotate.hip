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
#include "mx_core.h"

#include <algorithm>

namespace lbq {

// Natural-order rotation, one 128-block per wavefront (two values per lane);
// workgroup 0 also clears n_counters u32 counters (a product-VQ GEMM's split-K
// arrival counters) ahead of the GEMM launch that uses them.
__global__ void __launch_bounds__(256) rotate_kernel(const uint32_t *__restrict__ x, const int8_t *__restrict__ signs,
                                                     uint32_t *__restrict__ out, int M, int K,
                                                     uint32_t *__restrict__ counters, int n_counters) {
  if (blockIdx.x == 0)
    for (int i = static_cast<int>(threadIdx.x); i < n_counters; i += 256) counters[i] = 0;
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
// each 32-element chunk, u32 slot c holds (x'[c], x'[c + 16]). With tz non-null
// it also writes, per (token m, group g), the group sum T = sum_k x'_k of the
// fp16-rounded x' as the fp16 pair (T/16 rounded, the rounding of what is
// left) at tz[m * Gp + g], Gp = K/128 rounded up to a multiple of 16, and zero
// pairs for g in [K/128, Gp): the RTN GEMM's zero-point term. It clears
// n_counters u32 counters (the GEMM's split-K arrival counters) before the GEMM
// launch that uses them.
//
// Eight lanes rotate one (token, group) unit, sixteen values each, as in the
// matrix-core GEMV's prologue: three cross-lane butterfly stages as DPP
// multiply-adds, four in-lane stages (every exchange stays in registers; one
// block per wavefront with two values per lane needed seven LDS-crossbar
// shuffles for the butterflies and six more for the sum). Lane L holds the
// 16-value half L & 1 of chunk L >> 1; the even and odd lanes of a chunk swap
// half their values with one DPP move each, and each writes eight whole slots.
//
// With SWIGLU the rows are not read from x but formed from fp32 gate|up
// results h [M][2K] (gate in columns 0..K-1, up in K..2K-1): the value at k is
// silu(h[m][k]) h[m][K + k] rounded to fp16, the routed experts' SwiGLU
// intermediate, rotated with the ffn signs for their down linear.
template <bool SWIGLU>
__global__ void __launch_bounds__(256) rotate_folded_kernel(const uint32_t *__restrict__ x, const float *__restrict__ h,
                                                            const int8_t *__restrict__ signs,
                                                            uint32_t *__restrict__ out, uint32_t *__restrict__ tz,
                                                            int M, int K, int Gp, uint32_t *__restrict__ counters,
                                                            int n_counters) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n_counters; i += gridDim.x * 256) counters[i] = 0;
  const int G = K / kGroup;
  const int tid = static_cast<int>(threadIdx.x);
  const long unit = static_cast<long>(blockIdx.x) * 32 + mx::rot_unit_of(tid);
  const int L = mx::rot_lane_of(tid);
  const bool ok = unit < static_cast<long>(M) * G;   // the unit's eight lanes agree
  const int m = ok ? static_cast<int>(unit / G) : 0, g = ok ? static_cast<int>(unit - static_cast<long>(m) * G) : 0;
  // buffer loads: lanes without a unit load zeros (every lane takes part in the
  // DPP exchanges below)
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(signs), 0, K, 0x00020000);
  mx::RotIn in;
  if constexpr (SWIGLU) {
    const __amdgpu_buffer_rsrc_t hrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(h), 0, M * K * 8,
                                                                          0x00020000);
    const uint32_t bad = ok ? 0u : mx::kOutOfRange;
    const uint32_t go = static_cast<uint32_t>((m * 2 * K + g * kGroup + 16 * L) * 4) + bad;
    const uint32_t uo = go + static_cast<uint32_t>(K * 4);
    float gv[16], uv[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 a = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(hrs, go + 16 * q, 0, 0));
      const float4 c = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(hrs, uo + 16 * q, 0, 0));
      gv[4 * q] = a.x;
      gv[4 * q + 1] = a.y;
      gv[4 * q + 2] = a.z;
      gv[4 * q + 3] = a.w;
      uv[4 * q] = c.x;
      uv[4 * q + 1] = c.y;
      uv[4 * q + 2] = c.z;
      uv[4 * q + 3] = c.w;
    }
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float a0 = gv[2 * i] / (1.f + __expf(-gv[2 * i])) * uv[2 * i];
      const float a1 = gv[2 * i + 1] / (1.f + __expf(-gv[2 * i + 1])) * uv[2 * i + 1];
      w[i] = static_cast<uint32_t>(f32_to_f16_bits(a0)) | (static_cast<uint32_t>(f32_to_f16_bits(a1)) << 16);
    }
    in.xa = make_uint4(w[0], w[1], w[2], w[3]);
    in.xb = make_uint4(w[4], w[5], w[6], w[7]);
    in.sv = __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(srs, static_cast<uint32_t>(g * kGroup + 16 * L) + bad, 0, 0));
  } else {
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(x), 0,
                                                                          M * K * 2, 0x00020000);
    in = mx::rot_load(xrs, srs, K, m, g, L, ok);
  }
  float v[16];
  {
    const uint32_t xw[8] = {in.xa.x, in.xa.y, in.xa.z, in.xa.w, in.xb.x, in.xb.y, in.xb.z, in.xb.w};
    const uint32_t sw[4] = {in.sv.x, in.sv.y, in.sv.z, in.sv.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // sign bytes of elements 2i, 2i + 1 onto the fp16 sign bits 15 and 31
      const uint32_t sb = __builtin_amdgcn_perm(sw[i >> 1], sw[i >> 1], (i & 1) ? 0x030C020Cu : 0x010C000Cu);
      const uint32_t h = xw[i] ^ (sb & 0x80008000u);
      v[2 * i] = half_lo(h);
      v[2 * i + 1] = half_hi(h);
    }
  }
  // cross-lane stages: the lane whose bit is set gets the negated butterfly
  // output, so lane L ends up holding (-1)^popcount(L) times its values
  mx::dpp_butterfly16<0>(v, (L & 1) ? -1.f : 1.f);
  mx::dpp_butterfly16<1>(v, (L & 2) ? -1.f : 1.f);
  mx::dpp_butterfly16<2>(v, (L & 4) ? -1.f : 1.f);
#pragma unroll
  for (int hw = 1; hw < 16; hw <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & hw) == 0) {
        const float a = v[i], c = v[i + hw];
        v[i] = a + c;
        v[i + hw] = a - c;
      }
    }
  }
  const float c = (__builtin_popcount(L) & 1) ? -kInvSqrt128 : kInvSqrt128;
  uint32_t r[16];
  float T = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    r[i] = f32_to_f16_bits(v[i] * c);
    T += f16_bits_to_f32(r[i]);
  }
  // the even lane of a chunk needs its partner's values 0..7, the odd lane its
  // partner's 8..15
  const bool odd = L & 1;
  uint32_t got[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    got[i] = static_cast<uint32_t>(
        __builtin_amdgcn_mov_dpp(static_cast<int>(odd ? r[i] : r[8 + i]), mx::kDppXor1, 0xF, 0xF, true));
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = odd ? (got[i] | (r[8 + i] << 16)) : (r[i] | (got[i] << 16));
  if (ok) {
    uint4 *dst = reinterpret_cast<uint4 *>(out + ((static_cast<long>(m) * K + g * kGroup) >> 1) + (L >> 1) * 16 +
                                           (odd ? 8 : 0));
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
  if (!tz) return;
  T += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, T), mx::kDppXor1, 0xF, 0xF, true));
  T += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, T), mx::kDppXor2, 0xF, 0xF, true));
  T += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, T), mx::kDppXor8, 0xF, 0xF, true));
  if (!ok) return;
  uint32_t *row = tz + static_cast<long>(m) * Gp;
  if (L == 0) {
    const float t16 = T * 0.0625f;
    const uint32_t th = f32_to_f16_bits(t16);
    const uint32_t tl = f32_to_f16_bits(t16 - f16_bits_to_f32(th));
    row[g] = th | (tl << 16);
  }
  if (g == G - 1)
    for (int gz = G + L; gz < Gp; gz += 8) row[gz] = 0;
}

hipError_t launch_swiglu_rotate_folded(const float *h, int M, int K, const int8_t *signs, uint16_t *out,
                                       uint32_t *tz, hipStream_t s) {
  // 32 (row, group) units per workgroup; h is read through 32-bit buffer
  // offsets (M * 2K floats stay below 2 GiB: checked by the caller)
  const long nblk = static_cast<long>(M) * (K / kGroup);
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(rotate_folded_kernel<true>, dim3(static_cast<unsigned>((nblk + 31) / 32)), dim3(256), 0, s,
                     nullptr, h, signs, reinterpret_cast<uint32_t *>(out), tz, M, K, gemm_tz_stride(K), nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_rotate_folded(const uint16_t *x, int M, int K, const int8_t *signs, uint16_t *out, uint32_t *tz,
                                uint32_t *counters, int n_counters, hipStream_t s, int max_tokens) {
  // 32 (token, group) units per workgroup; buffer offsets are 32-bit, so the
  // tokens go in launches of under 1 GiB of activations each (the first also
  // clears the counters); max_tokens > 0 caps a launch lower
  const int Gp = gemm_tz_stride(K);
  int per = std::max(1, static_cast<int>((1L << 30) / (static_cast<long>(K) * 2)));
  if (max_tokens > 0 && max_tokens < per) per = max_tokens;
  int m0 = 0;
  do {
    const int Mc = std::min(per, M - m0);
    const long nblk = static_cast<long>(Mc) * (K / kGroup);
    const int nc = m0 == 0 ? n_counters : 0;
    const long need = std::max<long>((nblk + 31) / 32, (nc + 255) / 256);
    if (need > 0)
      hipLaunchKernelGGL(rotate_folded_kernel<false>, dim3(static_cast<unsigned>(need)), dim3(256), 0, s,
                         reinterpret_cast<const uint32_t *>(x + static_cast<long>(m0) * K), nullptr, signs,
                         reinterpret_cast<uint32_t *>(out + static_cast<long>(m0) * K),
                         tz ? tz + static_cast<long>(m0) * Gp : nullptr, Mc, K, Gp, counters, nc);
    m0 += Mc;
  } while (m0 < M);
  return hipGetLastError();
}

hipError_t launch_rotate_clear(const uint16_t *x, int M, int K, const int8_t *signs, uint16_t *out,
                               uint32_t *counters, int n_counters, hipStream_t s) {
  const long nblk = static_cast<long>(M) * (K / kGroup);
  if (nblk == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>((nblk + 3) / 4);
  hipLaunchKernelGGL(rotate_kernel, dim3(grid), dim3(256), 0, s, reinterpret_cast<const uint32_t *>(x), signs,
                     reinterpret_cast<uint32_t *>(out), M, K, counters, n_counters);
  return hipGetLastError();
}

hipError_t launch_rotate(const uint16_t *x, int M, int K, const int8_t *signs, uint16_t *out, hipStream_t s) {
  return launch_rotate_clear(x, M, K, signs, out, nullptr, 0, s);
}

}  // namespace lbq
