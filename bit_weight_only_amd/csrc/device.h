// Device-side building blocks shared by the HIP kernels: bit-plane merging and
// the fp16 "mantissa insert" decode that turns packed codes into operands of
// v_dot2_f32_f16 / MFMA without a per-weight integer-to-float conversion.
//
// Packed RTN format (include/lbq.h): bit j of word w of plane p is bit p of
// code q[128 g + 32 w + j] (bit-planes in 32-bit words: Qwen3-8B BPDQ model
// card, opening paragraph).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lbq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kGroup = 128;

// Single-instruction bit operations. Written as (non-volatile) inline asm so the
// compiler keeps one v_bfi_b32 per merged word and one v_and_or_b32 per decoded
// slot, with the masks in SGPRs and the fp16 constant in a VGPR; left to
// itself it fuses the merge into every slot extraction and splits the OR of the
// constant into a second instruction.
__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(mask), "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(c));
  return r;
}

// Two 1-bit planes of one 32-code word column -> two words of 2-bit fields.
// e: field p (bits 2p, 2p+1) = code 2p;  o: field p = code 2p + 1.
__device__ __forceinline__ void merge2(uint32_t p0, uint32_t p1, uint32_t &e, uint32_t &o) {
  e = bfi(0x55555555u, p0, p1 << 1);
  o = bfi(0x55555555u, p0 >> 1, p1);
}

// Three or four 1-bit planes -> four words of 4-bit fields (nibbles).
// n[r] nibble i (bits 4i..4i+3) = code 4i + r. A 3-bit code has a zero top bit.
template <int BITS>
__device__ __forceinline__ void merge_nibbles(const uint32_t *p, uint32_t n[4]) {
  uint32_t e01, o01, e23, o23;
  merge2(p[0], p[1], e01, o01);
  if constexpr (BITS == 4) {
    merge2(p[2], p[3], e23, o23);
  } else {
    e23 = p[2] & 0x55555555u;
    o23 = (p[2] >> 1) & 0x55555555u;
  }
  n[0] = bfi(0x33333333u, e01, e23 << 2);   // codes 4i
  n[2] = bfi(0x33333333u, e01 >> 2, e23);   // codes 4i + 2
  n[1] = bfi(0x33333333u, o01, o23 << 2);   // codes 4i + 1
  n[3] = bfi(0x33333333u, o01 >> 2, o23);   // codes 4i + 3
}

// fp16 1.0 in both halves. OR-ing a code q into mantissa bits m.. of 1.0 gives
// the exact fp16 value 1 + q * 2^(m - 10).
constexpr uint32_t kOne2 = 0x3C003C00u;

// fp16 2^(10 - m) in both halves. OR-ing a code q into mantissa bits m.. of it
// gives the exact fp16 value 2^(10 - m) + q: the code with a class-dependent
// offset and weight 1 in every class.
__host__ __device__ constexpr uint32_t biased_one2(int m) {
  return static_cast<uint32_t>(25 - m) << 10 | static_cast<uint32_t>(25 - m) << 26;
}

// Decode one 32-code word column into 16 half2 "slots". Slot c holds the codes
// of positions c and c + 16 (lo, hi half) encoded as 1 + q * 2^(m(c) - 10), with
// m(c) the class of the slot (BIASED: as 2^(10 - m(c)) + q). The activations
// are staged in the same slot order: slot c pairs x[c] with x[c + 16].
//
// 2-bit: slot 2p / 2p+1 comes from field p of e / o; fields 0..4 sit at
// m = 0, 2, 4, 6, 8 directly, fields 5..7 after a shift by 6 at m = 4, 6, 8.
// Class index (m / 2): {0,0,1,1,2,2,3,3,4,4,2,2,3,3,4,4}.
template <bool BIASED = false>
__device__ __forceinline__ void decode_slots2(uint32_t p0, uint32_t p1, uint32_t h[16]) {
  uint32_t e, o;
  merge2(p0, p1, e, o);
  const uint32_t e6 = e >> 6, o6 = o >> 6;
  const uint32_t c0 = BIASED ? biased_one2(0) : kOne2, c2 = BIASED ? biased_one2(2) : kOne2;
  const uint32_t c4 = BIASED ? biased_one2(4) : kOne2, c6 = BIASED ? biased_one2(6) : kOne2;
  const uint32_t c8 = BIASED ? biased_one2(8) : kOne2;
  h[0] = and_or(e, 0x00030003u, c0);
  h[1] = and_or(o, 0x00030003u, c0);
  h[2] = and_or(e, 0x000C000Cu, c2);
  h[3] = and_or(o, 0x000C000Cu, c2);
  h[4] = and_or(e, 0x00300030u, c4);
  h[5] = and_or(o, 0x00300030u, c4);
  h[6] = and_or(e, 0x00C000C0u, c6);
  h[7] = and_or(o, 0x00C000C0u, c6);
  h[8] = and_or(e, 0x03000300u, c8);
  h[9] = and_or(o, 0x03000300u, c8);
  h[10] = and_or(e6, 0x00300030u, c4);
  h[11] = and_or(o6, 0x00300030u, c4);
  h[12] = and_or(e6, 0x00C000C0u, c6);
  h[13] = and_or(o6, 0x00C000C0u, c6);
  h[14] = and_or(e6, 0x03000300u, c8);
  h[15] = and_or(o6, 0x03000300u, c8);
}
// Class of each 2-bit slot (index into scale 2^(10 - 2*cls)).
__host__ __device__ constexpr int slot_class2(int c) {
  return (c < 10) ? (c >> 1) : ((c >> 1) - 3);
}

// 3/4-bit: slot 4p + r comes from nibble word r; nibbles p and p+4 of the word
// (for p = 0, 1) or of the word shifted by 8 (p = 2, 3). m = 0 for even p,
// m = 4 for odd p. Class index: 0 (m = 0) or 1 (m = 4).
template <int BITS, bool BIASED = false>
__device__ __forceinline__ void decode_slots_nib(const uint32_t *p, uint32_t h[16]) {
  uint32_t n[4];
  merge_nibbles<BITS>(p, n);
  const uint32_t c0 = BIASED ? biased_one2(0) : kOne2, c4 = BIASED ? biased_one2(4) : kOne2;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t w = n[r], w8 = n[r] >> 8;
    h[r] = and_or(w, 0x000F000Fu, c0);
    h[4 + r] = and_or(w, 0x00F000F0u, c4);
    h[8 + r] = and_or(w8, 0x000F000Fu, c0);
    h[12 + r] = and_or(w8, 0x00F000F0u, c4);
  }
}
__host__ __device__ constexpr int slot_class_nib(int c) { return (c >> 2) & 1; }

// Weight 2^(10 - m) of a slot for the activation-sum correction.
template <int BITS>
__host__ __device__ constexpr float slot_weight(int c) {
  if constexpr (BITS == 2) {
    return static_cast<float>(1 << (10 - 2 * slot_class2(c)));
  } else {
    return slot_class_nib(c) ? 64.0f : 1024.0f;
  }
}
template <int BITS>
__host__ __device__ constexpr int num_classes() { return BITS == 2 ? 5 : 2; }
template <int BITS>
__host__ __device__ constexpr int slot_class(int c) {
  if constexpr (BITS == 2) return slot_class2(c);
  else return slot_class_nib(c);
}
template <int BITS>
__host__ __device__ constexpr int first_slot_of_class(int cls) {
  for (int c = 0; c < 16; ++c)
    if (slot_class<BITS>(c) == cls) return c;
  return -1;
}
template <int BITS>
__host__ __device__ constexpr float class_weight(int cls) {
  if constexpr (BITS == 2) return static_cast<float>(1 << (10 - 2 * cls));
  else return cls ? 64.0f : 1024.0f;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

__device__ __forceinline__ float half_lo(uint32_t v) {
  return static_cast<float>(__builtin_bit_cast(half2_t, v)[0]);
}
__device__ __forceinline__ float half_hi(uint32_t v) {
  return static_cast<float>(__builtin_bit_cast(half2_t, v)[1]);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

// Value of lane (l ^ X) for lane l, in registers (no LDS crossbar): DPP for
// X = 1, 2, 4 (half-row mirror then quad reversal), 8 (row rotate by 8);
// v_permlane16_swap / v_permlane32_swap of the value with itself for 16 / 32
// (each returns the two 16-lane (32-lane) halves exchanged in one of its two
// results; the lane picks the one holding its partner).
template <int X>
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t v) {
  const int i = static_cast<int>(v);
  if constexpr (X == 1) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, i, 0xB1, 0xF, 0xF, false));
  } else if constexpr (X == 2) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, i, 0x4E, 0xF, 0xF, false));
  } else if constexpr (X == 4) {
    const int m = __builtin_amdgcn_update_dpp(0, i, 0x141, 0xF, 0xF, false);
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, m, 0x1B, 0xF, 0xF, false));
  } else if constexpr (X == 8) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, i, 0x128, 0xF, 0xF, false));
  } else if constexpr (X == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
  } else {
    static_assert(X == 32, "xor distance");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
}

// fp8 e4m3 (OCP "fn": bias 7, no infinities, S.1111.111 = NaN) to fp16 bits.
// Every finite e4m3 value is exact in fp16.
__device__ __forceinline__ uint32_t e4m3_to_f16_bits(uint32_t b) {
  const uint32_t sign = (b & 0x80u) << 8;
  const uint32_t e = (b >> 3) & 0xFu, m = b & 7u;
  if (e == 15 && m == 7) return sign | 0x7E00u;
  if (e == 0) {  // subnormal m * 2^-9, normal in fp16
    return sign | f32_to_f16_bits(static_cast<float>(m) * 0.001953125f);
  }
  return sign | ((e + 8) << 10) | (m << 7);
}

// Fold a 32-element chunk of fp16 activations (16 dwords a[0..15], a[i] =
// x[2i] | x[2i+1] << 16) into the 16 slots: slot c = (x[c], x[c + 16]).
__device__ __forceinline__ void fold32(const uint32_t a[16], uint32_t s[16]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s[2 * i] = (a[i] & 0xFFFFu) | (a[i + 8] << 16);
    s[2 * i + 1] = (a[i] >> 16) | (a[i + 8] & 0xFFFF0000u);
  }
}

}  // namespace lbq
