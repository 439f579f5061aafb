// Shared inner loop of the RTN dequant-GEMVs (dense linear and MoE experts).
//
// Activations for MT tokens and a chunk of Gc groups are staged in LDS in the
// folded slot order (slot c of each 32-chunk = (x[c], x[c + 16])) together
// with per-group sums P_g = sum_k 2^(10-m_k) x_k and T_g = sum_k x_k. Each
// lane then decodes 128-code groups of one output row and accumulates
//   s * (sum_cls 2^(10-m_cls) acc_cls - P_g - z T_g) = s * sum_k x_k (q_k - z)
// into per-token partials (see device.h for the slot encoding).
#pragma once

#include "device.h"

namespace lbq {

constexpr int kGemvThreads = 256;
constexpr int kGroupStride = 68;   // u32 per staged group (64 slots + 16 B pad against bank conflicts)

// Bytes of LDS one staged group costs per token (slots + the float2 sums).
constexpr int kStagedGroupBytes = kGroupStride * 4 + 8;

// Stage groups [g0, g0 + gn) of MT tokens. Token m's rotated activations start
// at row_ptr(m) (u32 pairs of fp16); tokens m >= count are zero-filled.
template <int BITS, int MT, class RowPtr>
__device__ __forceinline__ void stage_groups(RowPtr row_ptr, int count, int g0, int gn, int Gc, uint32_t *xx,
                                             float2 *sums) {
  for (int u = threadIdx.x; u < MT * gn; u += blockDim.x) {
    const int m = u / gn, g = u - m * gn;
    uint32_t *dst = xx + (m * Gc + g) * kGroupStride;
    float P = 0.f, T = 0.f;
    if (m < count) {
      const uint4 *src = reinterpret_cast<const uint4 *>(row_ptr(m) + static_cast<size_t>(g0 + g) * 64);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t a[16], s[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 v = src[w * 4 + i];
          a[4 * i] = v.x;
          a[4 * i + 1] = v.y;
          a[4 * i + 2] = v.z;
          a[4 * i + 3] = v.w;
        }
        fold32(a, s);
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const float pair = half_lo(s[c]) + half_hi(s[c]);
          P += slot_weight<BITS>(c) * pair;
          T += pair;
        }
        uint4 *d4 = reinterpret_cast<uint4 *>(dst + w * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) d4[i] = make_uint4(s[4 * i], s[4 * i + 1], s[4 * i + 2], s[4 * i + 3]);
      }
    } else {
      uint4 *d4 = reinterpret_cast<uint4 *>(dst);
#pragma unroll
      for (int i = 0; i < 16; ++i) d4[i] = make_uint4(0, 0, 0, 0);
    }
    sums[m * Gc + g] = make_float2(P, T);
  }
}

// One lane's share of one row: groups g = j, j + L, ... < gn of the staged
// chunk. prow points at the row's planes for the chunk's first group, mrow at
// its (scale, zero) words. Adds into yacc[MT].
template <int BITS, int MT, int L>
__device__ __forceinline__ void row_partial(const uint4 *__restrict__ prow, const uint32_t *__restrict__ mrow,
                                            const uint32_t *xx, const float2 *sums, int Gc, int gn, int j,
                                            float yacc[MT]) {
  constexpr int NC = num_classes<BITS>();
  for (int g = j; g < gn; g += L) {
    uint4 pv[BITS];
#pragma unroll
    for (int p = 0; p < BITS; ++p) pv[p] = prow[g * BITS + p];
    const uint32_t mt = mrow[g];
    float acc[MT][NC];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[m][c] = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t pw[BITS];
#pragma unroll
      for (int p = 0; p < BITS; ++p) pw[p] = (w == 0) ? pv[p].x : (w == 1) ? pv[p].y : (w == 2) ? pv[p].z : pv[p].w;
      uint32_t h[16];
      if constexpr (BITS == 2) decode_slots2(pw[0], pw[1], h);
      else decode_slots_nib<BITS>(pw, h);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint4 *xs = reinterpret_cast<const uint4 *>(xx + (m * Gc + g) * kGroupStride + w * 16);
        uint32_t xv[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 v = xs[i];
          xv[4 * i] = v.x;
          xv[4 * i + 1] = v.y;
          xv[4 * i + 2] = v.z;
          xv[4 * i + 3] = v.w;
        }
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const int cls = slot_class<BITS>(c);
          // the first slot of a class in the first word starts its accumulator
          acc[m][cls] = dot2(h[c], xv[c], (w == 0 && c == first_slot_of_class<BITS>(cls)) ? 0.f : acc[m][cls]);
        }
      }
    }
    const float sc = f16_bits_to_f32(mt & 0xFFFFu);
    const float zp = f16_bits_to_f32(mt >> 16);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float2 pt = sums[m * Gc + g];
      float t = -pt.x;
#pragma unroll
      for (int c = 0; c < NC; ++c) t = fmaf(class_weight<BITS>(c), acc[m][c], t);
      t = fmaf(-zp, pt.y, t);
      yacc[m] = fmaf(sc, t, yacc[m]);
    }
  }
}

// U rows at once: the loads of all U rows' planes and (scale, zero) words for a
// group are issued before any of them is decoded, so U memory round trips
// overlap; the staged activations of a slot are read once for all U rows.
// prow[u] / mrow[u] as in row_partial; adds into yacc[u][MT].
template <int BITS, int MT, int L, int U>
__device__ __forceinline__ void rows_partial(const uint4 *const *prow, const uint32_t *const *mrow,
                                             const uint32_t *xx, const float2 *sums, int Gc, int gn, int j,
                                             float (&yacc)[U][MT]) {
  constexpr int NC = num_classes<BITS>();
  for (int g = j; g < gn; g += L) {
    uint4 pv[U][BITS];
    uint32_t mw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int p = 0; p < BITS; ++p) pv[u][p] = prow[u][g * BITS + p];
      mw[u] = mrow[u][g];
    }
    float acc[U][MT][NC];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t h[U][16];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        uint32_t pw[BITS];
#pragma unroll
        for (int p = 0; p < BITS; ++p)
          pw[p] = (w == 0) ? pv[u][p].x : (w == 1) ? pv[u][p].y : (w == 2) ? pv[u][p].z : pv[u][p].w;
        if constexpr (BITS == 2) decode_slots2(pw[0], pw[1], h[u]);
        else decode_slots_nib<BITS>(pw, h[u]);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint4 *xs = reinterpret_cast<const uint4 *>(xx + (m * Gc + g) * kGroupStride + w * 16);
        uint32_t xv[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 v = xs[i];
          xv[4 * i] = v.x;
          xv[4 * i + 1] = v.y;
          xv[4 * i + 2] = v.z;
          xv[4 * i + 3] = v.w;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            const int cls = slot_class<BITS>(c);
            acc[u][m][cls] =
                dot2(h[u][c], xv[c], (w == 0 && c == first_slot_of_class<BITS>(cls)) ? 0.f : acc[u][m][cls]);
          }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float sc = f16_bits_to_f32(mw[u] & 0xFFFFu);
      const float zp = f16_bits_to_f32(mw[u] >> 16);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float2 pt = sums[m * Gc + g];
        float t = -pt.x;
#pragma unroll
        for (int c = 0; c < NC; ++c) t = fmaf(class_weight<BITS>(c), acc[u][m][c], t);
        t = fmaf(-zp, pt.y, t);
        yacc[u][m] = fmaf(sc, t, yacc[u][m]);
      }
    }
  }
}

// Sum per-lane partials over the L lanes that share a row (aligned clusters).
template <int MT, int L>
__device__ __forceinline__ void reduce_cluster(float yacc[MT]) {
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int off = L / 2; off > 0; off >>= 1) yacc[m] += __shfl_xor(yacc[m], off);
  }
}

// Randomized Hadamard transform of one 128-block held two values per lane
// (element 2l + e in lane l): fp32 butterflies, in-lane first stage, then six
// cross-lane stages. Unnormalised; the caller multiplies by 1/sqrt(128).
__device__ __forceinline__ void fwht128_wave(float &v0, float &v1, int lane) {
  const float a = v0 + v1, b = v0 - v1;
  v0 = a;
  v1 = b;
#pragma unroll
  for (int hl = 1; hl < 64; hl <<= 1) {
    const float p0 = __shfl_xor(v0, hl);
    const float p1 = __shfl_xor(v1, hl);
    const bool upper = (lane & hl) != 0;
    v0 = upper ? (p0 - v0) : (v0 + p0);
    v1 = upper ? (p1 - v1) : (v1 + p1);
  }
}

constexpr float kInvSqrt128 = 0.08838834764831845f;

}  // namespace lbq
