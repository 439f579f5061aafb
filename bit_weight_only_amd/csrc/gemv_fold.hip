// Dequant-GEMV for one or two tokens, activation rotation fused into the
// prologue (one launch per linear).
//
// Each workgroup first rotates the raw activations x' = R x itself (eight
// lanes per 128-block, fp32 butterflies, fp16 out) straight into LDS, in the
// decoders' folded slot order (slot c of each 32-chunk = (x'[c], x'[c+16]))
// and transposed so chunk q of group g lives at [q][g]: lanes that decode
// consecutive groups read consecutive 16-byte words. Per group it also keeps
// the sums the decoders subtract (P over the slot classes, T = sum of x').
// The first code item is already in flight while this runs.
//
// Then it walks row tiles t = blockIdx.x, blockIdx.x + gridDim.x, ... as a
// persistent grid. L lanes share a row and each takes groups g = j, j + L, ...;
// RB rows per lane share every activation read. Codes are prefetched one work
// item ahead in registers, with unconditional loads at clamped indices so the
// compiler keeps exact wait counts (items past the end are computed and
// discarded).
//
// Every workgroup repeats the rotation, so this path only pays where K is
// small enough for that to hide behind the first loads (K <= 8192 at one
// token, K <= 4096 at two); longer rows and more tokens take the rotate +
// staged-GEMV path.
//
// Decode arithmetic is the one of gemv_core.h (mantissa insert into fp16 1.0,
// v_dot2_f32_f16, per-group correction s * (sum_cls w_cls acc_cls - P - z T)).
#include "gemv_core.h"
#include "kernels.h"

#include <hip/hip_ext.h>

namespace lbq {

namespace {

// Cross-lane moves within groups of 8 lanes (DPP, no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppQuadRev = 0x1B;  // quad_perm [3,2,1,0]; after the half-row mirror: lane ^ 4
template <int X>
__device__ __forceinline__ float xor_lane(float v) {
  if constexpr (X == 1) return dpp_f<kDppXor1>(v);
  else if constexpr (X == 2) return dpp_f<kDppXor2>(v);
  else return dpp_f<kDppQuadRev>(dpp_f<kDppHalfMirror>(v));
}

// Slot weight 2^(10-m) of slot c for the activation sums.
template <int BITS>
__device__ __forceinline__ float sum_weight(int c) { return slot_weight<BITS>(c); }

// Rotate the raw activations of MT tokens into LDS in the folded, chunk-major
// layout, with the group sums. Eight lanes per (token, group): lane b holds
// elements 16b .. 16b+15; four in-lane butterfly stages, three across lanes
// (lane ^ 1, ^ 2, ^ 4). Lanes b and b^1 hold the low and high halves of the
// same 16 slots and swap eight of them so each writes whole 16-byte words.
template <int BITS, int MT>
__device__ __forceinline__ void stage_rotate_fold(const uint4 *__restrict__ x, const uint4 *__restrict__ signs, int M,
                                                  int K, int G, uint4 *xs, float4 *ss) {
  const int lane8 = threadIdx.x & 7;
  const int units = MT * G;
  for (int q0 = threadIdx.x >> 3; q0 < units; q0 += blockDim.x >> 3) {
    const int m = q0 / G, g = q0 - (q0 / G) * G;
    uint4 xa = make_uint4(0, 0, 0, 0), xb = make_uint4(0, 0, 0, 0);
    if (m < M) {
      const uint4 *src = x + (static_cast<size_t>(m) * K + static_cast<size_t>(g) * kGroup + 16 * lane8) / 8;
      xa = src[0];
      xb = src[1];
    }
    const uint4 sv = signs[(g * kGroup + 16 * lane8) / 16];
    const uint32_t xw[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
    const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
    float v[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t sb = sw[i >> 1] >> (16 * (i & 1));       // sign bytes of elements 2i, 2i+1
      const uint32_t h = xw[i] ^ (((sb & 0x80u) << 8) | ((sb & 0x8000u) << 16));
      v[2 * i] = half_lo(h);
      v[2 * i + 1] = half_hi(h);
    }
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
    {
      const float sg = (lane8 & 1) ? -1.f : 1.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = fmaf(sg, v[i], xor_lane<1>(v[i]));
    }
    {
      const float sg = (lane8 & 2) ? -1.f : 1.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = fmaf(sg, v[i], xor_lane<2>(v[i]));
    }
    {
      const float sg = (lane8 & 4) ? -1.f : 1.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = fmaf(sg, v[i], xor_lane<4>(v[i]));
    }
    // round to fp16; element 16b + i is slot i of chunk b >> 1, half b & 1
    uint32_t r[16];
    float P = 0.f, T = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      r[i] = f32_to_f16_bits(v[i] * kInvSqrt128);
      const float rf = f16_bits_to_f32(r[i]);
      T += rf;
      P = fmaf(sum_weight<BITS>(i), rf, P);
    }
    // even lane keeps slots 0..7 (needs the partner's high halves of 0..7),
    // odd lane keeps slots 8..15 (needs the partner's low halves of 8..15)
    const bool odd = lane8 & 1;
    uint32_t out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t send = odd ? r[i] : r[8 + i];
      const uint32_t recv = dpp_u<kDppXor1>(send);
      out[i] = odd ? (recv | (r[8 + i] << 16)) : (r[i] | (recv << 16));
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
      P += (off == 1) ? xor_lane<1>(P) : (off == 2) ? xor_lane<2>(P) : xor_lane<4>(P);
      T += (off == 1) ? xor_lane<1>(T) : (off == 2) ? xor_lane<2>(T) : xor_lane<4>(T);
    }
    // 16-byte words of the group's 64 slots: chunk w = lane8 >> 1 holds words 4w .. 4w+3
    const int w = lane8 >> 1;
    const int q = 4 * w + (odd ? 2 : 0);
    xs[(m * 16 + q) * G + g] = make_uint4(out[0], out[1], out[2], out[3]);
    xs[(m * 16 + q + 1) * G + g] = make_uint4(out[4], out[5], out[6], out[7]);
    if (lane8 == 0) ss[m * G + g] = make_float4(BITS == 2 ? P : 0.f, BITS == 2 ? 0.f : P, T, 0.f);
  }
}

template <int BITS, int RB>
struct Item {
  uint4 p[RB][BITS];
  uint32_t m[RB];
};

// x: raw activations [M][K] fp16; signs: [K] int8 (+-1), 16-byte aligned.
template <int BITS, int MT, int L, int RB>
__global__ void __launch_bounds__(256) gemv_fold_kernel(const uint4 *__restrict__ planes,
                                                        const uint32_t *__restrict__ meta,
                                                        const uint4 *__restrict__ x, const uint4 *__restrict__ signs,
                                                        uint16_t *__restrict__ y, int M, int K, int N) {
  constexpr int RPW = 256 / L;        // row blocks per tile
  constexpr int ROWS = RPW * RB;      // rows per tile
  constexpr int NC = num_classes<BITS>();
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  const int G = K / kGroup;
  const int j = threadIdx.x % L, rb = threadIdx.x / L;
  const int U = (G + L - 1) / L;      // groups per lane per row
  const int tiles = (N + ROWS - 1) / ROWS;
  const int my_tiles = static_cast<int>(blockIdx.x) < tiles
                           ? (tiles - 1 - static_cast<int>(blockIdx.x)) / static_cast<int>(gridDim.x) + 1
                           : 0;
  const int n_items = my_tiles * U;

  // item i: tile blockIdx.x + (i / U) * gridDim.x, group j + (i % U) * L
  auto load_item = [&](int i, Item<BITS, RB> &it) {
    const int ic = min(i, max(n_items - 1, 0));
    const int t = min(static_cast<int>(blockIdx.x) + (ic / U) * static_cast<int>(gridDim.x), tiles - 1);
    const int g = min(j + (ic % U) * L, G - 1);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int row = min(t * ROWS + r * RPW + rb, N - 1);
      const uint4 *pr = planes + (static_cast<size_t>(row) * G + g) * BITS;
      it.m[r] = meta[static_cast<size_t>(row) * G + g];
#pragma unroll
      for (int p = 0; p < BITS; ++p) it.p[r][p] = pr[p];
    }
  };
  Item<BITS, RB> A, B;
  load_item(0, A);
  // activations of the MT tokens (tokens >= M are zero) and their group sums
  uint4 *xs = reinterpret_cast<uint4 *>(smem);
  float4 *ss = reinterpret_cast<float4 *>(smem + MT * G * 64);
  stage_rotate_fold<BITS, MT>(x, signs, M, K, G, xs, ss);
  __syncthreads();

  float yacc[MT][RB];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < RB; ++r) yacc[m][r] = 0.f;
  auto process = [&](int i, const Item<BITS, RB> &it) {
    const int t = static_cast<int>(blockIdx.x) + (i / U) * static_cast<int>(gridDim.x), u = i % U, g = j + u * L;
    if (g < G) {
      float acc[MT][RB][NC];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
          for (int c = 0; c < NC; ++c) acc[m][r][c] = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t h[RB][16];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          uint32_t pw[BITS];
#pragma unroll
          for (int p = 0; p < BITS; ++p)
            pw[p] = (w == 0) ? it.p[r][p].x : (w == 1) ? it.p[r][p].y : (w == 2) ? it.p[r][p].z : it.p[r][p].w;
          if constexpr (BITS == 2) decode_slots2(pw[0], pw[1], h[r]);
          else decode_slots_nib<BITS>(pw, h[r]);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          uint32_t xv[16];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint4 v = xs[(m * 16 + w * 4 + q) * G + g];
            xv[4 * q] = v.x;
            xv[4 * q + 1] = v.y;
            xv[4 * q + 2] = v.z;
            xv[4 * q + 3] = v.w;
          }
#pragma unroll
          for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int c = 0; c < 16; ++c) {
              const int cls = slot_class<BITS>(c);
              acc[m][r][cls] =
                  dot2(h[r][c], xv[c], (w == 0 && c == first_slot_of_class<BITS>(cls)) ? 0.f : acc[m][r][cls]);
            }
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float4 s4 = ss[m * G + g];
        const float P = (BITS == 2) ? s4.x : s4.y, T = s4.z;
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          float tt = -P;
#pragma unroll
          for (int c = 0; c < NC; ++c) tt = fmaf(class_weight<BITS>(c), acc[m][r][c], tt);
          tt = fmaf(-f16_bits_to_f32(it.m[r] >> 16), T, tt);
          yacc[m][r] = fmaf(f16_bits_to_f32(it.m[r] & 0xFFFFu), tt, yacc[m][r]);
        }
      }
    }
    if (u == U - 1) {   // row tile done: reduce over the L lanes of each row and store
#pragma unroll
      for (int m = 0; m < MT; ++m) reduce_cluster<RB, L>(yacc[m]);
      if (j == 0) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          const int row = t * ROWS + r * RPW + rb;
          if (row < N) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
              if (m < M) y[static_cast<size_t>(m) * N + row] = f32_to_f16_bits(yacc[m][r]);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < RB; ++r) yacc[m][r] = 0.f;
    }
  };
  for (int i = 0; i < n_items; i += 2) {
    load_item(i + 1, B);
    process(i, A);
    if (i + 1 >= n_items) break;
    load_item(i + 2, A);
    process(i + 1, B);
  }
}

template <int BITS, int MT, int L, int RB>
hipError_t launch_fold(const void *planes, const void *meta, const uint16_t *x, const int8_t *signs, uint16_t *y,
                       int M, int K, int N, int grid_cap, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  const int G = K / kGroup;
  const size_t lds = static_cast<size_t>(MT) * G * (256 + 16);
  auto kern = gemv_fold_kernel<BITS, MT, L, RB>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  constexpr int ROWS = (256 / L) * RB;
  const int tiles = (N + ROWS - 1) / ROWS;
  const unsigned grid = static_cast<unsigned>(min(tiles, grid_cap));
  const uint4 *pl = reinterpret_cast<const uint4 *>(planes);
  const uint32_t *mt = reinterpret_cast<const uint32_t *>(meta);
  const uint4 *xv = reinterpret_cast<const uint4 *>(x);
  const uint4 *sv = reinterpret_cast<const uint4 *>(signs);
  if (start || stop)   // the events take this kernel's own begin / end times
    hipExtLaunchKernelGGL(kern, dim3(grid), dim3(256), static_cast<uint32_t>(lds), s, start, stop, 0, pl, mt, xv, sv, y,
                          M, K, N);
  else
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, s, pl, mt, xv, sv, y, M, K, N);
  return hipGetLastError();
}

template <int BITS, int MT>
hipError_t launch_mt(const void *planes, const void *meta, const uint16_t *x, const int8_t *signs, uint16_t *y, int M,
                     int K, int N, int lanes, int rb, int grid_cap, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
#define LBQ_FOLD(LL, R)                                                                                   \
  if (lanes == LL && rb == R)                                                                             \
    return launch_fold<BITS, MT, LL, R>(planes, meta, x, signs, y, M, K, N, grid_cap, s, start, stop);
  LBQ_FOLD(16, 1) LBQ_FOLD(32, 1) LBQ_FOLD(64, 1) LBQ_FOLD(32, 2)
#undef LBQ_FOLD
  return hipErrorInvalidValue;
}

}  // namespace

void gemv_fold_shape(int M, int K, int N, int &lanes, int &rb, int &grid_cap) {
  const int G = K / kGroup;
  // lanes per row: the smallest of 16, 32, 64 that leaves each lane at most two groups
  lanes = 16;
  while (lanes * 2 < G && lanes < 64) lanes *= 2;
  rb = 1;
  grid_cap = 1024;
  (void)M;
  (void)N;
}

bool gemv_fold_supported(int M, int K) {
  const int G = K / kGroup;
  return (M == 1 && G <= 64) || (M == 2 && G <= 32);
}

hipError_t launch_gemv_fold(const void *planes, const void *meta, const uint16_t *x, const int8_t *signs, uint16_t *y,
                            int M, int K, int N, int bits, int lanes, int rb, int grid_cap, hipStream_t s,
                            hipEvent_t start, hipEvent_t stop) {
  if (M < 1 || M > 2 || (reinterpret_cast<uintptr_t>(signs) & 15u) != 0) return hipErrorInvalidValue;
  if (lanes <= 0) gemv_fold_shape(M, K, N, lanes, rb, grid_cap);
#define LBQ_MT(B)                                                                                  \
  return M == 1 ? launch_mt<B, 1>(planes, meta, x, signs, y, M, K, N, lanes, rb, grid_cap, s, start, stop) \
                : launch_mt<B, 2>(planes, meta, x, signs, y, M, K, N, lanes, rb, grid_cap, s, start, stop);
  switch (bits) {
    case 2: LBQ_MT(2)
    case 3: LBQ_MT(3)
    default: LBQ_MT(4)
  }
#undef LBQ_MT
}

}  // namespace lbq
