// Routed-expert MoE block on the RTN decoders (routed experts chosen top-k per
// token: Laguna-S-2.1 gridbook card, base-model line; per-expert code widths
// in a Hadamard-rotated basis: LLaDA2.2-mini Orin Nano card, "Routed Experts").
//
// Passes, all on the caller's stream:
//   1. route:   per pair of tokens (a workgroup of one wavefront each) the
//               top_k logits (ties to the lower expert id) and softmax weights
//               over them; then, in one workgroup, per-expert counts, exclusive
//               offsets, and the assignment list grouped by expert (a counting
//               sort over token chunks, one wavefront per chunk).
//   2. rotate:  x' = R_hidden x once per token (the rotate kernel).
//   3. gate|up: one workgroup per (expert, 128-wide block of the ffn axis);
//               inactive experts exit at once. It decodes the 128 gate rows and
//               the 128 matching up rows at the expert's own width, applies
//               SwiGLU, rounds to fp16, and rotates the 128-block with the ffn
//               signs (the down weight was quantized in that basis), writing the
//               rotated intermediate per assignment.
//   4. down:    one workgroup per (expert, 128 output rows); writes the fp32
//               expert output per assignment.
//   5. combine: y_t = sum_j w_tj o_tj in fp32, slot order, fp16 out.
// Nothing uses atomics on floating-point data, so repeated calls give
// bit-identical y.
#include "gemv_core.h"
#include "kernels.h"

namespace lbq {

namespace {

constexpr int kRouteThreads = 1024;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTokChunk = 8;

// ------------------------------------------------------------------ router

// Order-preserving map of a float to u32 (larger float -> larger u32) and back.
__device__ __forceinline__ uint32_t float_order(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float float_unorder(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}
template <int X>
__device__ __forceinline__ float add_xor(float v) {
  return v + __uint_as_float(xor_lane_u32<X>(__float_as_uint(v)));
}

// Largest u32 over the wavefront, in every lane (uniform): a DPP max
// reduction into lane 63 (row shifts by 1, 2, 4, 8 give each row's maximum
// in its lane 15; row broadcasts 15 and 31 carry them to lane 63), then a
// read of lane 63. Lanes without a DPP source keep their own value.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t max_dpp(uint32_t v) {
  const uint32_t o = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), CTRL, ROWS, 0xF, false));
  return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max_dpp<0x111, 0xF>(v);   // row_shr:1
  v = max_dpp<0x112, 0xF>(v);   // row_shr:2
  v = max_dpp<0x114, 0xF>(v);   // row_shr:4
  v = max_dpp<0x118, 0xF>(v);   // row_shr:8
  v = max_dpp<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v = max_dpp<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// The router runs as two launches. Its top-k rounds are chains of dependent
// lane exchanges; on one workgroup the waves of all tokens shared one compute
// unit's issue slots (about 7 us for 32 tokens), so the top-k launch spreads
// the token pairs over workgroups of one wavefront each, and a one-workgroup
// launch then sorts the assignments.

// PER: experts per lane (E <= 64 PER).
template <int PER>
__global__ void __launch_bounds__(64) moe_topk_kernel(const float *__restrict__ logits, int M, int E, int top_k,
                                                      int32_t *__restrict__ ids, float *__restrict__ weights) {
  const int lane = threadIdx.x & 63;

  // 1. top-k per token, one wavefront per pair of tokens (their dependent
  //    chains interleave). Expert e = lane + 64 i holds the order key of its
  //    logit (order-preserving u32; a selected or absent expert holds 0, below
  //    every finite logit's key). Each round takes the wavefront's largest key
  //    and, among the experts holding it, the lowest id (ties go to the lower
  //    id), and clears it. A pair's second token past M computes on copies of
  //    the first and stores nothing.
  for (int t0 = 2 * static_cast<int>(blockIdx.x); t0 < M; t0 += 2 * static_cast<int>(gridDim.x)) {
    const int tt[2] = {t0, min(t0 + 1, M - 1)};
    const bool ok1 = t0 + 1 < M;
    // all loads first, unconditionally at clamped indices, then the keys
    float lv[2][PER];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int i = 0; i < PER; ++i) lv[p][i] = logits[static_cast<size_t>(tt[p]) * E + min(lane + 64 * i, E - 1)];
    uint32_t key[2][PER];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int i = 0; i < PER; ++i) key[p][i] = lane + 64 * i < E ? float_order(lv[p][i] + 0.0f) : 0u;   // -0 -> +0
    // lane r keeps the r-th selected logit (selection order is descending)
    float sel0[2] = {0.f, 0.f}, mine[2] = {0.f, 0.f};
    for (int r = 0; r < top_k; ++r) {
      uint32_t best[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        uint32_t m = key[p][0];
#pragma unroll
        for (int i = 1; i < PER; ++i) m = key[p][i] > m ? key[p][i] : m;
        best[p] = m;
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) best[p] = wave_max_u32(best[p]);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        int e = 64 * PER;
#pragma unroll
        for (int i = PER - 1; i >= 0; --i) {
          const uint64_t bal = __ballot(key[p][i] == best[p]);
          if (bal) e = 64 * i + __builtin_ctzll(bal);
        }
#pragma unroll
        for (int i = 0; i < PER; ++i)
          if (i == (e >> 6) && lane == (e & 63)) key[p][i] = 0u;
        const float v = float_unorder(best[p]);
        if (r == 0) sel0[p] = v;
        if (lane == r) mine[p] = v;
        if (lane == 0 && (p == 0 || ok1)) ids[tt[p] * top_k + r] = e;
      }
    }
    // softmax over the selected logits (shifted by the largest)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const float ex = lane < top_k ? __expf(mine[p] - sel0[p]) : 0.f;
      float denom = add_xor<32>(ex);
      denom = add_xor<16>(denom);
      denom = add_xor<8>(denom);
      denom = add_xor<4>(denom);
      denom = add_xor<2>(denom);
      denom = add_xor<1>(denom);
      if (lane < top_k && (p == 0 || ok1)) weights[tt[p] * top_k + lane] = ex / denom;
    }
  }
}

__global__ void __launch_bounds__(kRouteThreads) moe_sort_kernel(const int32_t *__restrict__ ids, int M, int E,
                                                                  int top_k, int32_t *__restrict__ counts,
                                                                  int32_t *__restrict__ offsets,
                                                                  int32_t *__restrict__ perm) {
  constexpr int kWaves = kRouteThreads / 64;
  __shared__ int32_t s_cnt[kWaves * kMaxExperts];   // per (token chunk, expert): count, then run start
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // 2. counting sort of the assignments by expert, stable in the assignment
  //    index. Wave w owns the contiguous token chunk [w C, (w + 1) C); a
  //    token's top_k experts are distinct, so the lanes of one token never
  //    touch the same counter. (a) per-chunk counts cnt[w][e]; (b) per expert
  //    the total and, after an exclusive scan over experts, the start of each
  //    chunk's run; (c) each wave walks its tokens in order and places them.
  const int MK = M * top_k;
  const int chunk = (M + kWaves - 1) / kWaves;
  const int t_lo = min(M, wave * chunk), t_hi = min(M, t_lo + chunk);
  (void)MK;
  for (int i = threadIdx.x; i < kWaves * E; i += kRouteThreads) s_cnt[i] = 0;
  __syncthreads();
  for (int t = t_lo; t < t_hi; ++t)
    if (lane < top_k) s_cnt[wave * E + ids[t * top_k + lane]] += 1;
  __syncthreads();
  // exclusive offsets: thread i owns experts kPerThread i .. kPerThread (i + 1) - 1;
  // scan of the per-thread totals within each wave, then across the waves
  {
    constexpr int kPerThread = (kMaxExperts + kRouteThreads - 1) / kRouteThreads;
    __shared__ int32_t s_wave[kWaves];
    int own[kPerThread];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int e = threadIdx.x * kPerThread + j;
      int tot = 0;
      if (e < E)
        for (int w = 0; w < kWaves; ++w) tot += s_cnt[w * E + e];
      own[j] = tot;
      sum += tot;
    }
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int w = 0; w < wave; ++w) run += s_wave[w];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int e = threadIdx.x * kPerThread + j;
      if (e < E) {
        offsets[e] = run;
        counts[e] = own[j];
        // start of each chunk's run of expert e
        int pos = run;
        for (int w = 0; w < kWaves; ++w) {
          const int c = s_cnt[w * E + e];
          s_cnt[w * E + e] = pos;
          pos += c;
        }
      }
      run += own[j];
    }
    if (threadIdx.x == kRouteThreads - 1) offsets[E] = run;
  }
  __syncthreads();
  for (int t = t_lo; t < t_hi; ++t)
    if (lane < top_k) {
      const int a = t * top_k + lane;
      perm[s_cnt[wave * E + ids[a]]++] = a;
    }
}

// ------------------------------------------------------------------ gate|up

constexpr int kGuRows = 128;   // intermediate indices per workgroup (gate and up rows each)

template <int BITS, int MT>
__device__ void gateup_tile(const MoeArgs &a, int e, int ib, int first, int cnt, uint32_t *smem) {
  constexpr int L = 16;
  constexpr int R = kGemvThreads / L;   // rows per pass
  const int G = a.hidden / kGroup;
  const int Gc = G;                      // hidden fits LDS for MT <= 8 (checked by the host)
  uint32_t *xx = smem;
  float2 *sums = reinterpret_cast<float2 *>(xx + MT * Gc * kGroupStride);
  float *hbuf = reinterpret_cast<float *>(sums + MT * Gc);   // [2*kGuRows][MT]
  const int *perm = a.perm + first;
  auto row_ptr = [&](int m) {
    const int tok = perm[m] / a.top_k;
    return reinterpret_cast<const uint32_t *>(a.xr) + static_cast<size_t>(tok) * (a.hidden / 2);
  };
  stage_groups<BITS, MT>(row_ptr, cnt, 0, G, Gc, xx, sums);
  __syncthreads();
  const uint4 *planes = reinterpret_cast<const uint4 *>(a.planes + a.gu_plane_off[e]);
  const uint32_t *meta = reinterpret_cast<const uint32_t *>(a.meta + a.gu_meta_off[e]);
  const int j = threadIdx.x % L;
  // U passes of R rows at once (their loads in flight together)
  constexpr int U = MT <= 2 ? 4 : MT <= 4 ? 2 : 1;
  for (int p = 0; p < (2 * kGuRows) / R; p += U) {
    const uint4 *prow[U];
    const uint32_t *mrow[U];
    int local[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      local[u] = (p + u) * R + threadIdx.x / L;                 // 0..255: gate rows then up rows
      const int row =
          (local[u] < kGuRows) ? (ib * kGuRows + local[u]) : (a.ffn + ib * kGuRows + local[u] - kGuRows);
      prow[u] = planes + static_cast<size_t>(row) * G * BITS;
      mrow[u] = meta + static_cast<size_t>(row) * G;
    }
    float yacc[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < MT; ++m) yacc[u][m] = 0.f;
    rows_partial<BITS, MT, L, U>(prow, mrow, xx, sums, Gc, G, j, yacc);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      reduce_cluster<MT, L>(yacc[u]);
      if (j == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m) hbuf[local[u] * MT + m] = yacc[u][m];
      }
    }
  }
  __syncthreads();
  // SwiGLU, fp16 rounding, rotation of the 128-block, one wavefront per token.
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int m = wave; m < cnt; m += kGemvThreads / 64) {
    float v[2];
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
      const int r = 2 * lane + e2;
      const float g = hbuf[r * MT + m], u = hbuf[(kGuRows + r) * MT + m];
      const float act = g / (1.f + __expf(-g)) * u;
      const float act16 = f16_bits_to_f32(f32_to_f16_bits(act));
      v[e2] = act16 * static_cast<float>(a.signs_ffn[ib * kGuRows + r]);
    }
    fwht128_wave(v[0], v[1], lane);
    const uint32_t packed = static_cast<uint32_t>(f32_to_f16_bits(v[0] * kInvSqrt128)) |
                            (static_cast<uint32_t>(f32_to_f16_bits(v[1] * kInvSqrt128)) << 16);
    reinterpret_cast<uint32_t *>(a.act + static_cast<size_t>(perm[m]) * a.ffn + ib * kGuRows)[lane] = packed;
  }
  __syncthreads();
}

template <int BITS>
__device__ void gateup_bits(const MoeArgs &a, int e, int ib, int first, int n_e, uint32_t *smem) {
  for (int c0 = 0; c0 < n_e; c0 += kMaxTokChunk) {
    const int cnt = min(kMaxTokChunk, n_e - c0);
    if (cnt == 1) gateup_tile<BITS, 1>(a, e, ib, first + c0, cnt, smem);
    else if (cnt == 2) gateup_tile<BITS, 2>(a, e, ib, first + c0, cnt, smem);
    else if (cnt <= 4) gateup_tile<BITS, 4>(a, e, ib, first + c0, cnt, smem);
    else gateup_tile<BITS, 8>(a, e, ib, first + c0, cnt, smem);
  }
}

__global__ void __launch_bounds__(kGemvThreads) moe_gateup_kernel(MoeArgs a) {
  extern __shared__ uint32_t smem[];
  const int nb = a.ffn / kGuRows;
  const int e = blockIdx.x / nb, ib = blockIdx.x % nb;
  const int first = a.offsets[e];
  const int n_e = a.offsets[e + 1] - first;
  if (n_e == 0) return;
  switch (a.bits[e]) {
    case 2: gateup_bits<2>(a, e, ib, first, n_e, smem); break;
    case 3: gateup_bits<3>(a, e, ib, first, n_e, smem); break;
    default: gateup_bits<4>(a, e, ib, first, n_e, smem); break;
  }
}

// ------------------------------------------------------------------ down

constexpr int kDnRows = 128;   // output rows per workgroup

template <int BITS, int MT>
__device__ void down_tile(const MoeArgs &a, int e, int rb, int first, int cnt, uint32_t *smem) {
  constexpr int L = 8;
  constexpr int R = kGemvThreads / L;
  const int G = a.ffn / kGroup;
  const int Gc = G;
  uint32_t *xx = smem;
  float2 *sums = reinterpret_cast<float2 *>(xx + MT * Gc * kGroupStride);
  const int *perm = a.perm + first;
  auto row_ptr = [&](int m) {
    return reinterpret_cast<const uint32_t *>(a.act) + static_cast<size_t>(perm[m]) * (a.ffn / 2);
  };
  stage_groups<BITS, MT>(row_ptr, cnt, 0, G, Gc, xx, sums);
  __syncthreads();
  const uint4 *planes = reinterpret_cast<const uint4 *>(a.planes + a.dn_plane_off[e]);
  const uint32_t *meta = reinterpret_cast<const uint32_t *>(a.meta + a.dn_meta_off[e]);
  const int j = threadIdx.x % L;
  // U passes of R rows at once (their loads in flight together)
  constexpr int U = MT <= 2 ? 4 : MT <= 4 ? 2 : 1;
  for (int p = 0; p < kDnRows / R; p += U) {
    const uint4 *prow[U];
    const uint32_t *mrow[U];
    int row[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      row[u] = rb * kDnRows + (p + u) * R + threadIdx.x / L;
      prow[u] = planes + static_cast<size_t>(row[u]) * G * BITS;
      mrow[u] = meta + static_cast<size_t>(row[u]) * G;
    }
    float yacc[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < MT; ++m) yacc[u][m] = 0.f;
    rows_partial<BITS, MT, L, U>(prow, mrow, xx, sums, Gc, G, j, yacc);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      reduce_cluster<MT, L>(yacc[u]);
      if (j == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (m < cnt) a.out[static_cast<size_t>(perm[m]) * a.hidden + row[u]] = yacc[u][m];
      }
    }
  }
  __syncthreads();
}

template <int BITS>
__device__ void down_bits(const MoeArgs &a, int e, int rb, int first, int n_e, uint32_t *smem) {
  for (int c0 = 0; c0 < n_e; c0 += kMaxTokChunk) {
    const int cnt = min(kMaxTokChunk, n_e - c0);
    if (cnt == 1) down_tile<BITS, 1>(a, e, rb, first + c0, cnt, smem);
    else if (cnt == 2) down_tile<BITS, 2>(a, e, rb, first + c0, cnt, smem);
    else if (cnt <= 4) down_tile<BITS, 4>(a, e, rb, first + c0, cnt, smem);
    else down_tile<BITS, 8>(a, e, rb, first + c0, cnt, smem);
  }
}

__global__ void __launch_bounds__(kGemvThreads) moe_down_kernel(MoeArgs a) {
  extern __shared__ uint32_t smem[];
  const int nb = a.hidden / kDnRows;
  const int e = blockIdx.x / nb, rb = blockIdx.x % nb;
  const int first = a.offsets[e];
  const int n_e = a.offsets[e + 1] - first;
  if (n_e == 0) return;
  switch (a.bits[e]) {
    case 2: down_bits<2>(a, e, rb, first, n_e, smem); break;
    case 3: down_bits<3>(a, e, rb, first, n_e, smem); break;
    default: down_bits<4>(a, e, rb, first, n_e, smem); break;
  }
}

// ------------------------------------------------------------------ combine

__global__ void __launch_bounds__(256) moe_combine_kernel(const float *__restrict__ out,
                                                          const float *__restrict__ weights, int M, int hidden,
                                                          int top_k, uint16_t *__restrict__ y) {
  const long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<long>(M) * hidden) return;
  const int t = static_cast<int>(i / hidden), n = static_cast<int>(i % hidden);
  float acc = 0.f;
  for (int jj = 0; jj < top_k; ++jj)
    acc = fmaf(weights[t * top_k + jj], out[(static_cast<size_t>(t) * top_k + jj) * hidden + n], acc);
  y[i] = f32_to_f16_bits(acc);
}

}  // namespace

hipError_t launch_moe_route(const float *logits, int M, int E, int top_k, int32_t *ids, float *weights,
                            int32_t *counts, int32_t *offsets, int32_t *perm, hipStream_t s) {
  auto topk = E <= 64 ? moe_topk_kernel<1> : E <= 256 ? moe_topk_kernel<4> : E <= 512 ? moe_topk_kernel<8>
                                                                                : moe_topk_kernel<16>;
  if (M > 0) hipLaunchKernelGGL(topk, dim3(static_cast<unsigned>((M + 1) / 2)), dim3(64), 0, s, logits, M, E, top_k, ids, weights);
  hipLaunchKernelGGL(moe_sort_kernel, dim3(1), dim3(kRouteThreads), 0, s, ids, M, E, top_k, counts, offsets, perm);
  return hipGetLastError();
}

// Tile descriptors of the grouped expert GEMMs: expert e's list entries
// [offsets[e], offsets[e + 1]) in tiles of `per`, each (e, first entry,
// entries, bits[e]), experts in id order; *n_tiles = their number. One
// workgroup, one expert per thread.
__global__ void __launch_bounds__(kRouteThreads) moe_tiles_kernel(const int32_t *__restrict__ offsets,
                                                                   const uint8_t *__restrict__ bits, int E, int per,
                                                                   int4 *__restrict__ tiles,
                                                                   int32_t *__restrict__ n_tiles) {
  constexpr int kWaves = kRouteThreads / 64;
  __shared__ int32_t s_wave[kWaves];
  const int e = threadIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int first = e < E ? offsets[e] : 0;
  const int cnt = e < E ? offsets[e + 1] - first : 0;
  const int nt = (cnt + per - 1) / per;
  int incl = nt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int start = incl - nt;
  for (int w = 0; w < wave; ++w) start += s_wave[w];
  for (int k = 0; k < nt; ++k)
    tiles[start + k] = make_int4(e, first + k * per, min(per, cnt - k * per), e < E ? bits[e] : 0);
  if (threadIdx.x == kRouteThreads - 1) *n_tiles = start + nt;
}

size_t moe_gateup_lds(int hidden) {
  const int G = hidden / kGroup;
  return static_cast<size_t>(kMaxTokChunk) * G * kStagedGroupBytes + 2 * kGuRows * kMaxTokChunk * sizeof(float);
}
size_t moe_down_lds(int ffn) { return static_cast<size_t>(kMaxTokChunk) * (ffn / kGroup) * kStagedGroupBytes; }

int moe_prefill_tile_tokens(int M, int E, int top_k) {
  const long avg = (static_cast<long>(M) * top_k + E - 1) / E;   // list entries per expert
  return avg <= 16 ? 16 : avg <= 32 ? 32 : 64;
}

int moe_prefill_max_tiles(int M, int E, int top_k) {
  const int per = moe_prefill_tile_tokens(M, E, top_k);
  return static_cast<int>((static_cast<long>(M) * top_k + per - 1) / per) + E;
}

bool moe_prefill_supported(int hidden, int ffn, long assignments) {
  // the grouped GEMM stages a row tile's scale/zero words for the whole K in
  // LDS (two 16-row blocks per wave up to 40 groups), h is read through 32-bit
  // offsets
  return hidden / kGroup <= gemm_rtn_meta_max_groups(2) && ffn / kGroup <= gemm_rtn_meta_max_groups(2) &&
         assignments * 2 * ffn * 4 < (1L << 31);
}

hipError_t launch_moe_prefill(const MoeArgs &a, const MoePrefill &p, hipStream_t s) {
  const int per = moe_prefill_tile_tokens(a.M, a.E, a.top_k);
  const int max_tiles = moe_prefill_max_tiles(a.M, a.E, a.top_k);
  const int A = a.M * a.top_k;
  hipLaunchKernelGGL(moe_tiles_kernel, dim3(1), dim3(kRouteThreads), 0, s, a.offsets, a.bits, a.E, per,
                     reinterpret_cast<int4 *>(p.tiles), p.n_tiles);
  hipError_t e;
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // tokens rotated once with the hidden signs (folded order, zero-point sums)
  if ((e = launch_rotate_folded(a.x, a.M, a.hidden, a.signs_hidden, const_cast<uint16_t *>(a.xr), p.tz_hidden,
                                nullptr, 0, s)) != hipSuccess)
    return e;
  GroupedGemm g{};
  g.nb = 2;
  g.mt = per / 16;
  g.max_tiles = max_tiles;
  g.tiles = p.tiles;
  g.n_tiles = p.n_tiles;
  g.planes = a.planes;
  g.meta = a.meta;
  g.perm = a.perm;
  // gate|up: token rows perm[i] / top_k, results in list order
  g.K = a.hidden;
  g.N = 2 * a.ffn;
  g.plane_off = a.gu_plane_off;
  g.meta_off = a.gu_meta_off;
  g.xf = a.xr;
  g.tz = p.tz_hidden;
  g.act_div = a.top_k;
  g.out_perm = 0;
  g.out = a.h;
  if ((e = launch_gemm_rtn_grouped(g, s)) != hipSuccess) return e;
  // SwiGLU, fp16, rotated with the ffn signs, in list order
  if ((e = launch_swiglu_rotate_folded(a.h, A, a.ffn, a.signs_ffn, a.act, p.tz_ffn, s)) != hipSuccess) return e;
  // down: rows in list order, results by assignment index for the combine
  g.K = a.ffn;
  g.N = a.hidden;
  g.plane_off = a.dn_plane_off;
  g.meta_off = a.dn_meta_off;
  g.xf = a.act;
  g.tz = p.tz_ffn;
  g.act_div = 0;
  g.out_perm = 1;
  g.out = a.out;
  if ((e = launch_gemm_rtn_grouped(g, s)) != hipSuccess) return e;
  const long total = static_cast<long>(a.M) * a.hidden;
  hipLaunchKernelGGL(moe_combine_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s, a.out,
                     a.weights, a.M, a.hidden, a.top_k, a.y);
  return hipGetLastError();
}

hipError_t launch_moe_experts(const MoeArgs &a, hipStream_t s) {
  hipError_t e;
  if (moe_mx_supported(a.hidden, a.ffn, a.signs_hidden, a.signs_ffn)) {
    if ((e = launch_moe_mx(a, s)) != hipSuccess) return e;
  } else {
    if ((e = launch_rotate(a.x, a.M, a.hidden, a.signs_hidden, const_cast<uint16_t *>(a.xr), s)) != hipSuccess) return e;
    hipLaunchKernelGGL(moe_gateup_kernel, dim3(a.E * (a.ffn / kGuRows)), dim3(kGemvThreads), moe_gateup_lds(a.hidden),
                       s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(moe_down_kernel, dim3(a.E * (a.hidden / kDnRows)), dim3(kGemvThreads), moe_down_lds(a.ffn), s,
                       a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const long total = static_cast<long>(a.M) * a.hidden;
  hipLaunchKernelGGL(moe_combine_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s, a.out,
                     a.weights, a.M, a.hidden, a.top_k, a.y);
  return hipGetLastError();
}

}  // namespace lbq
