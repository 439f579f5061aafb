// Screened readout over the nibble-split planes of an 8-bit weight
// (LLaDA2.2-mini model card: property table, "Readout & Embeddings" row, and
// the file list: the readout's 8-bit codes are also kept as high and low
// nibble planes, which the engine's screened readout uses).
//
// The coarse logits of every row come from the high-nibble planes read as a
// 4-bit weight (the library's own linear path; scale 16 s and zero
// (z - 7.5) / 16 put each high nibble at the middle of its 16 codes). This
// file holds the other two steps:
//  * top-`cand` rows per token by coarse logit (larger first, ties to the
//    lower row): a threshold search on the fp16 logits' 16-bit order keys,
//    two bits per round, one workgroup per
//    (token, chunk of 4096 positions), repeated on the chunks' survivors
//    until one chunk is left;
//  * the exact logits of the survivors from both nibbles, q = lo + 16 hi, with
//    the 8-bit (s, z): one wavefront per (token, survivor), against x rotated
//    to fp16 by extra workgroups of the first selection launch.
#include "device.h"
#include "gemv_core.h"
#include "kernels.h"

namespace lbq {

namespace {

constexpr int kSelThreads = 256;
constexpr int kSelPer = 16;
constexpr int kSelChunk = kSelThreads * kSelPer;   // positions per workgroup

// Order key of an fp16 bit pattern: larger value, larger key (-0 folded onto +0).
__device__ __forceinline__ uint32_t order16(uint32_t h) {
  if (h == 0x8000u) h = 0;
  return (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u);
}

// A survivor: (order key << 32) | (0xFFFFFFFF - row); larger is better, and
// among equal keys the lower row is larger. 0 marks an empty slot.
__device__ __forceinline__ uint64_t make_key(uint32_t k16, uint32_t row) {
  return (static_cast<uint64_t>(k16 + 1) << 32) | (0xFFFFFFFFu - row);
}

// Lane exchanges go through xor_lane_u32 (DPP moves and permlane swaps): a
// ds_bpermute would cost a round trip through the LDS unit per step.
template <int STRIDE>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t v) {
  const uint32_t lo = xor_lane_u32<STRIDE>(static_cast<uint32_t>(v));
  const uint32_t hi = xor_lane_u32<STRIDE>(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
// Sum over the wave's 64 lanes, in every lane (xor butterfly, fixed order).
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += xor_lane_u32<32>(v);
  v += xor_lane_u32<16>(v);
  v += xor_lane_u32<8>(v);
  v += xor_lane_u32<4>(v);
  v += xor_lane_u32<2>(v);
  v += xor_lane_u32<1>(v);
  return v;
}

// One compare-exchange step of the bitonic network: runs of SIZE, partner ^ STRIDE.
template <int SIZE, int STRIDE>
__device__ __forceinline__ uint64_t bitonic_step(uint64_t v) {
  const int lane = threadIdx.x & 63;
  const uint64_t o = xor_lane64<STRIDE>(v);
  const bool desc = (lane & SIZE) == 0;          // this run sorts descending
  const bool low_half = (lane & STRIDE) == 0;    // keeps the larger in a descending run
  const bool keep_max = (desc == low_half);
  return keep_max ? (v > o ? v : o) : (v < o ? v : o);
}
template <int SIZE, int STRIDE>
__device__ __forceinline__ uint64_t bitonic_merge(uint64_t v) {
  v = bitonic_step<SIZE, STRIDE>(v);
  if constexpr (STRIDE > 1) v = bitonic_merge<SIZE, STRIDE / 2>(v);
  return v;
}

// Bitonic sort of 64 keys, one per lane, into descending order across the wave.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t v) {
  v = bitonic_merge<2, 1>(v);
  v = bitonic_merge<4, 2>(v);
  v = bitonic_merge<8, 4>(v);
  v = bitonic_merge<16, 8>(v);
  v = bitonic_merge<32, 16>(v);
  v = bitonic_merge<64, 32>(v);
  return v;
}

// One selection step. Stage 1 (keys_in == nullptr) reads fp16 logits
// vals[M][n] (position = row); later stages read the survivors of the previous
// one, keys_in[M][n] (each chunk's list sorted, chunks in row order, so
// position order is row order among equal values). Writes the chunk's `cand`
// best, sorted, to keys_out[M][chunks][cand] (0 where fewer exist).
// Thread tid holds positions i * 256 + tid (i < 16) of the chunk.
// Workgroups past the chunks (first stage only) rotate token blockIdx.y for
// the exact step instead, one 128-group per wavefront: xr = R x, fp32
// butterflies, fp16 out (a launch of its own would cost more than the work).
__global__ void __launch_bounds__(kSelThreads) select_kernel(const uint16_t *__restrict__ vals,
                                                             const uint64_t *__restrict__ keys_in, int n, int cand,
                                                             uint64_t *__restrict__ keys_out, int chunks,
                                                             const uint32_t *__restrict__ x,
                                                             const int8_t *__restrict__ signs,
                                                             uint32_t *__restrict__ xr, int K) {
  constexpr int W = kSelThreads / 64;
  static_assert(kSelPer * W == 64, "one scan entry per lane");
  __shared__ uint32_t cnt[2][W][2];          // per-wave counts of a search round (two rounds in flight)
  __shared__ uint32_t eq_base[kSelPer * W];  // equal-key counts per (step, wave), then their prefix
  __shared__ uint32_t sh_cnt_gt;
  __shared__ uint64_t sel[64];
  const int t = blockIdx.y, chunk = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (chunk >= chunks) {
    const int g = (chunk - chunks) * W + wave;
    if (g >= K / kGroup) return;
    const long base = static_cast<long>(t) * K + g * kGroup;   // element index
    const uint32_t xv = x[(base >> 1) + lane];
    const int k0 = g * kGroup + 2 * lane;
    float v0 = half_lo(xv) * static_cast<float>(signs[k0]);
    float v1 = half_hi(xv) * static_cast<float>(signs[k0 + 1]);
    fwht128_wave(v0, v1, lane);
    xr[(base >> 1) + lane] = static_cast<uint32_t>(f32_to_f16_bits(v0 * kInvSqrt128)) |
                             (static_cast<uint32_t>(f32_to_f16_bits(v1 * kInvSqrt128)) << 16);
    return;
  }

  uint64_t key[kSelPer];
  uint32_t val[kSelPer];   // order key of each held position (0 for empty: every real key is above it)
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const long p = static_cast<long>(chunk) * kSelChunk + i * kSelThreads + tid;
    uint64_t k = 0;
    if (p < n) {
      if (keys_in) k = keys_in[static_cast<size_t>(t) * n + p];
      else k = make_key(order16(vals[static_cast<size_t>(t) * n + p]), static_cast<uint32_t>(p));
    }
    key[i] = k;
    val[i] = static_cast<uint32_t>(k >> 32);   // order key + 1, or 0
  }
  if (tid < 64) sel[tid] = 0;
  if (tid == 0) sh_cnt_gt = 0;

  // The threshold X: the largest 16-bit order key that at least cand keys
  // reach, two bits per round from the top (the count of keys >= v falls as v
  // grows). Each round counts four thresholds in VALU registers (two per
  // 32-bit word: a thread holds at most 16 keys, a workgroup at most 4096),
  // adds them across the wave with xor shuffles and across the waves through
  // LDS, one barrier per round. Fewer than cand keys in all: no threshold,
  // every key survives. (val = order key + 1, 0 for empty slots.)
  int buf = 0;
  auto round_counts = [&](uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t out[4]) {
    uint32_t p01 = 0, p23 = 0;
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) {
      p01 += (val[i] >= c0 ? 1u : 0u) + (val[i] >= c1 ? 0x10000u : 0u);
      p23 += (val[i] >= c2 ? 1u : 0u) + (val[i] >= c3 ? 0x10000u : 0u);
    }
    p01 = wave_sum_u32(p01);
    p23 = wave_sum_u32(p23);
    if (lane == 0) {
      cnt[buf][wave][0] = p01;
      cnt[buf][wave][1] = p23;
    }
    __syncthreads();   // (a wave writes this buffer again only after the next round's barrier)
    uint32_t s01 = 0, s23 = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      s01 += cnt[buf][w][0];
      s23 += cnt[buf][w][1];
    }
    out[0] = s01 & 0xFFFFu;
    out[1] = s01 >> 16;
    out[2] = s23 & 0xFFFFu;
    out[3] = s23 >> 16;
    buf ^= 1;
  };
  const uint32_t c = static_cast<uint32_t>(cand);
  uint32_t tot[4];
  // first round: every valid key, and the top two bits
  round_counts(1, (1u << 14) + 1, (2u << 14) + 1, (3u << 14) + 1, tot);
  const bool all = tot[0] < c;
  uint32_t X = 0;
  if (!all) {
    X = tot[3] >= c ? 3u << 14 : tot[2] >= c ? 2u << 14 : tot[1] >= c ? 1u << 14 : 0u;
#pragma unroll 1
    for (int b = 12; b >= 0; b -= 2) {
      const uint32_t step = 1u << b;
      round_counts(X + step + 1, X + 2 * step + 1, X + 3 * step + 1, X + 3 * step + 1, tot);
      X += tot[2] >= c ? 3 * step : tot[1] >= c ? 2 * step : tot[0] >= c ? step : 0;
    }
  }
  const uint32_t T = X + 1;   // the threshold in val units

  // keys above the threshold (at most cand - 1 of them; every key when there
  // is none), then the lowest positions equal to it, in position order
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    if (val[i] != 0 && (all || val[i] > T)) {
      const uint32_t slot = atomicAdd(&sh_cnt_gt, 1u);
      if (slot < 64) sel[slot] = key[i];
    }
  }
  uint64_t bal[kSelPer];
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    bal[i] = all ? 0ull : __ballot(val[i] == T);
    if (lane == 0) eq_base[i * W + wave] = static_cast<uint32_t>(__popcll(bal[i]));
  }
  __syncthreads();
  if (!all) {
    const uint32_t g = sh_cnt_gt;
    const uint32_t need = c - g;
    // exclusive prefix of the (step, wave) counts in that order: lane l holds entry l
    uint32_t own = 0;
    if (wave == 0) {
      own = eq_base[lane];
      uint32_t incl = own;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(incl, d, 64);
        if (lane >= d) incl += o;
      }
      own = incl - own;
    }
    __syncthreads();
    if (wave == 0) eq_base[lane] = own;
    __syncthreads();
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) {
      if ((bal[i] >> lane) & 1ull) {
        const uint32_t r = eq_base[i * W + wave] + static_cast<uint32_t>(__popcll(bal[i] & below));
        if (r < need) sel[g + r] = key[i];
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    const uint64_t v = wave_sort_desc(sel[lane]);
    if (lane < cand) keys_out[(static_cast<size_t>(t) * chunks + chunk) * cand + lane] = v;
  }
}

// Exact logits of the survivors: wavefront (t, c) scores row r = the row of
// keys[t][c] from both nibble plane sets and the 8-bit (s, z), against the
// rotated activations xr [M][K] fp16. Per pass of 16 groups, lane l takes word
// column l mod 4 (32 consecutive codes) of group l / 4: its eight plane words,
// the group's (s, z) and 64 bytes of x' are all loaded before any use, so a
// pass costs one memory round trip.
__global__ void __launch_bounds__(256) refine_kernel(const uint64_t *__restrict__ keys, const uint32_t *__restrict__ hi,
                                                     const uint32_t *__restrict__ lo, const uint32_t *__restrict__ meta,
                                                     const uint16_t *__restrict__ xr, int M, int K, int N, int cand,
                                                     int32_t *__restrict__ ids, float *__restrict__ logits) {
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (item >= M * cand) return;
  const int t = item / cand;
  const uint64_t k = keys[item];
  const uint32_t rk = 0xFFFFFFFFu - static_cast<uint32_t>(k);
  if (k == 0 || rk >= static_cast<uint32_t>(N)) {   // fewer rows than cand
    if (lane == 0) {
      ids[item] = -1;
      logits[item] = 0.0f;
    }
    return;
  }
  const int row = static_cast<int>(rk);
  const int G = K / kGroup;
  const int w = lane & 3;
  float acc = 0.0f;
  for (int g0 = 0; g0 < G; g0 += 16) {
    const int g = g0 + (lane >> 2);
    if (g < G) {
      const size_t gi = static_cast<size_t>(row) * G + g;
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        hw[p] = hi[gi * 16 + p * 4 + w];
        lw[p] = lo[gi * 16 + p * 4 + w];
      }
      const uint32_t m = meta[gi];
      const uint4 *xp = reinterpret_cast<const uint4 *>(xr + static_cast<size_t>(t) * K + g * kGroup + 32 * w);
      uint4 xv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) xv[v] = xp[v];
      const float s = f16_bits_to_f32(m & 0xFFFFu);
      const float z = f16_bits_to_f32(m >> 16);
      float dot = 0.0f, xs = 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t pair[4] = {xv[v].x, xv[v].y, xv[v].z, xv[v].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = 8 * v + e;   // code 32 w + j
          uint32_t q = 0;
#pragma unroll
          for (int p = 0; p < 4; ++p) q |= (((lw[p] >> j) & 1u) << p) | (((hw[p] >> j) & 1u) << (p + 4));
          const float x = f16_bits_to_f32((pair[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
          dot += static_cast<float>(q) * x;
          xs += x;
        }
      }
      acc += s * (dot - z * xs);
    }
  }
  acc += __builtin_bit_cast(float, xor_lane_u32<32>(__builtin_bit_cast(uint32_t, acc)));
  acc += __builtin_bit_cast(float, xor_lane_u32<16>(__builtin_bit_cast(uint32_t, acc)));
  acc += __builtin_bit_cast(float, xor_lane_u32<8>(__builtin_bit_cast(uint32_t, acc)));
  acc += __builtin_bit_cast(float, xor_lane_u32<4>(__builtin_bit_cast(uint32_t, acc)));
  acc += __builtin_bit_cast(float, xor_lane_u32<2>(__builtin_bit_cast(uint32_t, acc)));
  acc += __builtin_bit_cast(float, xor_lane_u32<1>(__builtin_bit_cast(uint32_t, acc)));
  if (lane == 0) {
    ids[item] = row;
    logits[item] = acc;
  }
}

}  // namespace

int readout_chunks(int n) {
  return (n + kSelChunk - 1) / kSelChunk;
}

size_t readout_key_bytes(int M, int N, int cand) {
  // two ping-pong key buffers of the first stage's size
  const size_t first = static_cast<size_t>(M) * readout_chunks(N) * cand * 8;
  return 2 * ((first + 255) / 256 * 256);
}

hipError_t launch_readout_select(const uint16_t *coarse, int M, int N, int cand, uint64_t *keys,
                                 const uint64_t **final_keys, const uint16_t *x, const int8_t *signs, uint16_t *xr,
                                 int K, hipStream_t s) {
  *final_keys = keys;
  if (M <= 0) return hipSuccess;
  if (cand < 1 || cand > 64 || N < 1 || M > 65535) return hipErrorInvalidValue;
  const size_t half = readout_key_bytes(M, N, cand) / 2;
  uint64_t *buf[2] = {keys, reinterpret_cast<uint64_t *>(reinterpret_cast<uint8_t *>(keys) + half)};
  int n = N, chunks = readout_chunks(N), b = 0;
  // the first stage also rotates x for the exact step (kSelThreads / 64 groups per extra workgroup)
  const int rot_wgs = (K / kGroup + kSelThreads / 64 - 1) / (kSelThreads / 64);
  hipLaunchKernelGGL(select_kernel, dim3(chunks + rot_wgs, M), dim3(kSelThreads), 0, s, coarse,
                     static_cast<const uint64_t *>(nullptr), n, cand, buf[b], chunks,
                     reinterpret_cast<const uint32_t *>(x), signs, reinterpret_cast<uint32_t *>(xr), K);
  while (chunks > 1) {
    n = chunks * cand;
    chunks = readout_chunks(n);
    hipLaunchKernelGGL(select_kernel, dim3(chunks, M), dim3(kSelThreads), 0, s,
                       static_cast<const uint16_t *>(nullptr), buf[b], n, cand, buf[b ^ 1], chunks,
                       static_cast<const uint32_t *>(nullptr), static_cast<const int8_t *>(nullptr),
                       static_cast<uint32_t *>(nullptr), K);
    b ^= 1;
  }
  *final_keys = buf[b];   // [M][cand], sorted per token
  return hipGetLastError();
}

hipError_t launch_readout_refine(const uint64_t *keys, const void *hi, const void *lo, const void *meta,
                                 const uint16_t *xr, int M, int K, int N, int cand, int32_t *ids, float *logits,
                                 hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const int items = M * cand;
  hipLaunchKernelGGL(refine_kernel, dim3((items + 3) / 4), dim3(256), 0, s, keys, static_cast<const uint32_t *>(hi),
                     static_cast<const uint32_t *>(lo), static_cast<const uint32_t *>(meta), xr, M, K, N, cand, ids,
                     logits);
  return hipGetLastError();
}

}  // namespace lbq
