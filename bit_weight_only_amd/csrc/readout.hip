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
//    lower row): a radix select on the fp16 logits' 16-bit order keys, one
//    workgroup per (token, chunk of 16384 positions), repeated on the chunks'
//    survivors until one chunk is left;
//  * the exact logits of the survivors from both nibbles, q = lo + 16 hi, with
//    the 8-bit (s, z): one wavefront per (token, survivor).
#include "device.h"
#include "kernels.h"

namespace lbq {

namespace {

constexpr int kSelThreads = 1024;
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
__device__ __forceinline__ uint32_t key_value(uint64_t k) {
  return static_cast<uint32_t>(k >> 32) - 1;
}

// Bitonic sort of 64 keys, one per lane, into descending order across the wave.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), stride, 64);
      const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), stride, 64);
      const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
      const bool desc = (lane & size) == 0;          // this run sorts descending
      const bool low_half = (lane & stride) == 0;    // keeps the larger in a descending run
      const bool keep_max = (desc == low_half);
      v = keep_max ? (v > o ? v : o) : (v < o ? v : o);
    }
  }
  return v;
}

// One radix-select step. Stage 1 (keys_in == nullptr) reads fp16 logits
// vals[M][n] (position = row); later stages read the survivors of the previous
// one, keys_in[M][n] (each chunk's list sorted, chunks in row order, so
// position order is row order among equal values). Writes the chunk's `cand`
// best, sorted, to keys_out[M][gridDim.x][cand] (0 where fewer exist).
__global__ void __launch_bounds__(kSelThreads) select_kernel(const uint16_t *__restrict__ vals,
                                                             const uint64_t *__restrict__ keys_in, int n, int cand,
                                                             uint64_t *__restrict__ keys_out) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wave_cnt[kSelThreads / 64];
  __shared__ uint32_t sh_b, sh_above, sh_cnt_gt, sh_base;
  __shared__ uint64_t sel[64];
  const int t = blockIdx.y, chunk = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  uint64_t key[kSelPer];
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const long p = static_cast<long>(chunk) * kSelChunk + i * kSelThreads + tid;
    uint64_t k = 0;
    if (p < n) {
      if (keys_in) k = keys_in[static_cast<size_t>(t) * n + p];
      else k = make_key(order16(vals[static_cast<size_t>(t) * n + p]), static_cast<uint32_t>(p));
    }
    key[i] = k;
  }
  if (tid < 64) sel[tid] = 0;

  // two histogram passes: high byte, then low byte within the chosen high byte
  uint32_t T = 0, above = 0;
  for (int pass = 0; pass < 2; ++pass) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) {
      if (key[i] == 0) continue;
      const uint32_t v = key_value(key[i]);
      if (pass == 0) atomicAdd(&hist[v >> 8], 1u);
      else if ((v >> 8) == (T >> 8)) atomicAdd(&hist[v & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds bins 255 - 4l .. 252 - 4l (descending); counts from the top
      uint32_t c[4], s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hist[255 - 4 * lane - j];
        s += c[j];
      }
      uint32_t incl = s;   // inclusive prefix over lanes
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(incl, d, 64);
        if (lane >= d) incl += o;
      }
      uint32_t run = above + incl - s;   // keys above this lane's first bin
      int found = -1;
      uint32_t found_above = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (found < 0 && run + c[j] >= static_cast<uint32_t>(cand)) {
          found = 255 - 4 * lane - j;
          found_above = run;
        }
        run += c[j];
      }
      const uint64_t hit = __ballot(found >= 0);
      if (hit == 0) {
        // fewer than cand keys in all: take everything (threshold below every key)
        if (lane == 0) {
          sh_b = 0xFFFFFFFFu;
          sh_above = above + __shfl(incl, 63, 64);
        }
      } else {
        const int first = __ffsll(static_cast<unsigned long long>(hit)) - 1;
        const int b = __shfl(found, first, 64);
        const uint32_t ab = __shfl(found_above, first, 64);
        if (lane == 0) {
          sh_b = static_cast<uint32_t>(b);
          sh_above = ab;
        }
      }
    }
    __syncthreads();
    if (sh_b == 0xFFFFFFFFu) {   // take all: no threshold
      T = 0xFFFFFFFFu;
      above = sh_above;
      break;
    }
    T = pass == 0 ? (sh_b << 8) : ((T & 0xFF00u) | sh_b);
    above = sh_above;
    __syncthreads();
  }

  // keys above the threshold (at most cand - 1 of them; all when T is "none"),
  // then the lowest positions equal to it, in position order
  if (tid == 0) {
    sh_cnt_gt = 0;
    sh_base = 0;
  }
  __syncthreads();
  const bool all = T == 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    if (key[i] != 0 && (all || key_value(key[i]) > T)) {
      const uint32_t slot = atomicAdd(&sh_cnt_gt, 1u);
      if (slot < 64) sel[slot] = key[i];
    }
  }
  __syncthreads();
  if (!all) {
    const uint32_t g = sh_cnt_gt;
    const uint32_t need = static_cast<uint32_t>(cand) - g;
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) {
      // (sh_base is uniform: once it reaches need, no later key is taken)
      const bool eq = sh_base < need && key[i] != 0 && key_value(key[i]) == T;
      const uint64_t b = __ballot(eq);
      if (lane == 0) wave_cnt[wave] = static_cast<uint32_t>(__popcll(b));
      __syncthreads();
      uint32_t before = sh_base;
      for (int w = 0; w < wave; ++w) before += wave_cnt[w];
      before += static_cast<uint32_t>(__popcll(b & ((1ull << lane) - 1ull)));
      if (eq && before < need) sel[g + before] = key[i];
      __syncthreads();
      if (tid == 0) {
        uint32_t tot = 0;
        for (int w = 0; w < kSelThreads / 64; ++w) tot += wave_cnt[w];
        sh_base += tot;
      }
      __syncthreads();
    }
  }
  __syncthreads();
  if (wave == 0) {
    const uint64_t v = wave_sort_desc(sel[lane]);
    if (lane < cand) keys_out[(static_cast<size_t>(t) * gridDim.x + chunk) * cand + lane] = v;
  }
}

// Exact logits of the survivors: wavefront (t, c) scores row r = the row of
// keys[t][c] from both nibble plane sets and the 8-bit (s, z), against the
// rotated activations xr [M][K] fp16. Lane l takes codes 2l, 2l + 1 of every
// group (word l / 16, bits 2 (l mod 16) and the next).
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
  const int w = lane >> 4, j = 2 * (lane & 15);
  const uint32_t *hr = hi + static_cast<size_t>(row) * G * 16;
  const uint32_t *lr = lo + static_cast<size_t>(row) * G * 16;
  const uint32_t *mr = meta + static_cast<size_t>(row) * G;
  const uint32_t *xp = reinterpret_cast<const uint32_t *>(xr + static_cast<size_t>(t) * K) + lane;
  float acc = 0.0f;
  for (int g = 0; g < G; ++g) {
    uint32_t q0 = 0, q1 = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t lw = lr[g * 16 + p * 4 + w] >> j;
      const uint32_t hw = hr[g * 16 + p * 4 + w] >> j;
      q0 |= ((lw & 1u) | ((hw & 1u) << 4)) << p;
      q1 |= (((lw >> 1) & 1u) | (((hw >> 1) & 1u) << 4)) << p;
    }
    const uint32_t m = mr[g];
    const float s = f16_bits_to_f32(static_cast<uint16_t>(m & 0xFFFFu));
    const float z = f16_bits_to_f32(static_cast<uint16_t>(m >> 16));
    const uint32_t xv = xp[g * 64];
    const float x0 = f16_bits_to_f32(static_cast<uint16_t>(xv & 0xFFFFu));
    const float x1 = f16_bits_to_f32(static_cast<uint16_t>(xv >> 16));
    acc += s * ((static_cast<float>(q0) - z) * x0 + (static_cast<float>(q1) - z) * x1);
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) acc += __shfl_xor(acc, d, 64);
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
                                 const uint64_t **final_keys, hipStream_t s) {
  *final_keys = keys;
  if (M <= 0) return hipSuccess;
  if (cand < 1 || cand > 64 || N < 1 || M > 65535) return hipErrorInvalidValue;
  const size_t half = readout_key_bytes(M, N, cand) / 2;
  uint64_t *buf[2] = {keys, reinterpret_cast<uint64_t *>(reinterpret_cast<uint8_t *>(keys) + half)};
  int n = N, chunks = readout_chunks(N), b = 0;
  hipLaunchKernelGGL(select_kernel, dim3(chunks, M), dim3(kSelThreads), 0, s, coarse,
                     static_cast<const uint64_t *>(nullptr), n, cand, buf[b]);
  while (chunks > 1) {
    n = chunks * cand;
    chunks = readout_chunks(n);
    hipLaunchKernelGGL(select_kernel, dim3(chunks, M), dim3(kSelThreads), 0, s,
                       static_cast<const uint16_t *>(nullptr), buf[b], n, cand, buf[b ^ 1]);
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
