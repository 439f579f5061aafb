// MFMA dequant-GEMM for product-VQ codes: y = x' W'^T with W' = s_n C[idx]
// (Laguna-S-2.1 card, 8-bit codebook indices per 4-dim half vector, fp16 row
// scale), decoded inside the K mainloop into the B operand of
// v_mfma_f32_16x16x32_f16 (no expand-to-dense round trip through memory).
//
// Tiling. A workgroup of 4 wavefronts owns 64 * NB output columns (rows of W)
// and 16 * MT tokens; wave w owns NB blocks of 16 rows. The K range of the
// workgroup is one of S contiguous slices of the 128-groups (split-K when the
// tile grid alone would leave the chip idle). Per group:
//   * the token tile's rotated activations (natural order) and the wave's
//     index bytes are copied global -> LDS asynchronously (global_load_lds)
//     into a ring of R slots, R - 1 groups ahead of the contraction, one
//     barrier per group;
//   * lane (j, kq) of a wave looks up the codebook entries of word column kq
//     (weights 32 kq .. 32 kq + 31) of row j of each of its NB row blocks
//     (e4m3 values are exact in fp16, staged as a 2 KB fp16 table in LDS):
//     step t takes weights 32 kq + 8 t .. + 7, the two entries of index bytes
//     8 kq + 2 t and the next, whose four fp16 values each are already the
//     B operand's pairs. The A operand of lane (i, kq) is x[32 kq + 8 t .. + 7]
//     of token i, so A and B agree on which k each element is. The row scale
//     is constant along K and applied once at the end.
// Split-K: each workgroup writes its fp32 partial tile to the workspace; the
// last of the S workgroups of a tile to arrive (an atomic counter the rotation
// launch cleared) sums the S partials in slice order and writes y, so the
// result does not depend on arrival order. No workgroup ever waits on another.
#include "device.h"
#include "gemm_common.h"
#include "kernels.h"

#include <algorithm>

namespace lbq {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// ------------------------------------------------------------------ B decoders
//
// The decoder moves one group's index bytes for a wave into that wave's part
// of an LDS ring slot (kDma copies of 64 lanes per group) and later decodes
// them from there. Only the wave that copied a vector reads it back.

// Product-VQ indices: byte i of a row covers weights 4i..4i+3; a group's 32
// index bytes of a row are two 16-byte vectors (h = 0, 1), vector u = 2 nb + h
// of the lane set copied by lane (j, u). Lane (j, kq) needs word column kq
// (index bytes 8kq..8kq+7, weights 32kq..32kq+31): half kq & 1 of vector
// 2 nb + (kq >> 1).
// ST residual stages (stage t's indices at idx + t N K / 4, its row scales at
// row_scale + t N) fold into one fp16 B value per weight:
// C[i_1] + r_2 C[i_2] + r_3 C[i_3], r_t the fp16 ratio of stage t's row scale
// to stage 1's (two fused multiply-adds per weight pair); stage 1's row scale
// is applied at the end as for one stage.
template <int NB, int ST>
struct PvqTile {
  static constexpr int V = 2 * NB;
  static constexpr int T = (V + 3) / 4;
  static constexpr int kDma = T * ST;
  static constexpr int kBVecs = 64 * T;          // per wave and stage
  const uint8_t *idx;      // [ST][N][K/4]
  const uint32_t *lut;     // LDS: 256 entries x 2 u32 (4 fp16)
  int K, N;
  half2_t r[NB][ST > 1 ? ST : 1];   // stage ratios of this lane's rows (entry 0 unused)
  __device__ __forceinline__ void prepare(const uint16_t *row_scale, int row0) {
    if constexpr (ST > 1) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int row = min(row0 + nb * 16, N - 1);
        const float s1 = f16_bits_to_f32(row_scale[row]);
#pragma unroll
        for (int st = 1; st < ST; ++st) {
          const _Float16 q = static_cast<_Float16>(f16_bits_to_f32(row_scale[static_cast<size_t>(st) * N + row]) / s1);
          r[nb][st] = half2_t{q, q};
        }
      }
    }
  }
  __device__ __forceinline__ void request(uint4 *bslot, int row0, int g, int kq, int wave) const {
#pragma unroll
    for (int st = 0; st < ST; ++st)
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int u = min(kq + 4 * t, V - 1);
        const int row = min(row0 + (u >> 1) * 16, N - 1);
        copy16_to_lds(idx + (static_cast<size_t>(st) * N + row) * (K / 4) + g * 32 + (u & 1) * 16,
                      bslot + kBVecs * (kWaves * st + wave) + 64 * t);
      }
  }
  // Natural order: the fp16 pairs of k-step t are weights 8 t .. 8 t + 7 of the
  // lane's word column, i.e. the two codebook entries of index bytes 2 t and
  // 2 t + 1 as they stand (four fp16 values each, no repacking).
  __device__ __forceinline__ void decode(const uint4 *bslot, int wave, int lane, uint32_t b[NB][16]) const {
    const int j = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int u = 2 * nb + (kq >> 1);
#pragma unroll
      for (int st = 0; st < ST; ++st) {
        const uint2 w = reinterpret_cast<const uint2 *>(bslot + kBVecs * (kWaves * st + wave) + 64 * (u >> 2) +
                                                         (u & 3) * 16 + j)[kq & 1];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t word = t < 2 ? w.x : w.y;
          const uint32_t ia = (word >> (16 * (t & 1))) & 0xFFu;
          const uint32_t ib = (word >> (16 * (t & 1) + 8)) & 0xFFu;
          const uint2 ca = *reinterpret_cast<const uint2 *>(lut + 2 * ia);
          const uint2 cb = *reinterpret_cast<const uint2 *>(lut + 2 * ib);
          const uint32_t v[4] = {ca.x, ca.y, cb.x, cb.y};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (st == 0) {
              b[nb][4 * t + e] = v[e];
            } else {
              b[nb][4 * t + e] = __builtin_bit_cast(
                  uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(half2_t, v[e]), r[nb][st > 0 ? st : 0],
                                                      __builtin_bit_cast(half2_t, b[nb][4 * t + e])));
            }
          }
        }
      }
    }
  }
};

// ------------------------------------------------------------------ mainloop

struct GemmArgs {
  const uint4 *xf;            // rotated activations [M][K], natural order
  uint16_t *y;                // [M][N]
  float *part;                // split-K partial tiles (S > 1)
  uint32_t *counters;         // split-K arrival counters, one per tile, zero on entry
  const uint16_t *row_scale;  // fp16 [N]
  int M, K, N, S;
};

// Depth of the copy ring in groups: the copies for group g + R - 1 are issued
// while group g is contracted. Three slots at 64 tokens keep two workgroups
// per CU within LDS.
template <int MT>
constexpr int ring_depth() {
  return MT >= 4 ? 3 : 4;
}

// Ring slot pointers: activations (16 * MT tokens x 16 vectors of 16 bytes;
// logical column c of token t at physical column c ^ (t & 15), so the 16-byte
// reads of 16 consecutive tokens at one column, one pass of a ds_read_b128, hit
// 16 distinct bank groups) and the index bytes of the four waves.
template <int R>
struct Ring {
  uint4 *a[R];
  uint4 *b[R];
};

// pre() runs once the first R - 1 groups' copies are in flight (it fills the
// codebook table and passes a barrier).
template <int NB, int ST, int MT, int R, class Pre>
__device__ __forceinline__ void gemm_body(const PvqTile<NB, ST> &tile, const GemmArgs &a, const Ring<R> &ring,
                                          Pre pre) {
  constexpr int CA = MT;   // activation copies per wave per group
  const int G = a.K / kGroup;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane & 15, kq = lane >> 4;
  const int split = blockIdx.x;
  const int tile_id = blockIdx.z * gridDim.y + blockIdx.y;
  const int row0 = blockIdx.y * (kWaves * 16 * NB) + wave * 16 * NB + j;
  const int m0 = blockIdx.z * (16 * MT);
  const int g0 = static_cast<int>((static_cast<long>(split) * G) / a.S);
  const int g1 = static_cast<int>((static_cast<long>(split + 1) * G) / a.S);

  float4_t acc[NB][MT];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nb][mt] = float4_t{0.f, 0.f, 0.f, 0.f};

  // Activation copies: wave w fills physical vectors [64 CA w, 64 CA (w + 1))
  // of the slot, CA copies of 64 lanes x 16 bytes. Tokens past M repeat token
  // M - 1 (their outputs are never stored).
  const uint4 *asrc[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int p = 64 * (CA * wave + i) + lane;
    const int tok = p >> 4, c = (p & 15) ^ (tok & 15);
    asrc[i] = a.xf + static_cast<size_t>(min(m0 + tok, a.M - 1)) * (a.K / 8) + c;
  }
  // copies for group g (clamped into the slice) into ring slot q
  auto request = [&](int q, int g) {
    const int gc = min(g, g1 - 1);
#pragma unroll
    for (int i = 0; i < CA; ++i) copy16_to_lds(asrc[i] + static_cast<size_t>(gc) * 16, ring.a[q] + 64 * (CA * wave + i));
    tile.request(ring.b[q], row0, gc, kq, wave);
  };
  constexpr int kCopies = CA + PvqTile<NB, ST>::kDma;   // per wave per group

  auto contract = [&](int q) {
    uint32_t b[NB][16];
    tile.decode(ring.b[q], wave, lane, b);
    const uint4 *slot = ring.a[q];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int tok = mt * 16 + j;
        const uint4 av = slot[tok * 16 + ((4 * kq + t) ^ j)];
        const half8_t aop = __builtin_bit_cast(half8_t, av);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const half8_t bop = __builtin_bit_cast(
              half8_t, make_uint4(b[nb][4 * t], b[nb][4 * t + 1], b[nb][4 * t + 2], b[nb][4 * t + 3]));
          acc[nb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, acc[nb][mt], 0, 0, 0);
        }
      }
    }
  };

#pragma unroll
  for (int q = 0; q < R - 1; ++q) request(q, g0 + q);
  pre();
  for (int g = g0; g < g1; g += R) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      // group g + q: its copies are the oldest kCopies of this wave's R - 1
      // groups in flight; after the barrier every wave's copies are in LDS and
      // every wave is done reading the slot refilled next
      wait_vm_lds<(R - 2) * kCopies>();
      __builtin_amdgcn_s_barrier();
      request((q + R - 1) % R, g + q + R - 1);
      if (g + q < g1) contract(q);
    }
  }
  wait_vm_lds<0>();   // no copy into LDS may outlive the workgroup

  if (a.S > 1) {
    // publish this slice's partial tile; the last slice to arrive sums them all
    constexpr int kTileFloats = NB * MT * 4 * kThreads;
    float *mine = a.part + (static_cast<size_t>(tile_id) * a.S + split) * kTileFloats + threadIdx.x;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) store_coherent(mine + ((nb * MT + mt) * 4 + r) * kThreads, acc[nb][mt][r]);
    wait_vm_lds<0>();   // the stores above have completed
    __syncthreads();
    __shared__ uint32_t last;
    if (threadIdx.x == 0)
      last = (__hip_atomic_fetch_add(a.counters + tile_id, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              static_cast<uint32_t>(a.S - 1))
                 ? 1u
                 : 0u;
    __syncthreads();
    if (!last) return;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[nb][mt] = float4_t{0.f, 0.f, 0.f, 0.f};
    for (int s2 = 0; s2 < a.S; ++s2) {
      float *src = a.part + (static_cast<size_t>(tile_id) * a.S + s2) * kTileFloats + threadIdx.x;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[nb][mt][r] += load_coherent(src + ((nb * MT + mt) * 4 + r) * kThreads);
    }
  }

  // D layout: lane holds tokens 4*kq + r (r = 0..3) of token tile mt, row j of block nb.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int row = row0 + nb * 16;
    if (row < a.N) {
      const float rs = f16_bits_to_f32(a.row_scale[row]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = m0 + mt * 16 + kq * 4 + r;
          if (tok < a.M) a.y[static_cast<size_t>(tok) * a.N + row] = f32_to_f16_bits(acc[nb][mt][r] * rs);
        }
      }
    }
  }
}

// The ring slots are separate LDS objects so the compiler can tell that a
// read of one slot does not depend on the copies in flight into the others.
template <int NB, int ST, int MT>
__global__ void __launch_bounds__(kThreads) gemm_pvq_kernel(const uint8_t *__restrict__ idx,
                                                            const uint8_t *__restrict__ codebook, GemmArgs a) {
  using Tile = PvqTile<NB, ST>;
  constexpr int R = ring_depth<MT>();
#define LBQ_SLOT(I)                                                                      \
  __shared__ __attribute__((aligned(16))) uint4 a##I[(I) < R ? 16 * MT * 16 : 1];        \
  __shared__ __attribute__((aligned(16))) uint4 b##I[(I) < R ? kWaves * ST * Tile::kBVecs : 1];
  LBQ_SLOT(0) LBQ_SLOT(1) LBQ_SLOT(2) LBQ_SLOT(3)
#undef LBQ_SLOT
  Ring<R> ring;
  {
    uint4 *as[4] = {a0, a1, a2, a3};
    uint4 *bs[4] = {b0, b1, b2, b3};
    for (int i = 0; i < R; ++i) {
      ring.a[i] = as[i];
      ring.b[i] = bs[i];
    }
  }
  __shared__ __attribute__((aligned(16))) uint32_t lut[512];
  // e4m3 -> fp16 table: 256 entries x 4 values, 2 u32 per entry. The codebook
  // words are loaded first and written to LDS once the ring's first copies are
  // in flight, so the two round trips overlap.
  static_assert(2 * kThreads == 512, "two table words per thread");
  const uint16_t *cb16 = reinterpret_cast<const uint16_t *>(codebook);
  const uint32_t two0 = cb16[threadIdx.x], two1 = cb16[threadIdx.x + kThreads];
  Tile tile{idx, lut, a.K, a.N, {}};
  tile.prepare(a.row_scale, blockIdx.y * (kWaves * 16 * NB) + (threadIdx.x >> 6) * 16 * NB + (threadIdx.x & 15));
  auto fill_lut = [&]() {
    const uint32_t two[2] = {two0, two1};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint32_t out = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        out |= static_cast<uint32_t>(e4m3_to_f16_bits((two[i] >> (8 * h)) & 0xFFu)) << (16 * h);
      lut[threadIdx.x + i * kThreads] = out;
    }
    barrier_lds();   // the table is complete; the ring's copies stay in flight
  };
  gemm_body<NB, ST, MT, R>(tile, a, ring, fill_lut);
}

template <int NB, int ST>
void launch_pvq_nb(int mt, dim3 grid, const uint8_t *idx, const uint8_t *codebook, const GemmArgs &a, hipStream_t s) {
  switch (mt) {
    case 1: hipLaunchKernelGGL((gemm_pvq_kernel<NB, ST, 1>), grid, dim3(kThreads), 0, s, idx, codebook, a); break;
    case 2: hipLaunchKernelGGL((gemm_pvq_kernel<NB, ST, 2>), grid, dim3(kThreads), 0, s, idx, codebook, a); break;
    default: hipLaunchKernelGGL((gemm_pvq_kernel<NB, ST, 4>), grid, dim3(kThreads), 0, s, idx, codebook, a); break;
  }
}

template <int ST>
void launch_pvq_st(int nb, int mt, dim3 grid, const uint8_t *idx, const uint8_t *codebook, const GemmArgs &a,
                   hipStream_t s) {
  if (nb == 1) launch_pvq_nb<1, ST>(mt, grid, idx, codebook, a, s);
  else launch_pvq_nb<2, ST>(mt, grid, idx, codebook, a, s);
}

}  // namespace

GemmPlan gemm_plan(int M, int K, int N, int stages) {
  // Token tiles of 16, 32 or 64. Two row blocks per wave only with >= 512 such
  // tiles, else one; then split K until about 768 workgroups run at up to 16
  // tokens and 384 beyond, every slice keeping at least four groups (measured
  // on the product-VQ 4096 -> 14336 shape at 16 and 64 tokens). Residual
  // stages carry more index bytes per weight: two row blocks per wave and
  // half as many workgroups (4096 -> 14336 at three stages: 16 tokens
  // 32.9 -> 26.6 us, 64 tokens 57.4 -> 44.9 us).
  GemmPlan p;
  p.mt = M <= 16 ? 1 : M <= 32 ? 2 : 4;
  const int G = K / kGroup;
  p.m_tiles = M > 0 ? (M + 16 * p.mt - 1) / (16 * p.mt) : 0;
  const long tiles2 = static_cast<long>((N + 127) / 128) * p.m_tiles;
  p.nb = (tiles2 >= 512 || stages > 1) ? 2 : 1;
  p.n_tiles = (N + 64 * p.nb - 1) / (64 * p.nb);
  const long tiles = static_cast<long>(p.n_tiles) * p.m_tiles;
  const long target = (M <= 16 ? 768 : 384) / (stages > 1 ? 2 : 1);
  p.S = 1;
  while (tiles * p.S < target && p.S < 16) p.S *= 2;
  while (p.S > 1 && p.S * 4 > G) p.S /= 2;
  return p;
}

GemmPlan gemm_rtn_plan(int M, int K, int N, int bits) {
  // Measured on the dense-stack and FFN shapes (K up to 17408, N 4096..28672,
  // M 8..256). Up to 32 tokens the loop is bound by each compute unit's
  // vector-memory address path: one row block per wave, and K split until
  // about 384 workgroups run, every slice keeping at least eight groups. From
  // 33 tokens two row blocks per wave (each activation fragment read from LDS
  // feeds two MFMAs; one for rows of >= 64 groups below 128 tokens), four once
  // that alone gives >= 384 workgroups (two for 8-bit codes: registers for
  // their planes), and K split until 256 workgroups run (512 for rows of >= 64
  // groups at >= 128 tokens), slices of at least sixteen groups: split-K
  // partial tiles go through device-coherent memory and cost more than a
  // partly idle chip. (Sweeps of 32-token tiles and of more workgroups at 64
  // and 256 tokens were faster back to back but not under graph replay.)
  GemmPlan p;
  p.mt = M <= 16 ? 1 : M <= 32 ? 2 : 4;
  const int G = K / kGroup;
  p.m_tiles = M > 0 ? (M + 16 * p.mt - 1) / (16 * p.mt) : 0;
  p.S = 1;
  if (p.mt <= 2) {
    p.nb = 1;
    p.n_tiles = (N + 63) / 64;
    const long tiles = static_cast<long>(p.n_tiles) * p.m_tiles;
    while (tiles * p.S < 384 && G / (2 * p.S) >= 4) p.S *= 2;
  } else {
    const long t4 = static_cast<long>((N + 255) / 256) * p.m_tiles;
    // long rows below 128 tokens: one block per wave, the split carries the chip
    p.nb = (t4 >= 384 && bits != 8) ? 4 : (G >= 64 && M < 128) ? 1 : 2;
    p.n_tiles = (N + 64 * p.nb - 1) / (64 * p.nb);
    const long tiles = static_cast<long>(p.n_tiles) * p.m_tiles;
    const long target = (G >= 64 && M >= 128) ? 512 : 256;
    while (tiles * p.S < target && G / (2 * p.S) >= 8) p.S *= 2;
  }
  // slices short enough for the kernel to stage their scale/zero words in LDS
  while ((G + p.S - 1) / p.S > gemm_rtn_meta_max_groups(p.nb)) p.S *= 2;
  // Grids of up to two workgroups per compute unit leave one wavefront per
  // SIMD, which then waits alone on its loads and barriers: there two wave
  // sets per workgroup (alternate groups of the slice) run on half as many
  // workgroups, from two row blocks per wave (tiles of 64 tokens) or half the
  // split (fewer tokens), whichever the sweep favoured. Larger grids already
  // hold two workgroups per compute unit, and the 512-thread form, with twice
  // the activation ring in LDS, measured slower there.
  if (static_cast<long>(p.n_tiles) * p.m_tiles * p.S <= 512 && p.nb <= 2) {
    GemmPlan q = p;
    q.kw = 2;
    if (p.mt == 4 && p.nb == 1) {
      q.nb = 2;
      q.n_tiles = (N + 127) / 128;
    } else if (p.S >= 2) {
      q.S = p.S / 2;
    } else if (p.nb == 1) {
      q.nb = 2;
      q.n_tiles = (N + 127) / 128;
    }
    if ((G + q.S - 1) / q.S <= gemm_rtn_meta_max_groups(q.nb)) p = q;
  }
  return p;
}

size_t gemm_part_bytes(const GemmPlan &p) {
  const size_t tiles = static_cast<size_t>(p.n_tiles) * p.m_tiles;
  return ((tiles * p.S * p.nb * p.mt * 4 * kThreads * 4 + 255) / 256) * 256;
}

size_t gemm_scratch_bytes(const GemmPlan &p) {
  if (p.S <= 1) return 0;
  const size_t tiles = static_cast<size_t>(p.n_tiles) * p.m_tiles;
  return gemm_part_bytes(p) + ((tiles * 4 + 255) / 256) * 256;
}

int gemm_counters(const GemmPlan &p) {
  return p.S > 1 ? p.n_tiles * p.m_tiles : 0;
}

uint32_t *gemm_counter_ptr(const GemmPlan &p, void *scratch) {
  if (p.S <= 1) return nullptr;
  return reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(scratch) + gemm_part_bytes(p));
}

hipError_t launch_gemm_pvq(const GemmPlan &p, const void *idx, const void *row_scale, const uint8_t *codebook,
                           const uint16_t *xf, uint16_t *y, int M, int K, int N, int stages, void *scratch,
                           hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if ((p.nb != 1 && p.nb != 2) || (p.mt != 1 && p.mt != 2 && p.mt != 4) || p.S < 1) return hipErrorInvalidValue;
  if (stages < 1 || stages > 3 || static_cast<long long>(stages) * N * (K / 4) >= (1ll << 31)) return hipErrorInvalidValue;
  GemmArgs a;
  a.xf = reinterpret_cast<const uint4 *>(xf);
  a.y = y;
  a.part = static_cast<float *>(scratch);
  a.counters = gemm_counter_ptr(p, scratch);
  a.row_scale = static_cast<const uint16_t *>(row_scale);
  a.M = M;
  a.K = K;
  a.N = N;
  a.S = p.S;
  const dim3 grid(static_cast<unsigned>(p.S), static_cast<unsigned>(p.n_tiles), static_cast<unsigned>(p.m_tiles));
  const uint8_t *ix = static_cast<const uint8_t *>(idx);
  if (stages == 1) launch_pvq_st<1>(p.nb, p.mt, grid, ix, codebook, a, s);
  else if (stages == 2) launch_pvq_st<2>(p.nb, p.mt, grid, ix, codebook, a, s);
  else launch_pvq_st<3>(p.nb, p.mt, grid, ix, codebook, a, s);
  return hipGetLastError();
}

}  // namespace lbq
