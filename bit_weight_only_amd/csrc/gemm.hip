// MFMA dequant-GEMM: y = x' W'^T with W' decoded inside the K mainloop straight
// into the B operand of v_mfma_f32_16x16x32_f16 (no expand-to-dense round trip
// through memory; the gridbook card names exactly that round trip as its
// prefill gap: Laguna-S-2.1 card, "Reading it honestly").
//
// Tiling. A workgroup of 4 wavefronts owns 64 * NB output columns (rows of W)
// and 16 * MT tokens; wave w owns NB blocks of 16 rows. The K range of the
// workgroup is one of S contiguous slices of the 128-groups (split-K when the
// tile grid alone would leave the chip idle). Per group:
//   * everything the group needs (the token tile's rotated activations, already
//     in the folded slot order: slot c of a 32-chunk = (x[c], x[c+16]); the
//     codes and (s, z) words of the wave's rows; the tokens' activation sums)
//     is copied global -> LDS asynchronously (global_load_lds) into a ring of
//     R slots, R - 1 groups ahead of the contraction, one barrier per group;
//   * lane (j, kq) of a wave decodes word column kq of row j of each of its NB
//     row blocks: 16 slots, the B operands of the group's 4 k-steps (slots
//     4t..4t+3 for step t). The A operand of lane (i, kq) is slots 4t..4t+3 of
//     token i's chunk kq, so A and B agree on which k each element is.
//   * RTN codes arrive as 16-byte copies: the four lanes (j, 0..3) copy four
//     consecutive (row block, plane) vectors of the group and a 4x4 transpose
//     across the four 16-lane rows (v_permlane32_swap + v_permlane16_swap)
//     leaves each lane its own word column of every plane.
//   * RTN: a code q of slot class m is OR-ed into the mantissa of fp16
//     2^(10-m), which gives exactly 2^(10-m) + q: one instruction per two
//     weights and no further arithmetic before the MFMA. The group's
//     contraction then equals P + sum_k x_k q_k with P = sum_k 2^(10-m_k) x_k,
//     so the accumulator starts at -(P + z T) (T = sum_k x_k; P and T per token
//     from the rotation launch) and ends at sum_k x_k (q_k - z); the group scale
//     is applied once per group in fp32 (y += s * D_g).
//   * PVQ: the row scale is constant along K, so B holds the codebook values
//     themselves (e4m3 values are exact in fp16, staged as a 2 KB fp16 table in
//     LDS) and the scale is applied once at the end.
// Split-K: each workgroup writes its fp32 partial tile to the workspace; the
// last of the S workgroups of a tile to arrive (an atomic counter the rotation
// launch cleared) sums the S partials in slice order and writes y, so the
// result does not depend on arrival order. No workgroup ever waits on another.
#include "device.h"
#include "kernels.h"

#include <algorithm>

namespace lbq {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// Transpose a 4x4 matrix held as element e of lanes in 16-lane row r: after
// the call, element e of lane (j, row r) is the old element r of lane (j, row e).
__device__ __forceinline__ void transpose4(uint32_t &e0, uint32_t &e1, uint32_t &e2, uint32_t &e3) {
  const auto a = __builtin_amdgcn_permlane32_swap(e0, e2, false, false);
  e0 = a[0];
  e2 = a[1];
  const auto b = __builtin_amdgcn_permlane32_swap(e1, e3, false, false);
  e1 = b[0];
  e3 = b[1];
  const auto c = __builtin_amdgcn_permlane16_swap(e0, e1, false, false);
  e0 = c[0];
  e1 = c[1];
  const auto d = __builtin_amdgcn_permlane16_swap(e2, e3, false, false);
  e2 = d[0];
  e3 = d[1];
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void global_void_t;

// Asynchronous copies global -> LDS (global_load_lds): lane l of the wave
// sends 16 (4) bytes from its own address src to dst_base + 16 l (4 l);
// dst_base must be the same for the whole wave. Counted by the vector-memory
// counter.
__device__ __forceinline__ void copy16_to_lds(const void *src, void *dst_base) {
  __builtin_amdgcn_global_load_lds((global_void_t *)src, (lds_void_t *)dst_base, 16, 0, 0);
}
__device__ __forceinline__ void copy4_to_lds(const void *src, void *dst_base) {
  __builtin_amdgcn_global_load_lds((global_void_t *)src, (lds_void_t *)dst_base, 4, 0, 0);
}

// s_waitcnt: at most N vector-memory operations of this wave outstanding, and
// every LDS operation done (gfx9 encoding: vmcnt bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// ------------------------------------------------------------------ B decoders
//
// Each decoder moves one group's codes for a wave into that wave's part of an
// LDS ring slot (kDma copies of 64 lanes per group) and later decodes them
// from there. Only the wave that copied a vector reads it back.

// RTN bit planes, NB row blocks per lane. The group's NB * BITS 16-byte
// vectors (row block nb, plane p) at u = nb * BITS + p are spread over the four
// kq lanes, T per lane (the last ones padded with repeats); after the copy back
// a 4x4 transpose across the four 16-lane rows leaves lane (j, kq) word kq of
// every plane. The (s, z) word of row block nb is copied by lane (j, nb).
template <int BITS, int NB>
struct RtnTile {
  static constexpr int U = NB * BITS;
  static constexpr int T = (U + 3) / 4;
  static constexpr bool kGroupScale = true;
  static constexpr int kDma = T + 1;          // copies per wave per group
  static constexpr int kBVecs = 64 * T;       // 16-byte vectors per wave per slot
  static constexpr int kCWords = 64;          // meta words per wave per slot
  const uint4 *planes;     // [N][G][BITS] 16-byte vectors
  const uint32_t *meta;    // [N][G] (fp16 s, fp16 z)
  int G, N;
  __device__ __forceinline__ void request(uint4 *bslot, uint32_t *cslot, int row0, int g, int kq, int wave) const {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int u = min(kq + 4 * t, U - 1);
      const int nb = u / BITS, p = u - (u / BITS) * BITS;
      const int row = min(row0 + nb * 16, N - 1);
      copy16_to_lds(planes + (static_cast<size_t>(row) * G + g) * BITS + p, bslot + kBVecs * wave + 64 * t);
    }
    const int row = min(row0 + min(kq, NB - 1) * 16, N - 1);
    copy4_to_lds(meta + static_cast<size_t>(row) * G + g, cslot + kCWords * wave);
  }
  // b[nb][c]: slot c of the lane's word column as fp16 pairs 2^(10 - m_c) + q
  // (the class offsets leave the contraction as the activation sum P, which
  // the caller removes together with z T); sc, zr: the row's scale and zero.
  __device__ __forceinline__ void decode(const uint4 *bslot, const uint32_t *cslot, int wave, int lane,
                                         uint32_t b[NB][16], float sc[NB], float zr[NB]) const {
    uint32_t w[4 * T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const uint4 v = bslot[kBVecs * wave + 64 * t + lane];
      uint32_t e0 = v.x, e1 = v.y, e2 = v.z, e3 = v.w;
      transpose4(e0, e1, e2, e3);
      w[4 * t] = e0;
      w[4 * t + 1] = e1;
      w[4 * t + 2] = e2;
      w[4 * t + 3] = e3;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint32_t mt = cslot[kCWords * wave + nb * 16 + (lane & 15)];
      if constexpr (BITS == 2) decode_slots2<true>(w[nb * BITS], w[nb * BITS + 1], b[nb]);
      else decode_slots_nib<BITS, true>(&w[nb * BITS], b[nb]);
      sc[nb] = f16_bits_to_f32(mt & 0xFFFFu);
      zr[nb] = f16_bits_to_f32(mt >> 16);
    }
  }
};

// Product-VQ indices: byte i of a row covers weights 4i..4i+3; a group's 32
// index bytes of a row are two 16-byte vectors (h = 0, 1), vector u = 2 nb + h
// of the lane set copied by lane (j, u). Lane (j, kq) needs word column kq
// (index bytes 8kq..8kq+7, weights 32kq..32kq+31): half kq & 1 of vector
// 2 nb + (kq >> 1).
template <int NB>
struct PvqTile {
  static constexpr int V = 2 * NB;
  static constexpr int T = (V + 3) / 4;
  static constexpr bool kGroupScale = false;
  static constexpr int kDma = T;
  static constexpr int kBVecs = 64 * T;
  static constexpr int kCWords = 1;
  const uint8_t *idx;      // [N][K/4]
  const uint32_t *lut;     // LDS: 256 entries x 2 u32 (4 fp16)
  int K, N;
  __device__ __forceinline__ void request(uint4 *bslot, uint32_t *, int row0, int g, int kq, int wave) const {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int u = min(kq + 4 * t, V - 1);
      const int row = min(row0 + (u >> 1) * 16, N - 1);
      copy16_to_lds(idx + static_cast<size_t>(row) * (K / 4) + g * 32 + (u & 1) * 16,
                      bslot + kBVecs * wave + 64 * t);
    }
  }
  // slot c = (w[c], w[c+16]); weights 4t..4t+3 use index byte t, weights
  // 16+4t.. use index byte t+4.
  __device__ __forceinline__ void decode(const uint4 *bslot, const uint32_t *, int wave, int lane, uint32_t b[NB][16],
                                         float sc[NB], float zr[NB]) const {
    const int j = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int u = 2 * nb + (kq >> 1);
      const uint2 w = reinterpret_cast<const uint2 *>(bslot + kBVecs * wave + 64 * (u >> 2) + (u & 3) * 16 + j)[kq & 1];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t ia = (w.x >> (8 * t)) & 0xFFu;
        const uint32_t ib = (w.y >> (8 * t)) & 0xFFu;
        const uint2 ca = *reinterpret_cast<const uint2 *>(lut + 2 * ia);
        const uint2 cb = *reinterpret_cast<const uint2 *>(lut + 2 * ib);
        b[nb][4 * t + 0] = (ca.x & 0xFFFFu) | (cb.x << 16);
        b[nb][4 * t + 1] = (ca.x >> 16) | (cb.x & 0xFFFF0000u);
        b[nb][4 * t + 2] = (ca.y & 0xFFFFu) | (cb.y << 16);
        b[nb][4 * t + 3] = (ca.y >> 16) | (cb.y & 0xFFFF0000u);
      }
      sc[nb] = 1.0f;
      zr[nb] = 0.0f;
    }
  }
};

// ------------------------------------------------------------------ mainloop

struct GemmArgs {
  const uint4 *xf;            // rotated activations [M][K], folded slot order
  const float2 *sums;         // RTN: per (group, token) (P, T) of the activations, [G][M]
  uint16_t *y;                // [M][N]
  float *part;                // split-K partial tiles (S > 1)
  uint32_t *counters;         // split-K arrival counters, one per tile, zero on entry
  const uint16_t *row_scale;  // PVQ: fp16 [N]; RTN: null
  int M, K, N, S;
};

// Depth of the copy ring in groups: the copies for group g + R - 1 are issued
// while group g is contracted. Three slots at 64 tokens keep two workgroups
// per CU within LDS.
template <int MT>
constexpr int ring_depth() {
  return MT >= 4 ? 3 : 4;
}

// Partial tiles cross workgroups (and L2 slices): agent-scope relaxed atomics
// read and write them at the device-coherent level, so no cache flush or
// invalidate is needed; a wait for the stores' completion orders them before
// the arrival counter.
__device__ __forceinline__ void store_coherent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Ring slot pointers: activations (16 * MT tokens x 16 vectors of 16 bytes;
// logical column c of token t at physical column c ^ (t & 7), so 16-byte reads
// of 8 consecutive tokens at one column hit 8 distinct bank groups), codes and
// meta words of the four waves.
template <int R>
struct Ring {
  uint4 *a[R];
  uint4 *b[R];
  uint32_t *c[R];
  float *p[R];   // per wave: (P, T) of the token tile's tokens
};

// dword copies per wave per group for the (P, T) pairs of 16 * MT tokens
template <int MT>
constexpr int pt_copies() {
  return MT >= 4 ? 2 : 1;
}

template <int NB, int MT, int R, class Tile>
__device__ __forceinline__ void gemm_body(const Tile &tile, const GemmArgs &a, const Ring<R> &ring) {
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
  float4_t yacc[NB][MT];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[nb][mt] = float4_t{0.f, 0.f, 0.f, 0.f};
      yacc[nb][mt] = float4_t{0.f, 0.f, 0.f, 0.f};
    }

  // Activation copies: wave w fills physical vectors [64 MT w, 64 MT (w + 1))
  // of the slot, MT copies of 64 lanes x 16 bytes. Tokens past M repeat token
  // M - 1 (their outputs are never stored).
  const uint4 *asrc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int p = 64 * (MT * wave + i) + lane;
    const int tok = p >> 4, c = (p & 15) ^ (tok & 7);
    asrc[i] = a.xf + static_cast<size_t>(min(m0 + tok, a.M - 1)) * (a.K / 8) + c;
  }
  // copies for group g (clamped into the slice) into ring slot q
  // (P, T) pairs of the token tile: dword d of a wave's copy is pair
  // (m0 + d / 2) of the group (tokens past M repeat token M - 1)
  constexpr int kPT = Tile::kGroupScale ? pt_copies<MT>() : 0;
  const float *psrc[kPT > 0 ? kPT : 1];
#pragma unroll
  for (int i = 0; i < kPT; ++i)
    psrc[i] = reinterpret_cast<const float *>(a.sums + min(m0 + (64 * i + lane) / 2, a.M - 1)) + (lane & 1);
  auto request = [&](int q, int g) {
    const int gc = min(g, g1 - 1);
#pragma unroll
    for (int i = 0; i < MT; ++i) copy16_to_lds(asrc[i] + static_cast<size_t>(gc) * 16, ring.a[q] + 64 * (MT * wave + i));
    tile.request(ring.b[q], ring.c[q], row0, gc, kq, wave);
#pragma unroll
    for (int i = 0; i < kPT; ++i)
      copy4_to_lds(psrc[i] + static_cast<size_t>(gc) * a.M * 2, ring.p[q] + 64 * (kPT * wave + i));
  };
  constexpr int kCopies = MT + Tile::kDma + kPT;   // per wave per group

  auto contract = [&](int q) {
    uint32_t b[NB][16];
    float sc[NB], zr[NB];
    tile.decode(ring.b[q], ring.c[q], wave, lane, b, sc, zr);
    const uint4 *slot = ring.a[q];
    if constexpr (Tile::kGroupScale) {
      // the group's contraction starts at -(P + z T) for the lane's 4 tokens
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const float4 *pt = reinterpret_cast<const float4 *>(ring.p[q] + 64 * kPT * wave + 2 * (mt * 16 + 4 * kq));
        const float4 u = pt[0], v = pt[1];   // (P, T) of tokens 4kq .. 4kq + 3
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[nb][mt] = float4_t{fmaf(-zr[nb], u.y, -u.x), fmaf(-zr[nb], u.w, -u.z), fmaf(-zr[nb], v.y, -v.x),
                                 fmaf(-zr[nb], v.w, -v.z)};
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int tok = mt * 16 + j;
        const uint4 av = slot[tok * 16 + ((4 * kq + t) ^ (tok & 7))];
        const half8_t aop = __builtin_bit_cast(half8_t, av);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const half8_t bop = __builtin_bit_cast(
              half8_t, make_uint4(b[nb][4 * t], b[nb][4 * t + 1], b[nb][4 * t + 2], b[nb][4 * t + 3]));
          acc[nb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, acc[nb][mt], 0, 0, 0);
        }
      }
    }
    if constexpr (Tile::kGroupScale) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) yacc[nb][mt] += sc[nb] * acc[nb][mt];
    }
  };

#pragma unroll
  for (int q = 0; q < R - 1; ++q) request(q, g0 + q);
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

  if constexpr (!Tile::kGroupScale) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) yacc[nb][mt] = acc[nb][mt];
  }

  if (a.S > 1) {
    // publish this slice's partial tile; the last slice to arrive sums them all
    constexpr int kTileFloats = NB * MT * 4 * kThreads;
    float *mine = a.part + (static_cast<size_t>(tile_id) * a.S + split) * kTileFloats + threadIdx.x;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) store_coherent(mine + ((nb * MT + mt) * 4 + r) * kThreads, yacc[nb][mt][r]);
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
      for (int mt = 0; mt < MT; ++mt) yacc[nb][mt] = float4_t{0.f, 0.f, 0.f, 0.f};
    for (int s2 = 0; s2 < a.S; ++s2) {
      float *src = a.part + (static_cast<size_t>(tile_id) * a.S + s2) * kTileFloats + threadIdx.x;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) yacc[nb][mt][r] += load_coherent(src + ((nb * MT + mt) * 4 + r) * kThreads);
    }
  }

  // D layout: lane holds tokens 4*kq + r (r = 0..3) of token tile mt, row j of block nb.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int row = row0 + nb * 16;
    if (row < a.N) {
      const float rs = a.row_scale ? f16_bits_to_f32(a.row_scale[row]) : 1.0f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = m0 + mt * 16 + kq * 4 + r;
          if (tok < a.M) a.y[static_cast<size_t>(tok) * a.N + row] = f32_to_f16_bits(yacc[nb][mt][r] * rs);
        }
      }
    }
  }
}

// The ring slots are separate LDS objects so the compiler can tell that a
// read of one slot does not depend on the copies in flight into the others.
#define LBQ_SLOT(I)                                                                      \
  __shared__ __attribute__((aligned(16))) uint4 a##I[16 * MT * 16];                     \
  __shared__ __attribute__((aligned(16))) uint4 b##I[kWaves * Tile::kBVecs];            \
  __shared__ __attribute__((aligned(16))) uint32_t c##I[kWaves * Tile::kCWords];        \
  __shared__ __attribute__((aligned(16))) float p##I[Tile::kGroupScale ? kWaves * 64 * pt_copies<MT>() : 4];
#define LBQ_RING                                                                         \
  constexpr int R = ring_depth<MT>();                                                    \
  LBQ_SLOT(0) LBQ_SLOT(1) LBQ_SLOT(2) LBQ_SLOT(3)                                        \
  Ring<R> ring;                                                                          \
  {                                                                                      \
    uint4 *as[4] = {a0, a1, a2, a3};                                                     \
    uint4 *bs[4] = {b0, b1, b2, b3};                                                     \
    uint32_t *cs[4] = {c0, c1, c2, c3};                                                  \
    float *ps[4] = {p0, p1, p2, p3};                                                     \
    for (int i = 0; i < R; ++i) {                                                        \
      ring.a[i] = as[i];                                                                 \
      ring.b[i] = bs[i];                                                                 \
      ring.c[i] = cs[i];                                                                 \
      ring.p[i] = ps[i];                                                                 \
    }                                                                                    \
  }

template <int BITS, int NB, int MT>
__global__ void __launch_bounds__(kThreads) gemm_rtn_kernel(const uint4 *__restrict__ planes,
                                                            const uint32_t *__restrict__ meta, GemmArgs a) {
  using Tile = RtnTile<BITS, NB>;
  LBQ_RING
  Tile tile{planes, meta, a.K / kGroup, a.N};
  gemm_body<NB, MT, R>(tile, a, ring);
}

template <int NB, int MT>
__global__ void __launch_bounds__(kThreads) gemm_pvq_kernel(const uint8_t *__restrict__ idx,
                                                            const uint8_t *__restrict__ codebook, GemmArgs a) {
  using Tile = PvqTile<NB>;
  LBQ_RING
  __shared__ __attribute__((aligned(16))) uint32_t lut[512];
  // e4m3 -> fp16 table: 256 entries x 4 values, 2 u32 per entry.
  for (int e = threadIdx.x; e < 512; e += kThreads) {
    const uint32_t two = reinterpret_cast<const uint16_t *>(codebook)[e];
    uint32_t out = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) out |= static_cast<uint32_t>(e4m3_to_f16_bits((two >> (8 * h)) & 0xFFu)) << (16 * h);
    lut[e] = out;
  }
  __syncthreads();
  Tile tile{idx, lut, a.K, a.N};
  gemm_body<NB, MT, R>(tile, a, ring);
}

#undef LBQ_RING
#undef LBQ_SLOT

}  // namespace

GemmPlan gemm_plan(int M, int K, int N) {
  // Measured on the dense-stack and FFN shapes (K, N up to 17408, M 4..256):
  // two row blocks per wave once that still gives >= 128 tiles, else one; with
  // few tiles split K until about 192 workgroups run (384 for long rows at
  // >= 64 tokens); with many tiles at >= 64 tokens split 2 (4 for long rows)
  // unless there are >= 512 tiles. Every slice keeps at least four groups.
  GemmPlan p;
  p.mt = M <= 16 ? 1 : M <= 32 ? 2 : 4;
  const int G = K / kGroup;
  p.m_tiles = M > 0 ? (M + 16 * p.mt - 1) / (16 * p.mt) : 0;
  const long tiles2 = static_cast<long>((N + 127) / 128) * p.m_tiles;
  p.nb = tiles2 >= 128 ? 2 : 1;
  p.n_tiles = (N + kWaves * 16 * p.nb - 1) / (kWaves * 16 * p.nb);
  const long tiles = static_cast<long>(p.n_tiles) * p.m_tiles;
  p.S = 1;
  if (p.nb == 2) {
    if (M >= 64 && tiles < 512) p.S = G > 64 ? 4 : 2;
  } else {
    const long target = (M >= 64 && G > 64) ? 384 : 192;
    while (tiles * p.S < target && p.S < 16) p.S *= 2;
  }
  while (p.S > 1 && p.S * 4 > G) p.S /= 2;
  return p;
}

size_t gemm_part_bytes(const GemmPlan &p) {
  const size_t tiles = static_cast<size_t>(p.n_tiles) * p.m_tiles;
  return ((tiles * p.S * p.nb * p.mt * kThreads * 16 + 255) / 256) * 256;
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

namespace {

template <int NB, int MT>
void launch_pvq_nb(dim3 grid, const uint8_t *idx, const uint8_t *codebook, const GemmArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((gemm_pvq_kernel<NB, MT>), grid, dim3(kThreads), 0, s, idx, codebook, a);
}

template <int BITS, int NB>
void launch_rtn_nb(int mt, dim3 grid, const uint4 *pl, const uint32_t *meta, const GemmArgs &a, hipStream_t s) {
  switch (mt) {
    case 1: hipLaunchKernelGGL((gemm_rtn_kernel<BITS, NB, 1>), grid, dim3(kThreads), 0, s, pl, meta, a); break;
    case 2: hipLaunchKernelGGL((gemm_rtn_kernel<BITS, NB, 2>), grid, dim3(kThreads), 0, s, pl, meta, a); break;
    default: hipLaunchKernelGGL((gemm_rtn_kernel<BITS, NB, 4>), grid, dim3(kThreads), 0, s, pl, meta, a); break;
  }
}

template <int BITS>
void launch_rtn_bits(const GemmPlan &p, dim3 grid, const uint4 *pl, const uint32_t *meta, const GemmArgs &a,
                     hipStream_t s) {
  if (p.nb == 1) launch_rtn_nb<BITS, 1>(p.mt, grid, pl, meta, a, s);
  else launch_rtn_nb<BITS, 2>(p.mt, grid, pl, meta, a, s);
}

}  // namespace

hipError_t launch_gemm(const GemmPlan &p, int format, int bits, const void *planes, const void *meta,
                       const uint8_t *codebook, const uint16_t *xf, const float2 *sums, uint16_t *y, int M, int K,
                       int N, void *scratch, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if ((p.nb != 1 && p.nb != 2) || (p.mt != 1 && p.mt != 2 && p.mt != 4) || p.S < 1) return hipErrorInvalidValue;
  GemmArgs a;
  a.xf = reinterpret_cast<const uint4 *>(xf);
  a.sums = sums;
  a.y = y;
  a.part = static_cast<float *>(scratch);
  a.counters = gemm_counter_ptr(p, scratch);
  a.row_scale = format == 1 ? static_cast<const uint16_t *>(meta) : nullptr;
  a.M = M;
  a.K = K;
  a.N = N;
  a.S = p.S;
  const dim3 grid(static_cast<unsigned>(p.S), static_cast<unsigned>(p.n_tiles), static_cast<unsigned>(p.m_tiles));
  if (format == 1) {
    const uint8_t *idx = static_cast<const uint8_t *>(planes);
    if (p.nb == 1) {
      if (p.mt == 1) launch_pvq_nb<1, 1>(grid, idx, codebook, a, s);
      else if (p.mt == 2) launch_pvq_nb<1, 2>(grid, idx, codebook, a, s);
      else launch_pvq_nb<1, 4>(grid, idx, codebook, a, s);
    } else {
      if (p.mt == 1) launch_pvq_nb<2, 1>(grid, idx, codebook, a, s);
      else if (p.mt == 2) launch_pvq_nb<2, 2>(grid, idx, codebook, a, s);
      else launch_pvq_nb<2, 4>(grid, idx, codebook, a, s);
    }
    return hipGetLastError();
  }
  const uint4 *pl = static_cast<const uint4 *>(planes);
  const uint32_t *mt = static_cast<const uint32_t *>(meta);
  switch (bits) {
    case 2: launch_rtn_bits<2>(p, grid, pl, mt, a, s); break;
    case 3: launch_rtn_bits<3>(p, grid, pl, mt, a, s); break;
    default: launch_rtn_bits<4>(p, grid, pl, mt, a, s); break;
  }
  return hipGetLastError();
}

}  // namespace lbq
