// MFMA dequant-GEMM for RTN codes: y = x' W'^T with W' = s (q - z) per
// 128-group (Qwen3-8B BPDQ model card, group-wise scale and zero), decoded
// inside the K mainloop into the B operand of v_mfma_f32_16x16x32_f16 (no
// expand-to-dense round trip through memory, the gap the Laguna-S-2.1 card
// names for its prefill path in "Reading it honestly").
//
// B = round_fp16(s q). A code q of slot class m OR-ed into the mantissa of fp16
// 2^(10 - m) is exactly h = 2^(10 - m) + q, and one v_pk_fma_f16
// h * s + (-s 2^(10 - m)) is round(s q) for two weights at once: inside the
// fused operation h * s is exact and the addend cancels the offset exactly.
// So each pair of weights costs two VALU operations (mask-insert, fma) and the
// accumulators run through the whole K range with no per-group rescaling.
// Every class sits at mantissa bit 4 or above (offsets 64, 16, 4), which keeps
// the addends finite for every scale below 2^10.
// The zero-point term -s z T_g (T_g = sum of the group's rotated activations)
// is one MFMA per 16 groups at the end of the slice: A holds (T_g/16 high,
// T_g/16 low) fp16 pairs per (token, group), B the pairs (-16 s z, -16 s z).
//
// Tiling: a workgroup of 4 KW wavefronts owns 64 NB output rows and 16 MT
// tokens; row wave w (= wave mod 4) owns NB blocks of 16 rows, so each A
// fragment read from LDS feeds NB MFMAs. The workgroup's K range is one of S
// slices of the 128-groups (split-K when the tile grid alone leaves the chip
// idle). With KW = 2 the two wave sets take alternate groups of the slice, so
// each SIMD holds two wavefronts that hide each other's waits, and their
// accumulators are added in LDS at the end (set 0 + set 1: a fixed order).
// Per group:
//  * the token tile's rotated activations (folded slot order: u32 slot c of a
//    32-chunk = (x[c], x[c + 16])) are copied global -> LDS asynchronously into
//    a ring of three slots, two groups ahead, one barrier per group;
//  * each wave's code vectors go straight into registers by buffer loads, two
//    groups ahead (offsets past the end return zeros without a memory access:
//    rows past N, groups past the slice); a 4x4 lane transpose gives lane
//    (j, kq) word column kq of every plane of its rows;
//  * the (s, z) words of the workgroup's rows over its slice are staged in LDS
//    once, in whole 16-byte vectors, before the loop (per group and row they
//    would cost one 128-byte line request each for 4 bytes);
//  * for k-step t, lane (i, kq) supplies slots 4t..4t+3 of token i's chunk kq
//    as A and slots 4t..4t+3 of row j's word column kq as B, so both operands
//    agree on which k each element is.
// Split-K: each workgroup writes its fp32 partial tile to the workspace; the
// last of the S workgroups of a tile to arrive (an atomic counter the rotation
// launch cleared) sums the S partials in slice order and writes y, so the
// result does not depend on arrival order. No workgroup ever waits on another.
#include "device.h"
#include "gemm_common.h"
#include "kernels.h"

namespace lbq {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// Ring slots: loads run kRing - 1 groups ahead. Deeper rings measured no
// faster: at few tokens the loop is bound by the compute unit's vector-memory
// address path (about one 128-byte line per few cycles), not by latency.
#ifndef LBQ_GEMM_RING
#define LBQ_GEMM_RING 3
#endif
constexpr int kRing = LBQ_GEMM_RING;
static_assert(kRing >= 3 && kRing <= 8, "ring depth");
constexpr int kBufferFlags = 0x00020000;        // buffer descriptor word 3 (32-bit data, no swizzle)
constexpr uint32_t kOutOfRange = 0x80000000u;   // buffer offset past every supported size

// Slice length (groups) up to which the scale/zero words of a workgroup's rows
// are staged in LDS (about 24 KB); the plans split K further when needed.
__host__ __device__ constexpr int meta_max_groups(int nb) {
  return nb == 1 ? 88 : nb == 2 ? 40 : 16;
}
// 16-byte meta vectors per row of a slice of ns groups (4-group aligned ends)
__host__ __device__ constexpr int meta_vectors(int ns) {
  return (ns + 6) / 4;
}

struct RtnGemmArgs {
  const uint4 *xf;         // rotated activations [M][K] fp16, folded slot order
  const uint4 *tz;         // [M][Gp / 4] of 4 u32: (T/16 high, T/16 low) fp16 per (token, group)
  const uint4 *planes;     // [N][G][BITS] 16-byte plane vectors (grouped: base of all experts' planes)
  const uint32_t *meta;    // [N][G] (fp16 s, fp16 z) (grouped: base of all experts' meta)
  uint16_t *y;             // [M][N]
  float *part;             // split-K partial tiles (S > 1)
  uint32_t *counters;      // split-K arrival counters, one per tile, zero on entry
  int M, K, N, S, Gp;
  int MS;                  // LDS row stride (words) of the staged scale/zero words: 4 vectors + 1
  // grouped GEMM over routed experts (gemm_rtn_grouped_kernel): a workgroup's
  // token tile is entries i0 .. i0 + cnt - 1 of the expert-sorted assignment
  // list, all routed to one expert e, whose weight sits at the byte offsets
  // plane_off[e] / meta_off[e]
  const int4 *tiles;       // [max tiles] (e, i0, cnt, bits), from moe_tiles
  const int32_t *n_tiles;  // tiles in use
  const uint64_t *plane_off, *meta_off;
  const int32_t *perm;     // list entry -> assignment index t * top_k + j
  int act_div;             // activation row of entry i: perm[i] / act_div, or i when 0
  int out_perm;            // output row of entry i: perm[i] when 1, else i
  float *out;              // fp32 outputs [rows][N]
};

// The token tile of one workgroup: dense, tokens m0 .. m0 + 16 MT - 1 of x;
// grouped, entries i0 .. i0 + cnt - 1 of the assignment list.
struct TokenTile {
  int m0, i0, cnt;
};

__device__ __forceinline__ uint32_t pk_fma(uint32_t h, half2_t s2, half2_t c) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(half2_t, h), s2, c));
}

// Slot classes. 2-bit: slot 2p / 2p + 1 is field p of the even / odd merged
// word; fields 2..4 sit at mantissa bits 4, 6, 8, fields 5..7 land there after
// a shift right by 6 and fields 0, 1 at bits 4, 6 after a shift left by 4.
// Class index (m - 4) / 2. 3/4-bit: nibble i of the merged nibble words, moved
// to bits 4..7 (class 0, m = 4) by a shift of 4 - 4i. 8-bit: the low nibble at
// bits 2..5 and the high nibble at bits 6..9 (one class, m = 2).
template <int BITS>
__host__ __device__ constexpr int gemm_slot_class(int c) {
  if constexpr (BITS == 2) {
    constexpr int kField[8] = {0, 1, 0, 1, 2, 0, 1, 2};
    return kField[c >> 1];
  } else {
    return 0;
  }
}
template <int BITS>
constexpr int gemm_num_classes() {
  return BITS == 2 ? 3 : 1;
}
// The offset 2^(10 - m) of class c (the decode removes s times it).
template <int BITS>
__host__ __device__ constexpr float gemm_class_offset(int c) {
  return BITS == 8 ? 256.0f : static_cast<float>(1 << (6 - 2 * c));
}

// Biased decode of one 32-code word column into the 16 slots (fp16 pairs
// 2^(10 - m) + q for the codes of positions c and c + 16).
template <int BITS>
__device__ __forceinline__ void decode_biased(const uint32_t *w, uint32_t h[16]) {
  if constexpr (BITS == 2) {
    uint32_t e, o;
    merge2(w[0], w[1], e, o);
    const uint32_t el = e << 4, ol = o << 4, er = e >> 6, orr = o >> 6;
    const uint32_t c4 = biased_one2(4), c6 = biased_one2(6), c8 = biased_one2(8);
    h[0] = and_or(el, 0x00300030u, c4);
    h[1] = and_or(ol, 0x00300030u, c4);
    h[2] = and_or(el, 0x00C000C0u, c6);
    h[3] = and_or(ol, 0x00C000C0u, c6);
    h[4] = and_or(e, 0x00300030u, c4);
    h[5] = and_or(o, 0x00300030u, c4);
    h[6] = and_or(e, 0x00C000C0u, c6);
    h[7] = and_or(o, 0x00C000C0u, c6);
    h[8] = and_or(e, 0x03000300u, c8);
    h[9] = and_or(o, 0x03000300u, c8);
    h[10] = and_or(er, 0x00300030u, c4);
    h[11] = and_or(orr, 0x00300030u, c4);
    h[12] = and_or(er, 0x00C000C0u, c6);
    h[13] = and_or(orr, 0x00C000C0u, c6);
    h[14] = and_or(er, 0x03000300u, c8);
    h[15] = and_or(orr, 0x03000300u, c8);
  } else if constexpr (BITS == 8) {
    // nibble i of lo[r] / hi[r] is the low / high half of code 4i + r; slot
    // 4p + r takes nibbles p (low half of the slot) and p + 4 (high half)
    uint32_t lo[4], hi[4];
    merge_nibbles<4>(w, lo);
    merge_nibbles<4>(w + 4, hi);
    const uint32_t c2 = biased_one2(2);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      h[r] = and_or(hi[r] << 6, 0x03C003C0u, and_or(lo[r] << 2, 0x003C003Cu, c2));
      h[4 + r] = and_or(hi[r] << 2, 0x03C003C0u, and_or(lo[r] >> 2, 0x003C003Cu, c2));
      h[8 + r] = and_or(hi[r] >> 2, 0x03C003C0u, and_or(lo[r] >> 6, 0x003C003Cu, c2));
      h[12 + r] = and_or(hi[r] >> 6, 0x03C003C0u, and_or(lo[r] >> 10, 0x003C003Cu, c2));
    }
  } else {
    uint32_t n[4];
    merge_nibbles<BITS>(w, n);
    const uint32_t c4 = biased_one2(4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      h[r] = and_or(n[r] << 4, 0x00F000F0u, c4);
      h[4 + r] = and_or(n[r], 0x00F000F0u, c4);
      h[8 + r] = and_or(n[r] >> 4, 0x00F000F0u, c4);
      h[12 + r] = and_or(n[r] >> 8, 0x00F000F0u, c4);
    }
  }
}

// One workgroup's tile: the mainloop shared by the dense and the grouped GEMM.
template <int BITS, int NB, int MT, int KW, bool GROUPED>
__device__ __forceinline__ void gemm_rtn_body(const RtnGemmArgs &a, const uint4 *planes, const uint32_t *meta,
                                              const TokenTile tt, uint4 *const *xs, uint32_t *msm) {
  static_assert(KW == 1 || (KW == 2 && NB <= 2), "wave sets");
  constexpr int kAll = kThreads * KW;    // threads of the workgroup
  constexpr int kSlot = 16 * MT * 16;    // 16-byte vectors of one group's activations in a ring slot
  constexpr int U = NB * BITS;           // 16-byte plane vectors of a wave's rows per group
  constexpr int T = (U + 3) / 4;         // of them per lane
  constexpr int D = kRing - 1;           // groups in flight
  constexpr int CA = MT;                 // activation copies per wave per group (16 MT rows x 256 B)
  constexpr int kLoads = CA + T;         // vector-memory operations per wave per group
  constexpr int kRowsWG = kWaves * 16 * NB;
  constexpr int kMetaIters = (kRowsWG * meta_vectors(meta_max_groups(NB)) + kAll - 1) / kAll;
  constexpr int C = gemm_num_classes<BITS>();
  // msm: [kRowsWG][a.MS] (s, z) of group gb0 + c at column c; xs: the ring slots

  const int lane = threadIdx.x & 63;
  const int wave = (threadIdx.x >> 6) & (kWaves - 1);   // row wave
  const int kh = static_cast<int>(threadIdx.x) / kThreads;   // wave set: groups g0 + kh, g0 + kh + KW, ...
  const int j = lane & 15, kq = lane >> 4;
  const int G = a.K / kGroup;
  const int split = blockIdx.x;
  const int tile_id = blockIdx.z * gridDim.y + blockIdx.y;
  const int row0 = blockIdx.y * (kWaves * 16 * NB) + wave * 16 * NB + j;   // the lane's row of block 0
  const int g0 = static_cast<int>((static_cast<long>(split) * G) / a.S);
  const int g1 = static_cast<int>((static_cast<long>(split + 1) * G) / a.S);

  const int m0 = tt.m0;
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint4 *>(planes), 0, a.N * G * BITS * 16, kBufferFlags);
  const __amdgpu_buffer_rsrc_t mrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(meta), 0, a.N * G * 4, kBufferFlags);
  // x / tz row of token slot tok of the tile (slots past the tile repeat its
  // last token; their outputs are never stored)
  auto act_row = [&](int tok) -> size_t {
    if constexpr (GROUPED) {
      const int i = tt.i0 + min(tok, tt.cnt - 1);
      return static_cast<size_t>(a.act_div ? a.perm[i] / a.act_div : i);
    } else {
      return static_cast<size_t>(min(m0 + tok, a.M - 1));
    }
  };

  // lane (j, kq) loads plane vectors u = kq + 4t of its rows: block u / BITS, plane u % BITS
  uint32_t poff[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int u = kq + 4 * t;
    const int row = row0 + (u / BITS) * 16;
    poff[t] = (u < U && row < a.N) ? (static_cast<uint32_t>(row) * G * BITS + u % BITS) * 16 : kOutOfRange;
  }
  // scale/zero staging loads: thread i + kThreads it takes vector v of local
  // row r (consecutive threads, consecutive vectors of a row). Issued first, so
  // they arrive ahead of the ring's loads.
  const int gb0 = g0 & ~3;
  const int nq = (((g1 + 3) & ~3) - gb0) / 4;
  uint4 mst[kMetaIters];
#pragma unroll
  for (int it = 0; it < kMetaIters; ++it) {
    const int i = static_cast<int>(threadIdx.x) + it * kAll;
    const int r = i / nq, v = i - r * nq, row = blockIdx.y * kRowsWG + r;
    const uint32_t off = (r < kRowsWG && row < a.N) ? (static_cast<uint32_t>(row) * G + gb0) * 4 + v * 16 : kOutOfRange;
    mst[it] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(mrs, off, 0, 0));
  }
  // activation copies: wave w fills physical vectors [64 CA w, 64 CA (w + 1)) of
  // a slot. Logical column c of token t sits at physical column c ^ (t & 15), so
  // the 16-byte reads of 16 consecutive tokens at one column (one pass of a
  // ds_read_b128) hit 16 distinct bank groups. Tokens past M repeat token M - 1
  // (their outputs are never stored).
  const uint4 *asrc[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int p = 64 * (CA * wave + i) + lane;
    const int tok = p >> 4, c = (p & 15) ^ (tok & 15);
    asrc[i] = a.xf + act_row(tok) * (a.K / 8) + c;
  }

  uint4 bv[kRing][T];
  float4_t acc[NB][MT];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nb][mt] = float4_t{0.f, 0.f, 0.f, 0.f};

  // loads of step st (this wave set's group g0 + KW st + kh) into ring slot q
  // (past the slice: the activation copies repeat the slice's last group, the
  // code loads return zeros)
  auto issue = [&](int q, int st) {
    const int g = g0 + KW * st + kh;
    const int gc = min(g, g1 - 1);
#pragma unroll
    for (int i = 0; i < CA; ++i)
      copy16_to_lds(asrc[i] + static_cast<size_t>(gc) * 16, xs[q] + kh * kSlot + 64 * (CA * wave + i));
    const uint32_t past = g < g1 ? 0u : kOutOfRange;
#pragma unroll
    for (int t = 0; t < T; ++t)
      bv[q][t] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(prs, (poff[t] | past) + g * (BITS * 16), 0, 0));
  };
  // this lane's row of block nb in the staged scale/zero words
  const uint32_t *mrow = msm + (wave * 16 * NB + j) * a.MS - gb0;

  auto contract = [&](int q, int g) {
    // the group's A fragments first: their LDS latency overlaps the decode
    const uint4 *slot = xs[q] + kh * kSlot;
    half8_t av[4][MT];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        av[t][mt] = __builtin_bit_cast(half8_t, slot[(mt * 16 + j) * 16 + ((4 * kq + t) ^ j)]);
    __builtin_amdgcn_sched_barrier(0);
    uint32_t w[4 * T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      uint32_t e0 = bv[q][t].x, e1 = bv[q][t].y, e2 = bv[q][t].z, e3 = bv[q][t].w;
      transpose4(e0, e1, e2, e3);
      w[4 * t] = e0;
      w[4 * t + 1] = e1;
      w[4 * t + 2] = e2;
      w[4 * t + 3] = e3;
    }
    half2_t s2[NB], nc[NB][C];
    uint32_t h[NB][16];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const _Float16 s = __builtin_bit_cast(half2_t, mrow[nb * 16 * a.MS + g])[0];
      s2[nb] = half2_t{s, s};
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const _Float16 off = static_cast<_Float16>(-gemm_class_offset<BITS>(c));   // -2^(10 - m)
        nc[nb][c] = s2[nb] * half2_t{off, off};
      }
      decode_biased<BITS>(&w[nb * BITS], h[nb]);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        uint32_t b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          b[e] = pk_fma(h[nb][4 * t + e], s2[nb], nc[nb][gemm_slot_class<BITS>(4 * t + e)]);
        const half8_t bop = __builtin_bit_cast(half8_t, make_uint4(b[0], b[1], b[2], b[3]));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[nb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[t][mt], bop, acc[nb][mt], 0, 0, 0);
      }
    }
  };

#pragma unroll
  for (int q = 0; q < D; ++q) issue(q, q);
  // the staged words into LDS (visible after the loop's first barrier)
#pragma unroll
  for (int it = 0; it < kMetaIters; ++it) {
    const int i = static_cast<int>(threadIdx.x) + it * kAll;
    const int r = i / nq, v = i - r * nq;
    if (r < kRowsWG) {
      uint32_t *dst = msm + r * a.MS + 4 * v;
      dst[0] = mst[it].x;
      dst[1] = mst[it].y;
      dst[2] = mst[it].z;
      dst[3] = mst[it].w;
    }
  }
  const int nst = (g1 - g0 + KW - 1) / KW;   // steps (the same count for every wave set)
  for (int st = 0; st < nst; st += kRing) {
#pragma unroll
    for (int q = 0; q < kRing; ++q) {
      // step st + q: its loads are the oldest kLoads of this wave's D steps in
      // flight; after the barrier every wave's copies are in LDS and every wave
      // is done reading the slot refilled next
      wait_vm_lds<(D - 1) * kLoads>();
      __builtin_amdgcn_s_barrier();
      issue((q + D) % kRing, st + q + D);
      const int g = g0 + KW * (st + q) + kh;
      if (g < g1) contract(q, g);
    }
  }

  // zero-point term of the slice: K = (group, high/low) over 16 groups per MFMA;
  // lane (j, kq) covers groups 16 c + 4 kq .. + 3 (the wave sets alternate)
  for (int c16 = g0 / 16 + kh; c16 <= (g1 - 1) / 16; c16 += KW) {
    half8_t za[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      za[mt] = __builtin_bit_cast(half8_t, a.tz[act_row(mt * 16 + j) * (a.Gp / 4) + 4 * c16 + kq]);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      uint32_t b[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int g = 16 * c16 + 4 * kq + e;
        const half2_t sz = __builtin_bit_cast(half2_t, (g >= g0 && g < g1) ? mrow[nb * 16 * a.MS + g] : 0u);
        const _Float16 v = static_cast<_Float16>(-16.0f) * (sz[0] * sz[1]);
        b[e] = __builtin_bit_cast(uint32_t, half2_t{v, v});
      }
      const half8_t bop = __builtin_bit_cast(half8_t, make_uint4(b[0], b[1], b[2], b[3]));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[nb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(za[mt], bop, acc[nb][mt], 0, 0, 0);
    }
  }
  wait_vm_lds<0>();   // no copy into LDS may outlive the workgroup
  if constexpr (KW > 1) {
    // set 1 hands its accumulators to set 0 through the first ring slot
    // (NB MT 4 floats per thread: NB MT 4 KB per wave set)
    static_assert(NB * MT * 4 * kThreads * 4 <= kSlot * 16 * KW, "reduction buffer");
    float *red = reinterpret_cast<float *>(xs[0]) + threadIdx.x % kThreads;
    __syncthreads();   // every wave is done with the ring
    if (kh == 1) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[((nb * MT + mt) * 4 + r) * kThreads] = acc[nb][mt][r];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[nb][mt][r] += red[((nb * MT + mt) * 4 + r) * kThreads];
    }
  }
  const bool lead = kh == 0;   // the wave set that holds the sums

  if constexpr (GROUPED) {
    if (!lead) return;
    // fp32 results by output row of each list entry (no split-K here)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = mt * 16 + kq * 4 + r;
        if (tok < tt.cnt) {
          const int i = tt.i0 + tok;
          float *orow = a.out + static_cast<size_t>(a.out_perm ? a.perm[i] : i) * a.N;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int row = row0 + nb * 16;
            if (row < a.N) orow[row] = acc[nb][mt][r];
          }
        }
      }
    }
    return;
  }
  if (a.S > 1) {
    // publish this slice's partial tile; the last slice to arrive sums them all
    constexpr int kTileFloats = NB * MT * 4 * kThreads;
    float *mine = a.part + (static_cast<size_t>(tile_id) * a.S + split) * kTileFloats + threadIdx.x;
    if (lead) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) store_coherent(mine + ((nb * MT + mt) * 4 + r) * kThreads, acc[nb][mt][r]);
    }
    wait_vm_lds<0>();   // the stores above have completed
    __syncthreads();
    __shared__ uint32_t last;
    if (threadIdx.x == 0)
      last = (__hip_atomic_fetch_add(a.counters + tile_id, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              static_cast<uint32_t>(a.S - 1))
                 ? 1u
                 : 0u;
    __syncthreads();
    if (!last || !lead) return;
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

  if (!lead) return;
  // D layout: lane holds tokens 4 kq + r (r = 0..3) of token tile mt, row j of block nb
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int row = row0 + nb * 16;
    if (row < a.N) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = m0 + mt * 16 + kq * 4 + r;
          if (tok < a.M) a.y[static_cast<size_t>(tok) * a.N + row] = f32_to_f16_bits(acc[nb][mt][r]);
        }
      }
    }
  }
}

// The ring slots are separate LDS objects so the compiler can tell that a read
// of one slot does not depend on the copies in flight into the others.
#define LBQ_RING_SLOTS(MT, KW)                                                                          \
  __shared__ __attribute__((aligned(16))) uint4 xs0[(KW) * 16 * (MT) * 16];                             \
  __shared__ __attribute__((aligned(16))) uint4 xs1[(KW) * 16 * (MT) * 16];                             \
  __shared__ __attribute__((aligned(16))) uint4 xs2[kRing > 2 ? (KW) * 16 * (MT) * 16 : 1];            \
  __shared__ __attribute__((aligned(16))) uint4 xs3[kRing > 3 ? (KW) * 16 * (MT) * 16 : 1];            \
  __shared__ __attribute__((aligned(16))) uint4 xs4[kRing > 4 ? (KW) * 16 * (MT) * 16 : 1];            \
  __shared__ __attribute__((aligned(16))) uint4 xs5[kRing > 5 ? (KW) * 16 * (MT) * 16 : 1];            \
  __shared__ __attribute__((aligned(16))) uint4 xs6[kRing > 6 ? (KW) * 16 * (MT) * 16 : 1];            \
  __shared__ __attribute__((aligned(16))) uint4 xs7[kRing > 7 ? (KW) * 16 * (MT) * 16 : 1];            \
  uint4 *const xs[8] = {xs0, xs1, xs2, xs3, xs4, xs5, xs6, xs7};                                        \
  extern __shared__ uint32_t msm[];

template <int BITS, int NB, int MT, int KW>
__global__ void __launch_bounds__(kThreads * KW) gemm_rtn_kernel(RtnGemmArgs a) {
  LBQ_RING_SLOTS(MT, KW)
  gemm_rtn_body<BITS, NB, MT, KW, false>(a, a.planes, a.meta, TokenTile{static_cast<int>(blockIdx.z) * 16 * MT, 0, 0},
                                         xs, msm);
}

// Grouped GEMM over routed experts: workgroup (., y, z) takes row tile y of
// the expert of tile descriptor z, at that expert's own code width.
template <int NB, int MT>
__global__ void __launch_bounds__(kThreads) gemm_rtn_grouped_kernel(RtnGemmArgs a) {
  if (static_cast<int>(blockIdx.z) >= *a.n_tiles) return;
  LBQ_RING_SLOTS(MT, 1)
  const int4 d = a.tiles[blockIdx.z];   // (e, i0, cnt, bits)
  const uint4 *pl = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint8_t *>(a.planes) + a.plane_off[d.x]);
  const uint32_t *mt = reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint8_t *>(a.meta) + a.meta_off[d.x]);
  const TokenTile tt{0, d.y, d.z};
  if (d.w == 2) gemm_rtn_body<2, NB, MT, 1, true>(a, pl, mt, tt, xs, msm);
  else if (d.w == 3) gemm_rtn_body<3, NB, MT, 1, true>(a, pl, mt, tt, xs, msm);
  else gemm_rtn_body<4, NB, MT, 1, true>(a, pl, mt, tt, xs, msm);
}
#undef LBQ_RING_SLOTS

template <int BITS, int NB, int MT, int KW>
hipError_t launch_rtn(dim3 grid, const RtnGemmArgs &a, hipStream_t s) {
  const size_t lds = static_cast<size_t>(kWaves * 16 * NB) * a.MS * 4;
  const size_t ring = static_cast<size_t>(kRing) * KW * 16 * MT * 16 * 16;   // the static activation slots
  auto kern = gemm_rtn_kernel<BITS, NB, MT, KW>;
  if (ring + lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, grid, dim3(kThreads * KW), lds, s, a);
  return hipGetLastError();
}

template <int BITS, int NB>
hipError_t launch_rtn_mt(const GemmPlan &p, dim3 grid, const RtnGemmArgs &a, hipStream_t s) {
  if (NB <= 2 && p.kw == 2) {
    constexpr int KW = NB <= 2 ? 2 : 1;
    if (p.mt == 1) return launch_rtn<BITS, NB, 1, KW>(grid, a, s);
    if (p.mt == 2) return launch_rtn<BITS, NB, 2, KW>(grid, a, s);
    return launch_rtn<BITS, NB, 4, KW>(grid, a, s);
  }
  if (p.mt == 1) return launch_rtn<BITS, NB, 1, 1>(grid, a, s);
  if (p.mt == 2) return launch_rtn<BITS, NB, 2, 1>(grid, a, s);
  return launch_rtn<BITS, NB, 4, 1>(grid, a, s);
}

template <int BITS>
hipError_t launch_rtn_bits(const GemmPlan &p, dim3 grid, const RtnGemmArgs &a, hipStream_t s) {
  if (BITS != 8 && p.nb == 4) return launch_rtn_mt<BITS, BITS == 8 ? 2 : 4>(p, grid, a, s);   // (8-bit: no four-block plans)
  if (p.nb == 2) return launch_rtn_mt<BITS, 2>(p, grid, a, s);
  return launch_rtn_mt<BITS, 1>(p, grid, a, s);
}

}  // namespace

int gemm_rtn_meta_max_groups(int nb) {
  return meta_max_groups(nb);
}

hipError_t launch_gemm_rtn_grouped(const GroupedGemm &g, hipStream_t s) {
  if (g.max_tiles <= 0) return hipSuccess;
  if ((g.nb != 1 && g.nb != 2) || (g.mt != 1 && g.mt != 2 && g.mt != 4)) return hipErrorInvalidValue;
  const int G = g.K / kGroup;
  if (g.K % kGroup != 0 || G > meta_max_groups(g.nb) || g.max_tiles > 65535) return hipErrorInvalidValue;
  RtnGemmArgs a{};
  a.xf = reinterpret_cast<const uint4 *>(g.xf);
  a.tz = reinterpret_cast<const uint4 *>(g.tz);
  a.planes = static_cast<const uint4 *>(g.planes);
  a.meta = static_cast<const uint32_t *>(g.meta);
  a.K = g.K;
  a.N = g.N;
  a.S = 1;
  a.Gp = gemm_tz_stride(g.K);
  a.MS = 4 * meta_vectors(G) + 1;
  a.tiles = reinterpret_cast<const int4 *>(g.tiles);
  a.n_tiles = g.n_tiles;
  a.plane_off = g.plane_off;
  a.meta_off = g.meta_off;
  a.perm = g.perm;
  a.act_div = g.act_div;
  a.out_perm = g.out_perm;
  a.out = g.out;
  const dim3 grid(1, static_cast<unsigned>((g.N + 64 * g.nb - 1) / (64 * g.nb)), static_cast<unsigned>(g.max_tiles));
  const size_t lds = static_cast<size_t>(kWaves * 16 * g.nb) * a.MS * 4;
  auto kern = g.nb == 1 ? (g.mt == 1 ? gemm_rtn_grouped_kernel<1, 1> : g.mt == 2 ? gemm_rtn_grouped_kernel<1, 2>
                                                                                  : gemm_rtn_grouped_kernel<1, 4>)
                        : (g.mt == 1 ? gemm_rtn_grouped_kernel<2, 1> : g.mt == 2 ? gemm_rtn_grouped_kernel<2, 2>
                                                                                  : gemm_rtn_grouped_kernel<2, 4>);
  const size_t ring = static_cast<size_t>(kRing) * 16 * g.mt * 16 * 16;
  if (ring + lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

int gemm_tz_stride(int K) {
  return (K / kGroup + 15) / 16 * 16;
}

bool gemm_rtn_supported(int K, int N, int bits) {
  // 32-bit buffer offsets over the planes and meta words
  return static_cast<long long>(N) * (K / kGroup) * bits * 16 < static_cast<long long>(kOutOfRange) - 4096;
}

hipError_t launch_gemm_rtn(const GemmPlan &p, int bits, const void *planes, const void *meta, const uint16_t *xf,
                           const uint32_t *tz, uint16_t *y, int M, int K, int N, void *scratch, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if ((p.nb != 1 && p.nb != 2 && p.nb != 4) || (p.mt != 1 && p.mt != 2 && p.mt != 4) || p.S < 1 ||
      (p.kw != 1 && p.kw != 2) || (p.kw == 2 && p.nb == 4))
    return hipErrorInvalidValue;
  if ((bits < 2 || bits > 4) && bits != 8) return hipErrorInvalidValue;
  if (!gemm_rtn_supported(K, N, bits) || (bits == 8 && p.nb > 2)) return hipErrorInvalidValue;
  const int G = K / kGroup, ns = (G + p.S - 1) / p.S;   // longest slice
  if (p.S > G || ns > meta_max_groups(p.nb)) return hipErrorInvalidValue;
  RtnGemmArgs a;
  a.xf = reinterpret_cast<const uint4 *>(xf);
  a.tz = reinterpret_cast<const uint4 *>(tz);
  a.planes = static_cast<const uint4 *>(planes);
  a.meta = static_cast<const uint32_t *>(meta);
  a.y = y;
  a.part = static_cast<float *>(scratch);
  a.counters = gemm_counter_ptr(p, scratch);
  a.M = M;
  a.K = K;
  a.N = N;
  a.S = p.S;
  a.Gp = gemm_tz_stride(K);
  a.MS = 4 * meta_vectors(ns) + 1;
  const dim3 grid(static_cast<unsigned>(p.S), static_cast<unsigned>(p.n_tiles), static_cast<unsigned>(p.m_tiles));
  switch (bits) {
    case 2: return launch_rtn_bits<2>(p, grid, a, s);
    case 3: return launch_rtn_bits<3>(p, grid, a, s);
    case 4: return launch_rtn_bits<4>(p, grid, a, s);
    default: return launch_rtn_bits<8>(p, grid, a, s);
  }
}

}  // namespace lbq
