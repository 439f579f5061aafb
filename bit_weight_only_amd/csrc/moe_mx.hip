// Routed-expert linears on the matrix cores (fp8 activation pieces x fp4
// codes, the operand encoding of mx_core.h), one launch per linear of the
// block: gate|up over the routed tokens, then down over the SwiGLU outputs
// (routed experts at their own 2/3/4-bit widths in a Hadamard-rotated basis:
// LLaDA2.2-mini Orin Nano card, "Routed Experts"; top-k routing: Laguna-S-2.1
// gridbook card, base-model line).
//
// Workgroup b of expert e owns row tiles b, b + grid, ... of that expert's
// weight (grid workgroups per expert; experts with no tokens exit at once).
// It walks the expert's assignment list in chunks of up to four: each chunk's
// activation rows are gathered (row perm[i] / row_div), rotated with the
// layer's signs in the prologue and split into A pieces. For down, the
// prologue forms the SwiGLU intermediate itself from the gate|up results
// (fp32 gate and up, silu(g) u rounded to fp16). Wave w then streams whole
// tiles w, w + 8, ... of the workgroup (every batch of groups of a tile, in
// order) and writes each finished tile's fp32 results per assignment,
// out[perm[i]][row], so no partial sums cross waves and repeat calls are
// bit-identical. Later chunks of a crowded expert read the same weights again
// (from the caches).
#include "kernels.h"
#include "mx_core.h"

#include <algorithm>
#include <type_traits>

namespace lbq {

namespace {

using namespace mx;

constexpr int kMoeMxThreads = 512;   // eight wavefronts
constexpr int kChunk = 4;            // tokens per pass: A rows 4t .. 4t + 2

struct MoeMxArgs {
  const uint8_t *planes, *meta;           // all experts' buffers
  const uint64_t *plane_off, *meta_off;   // [E] byte offsets of this linear
  const uint8_t *bits;                    // [E]
  const uint16_t *x;                      // activation rows fp16 [x_rows][K] (not rotated), or
  const float *h;                         //   gate|up results fp32 [x_rows][2 K]: SwiGLU in the prologue
  const int8_t *signs;                    // [K] +-1, 16-byte aligned
  const int32_t *offsets;                 // [E + 1]
  const int32_t *perm;                    // assignment indices grouped by expert
  float *out;                             // fp32 [assignments][N], by assignment index
  int x_rows, row_div;                    // x row of list entry i: perm[i] / row_div
  MxShape sh[3];                          // one expert's linear at 2, 3, 4 bits (kChunk tokens)
};

// Activations of one rotation unit (token row, group g, lane L: 16 values)
// from the SwiGLU of gate|up results: silu(h[row][16 i + c]) h[row][K + ...]
// rounded to fp16, as rot_load would have read them; signs as rot_load.
__device__ __forceinline__ RotIn swiglu_load(__amdgpu_buffer_rsrc_t hrs, __amdgpu_buffer_rsrc_t srs, int K, int row,
                                             int g, int L, bool ok) {
  const uint32_t bad = ok ? 0u : kOutOfRange;
  const uint32_t go = static_cast<uint32_t>((row * 2 * K + g * kGroup + 16 * L) * 4) + bad;
  const uint32_t uo = go + static_cast<uint32_t>(K * 4);
  const uint32_t so = static_cast<uint32_t>(g * kGroup + 16 * L) + bad;
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
  RotIn r;
  r.xa = make_uint4(w[0], w[1], w[2], w[3]);
  r.xb = make_uint4(w[4], w[5], w[6], w[7]);
  r.sv = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(srs, so, 0, 0));
  return r;
}

template <int BITS, int DEPTH, bool SWIGLU>
__device__ void expert_linear(const MoeMxArgs &a, int e, int b, uint32_t *smem) {
  constexpr int GB = MxBatch<BITS>::GB, NV = MxBatch<BITS>::NV;
  const MxShape &sh = a.sh[BITS - 2];
  const int K = sh.K, N = sh.N, G = sh.G, Gp = sh.Gp, NB = sh.NB;
  const int VR = G * BITS;                       // 16-byte plane vectors per row
  const int ntl = sh.tq + (b < sh.tr ? 1 : 0);   // this workgroup's tiles: b + k grid, k < ntl
  constexpr int nw = kMoeMxThreads / 64;
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));   // wave-uniform
  const int lane = static_cast<int>(threadIdx.x & 63), j = lane & 15, kq = lane >> 4;
  const int first = a.offsets[e], n_e = a.offsets[e + 1] - first;
  // this wave's tiles: k = wv, wv + nw, ... < ntl, each NB items (batches) in order
  const int tiles_w = ntl > wv ? (ntl - wv + nw - 1) / nw : 0;
  const int items = tiles_w * NB;

  // LDS (laid out for kChunk tokens): piece sets [kChunk][Gp], (2/sc, T) per
  // (token, group) [kChunk][Gp], the meta words of this workgroup's rows
  // [ntl * 16][meta_stride(G)].
  const int MS = meta_stride(G);
  uint32_t *xa = smem;
  float2 *ss = reinterpret_cast<float2 *>(xa + kChunk * Gp * (kSetBytes / 4));
  uint32_t *ml = reinterpret_cast<uint32_t *>(ss + kChunk * Gp);

  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(a.planes + a.plane_off[e]), 0, N * VR * 16, kBufferFlags);
  const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(a.meta + a.meta_off[e]), 0, N * G * 4, kBufferFlags);
  const __amdgpu_buffer_rsrc_t xrs =
      SWIGLU ? __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.h), 0, a.x_rows * K * 8, kBufferFlags)
             : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a.x), 0, a.x_rows * K * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(a.signs), 0, K, kBufferFlags);
  const uint32_t pbase = static_cast<uint32_t>(((b * 16 + j) * VR + kq) * 16);
  const int tstride = sh.grid * 16;              // rows between a workgroup's consecutive tiles
  auto unit_load = [&](int row, int g, int L, bool ok) {
    if constexpr (SWIGLU) return swiglu_load(xrs, srs, K, row, g, L, ok);
    else return rot_load(xrs, srs, K, row, g, L, ok);
  };

  // meta staging of this workgroup's rows, once for all chunks (G % 4 == 0):
  // tile k (rows 16 (b + k grid) .. +15) is 16 G contiguous words. The first
  // two vectors of each thread are loaded with the first chunk's activations
  // and stored after its rotation; any further ones right there.
  const int per_tile = 4 * G, n_meta = ntl * per_tile;
  auto meta_load = [&](int i) {
    const int k = i / per_tile, v = i - k * per_tile;
    const uint32_t off = static_cast<uint32_t>(((b + k * sh.grid) * per_tile + v) * 16) +
                         (i < n_meta ? 0u : kOutOfRange);
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(mrs, off, 0, 0));
  };
  auto meta_store = [&](int i, uint4 v4) {
    const int k = i / per_tile, v = i - k * per_tile;
    const int w = v * 4, r = w / G, c = w - r * G;   // row r of tile k, word c (a vector never spans rows)
    *reinterpret_cast<uint4 *>(ml + (k * 16 + r) * MS + c) = v4;
  };
  const int t0 = static_cast<int>(threadIdx.x);
  const uint4 mv0 = meta_load(t0), mv1 = meta_load(t0 + kMoeMxThreads);

  const int units_max = kChunk * G, ustep = kMoeMxThreads >> 3;
  const int u0 = rot_unit_of(static_cast<int>(threadIdx.x)), rL = rot_lane_of(static_cast<int>(threadIdx.x));

  auto chunk = [&](int c0, auto first_tag) {
    constexpr bool kFirst = decltype(first_tag)::value;
    const int M = min(kChunk, n_e - c0);
    const int units = M * G;
    // gathered activation rows and output assignments of the chunk (uniform)
    int xrow[kChunk], asg[kChunk];
#pragma unroll
    for (int m = 0; m < kChunk; ++m) {
      asg[m] = a.perm[first + c0 + min(m, M - 1)];
      xrow[m] = asg[m] / a.row_div;
    }
    auto row_of = [&](int m) { return m == 0 ? xrow[0] : m == 1 ? xrow[1] : m == 2 ? xrow[2] : xrow[3]; };
    const int out_asg = kq == 0 ? asg[0] : kq == 1 ? asg[1] : kq == 2 ? asg[2] : asg[3];

    // load cursor (lt = the wave's tile ordinal, lb = batch) and process cursor
    int li = 0, lt = 0, lb = 0;
    auto load = [&](MxItem<BITS> &it) {
      const uint32_t past = li < items ? 0u : kOutOfRange;
      const int k = wv + lt * nw;   // workgroup tile
      const uint32_t pstep = static_cast<uint32_t>((k * tstride * VR + lb * GB * BITS) * 16) + past;
#pragma unroll
      for (int q = 0; q < NV; ++q)
        it.v[q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(prs, pbase + pstep + 64 * q, 0, 0));
      ++li;
      const int wrap = lb + 1 >= NB ? 1 : 0;
      lb = wrap ? 0 : lb + 1;
      lt += wrap;
    };
    const int m0 = (u0 >= G) + (u0 >= 2 * G) + (u0 >= 3 * G);
    // Order of the loads (a compute unit's vector memory path returns data in
    // request order): every wave's activations go out first, all waves pass one
    // barrier that waits for no data, then the code loads. Waves with rotation
    // units issue two ring slots, rotate, and issue the rest; the others skip
    // the rotation and issue every slot at once. Both branches leave the same
    // loads outstanding in the same order.
    constexpr int kEarly = DEPTH < 2 ? DEPTH : 2;
    const bool rotating = wv * 8 < units;   // wave-uniform
    MxItem<BITS> ring[DEPTH];
    if (rotating) {
      const RotIn rin = unit_load(row_of(min(m0, M - 1)), u0 - m0 * G, rL, u0 < units);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int d = 0; d < kEarly; ++d) {
        load(ring[d]);
        __builtin_amdgcn_sched_barrier(0);   // keep the slots' loads in slot order, as in the loop
      }
      // the first pass runs on every lane of the wave; lanes without a unit
      // compute on zeros and store nothing
      rot_pieces(rin, Gp, min(m0, M - 1), u0 - m0 * G, rL, u0 < units, xa, ss);
      for (int u = u0 + ustep; u < units; u += ustep) {
        const int m = (u >= G) + (u >= 2 * G) + (u >= 3 * G), g = u - m * G;
        rot_pieces(unit_load(row_of(m), g, rL, true), Gp, m, g, rL, true, xa, ss);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int d = kEarly; d < DEPTH; ++d) {
        load(ring[d]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        load(ring[d]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (kFirst) {
      if (t0 < n_meta) meta_store(t0, mv0);
      if (t0 + kMoeMxThreads < n_meta) meta_store(t0 + kMoeMxThreads, mv1);
      for (int i = t0 + 2 * kMoeMxThreads; i < n_meta; i += kMoeMxThreads) meta_store(i, meta_load(i));
    }
    {   // zero the padding groups' pieces and sums, and every set's zero piece
      const int pad = (Gp - G) * kChunk;
      for (int i = static_cast<int>(threadIdx.x); i < pad * (kSetBytes / 4); i += kMoeMxThreads) {
        const int q = i / (kSetBytes / 4), m = q / (Gp - G), g = G + q - m * (Gp - G);
        xa[(m * Gp + g) * (kSetBytes / 4) + i - q * (kSetBytes / 4)] = 0u;
      }
      for (int i = static_cast<int>(threadIdx.x); i < pad; i += kMoeMxThreads) {
        const int m = i / (Gp - G);
        ss[m * Gp + G + i - m * (Gp - G)] = make_float2(0.f, 0.f);
      }
      for (int i = static_cast<int>(threadIdx.x); i < units_max * (kPieceBytes / 16); i += kMoeMxThreads) {
        const int q = i / (kPieceBytes / 16);
        reinterpret_cast<uint4 *>(xa + q * (kSetBytes / 4) + piece_offset(3) / 4)[i - q * (kPieceBytes / 16)] =
            make_uint4(0, 0, 0, 0);
      }
    }
    barrier_lds();   // the ring's code loads stay in flight

    // A operand source of this lane: row i = lane & 15 holds piece i & 3 of token
    // i >> 2; rows of tokens >= M read token 0's zero piece
    const int ai = lane & 15, at = ai >> 2, ap = ai & 3;
    const uint32_t a_base =
        static_cast<uint32_t>(at < M ? at * Gp * kSetBytes + piece_offset(ap) : piece_offset(3)) + kq * 32;
    constexpr uint32_t a_step = kSetBytes;
    const char *lds = reinterpret_cast<const char *>(smem);
    // (2/sc, T) of this lane's token (lanes of tokens >= M read token M - 1's and never store)
    const bool t_ok = kq < M;
    const uint32_t s_base = static_cast<uint32_t>(reinterpret_cast<const char *>(ss) - lds) +
                            static_cast<uint32_t>(min(kq, M - 1) * Gp * 8);

    int pt = 0, pb = 0;   // process cursor: tile ordinal, batch
    float yacc = 0.f;
    auto process = [&](const MxItem<BITS> &it) {
      const int g0 = pb * GB;
      const int k = wv + pt * nw;   // workgroup tile
      uint32_t w[NV][4];
#pragma unroll
      for (int q = 0; q < NV; ++q) {
        w[q][0] = it.v[q].x;
        w[q][1] = it.v[q].y;
        w[q][2] = it.v[q].z;
        w[q][3] = it.v[q].w;
        transpose4(w[q][0], w[q][1], w[q][2], w[q][3]);
      }
      const uint32_t a0off = a_base + static_cast<uint32_t>(g0) * a_step;
      const uint32_t *mrow = ml + (k * 16 + j) * MS + g0;   // meta words of this lane's row
      float2 st[GB];
#pragma unroll
      for (int u = 0; u < GB; u += 2) {
        if (u + 1 < GB) {
          const float4 s4 = *reinterpret_cast<const float4 *>(lds + s_base + (g0 + u) * 8);
          st[u] = make_float2(s4.x, s4.y);
          st[u + 1] = make_float2(s4.z, s4.w);
        } else {
          st[u] = *reinterpret_cast<const float2 *>(lds + s_base + (g0 + u) * 8);
        }
      }
      v4f_t acc[GB];
#pragma unroll
      for (int u = 0; u < GB; ++u) {
        uint32_t pl[BITS];
#pragma unroll
        for (int p = 0; p < BITS; ++p) pl[p] = w[(u * BITS + p) >> 2][(u * BITS + p) & 3];
        const uint4 *ap4 = reinterpret_cast<const uint4 *>(lds + a0off + u * a_step);
        const uint4 x0 = ap4[0], x1 = ap4[1];
        const v8i_t av = {static_cast<int>(x0.x), static_cast<int>(x0.y), static_cast<int>(x0.z),
                          static_cast<int>(x0.w), static_cast<int>(x1.x), static_cast<int>(x1.y),
                          static_cast<int>(x1.z), static_cast<int>(x1.w)};
        uint32_t lo[4];
        fp4_from_pair(pl[0], pl[1], lo);
        const v8i_t bl = {static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                          static_cast<int>(lo[3]), 0, 0, 0, 0};
        acc[u] = v4f_t{0.f, 0.f, 0.f, 0.f};
        acc[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bl, acc[u], 0, 4, 0, 127, 0, 127);
        if constexpr (BITS > 2) {
          uint32_t hi[4];
          if constexpr (BITS == 3) fp4_from_single(pl[2], hi);
          else fp4_from_pair(pl[2], pl[3], hi);
          const v8i_t bh = {static_cast<int>(hi[0]), static_cast<int>(hi[1]), static_cast<int>(hi[2]),
                            static_cast<int>(hi[3]), 0, 0, 0, 0};
          acc[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bh, acc[u], 0, 4, 0, 127, 0, 129);
        }
      }
#pragma unroll
      for (int u = 0; u < GB; ++u) {
        // groups past G: zero pieces and zero (2/sc, T), so the term vanishes
        const float d = acc[u][0] + acc[u][1] + acc[u][2];
        const uint32_t mt = mrow[min(u, G - 1 - g0)];
        const float sc = f16_bits_to_f32(mt & 0xFFFFu), z = f16_bits_to_f32(mt >> 16);
        yacc = fmaf(sc, fmaf(d, st[u].x, -z * st[u].y), yacc);
      }
      // the tile's last batch: its rows are complete
      if (pb + 1 >= NB) {
        const int row = (b + k * sh.grid) * 16 + j;
        if (t_ok && row < N) a.out[static_cast<size_t>(out_asg) * N + row] = yacc;
        yacc = 0.f;
        pb = 0;
        ++pt;
      } else {
        ++pb;
      }
    };
    // ring slot d holds items d, d + DEPTH, ... of the wave's sequence; every slot
    // is refilled on every pass (also past the wave's last item) so the loads stay
    // unconditional and the compiler keeps exact wait counts
    for (int i = 0; i < items; i += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        if (d == 0 || i + d < items) process(ring[d]);
        load(ring[d]);
      }
    }
    __syncthreads();   // the next chunk overwrites the pieces
  };
  chunk(0, std::true_type{});
  for (int c0 = kChunk; c0 < n_e; c0 += kChunk) chunk(c0, std::false_type{});
}

template <bool SWIGLU>
__global__ void __launch_bounds__(kMoeMxThreads) moe_mx_kernel(MoeMxArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  const int grid = a.sh[0].grid;   // workgroups per expert (the same at every width)
  const int e = static_cast<int>(blockIdx.x) / grid, b = static_cast<int>(blockIdx.x) - e * grid;
  if (a.offsets[e + 1] == a.offsets[e]) return;
  switch (a.bits[e]) {
    case 2: expert_linear<2, 2, SWIGLU>(a, e, b, smem); break;
    case 3: expert_linear<3, 2, SWIGLU>(a, e, b, smem); break;
    default: expert_linear<4, 3, SWIGLU>(a, e, b, smem); break;
  }
}

// Row tiles per workgroup: two per wave, four for rows of up to 1024 inputs
// (less streaming per tile, so more tiles carry each workgroup's prologue).
int moe_tiles_per_wg(int K) { return K <= 1024 ? 32 : 16; }

size_t moe_mx_lds(int K) {
  const int G = K / kGroup, Gp = padded_groups(G, 3);
  const int rows = moe_tiles_per_wg(K) * 16;
  return static_cast<size_t>(kChunk) * Gp * (kSetBytes + 8) + static_cast<size_t>(rows) * meta_stride(G) * 4;
}

hipError_t launch_linear(const MoeArgs &m, const uint64_t *poff, const uint64_t *moff, const uint16_t *x,
                         const float *h, int x_rows, const int8_t *signs, int row_div, int K, int N, float *out,
                         hipStream_t s) {
  MoeMxArgs a;
  a.planes = m.planes;
  a.meta = m.meta;
  a.plane_off = poff;
  a.meta_off = moff;
  a.bits = m.bits;
  a.x = x;
  a.h = h;
  a.signs = signs;
  a.offsets = m.offsets;
  a.perm = m.perm;
  a.out = out;
  a.x_rows = x_rows;
  a.row_div = row_div;
  const int grid = (N / 16) / moe_tiles_per_wg(K);
  for (int w = 0; w < 3; ++w) a.sh[w] = make_shape(kChunk, K, N, w + 2, grid, kMoeMxThreads);
  auto kern = h ? moe_mx_kernel<true> : moe_mx_kernel<false>;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(m.E * grid)), dim3(kMoeMxThreads), moe_mx_lds(K), s, a);
  return hipGetLastError();
}

}  // namespace

bool moe_mx_supported(int hidden, int ffn, const int8_t *signs_hidden, const int8_t *signs_ffn) {
  // K a multiple of 512 (whole meta vectors per row), rows in whole workgroup
  // tiles, LDS within 64 KB, 16-byte aligned signs (vector loads)
  auto aligned = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  return hidden % 512 == 0 && ffn % 512 == 0 && (2 * ffn) % (16 * moe_tiles_per_wg(hidden)) == 0 &&
         hidden % (16 * moe_tiles_per_wg(ffn)) == 0 && moe_mx_lds(hidden) <= 64 * 1024 && moe_mx_lds(ffn) <= 64 * 1024 &&
         aligned(signs_hidden) && aligned(signs_ffn);
}

hipError_t launch_moe_mx(const MoeArgs &m, hipStream_t s) {
  hipError_t e = launch_linear(m, m.gu_plane_off, m.gu_meta_off, m.x, nullptr, m.M, m.signs_hidden, m.top_k,
                               m.hidden, 2 * m.ffn, m.h, s);
  if (e != hipSuccess) return e;
  // down: the prologue forms silu(gate) * up from the gate|up results of each assignment
  return launch_linear(m, m.dn_plane_off, m.dn_meta_off, nullptr, m.h, m.M * m.top_k, m.signs_ffn, 1, m.ffn,
                       m.hidden, m.out, s);
}

}  // namespace lbq
