// Dequant-GEMV for one to four tokens on the matrix cores, activation rotation
// fused into the prologue (one launch per linear).
//
// Operands of v_mfma_scale_f32_16x16x128_f8f6f4 (A fp8 e4m3, B fp4 e2m1):
//  * B = codes. A 2-bit code q dropped into the two low bits of an fp4 nibble
//    is the exact value q / 2, so decoding a 32-code word column of two bit
//    planes is ten bit operations (two v_bfi to merge the planes, six shifts
//    and masks into four nibble words). 3- and 4-bit codes q = ql + 4 qh
//    take a second MFMA on the high part with the B scale 2^2.
//  * A = activations. Each rotated group x'_g (fp32) is scaled by a power of
//    two sc_g that puts its largest magnitude in [128, 256) and split into
//    three e4m3 pieces h + l + l2 (each piece the rounding of what the
//    previous ones left): about twelve significant bits, at least fp16's.
//    Token t's pieces sit on A rows 4t, 4t + 1, 4t + 2 (row 4t + 3 is zero),
//    so one MFMA serves up to four tokens and lane (j, t) of the result holds
//    the three piece products of token t and output row j in its first three
//    accumulator registers.
// The group's contribution to y_j is then s (2 d / sc_g - z T_g) with d the
// sum of the three products and T_g = sum_k x'_k (RTN dequantisation
// s (q - z): Qwen3-8B BPDQ model card, group-wise scale and zero).
//
// Layout of one wave's work: 16 output rows (the MFMA's 16 B columns) times a
// batch of groups whose packed planes are 64 contiguous bytes of each row
// (two groups at 2 bits, one at 4) or 192 (four groups at 3 bits); lane
// (j, kq) loads 16 bytes at offset 16 kq of row j and a 4x4 lane transpose
// hands it word column kq of every plane vector of the batch. Each workgroup
// owns a set of 16-row tiles, its waves split the (tile, batch) items evenly
// and leave per-tile partial sums in LDS; one pass at the end adds them in a
// fixed order (repeat calls are bit-identical) and writes y.
// Tiles are dealt round-robin (workgroup b takes b, b + grid,
// ...), so at any moment the whole grid streams one contiguous stretch of the
// packed matrix.
//
// Element order: B element b (nibble b & 7 of register b >> 3) of lane
// (j, kq) holds code 32 kq + 4 (b & 7) + sigma(b >> 3) of the group, sigma =
// (0, 2, 1, 3); fp8 A element b_a of lane (i, kq_a) meets the fp4 B element
// of lane group kq_b = (kq_a >> 1) + 2 (b_a >> 4), b_b = (b_a & 15) +
// 16 (kq_a & 1) (the operand layouts of the mixed-format instruction). The
// rotation writes each piece straight into that order.
#include "device.h"
#include "kernels.h"
#include "mx_core.h"

#include <hip/hip_ext.h>

namespace lbq {

namespace {

using namespace mx;

constexpr int kMxMaxThreads = 1024;

// Scale/zero pairs staged in LDS as fp32 (s, s z), one row of the workgroup's
// tiles per MS pairs. A lane reads the GB pairs of its row and batch at once;
// the sixteen rows of a tile land in distinct bank groups when the row stride
// is an odd number of the read's width (8 bytes at GB = 1, 16 bytes otherwise).
template <int GB>
__host__ __device__ constexpr int fp32_meta_stride(int G) {
  return GB == 1 ? (G | 1) : ((G + 1) / 2 | 1) * 2;
}
// the largest over the code widths (LDS sizing before the width is known)
inline int fp32_meta_stride_any(int G) {
  const int a = fp32_meta_stride<1>(G), b = fp32_meta_stride<2>(G);
  return a > b ? a : b;
}
__device__ __forceinline__ float4 meta_pair(uint32_t w0, uint32_t w1) {
  const float s0 = f16_bits_to_f32(w0 & 0xFFFFu), z0 = f16_bits_to_f32(w0 >> 16);
  const float s1 = f16_bits_to_f32(w1 & 0xFFFFu), z1 = f16_bits_to_f32(w1 >> 16);
  return make_float4(s0, s0 * z0, s1, s1 * z1);
}

// x: raw activations [M][K] fp16 (M <= 4); signs: [K] int8 (+-1), 16-byte aligned.
// PASSES: the tokens go in passes of mp (else all M in one, mp == M).
template <int BITS, int DEPTH, bool PASSES>
__global__ void __launch_bounds__(kMxMaxThreads) gemv_mfma_kernel(const uint4 *__restrict__ planes,
                                                                 const uint32_t *__restrict__ meta,
                                                                 const uint4 *__restrict__ x,
                                                                 const uint4 *__restrict__ signs,
                                                                 uint16_t *__restrict__ y, const MxShape sh,
                                                                 const int mp) {
  constexpr int GB = MxBatch<BITS>::GB, NV = MxBatch<BITS>::NV;
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  const int K = sh.K, N = sh.N, G = sh.G, Gp = sh.Gp;
  const int VR = G * BITS;                       // 16-byte plane vectors per row
  const int b = static_cast<int>(blockIdx.x);
  const int ntl = sh.tq + (b < sh.tr ? 1 : 0);   // this workgroup's tiles: b + k grid, k < ntl
  const int rows = ntl * 16;
  const int items = ntl * sh.NB;
  const int nw = static_cast<int>(blockDim.x >> 6);
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));   // wave-uniform
  const int lane = static_cast<int>(threadIdx.x & 63), j = lane & 15, kq = lane >> 4;

  // The tokens go in passes of up to mp (all of them when their pieces fit in
  // LDS; a later pass re-reads the codes, mostly from L2). LDS, sized for mp
  // tokens: piece sets [mp][Gp] (kSetBytes each; groups past G zero), (2/sc, T)
  // per (token, group) [mp][Gp] (past G zero), the waves' row partial sums
  // [nw][mp][rows], and, staged once by the first pass, the scale and scale x
  // zero of this workgroup's rows as fp32 pairs [rows][MS] (MS =
  // fp32_meta_stride(G, GB)).
  const int MS = fp32_meta_stride<GB>(G);
  uint32_t *xa = smem;
  float2 *ss = reinterpret_cast<float2 *>(xa + mp * Gp * (kSetBytes / 4));
  float *yl = reinterpret_cast<float *>(ss + mp * Gp);
  float2 *ml = reinterpret_cast<float2 *>(yl + nw * mp * rows);
  const int npass = PASSES ? (sh.M + mp - 1) / mp : 1;
  for (int pass = 0; pass < npass; ++pass) {
  const int t0 = PASSES ? pass * mp : 0;
  const int M = PASSES ? min(mp, sh.M - t0) : sh.M;
  const bool first = pass == 0;

  // All first-round loads go out before anything waits: the activations of the
  // first rotation pass, the code items (ring slots), the first pass of the
  // meta staging. Buffer loads return zeros past a buffer's end, so every one
  // of them is unconditional. Rows past N fall past the end by themselves
  // (row-major data); loads past the wave's last item add 2^31.
  const __amdgpu_buffer_rsrc_t prs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4 *>(planes), 0, N * VR * 16, kBufferFlags);
  const __amdgpu_buffer_rsrc_t mrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(meta), 0, N * G * 4, kBufferFlags);
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4 *>(x + t0 * (K / 8)), 0, M * K * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4 *>(signs), 0, K, kBufferFlags);
  const uint32_t pbase = static_cast<uint32_t>(((b * 16 + j) * VR + kq) * 16);
  const int tstride = sh.grid * 16;              // rows between a workgroup's consecutive tiles
  // item w of the wave: tile w / NB, batch w % NB (w < nw <= 16)
  MxCursor lc{wv, 0, wv};
  while (lc.batch >= sh.NB) {
    lc.batch -= sh.NB;
    ++lc.tile;
  }
  MxCursor pc = lc;
  auto load = [&](MxItem<BITS> &it) {
    const uint32_t past = lc.i < items ? 0u : kOutOfRange;
    const uint32_t pstep = static_cast<uint32_t>((lc.tile * tstride * VR + lc.batch * GB * BITS) * 16) + past;
#pragma unroll
    for (int a = 0; a < NV; ++a)
      it.v[a] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(prs, pbase + pstep + 64 * a, 0, 0));
    lc.advance(sh, nw);
  };
  const int units = M * G, ustep = static_cast<int>(blockDim.x >> 3);
  const int u0 = rot_unit_of(static_cast<int>(threadIdx.x)), rL = rot_lane_of(static_cast<int>(threadIdx.x));
  const int m0 = (u0 >= G) + (u0 >= 2 * G) + (u0 >= 3 * G);
  // meta staging in 16-byte vectors (G % 4 == 0): tile k (rows 16 (b + k grid)
  // .. +15) is 16 G contiguous words of the meta array
  const int per_tile = 4 * G, n_meta = first ? ntl * per_tile : 0;   // the first pass stages them
  auto meta_load = [&](int i) {
    const int k = i / per_tile, v = i - k * per_tile;
    const uint32_t off = static_cast<uint32_t>(((b + k * sh.grid) * per_tile + v) * 16) +
                         (i < n_meta ? 0u : kOutOfRange);
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(mrs, off, 0, 0));
  };
  auto meta_store = [&](int i, uint4 v4) {
    const int k = i / per_tile, v = i - k * per_tile;
    const int w = v * 4, r = w / G, c = w - r * G;   // row r of tile k, word c (a vector never spans rows)
    float2 *dst = ml + (k * 16 + r) * MS + c;   // 8-byte aligned (MS may be odd)
    const float4 p0 = meta_pair(v4.x, v4.y), p1 = meta_pair(v4.z, v4.w);
    dst[0] = make_float2(p0.x, p0.y);
    dst[1] = make_float2(p0.z, p0.w);
    dst[2] = make_float2(p1.x, p1.y);
    dst[3] = make_float2(p1.z, p1.w);
  };
  // Order of the first loads. Every wave's activations and first scale/zero
  // words go out before any wave's code loads: a compute unit's vector memory
  // path returns data in request order, so the prologue would otherwise wait
  // for the code loads' trip to HBM (the barrier waits for no data). Waves that
  // rotate then issue two ring slots, rotate, and issue the rest (issuing a load
  // stalls the wave while the unit's address queue is full, and the rotation is
  // the prologue's critical path); waves without rotation units issue every
  // slot at once. Both branches leave the same loads outstanding in the same
  // order, and each wave passes one barrier.
  constexpr int kEarly = DEPTH < 2 ? DEPTH : 2;
  const bool rotating = wv * 8 < units;   // wave-uniform: the wave's first unit exists
  MxItem<BITS> ring[DEPTH];
  // each thread's first two meta vectors go out with the activations; any
  // further ones (none at the usual shapes) are loaded and stored on the spot
  const bool two_meta = n_meta > static_cast<int>(blockDim.x);   // workgroup-uniform
  uint4 mv0, mv1 = make_uint4(0, 0, 0, 0);
  if (rotating) {
    const RotIn rin = rot_load(xrs, srs, K, m0, u0 - m0 * G, rL, u0 < units);
    mv0 = meta_load(static_cast<int>(threadIdx.x));
    if (two_meta) mv1 = meta_load(static_cast<int>(threadIdx.x + blockDim.x));
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
      rot_pieces(rot_load(xrs, srs, K, m, g, rL, true), Gp, m, g, rL, true, xa, ss);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = kEarly; d < DEPTH; ++d) {
      load(ring[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    mv0 = meta_load(static_cast<int>(threadIdx.x));
    if (two_meta) mv1 = meta_load(static_cast<int>(threadIdx.x + blockDim.x));
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      load(ring[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (static_cast<int>(threadIdx.x) < n_meta) meta_store(static_cast<int>(threadIdx.x), mv0);
  if (static_cast<int>(threadIdx.x + blockDim.x) < n_meta) meta_store(static_cast<int>(threadIdx.x + blockDim.x), mv1);
  for (int i = static_cast<int>(threadIdx.x + 2 * blockDim.x); i < n_meta; i += static_cast<int>(blockDim.x))
    meta_store(i, meta_load(i));
  {   // zero the padding groups' pieces and sums, every set's zero piece, the row sums
    const int pad = (Gp - G) * M;
    for (int i = static_cast<int>(threadIdx.x); i < pad * (kSetBytes / 4); i += static_cast<int>(blockDim.x)) {
      const int q = i / (kSetBytes / 4), m = q / (Gp - G), g = G + q - m * (Gp - G);
      xa[(m * Gp + g) * (kSetBytes / 4) + i - q * (kSetBytes / 4)] = 0u;
    }
    for (int i = static_cast<int>(threadIdx.x); i < pad; i += static_cast<int>(blockDim.x)) {
      const int m = i / (Gp - G);
      ss[m * Gp + G + i - m * (Gp - G)] = make_float2(0.f, 0.f);
    }
    for (int i = static_cast<int>(threadIdx.x); i < M * G * (kPieceBytes / 16); i += static_cast<int>(blockDim.x)) {
      const int q = i / (kPieceBytes / 16);
      reinterpret_cast<uint4 *>(xa + q * (kSetBytes / 4) + piece_offset(3) / 4)[i - q * (kPieceBytes / 16)] =
          make_uint4(0, 0, 0, 0);
    }
    for (int i = static_cast<int>(threadIdx.x); i < nw * M * rows; i += static_cast<int>(blockDim.x)) yl[i] = 0.f;
  }
  barrier_lds();   // the ring's code loads stay in flight

  // A operand source of this lane: row i = lane & 15 holds piece i & 3 of token
  // i >> 2; rows of tokens >= M read token 0's zero piece
  const int ai = lane & 15, at = ai >> 2, ap = ai & 3;
  const uint32_t a_base = static_cast<uint32_t>(at < M ? at * Gp * kSetBytes + piece_offset(ap) : piece_offset(3)) +
                          kq * 32;
  constexpr uint32_t a_step = kSetBytes;
  const char *lds = reinterpret_cast<const char *>(smem);
  // (2/sc, T) of this lane's token (lanes of tokens >= M read token M - 1's and never store)
  const bool t_ok = kq < M;
  const uint32_t s_base = static_cast<uint32_t>(reinterpret_cast<const char *>(ss) - lds) +
                          static_cast<uint32_t>(min(kq, M - 1) * Gp * 8);
  float *ylane = yl + (wv * M + kq) * rows + j;   // this wave's partial sums (one per tile it touches)
  const float2 *mlane = ml + j * MS;

  float yacc = 0.f;
  auto process = [&](const MxItem<BITS> &it) {
    const int g0 = pc.batch * GB;
    uint32_t w[NV][4];
#pragma unroll
    for (int a = 0; a < NV; ++a) {
      w[a][0] = it.v[a].x;
      w[a][1] = it.v[a].y;
      w[a][2] = it.v[a].z;
      w[a][3] = it.v[a].w;
      transpose4(w[a][0], w[a][1], w[a][2], w[a][3]);
    }
    const uint32_t a0off = a_base + static_cast<uint32_t>(g0) * a_step;
    const float2 *mrow = mlane + (pc.tile * 16 * MS + g0);   // this lane's row: (s, s z) of the batch's groups
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
      const uint4 a0 = ap4[0], a1 = ap4[1];
      const v8i_t av = {static_cast<int>(a0.x), static_cast<int>(a0.y), static_cast<int>(a0.z),
                        static_cast<int>(a0.w), static_cast<int>(a1.x), static_cast<int>(a1.y),
                        static_cast<int>(a1.z), static_cast<int>(a1.w)};
      uint32_t lo[4];
      fp4_from_pair(pl[0], pl[1], lo);
      const v8i_t bl = {static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                        static_cast<int>(lo[3]), 0, 0, 0, 0};
      acc[u] = v4f_t{0.f, 0.f, 0.f, 0.f};
      acc[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bl, acc[u], 0, 4, 0, 127, 0, 127);
      if constexpr (BITS == 8) {
        // q = q0 + 4 q1 + 16 q2 + 64 q3, 2-bit digits from plane pairs (2d, 2d + 1),
        // digit d on the matrix cores with the B scale 2^(2d)
#pragma unroll
        for (int d = 1; d < 4; ++d) {
          uint32_t dg[4];
          fp4_from_pair(pl[2 * d], pl[2 * d + 1], dg);
          const v8i_t bd = {static_cast<int>(dg[0]), static_cast<int>(dg[1]), static_cast<int>(dg[2]),
                            static_cast<int>(dg[3]), 0, 0, 0, 0};
          acc[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bd, acc[u], 0, 4, 0, 127, 0, 127 + 2 * d);
        }
      } else if constexpr (BITS > 2) {
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
      // groups past G: zero pieces and zero (2/sc, T), so the term vanishes (their
      // codes are the next row's)
      const float d = acc[u][0] + acc[u][1] + acc[u][2];
      const float2 sz = mrow[u];   // K a multiple of 512: no padding groups
      yacc = fmaf(sz.x, d * st[u].x, yacc);
      yacc = fmaf(-sz.y, st[u].y, yacc);
    }
    // row tile done (the next item starts another tile, or this was the wave's last): add into LDS
    const int tile = pc.tile;
    pc.advance(sh, nw);
    if (pc.i >= items || pc.tile != tile) {
      if (t_ok) ylane[tile * 16] = yacc;
      yacc = 0.f;
    }
  };
  // ring slot d holds items d, d + DEPTH, ... of the wave's sequence. Full
  // passes refill every slot unconditionally, in one fixed order, so the
  // compiler keeps exact wait counts; the last pass refills only slots with an
  // item left and the drain processes them, so no load goes past the end (each
  // costs address-unit time even when it returns zeros).
  const int nwi = items > wv ? (items - wv + nw - 1) / nw : 0;   // this wave's items
  int k = 0;
  for (; k + 2 * DEPTH <= nwi; k += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      process(ring[d]);
      load(ring[d]);
    }
  }
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    if (k + d < nwi) process(ring[d]);
    if (k + d + DEPTH < nwi) load(ring[d]);
  }
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (k + DEPTH + d < nwi) process(ring[d]);
  __syncthreads();
  // the waves' partials summed in wave order: the result does not depend on timing
  for (int idx = static_cast<int>(threadIdx.x); idx < M * rows; idx += static_cast<int>(blockDim.x)) {
    const int m = idx / rows, r = idx - m * rows, row = (b + (r >> 4) * sh.grid) * 16 + (r & 15);
    float acc = 0.f;
    for (int w = 0; w < nw; ++w) acc += yl[w * M * rows + idx];
    if (row < N) y[static_cast<size_t>(t0 + m) * N + row] = f32_to_f16_bits(acc);
  }
  if (PASSES) __syncthreads();   // the next pass overwrites the pieces and partial sums
  }
}

size_t mfma_lds_bytes(int M, int G, int Gp, int rows, int nw) {
  return static_cast<size_t>(M) * Gp * (kSetBytes + 8) + static_cast<size_t>(nw) * M * rows * 4 +
         static_cast<size_t>(rows) * fp32_meta_stride_any(G) * 8;
}

template <int BITS, int DEPTH>
hipError_t launch_depth(const void *planes, const void *meta, const uint16_t *x, const int8_t *signs, uint16_t *y,
                        const MxShape &sh, int grid, int block, int mp, hipStream_t s, hipEvent_t start,
                        hipEvent_t stop) {
  const int rows = (sh.tq + (sh.tr ? 1 : 0)) * 16;
  const size_t lds = mfma_lds_bytes(mp, sh.G, sh.Gp, rows, block / 64);
  auto kern = mp < sh.M ? gemv_mfma_kernel<BITS, DEPTH, true> : gemv_mfma_kernel<BITS, DEPTH, false>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  const uint4 *pl = reinterpret_cast<const uint4 *>(planes);
  const uint32_t *mt = reinterpret_cast<const uint32_t *>(meta);
  const uint4 *xv = reinterpret_cast<const uint4 *>(x);
  const uint4 *sv = reinterpret_cast<const uint4 *>(signs);
  if (start || stop)   // the events take this kernel's own begin / end times
    hipExtLaunchKernelGGL(kern, dim3(grid), dim3(block), static_cast<uint32_t>(lds), s, start, stop, 0, pl, mt, xv,
                          sv, y, sh, mp);
  else
    hipLaunchKernelGGL(kern, dim3(grid), dim3(block), lds, s, pl, mt, xv, sv, y, sh, mp);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const void *planes, const void *meta, const uint16_t *x, const int8_t *signs, uint16_t *y,
                       const MxShape &sh, int grid, int block, int depth, int mp, hipStream_t s, hipEvent_t start,
                       hipEvent_t stop) {
  switch (depth) {
    case 1: return launch_depth<BITS, 1>(planes, meta, x, signs, y, sh, grid, block, mp, s, start, stop);
    case 2: return launch_depth<BITS, 2>(planes, meta, x, signs, y, sh, grid, block, mp, s, start, stop);
    case 3: return launch_depth<BITS, 3>(planes, meta, x, signs, y, sh, grid, block, mp, s, start, stop);
    default: return launch_depth<BITS, 4>(planes, meta, x, signs, y, sh, grid, block, mp, s, start, stop);
  }
}

constexpr int kComputeUnits = 256;
constexpr size_t kMaxLds = 160 * 1024;

}  // namespace

namespace {

// Tokens per pass: all of them when their pieces fit in LDS next to the
// workgroup's rows, else two (a second pass re-reads the codes, mostly from L2);
// 0 when not even that fits.
int tokens_per_pass(int M, int G, int Gp, int rows, int nw) {
  if (mfma_lds_bytes(M, G, Gp, rows, nw) <= kMaxLds) return M;
  return (M > 2 && mfma_lds_bytes(2, G, Gp, rows, nw) <= kMaxLds) ? 2 : 0;
}

}  // namespace

void gemv_mfma_shape(int M, int K, int N, int bits, int &grid, int &block, int &depth) {
  const int G = K / kGroup, T = (N + 15) / 16;
  // One workgroup per compute unit. Eight waves rotate up to 64 (token, group)
  // units in one pass and suit up to one tile per workgroup; larger rotations
  // or more tiles take sixteen (measured on the dense-stack shapes).
  block = (M * G <= 64 && T <= kComputeUnits) ? 512 : kMxMaxThreads;
  grid = T < kComputeUnits ? T : kComputeUnits;
  // 4-bit codes of tall matrices with small rotations: two workgroups of eight
  // waves per compute unit stream the doubled bytes better (4096 -> 28672 at
  // one token: 14.0 -> 12.7 us; 2- and 3-bit shapes measured best as above)
  if (bits == 4 && M * G <= 64 && T >= 4 * kComputeUnits) {
    block = 512;
    grid = 2 * kComputeUnits;
  }
  // very tall matrices: more workgroups until a workgroup's rows fit in LDS
  while (grid < T && tokens_per_pass(M, G, padded_groups(G, 3), ((T + grid - 1) / grid) * 16, block / 64) == 0)
    grid = grid * 2 < T ? grid * 2 : T;
  // ring depth: a third slot pays once each wave streams several tiles or long rows
  depth = bits == 3 ? 2 : (bits >= 4 || T >= 4 * kComputeUnits || G >= 64) ? 3 : 2;
}

bool gemv_mfma_one_pass(int M, int K, int N, int bits) {
  int grid, block, depth;
  gemv_mfma_shape(M, K, N, bits, grid, block, depth);
  const int G = K / kGroup, T = (N + 15) / 16;
  return tokens_per_pass(M, G, padded_groups(G, bits), ((T + grid - 1) / grid) * 16, block / 64) == M;
}

bool gemv_mfma_supported_8bit(int K, int N) {
  // buffer offsets are 32-bit and kOutOfRange must lie past the planes of 8-bit codes
  return static_cast<long long>(N + 16) * (K / kGroup) * 8 * 16 < static_cast<long long>(kOutOfRange);
}

bool gemv_mfma_supported(int M, int K, int N) {
  // K a multiple of 512: whole 16-byte vectors of meta words per row
  if (M < 1 || M > 4 || K < 4 * kGroup || K % (4 * kGroup) != 0 || N < 1) return false;
  // buffer offsets are 32-bit and kOutOfRange must lie past the planes of 4-bit codes
  if (static_cast<long long>(N + 16) * (K / kGroup) * 4 * 16 >= static_cast<long long>(kOutOfRange)) return false;
  int grid, block, depth;
  gemv_mfma_shape(M, K, N, 2, grid, block, depth);
  const int T = (N + 15) / 16;
  return tokens_per_pass(M, K / kGroup, padded_groups(K / kGroup, 3), ((T + grid - 1) / grid) * 16, block / 64) > 0;
}

hipError_t launch_gemv_mfma(const void *planes, const void *meta, const uint16_t *x, const int8_t *signs,
                            uint16_t *y, int M, int K, int N, int bits, int grid, int block, int depth,
                            hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  if (M < 1 || M > 4 || (reinterpret_cast<uintptr_t>(signs) & 15u) != 0 || (reinterpret_cast<uintptr_t>(x) & 15u) != 0)
    return hipErrorInvalidValue;
  if ((bits < 2 || bits > 4) && bits != 8) return hipErrorInvalidValue;
  if (!gemv_mfma_supported(M, K, N) || (bits == 8 && !gemv_mfma_supported_8bit(K, N))) return hipErrorInvalidValue;
  int g0, b0, d0;
  gemv_mfma_shape(M, K, N, bits, g0, b0, d0);
  if (grid <= 0) grid = g0;
  if (block <= 0) block = b0;
  if (depth <= 0) depth = d0;
  if (block % 64 != 0 || block < 64 || block > kMxMaxThreads || grid < 1) return hipErrorInvalidValue;
  const MxShape sh = make_shape(M, K, N, bits, grid, block);
  const int mp = tokens_per_pass(M, sh.G, sh.Gp, (sh.tq + (sh.tr ? 1 : 0)) * 16, block / 64);
  if (mp == 0) return hipErrorInvalidValue;
  switch (bits) {
    case 2: return launch_bits<2>(planes, meta, x, signs, y, sh, grid, block, depth, mp, s, start, stop);
    case 3: return launch_bits<3>(planes, meta, x, signs, y, sh, grid, block, depth, mp, s, start, stop);
    case 4: return launch_bits<4>(planes, meta, x, signs, y, sh, grid, block, depth, mp, s, start, stop);
    default: return launch_bits<8>(planes, meta, x, signs, y, sh, grid, block, depth, mp, s, start, stop);
  }
}

}  // namespace lbq
