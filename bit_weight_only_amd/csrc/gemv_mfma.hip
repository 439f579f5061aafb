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

#include <hip/hip_ext.h>

namespace lbq {

namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

constexpr int kMxMaxThreads = 1024;
constexpr int kPieceBytes = 128;               // one e4m3 piece of one (token, group)
// LDS set of one (token, group): pieces 0..2 and a zero piece 3 at byte offsets
// 0, 128, 272, 400. Lane (i, kq) of a ds_read reads 16 bytes at piece i & 3,
// offset 32 kq: these sixteen addresses fall in sixteen distinct 16-byte bank
// groups (offsets mod 256), so the A reads are conflict-free.
constexpr int kSetBytes = 528;
__host__ __device__ constexpr int piece_offset(int p) { return p == 0 ? 0 : p == 1 ? 128 : p == 2 ? 272 : 400; }
// Meta rows in LDS: a stride of 4 x (odd number) words puts the sixteen rows
// of a tile in distinct banks.
__host__ __device__ constexpr int meta_stride(int G) { return 4 * (((G + 3) / 4) | 1); }
constexpr float kInvSqrt128 = 0.08838834764831845f;
constexpr int kBufferFlags = 0x00020000;        // buffer descriptor word 3 (32-bit data, no swizzle)
constexpr uint32_t kOutOfRange = 0x80000000u;   // buffer offset past every supported size

template <int BITS>
struct MxBatch;
template <>
struct MxBatch<2> {
  static constexpr int GB = 2, NV = 1;   // groups per batch, 16-byte vectors per lane
};
template <>
struct MxBatch<3> {
  static constexpr int GB = 4, NV = 3;
};
template <>
struct MxBatch<4> {
  static constexpr int GB = 1, NV = 1;
};

template <int BITS>
struct MxItem {
  uint4 v[MxBatch<BITS>::NV];
};

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

// Two bit planes of one 32-code word column -> four fp4 words. Nibble t of
// word r holds code 4t + sigma(r) in its two low bits (value code / 2).
__device__ __forceinline__ void fp4_from_pair(uint32_t p0, uint32_t p1, uint32_t o[4]) {
  uint32_t e, od;
  merge2(p0, p1, e, od);   // e: 2-bit field f = code 2f; od: code 2f + 1
  o[0] = e & 0x33333333u;
  o[1] = (e >> 2) & 0x33333333u;
  o[2] = od & 0x33333333u;
  o[3] = (od >> 2) & 0x33333333u;
}
// One bit plane -> four fp4 words in the same order (value bit / 2).
__device__ __forceinline__ void fp4_from_single(uint32_t p, uint32_t o[4]) {
  o[0] = p & 0x11111111u;
  o[1] = (p >> 2) & 0x11111111u;
  o[2] = (p >> 1) & 0x11111111u;
  o[3] = (p >> 3) & 0x11111111u;
}

__host__ __device__ constexpr int sigma(int r) { return r == 1 ? 2 : (r == 2 ? 1 : r); }

__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  uint32_t w = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false));
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, static_cast<int>(w), true));
}

// Rotation of one (token m, group g) unit by eight lanes: logical lane L
// (0..7) holds positions 16 L .. 16 L + 15. The eight lanes of a unit sit at
// wave lanes {0..3, 8..11} (+4 for the second unit of a 16-lane row), so the
// cross-lane partners L ^ 1, L ^ 2, L ^ 4 are wave lanes ^ 1, ^ 2, ^ 8: single
// DPP moves (quad permutes, row rotate by 8).
__device__ __forceinline__ int rot_unit_of(int tid) {
  const int l = tid & 63;
  return (tid >> 6) * 8 + (l >> 4) * 2 + ((l >> 2) & 1);
}
__device__ __forceinline__ int rot_lane_of(int tid) {
  const int l = tid & 63;
  return (l & 3) | (((l >> 3) & 1) << 2);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;    // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;    // quad_perm [2, 3, 0, 1]
constexpr int kDppXor8 = 0x128;   // row_ror 8: lane ^ 8 inside a 16-lane row

// Buffer loads (an offset past the end returns zeros): lanes without a unit
// pass ok = false and load nothing.
struct RotIn {
  uint4 xa, xb, sv;
};
__device__ __forceinline__ RotIn rot_load(__amdgpu_buffer_rsrc_t xrs, __amdgpu_buffer_rsrc_t srs, int K, int m, int g,
                                          int L, bool ok) {
  const uint32_t bad = ok ? 0u : kOutOfRange;
  const uint32_t xo = static_cast<uint32_t>((m * K + g * kGroup + 16 * L) * 2) + bad;
  const uint32_t so = static_cast<uint32_t>(g * kGroup + 16 * L) + bad;
  RotIn r;
  r.xa = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xo, 0, 0));
  r.xb = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xo + 16, 0, 0));
  r.sv = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(srs, so, 0, 0));
  return r;
}

// Rotate one unit and split it into the A pieces, (H_128 D x)_g with the
// 1/sqrt(128) normalisation folded into the piece scale.
//  * Cross-lane stages first, on the signed inputs, each one v_fmac with a DPP
//    operand: v += sg * partner with sg = -1 on the lane whose bit is set.
//    That lane gets v - partner, the negated butterfly output; the pair
//    partners always carry the same accumulated sign, so after the three
//    stages lane L holds (-1)^popcount(L) times the exact value, and the
//    factor goes into the lane's piece scale.
//  * Four in-lane stages.
//  * Positions 16 L + s + 4 e (e = 0..3) form one 4-byte word of the A layout
//    (see the file comment): four words per piece per lane.
// Sylvester's H_128 has column sums 128, 0, 0, ..., so the group sum is
// T_g = sqrt(128) s_0 x_0 (exact, no reduction). ss[t * Gp + g] = (2 / sc_g,
// T_g). store = false computes without writing.
__device__ __forceinline__ void rot_pieces(const RotIn &in, int Gp, int m, int g, int L, bool store, uint32_t *xa,
                                           float2 *ss) {
  const uint32_t xw[8] = {in.xa.x, in.xa.y, in.xa.z, in.xa.w, in.xb.x, in.xb.y, in.xb.z, in.xb.w};
  const uint32_t sw[4] = {in.sv.x, in.sv.y, in.sv.z, in.sv.w};
  float v[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t sb = sw[i >> 1] >> (16 * (i & 1));   // sign bytes of elements 2i, 2i + 1
    const uint32_t h = xw[i] ^ (((sb & 0x80u) << 8) | ((sb & 0x8000u) << 16));
    v[2 * i] = half_lo(h);
    v[2 * i + 1] = half_hi(h);
  }
  const float first = v[0];   // s_0 x_0 on lane 0
  {
    const float sg = (L & 1) ? -1.f : 1.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = fmaf(dpp_f<kDppXor1>(v[i]), sg, v[i]);
  }
  {
    const float sg = (L & 2) ? -1.f : 1.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = fmaf(dpp_f<kDppXor2>(v[i]), sg, v[i]);
  }
  {
    const float sg = (L & 4) ? -1.f : 1.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = fmaf(dpp_f<kDppXor8>(v[i]), sg, v[i]);
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
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(v[i]));
  mx = fmaxf(mx, dpp_f<kDppXor1>(mx));
  mx = fmaxf(mx, dpp_f<kDppXor2>(mx));
  mx = fmaxf(mx, dpp_f<kDppXor8>(mx));
  // sc = 2^(8 - E) with max |x'| = f 2^E, f in [0.5, 1): scaled maximum in [128, 256)
  const int E = __builtin_amdgcn_frexp_expf(mx * kInvSqrt128);
  const float flip = (__builtin_popcount(L) & 1) ? -1.f : 1.f;
  const float c = __builtin_amdgcn_ldexpf(flip * kInvSqrt128, 8 - E);
  uint32_t *blk = xa + static_cast<size_t>(m * Gp + g) * (kSetBytes / 4);
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    float a[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = v[s4 + 4 * e] * c;
    // word (kq_a, w) of the A layout that holds positions 16 L + s4 + 4 e
    const int r = sigma(s4), kqb = L >> 1;
    const int off = (2 * (kqb & 1) + (r >> 1)) * 8 + 4 * (kqb >> 1) + 2 * (r & 1) + (L & 1);
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const uint32_t word = e4m3x4(a[0], a[1], a[2], a[3]);
      if (store) blk[piece_offset(p) / 4 + off] = word;
      if (p < 2) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(word), false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(word), true);
        a[0] -= lo[0];
        a[1] -= lo[1];
        a[2] -= hi[0];
        a[3] -= hi[1];
      }
    }
  }
  if (store && L == 0) ss[m * Gp + g] = make_float2(__builtin_amdgcn_ldexpf(1.f, E - 7), first * 11.313708498984761f);
}

// Launch constants the host derives once (no integer division in the kernel).
struct MxShape {
  int M, K, N;
  int G, Gp;        // groups per row; padded to whole batches (Gp = NB * GB)
  int NB, T;        // batches per row tile, 16-row tiles
  int tq, tr;       // tiles per workgroup: tq, plus one for the first tr workgroups
  int grid;         // workgroup b owns tiles b, b + grid, b + 2 grid, ...
  int dt, db;       // one step of nw items = dt tiles + db batches (nw = waves per workgroup)
};

// Position of one wave in its item sequence: items w, w + nw, w + 2 nw, ... of
// the workgroup's (tile, batch) list, tile-major.
struct MxCursor {
  int i, tile, batch;
  __device__ __forceinline__ void advance(const MxShape &sh, int nw) {   // scalar, branch-free
    i += nw;
    int b = batch + sh.db;
    const int wrap = b >= sh.NB ? 1 : 0;
    batch = b - (wrap ? sh.NB : 0);
    tile += sh.dt + wrap;
  }
};

// x: raw activations [M][K] fp16 (M <= 4); signs: [K] int8 (+-1), 16-byte aligned.
template <int BITS, int DEPTH>
__global__ void __launch_bounds__(kMxMaxThreads) gemv_mfma_kernel(const uint4 *__restrict__ planes,
                                                                 const uint32_t *__restrict__ meta,
                                                                 const uint4 *__restrict__ x,
                                                                 const uint4 *__restrict__ signs,
                                                                 uint16_t *__restrict__ y, const MxShape sh) {
  constexpr int GB = MxBatch<BITS>::GB, NV = MxBatch<BITS>::NV;
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  const int M = sh.M, K = sh.K, N = sh.N, G = sh.G, Gp = sh.Gp;
  const int VR = G * BITS;                       // 16-byte plane vectors per row
  const int b = static_cast<int>(blockIdx.x);
  const int ntl = sh.tq + (b < sh.tr ? 1 : 0);   // this workgroup's tiles: b + k grid, k < ntl
  const int rows = ntl * 16;
  const int items = ntl * sh.NB;
  const int nw = static_cast<int>(blockDim.x >> 6);
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));   // wave-uniform
  const int lane = static_cast<int>(threadIdx.x & 63), j = lane & 15, kq = lane >> 4;

  // LDS: piece sets [M][Gp] (kSetBytes each; groups past G zero), (2/sc, T) per
  // (token, group) [M][Gp] (past G zero), the waves' row partial sums
  // [nw][M][rows], the meta words of this workgroup's rows [rows][meta_stride(G)].
  const int MS = meta_stride(G);
  uint32_t *xa = smem;
  float2 *ss = reinterpret_cast<float2 *>(xa + M * Gp * (kSetBytes / 4));
  float *yl = reinterpret_cast<float *>(ss + M * Gp);
  uint32_t *ml = reinterpret_cast<uint32_t *>(yl + nw * M * rows);

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
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4 *>(x), 0, M * K * 2, kBufferFlags);
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
  const RotIn rin = rot_load(xrs, srs, K, m0, u0 - m0 * G, rL, u0 < units);
  __builtin_amdgcn_sched_barrier(0);   // the activations go out first: the rotation waits on them only
  MxItem<BITS> ring[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    load(ring[d]);
    __builtin_amdgcn_sched_barrier(0);   // keep the slots' loads in slot order, as in the loop
  }

  // meta staging in 16-byte vectors (G % 4 == 0): tile k (rows 16 (b + k grid)
  // .. +15) is 16 G contiguous words of the meta array
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
  const uint4 mv0 = meta_load(static_cast<int>(threadIdx.x));

  // the first pass runs on every lane (its loads must not be sunk into a branch);
  // lanes without a unit compute on zeros and store nothing
  rot_pieces(rin, Gp, min(m0, M - 1), u0 - m0 * G, rL, u0 < units, xa, ss);
  for (int u = u0 + ustep; u < units; u += ustep) {
    const int m = (u >= G) + (u >= 2 * G) + (u >= 3 * G), g = u - m * G;
    rot_pieces(rot_load(xrs, srs, K, m, g, rL, true), Gp, m, g, rL, true, xa, ss);
  }
  if (static_cast<int>(threadIdx.x) < n_meta) meta_store(static_cast<int>(threadIdx.x), mv0);
  for (int i = static_cast<int>(threadIdx.x + blockDim.x); i < n_meta; i += static_cast<int>(blockDim.x))
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
  __syncthreads();

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
    const uint32_t *mrow = ml + (pc.tile * 16 + j) * MS + g0;   // meta words of this lane's row
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
      // groups past G: zero pieces and zero (2/sc, T), so the term vanishes (their
      // codes are the next row's)
      const float d = acc[u][0] + acc[u][1] + acc[u][2];
      const uint32_t mt = mrow[min(u, G - 1 - g0)];   // groups past G: any finite word (the term is zero)
      const float sc = f16_bits_to_f32(mt & 0xFFFFu), z = f16_bits_to_f32(mt >> 16);
      yacc = fmaf(sc, fmaf(d, st[u].x, -z * st[u].y), yacc);
    }
    // row tile done (the next item starts another tile, or this was the wave's last): add into LDS
    const int tile = pc.tile;
    pc.advance(sh, nw);
    if (pc.i >= items || pc.tile != tile) {
      if (t_ok) ylane[tile * 16] = yacc;
      yacc = 0.f;
    }
  };
  // ring slot d holds items d, d + DEPTH, ... of the wave's sequence. Every
  // slot is refilled on every pass, also past the wave's last item, and only
  // the processing is skipped there: the loads stay unconditional and in one
  // fixed order, so the compiler keeps exact wait counts.
  for (int i = wv; i < items; i += DEPTH * nw) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      if (d == 0 || i + d * nw < items) process(ring[d]);
      load(ring[d]);
    }
  }
  __syncthreads();
  // the waves' partials summed in wave order: the result does not depend on timing
  for (int idx = static_cast<int>(threadIdx.x); idx < M * rows; idx += static_cast<int>(blockDim.x)) {
    const int m = idx / rows, r = idx - m * rows, row = (b + (r >> 4) * sh.grid) * 16 + (r & 15);
    float acc = 0.f;
    for (int w = 0; w < nw; ++w) acc += yl[w * M * rows + idx];
    if (row < N) y[static_cast<size_t>(m) * N + row] = f32_to_f16_bits(acc);
  }
}

size_t mfma_lds_bytes(int M, int G, int Gp, int rows, int nw) {
  return static_cast<size_t>(M) * Gp * (kSetBytes + 8) + static_cast<size_t>(nw) * M * rows * 4 +
         static_cast<size_t>(rows) * meta_stride(G) * 4;
}

int padded_groups(int G, int bits) {
  const int gb = bits == 2 ? MxBatch<2>::GB : bits == 3 ? MxBatch<3>::GB : MxBatch<4>::GB;
  return (G + gb - 1) / gb * gb;
}

MxShape make_shape(int M, int K, int N, int bits, int grid, int block) {
  MxShape sh;
  const int gb = bits == 2 ? MxBatch<2>::GB : bits == 3 ? MxBatch<3>::GB : MxBatch<4>::GB;
  sh.M = M;
  sh.K = K;
  sh.N = N;
  sh.G = K / kGroup;
  sh.NB = (sh.G + gb - 1) / gb;
  sh.Gp = sh.NB * gb;
  sh.T = (N + 15) / 16;
  sh.tq = sh.T / grid;
  sh.tr = sh.T % grid;
  sh.grid = grid;
  const int nw = block / 64;
  sh.dt = nw / sh.NB;
  sh.db = nw % sh.NB;
  return sh;
}

template <int BITS, int DEPTH>
hipError_t launch_depth(const void *planes, const void *meta, const uint16_t *x, const int8_t *signs, uint16_t *y,
                        const MxShape &sh, int grid, int block, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  const int rows = (sh.tq + (sh.tr ? 1 : 0)) * 16;
  const size_t lds = mfma_lds_bytes(sh.M, sh.G, sh.Gp, rows, block / 64);
  auto kern = gemv_mfma_kernel<BITS, DEPTH>;
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
                          sv, y, sh);
  else
    hipLaunchKernelGGL(kern, dim3(grid), dim3(block), lds, s, pl, mt, xv, sv, y, sh);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const void *planes, const void *meta, const uint16_t *x, const int8_t *signs, uint16_t *y,
                       const MxShape &sh, int grid, int block, int depth, hipStream_t s, hipEvent_t start,
                       hipEvent_t stop) {
  switch (depth) {
    case 1: return launch_depth<BITS, 1>(planes, meta, x, signs, y, sh, grid, block, s, start, stop);
    case 2: return launch_depth<BITS, 2>(planes, meta, x, signs, y, sh, grid, block, s, start, stop);
    case 3: return launch_depth<BITS, 3>(planes, meta, x, signs, y, sh, grid, block, s, start, stop);
    default: return launch_depth<BITS, 4>(planes, meta, x, signs, y, sh, grid, block, s, start, stop);
  }
}

constexpr int kComputeUnits = 256;
constexpr size_t kMaxLds = 160 * 1024;

}  // namespace

void gemv_mfma_shape(int M, int K, int N, int bits, int &grid, int &block, int &depth) {
  const int G = K / kGroup, T = (N + 15) / 16;
  // eight waves rotate up to 64 (token, group) units in one pass; more units take sixteen
  block = M * G <= 64 ? 512 : kMxMaxThreads;
  // two workgroups per compute unit when there are many tiles and the workgroups are small
  grid = (block == 512 && T >= 4 * kComputeUnits) ? 2 * kComputeUnits : (T < kComputeUnits ? T : kComputeUnits);
  depth = bits == 4 ? 3 : 2;
}

bool gemv_mfma_supported(int M, int K, int N) {
  // K a multiple of 512: whole 16-byte vectors of meta words per row
  if (M < 1 || M > 4 || K < 4 * kGroup || K % (4 * kGroup) != 0 || N < 1) return false;
  // buffer offsets are 32-bit and kOutOfRange must lie past the planes of 4-bit codes
  if (static_cast<long long>(N + 16) * (K / kGroup) * 4 * 16 >= static_cast<long long>(kOutOfRange)) return false;
  int grid, block, depth;
  gemv_mfma_shape(M, K, N, 2, grid, block, depth);
  const int T = (N + 15) / 16;
  return mfma_lds_bytes(M, K / kGroup, padded_groups(K / kGroup, 3), ((T + grid - 1) / grid) * 16, block / 64) <=
         kMaxLds;
}

hipError_t launch_gemv_mfma(const void *planes, const void *meta, const uint16_t *x, const int8_t *signs,
                            uint16_t *y, int M, int K, int N, int bits, int grid, int block, int depth,
                            hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  if (M < 1 || M > 4 || (reinterpret_cast<uintptr_t>(signs) & 15u) != 0 || (reinterpret_cast<uintptr_t>(x) & 15u) != 0)
    return hipErrorInvalidValue;
  if (bits < 2 || bits > 4 || !gemv_mfma_supported(M, K, N)) return hipErrorInvalidValue;
  int g0, b0, d0;
  gemv_mfma_shape(M, K, N, bits, g0, b0, d0);
  if (grid <= 0) grid = g0;
  if (block <= 0) block = b0;
  if (depth <= 0) depth = d0;
  if (block % 64 != 0 || block < 64 || block > kMxMaxThreads || grid < 1) return hipErrorInvalidValue;
  const MxShape sh = make_shape(M, K, N, bits, grid, block);
  if (mfma_lds_bytes(M, sh.G, sh.Gp, (sh.tq + (sh.tr ? 1 : 0)) * 16, block / 64) > kMaxLds) return hipErrorInvalidValue;
  switch (bits) {
    case 2: return launch_bits<2>(planes, meta, x, signs, y, sh, grid, block, depth, s, start, stop);
    case 3: return launch_bits<3>(planes, meta, x, signs, y, sh, grid, block, depth, s, start, stop);
    default: return launch_bits<4>(planes, meta, x, signs, y, sh, grid, block, depth, s, start, stop);
  }
}

}  // namespace lbq
