// Matrix-core decode of RTN codes against fp8 activation pieces
// (v_mfma_scale_f32_16x16x128_f8f6f4, A fp8 e4m3, B fp4 e2m1), shared by the
// dense GEMV and the grouped MoE expert kernels.
//
// Operands:
//  * B = codes. A 2-bit code q dropped into the two low bits of an fp4 nibble
//    is the exact value q / 2, so a 32-code word column of two bit planes
//    becomes four nibble words in ten bit operations. 3- and 4-bit codes
//    q = ql + 4 qh take a second MFMA on the high part with the B scale 2^2.
//  * A = activations. Each rotated group x'_g (fp32) is scaled by a power of
//    two sc_g that puts its largest magnitude in [128, 256) and split into
//    three e4m3 pieces h + l + l2 (each piece the rounding of what the
//    previous ones left): about twelve significant bits, at least fp16's.
//    Token t's pieces sit on A rows 4t, 4t + 1, 4t + 2 (row 4t + 3 is zero),
//    so one MFMA serves up to four tokens and lane (j, t) of the result holds
//    the three piece products of token t and output row j in its first three
//    accumulator registers.
// A group's contribution to y_j is then s (2 d / sc_g - z T_g) with d the sum
// of the three products and T_g = sum_k x'_k (RTN dequantisation s (q - z):
// Qwen3-8B BPDQ model card, group-wise scale and zero).
//
// Element order: B element b (nibble b & 7 of register b >> 3) of lane
// (j, kq) holds code 32 kq + 4 (b & 7) + sigma(b >> 3) of the group, sigma =
// (0, 2, 1, 3); fp8 A element b_a of lane (i, kq_a) meets the fp4 B element
// of lane group kq_b = (kq_a >> 1) + 2 (b_a >> 4), b_b = (b_a & 15) +
// 16 (kq_a & 1) (the operand layouts of the mixed-format instruction). The
// rotation writes each piece straight into that order.
#pragma once

#include "device.h"
#include "gemm_common.h"

namespace lbq {
namespace mx {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

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
template <>
struct MxBatch<8> {
  static constexpr int GB = 1, NV = 2;   // one group of eight planes: 128 bytes per row
};

template <int BITS>
struct MxItem {
  uint4 v[MxBatch<BITS>::NV];
};

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

// One cross-lane butterfly stage over sixteen values: v += sg * (v of the
// partner lane), each a single v_fmac_f32 with a DPP source (partner lane ^ 1,
// ^ 2 or ^ 8 for STAGE 0, 1, 2). Written out because the compiler keeps the DPP
// move and the multiply-add apart (two instructions and a hazard wait each).
// The leading s_nop covers the DPP read-after-VALU-write hazard of values the
// compiler wrote just before; inside the block each value is read sixteen
// instructions after its last write.
#define LBQ_FMAC_DPP(I, CTRL) "v_fmac_f32_dpp %" #I ", %" #I ", %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"
#define LBQ_FMAC_DPP16(CTRL)                                                                                        \
  "s_nop 1\n\t" LBQ_FMAC_DPP(0, CTRL) LBQ_FMAC_DPP(1, CTRL) LBQ_FMAC_DPP(2, CTRL) LBQ_FMAC_DPP(3, CTRL)            \
      LBQ_FMAC_DPP(4, CTRL) LBQ_FMAC_DPP(5, CTRL) LBQ_FMAC_DPP(6, CTRL) LBQ_FMAC_DPP(7, CTRL) LBQ_FMAC_DPP(8, CTRL)   \
          LBQ_FMAC_DPP(9, CTRL) LBQ_FMAC_DPP(10, CTRL) LBQ_FMAC_DPP(11, CTRL) LBQ_FMAC_DPP(12, CTRL)                  \
              LBQ_FMAC_DPP(13, CTRL) LBQ_FMAC_DPP(14, CTRL) LBQ_FMAC_DPP(15, CTRL)
template <int STAGE>
__device__ __forceinline__ void dpp_butterfly16(float v[16], float sg) {
  static_assert(STAGE >= 0 && STAGE < 3, "stage");
#define LBQ_DPP_OPERANDS                                                                                             \
  : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]), "+v"(v[8]),      \
    "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15])                       \
  : "v"(sg)
  if constexpr (STAGE == 0) asm volatile(LBQ_FMAC_DPP16("quad_perm:[1,0,3,2]") LBQ_DPP_OPERANDS);
  else if constexpr (STAGE == 1) asm volatile(LBQ_FMAC_DPP16("quad_perm:[2,3,0,1]") LBQ_DPP_OPERANDS);
  else asm volatile(LBQ_FMAC_DPP16("row_ror:8") LBQ_DPP_OPERANDS);
#undef LBQ_DPP_OPERANDS
}
#undef LBQ_FMAC_DPP16
#undef LBQ_FMAC_DPP

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

// Rotation of one unit: the 16 values of lane L, (H_128 D x) at positions
// 16 L .. 16 L + 15 of the group, up to a sign, with the 1/sqrt(128)
// normalisation and the group's power-of-two scale folded into c: v[i] * c is
// the scaled rotated value (largest magnitude of the group in [128, 256)).
//  * Cross-lane stages first, on the signed inputs, each one v_fmac with a DPP
//    operand: v += sg * partner with sg = -1 on the lane whose bit is set.
//    That lane gets v - partner, the negated butterfly output; the pair
//    partners always carry the same accumulated sign, so after the three
//    stages lane L holds (-1)^popcount(L) times the exact value, and the
//    factor goes into c.
//  * Four in-lane stages.
// E is the group's exponent (max |x'| = f 2^E, f in [0.5, 1); scale 2^(8 - E)).
// first = s_0 x_0 on lane 0: Sylvester's H_128 has column sums 128, 0, 0, ...,
// so the group sum is T_g = sqrt(128) s_0 x_0 (exact, no reduction).
struct RotUnit {
  float v[16];
  float c, first;
  int E;
};
__device__ __forceinline__ RotUnit rot_unit(const RotIn &in, int L) {
  RotUnit u;
  float *v = u.v;
  const uint32_t xw[8] = {in.xa.x, in.xa.y, in.xa.z, in.xa.w, in.xb.x, in.xb.y, in.xb.z, in.xb.w};
  const uint32_t sw[4] = {in.sv.x, in.sv.y, in.sv.z, in.sv.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // sign bytes of elements 2i, 2i + 1 moved to bytes 1 and 3 (their bit 7 onto
    // the fp16 sign bits 15 and 31); selector 0x0C gives a zero byte
    const uint32_t sel = (i & 1) ? 0x030C020Cu : 0x010C000Cu;
    const uint32_t sb = __builtin_amdgcn_perm(sw[i >> 1], sw[i >> 1], sel);
    const uint32_t h = xw[i] ^ (sb & 0x80008000u);
    v[2 * i] = half_lo(h);
    v[2 * i + 1] = half_hi(h);
  }
  u.first = v[0];   // s_0 x_0 on lane 0
  dpp_butterfly16<0>(v, (L & 1) ? -1.f : 1.f);
  dpp_butterfly16<1>(v, (L & 2) ? -1.f : 1.f);
  dpp_butterfly16<2>(v, (L & 4) ? -1.f : 1.f);
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
  // across the unit's lanes on the bit patterns (non-negative floats order as
  // unsigned integers; no NaN quieting needed)
  uint32_t mb = __builtin_bit_cast(uint32_t, mx);
  mb = max(mb, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(mb), kDppXor1, 0xF, 0xF, true)));
  mb = max(mb, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(mb), kDppXor2, 0xF, 0xF, true)));
  mb = max(mb, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(mb), kDppXor8, 0xF, 0xF, true)));
  mx = __builtin_bit_cast(float, mb);
  u.E = __builtin_amdgcn_frexp_expf(mx * kInvSqrt128);
  const float flip = (__builtin_popcount(L) & 1) ? -1.f : 1.f;
  u.c = __builtin_amdgcn_ldexpf(flip * kInvSqrt128, 8 - u.E);
  return u;
}

// Three e4m3 pieces of four scaled values (each the rounding of what the
// previous ones left), one word each.
__device__ __forceinline__ void split3(float a[4], uint32_t w[3]) {
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    w[p] = e4m3x4(a[0], a[1], a[2], a[3]);
    if (p < 2) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[p]), false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[p]), true);
      a[0] -= lo[0];
      a[1] -= lo[1];
      a[2] -= hi[0];
      a[3] -= hi[1];
    }
  }
}

// Rotate one unit and write its A pieces in the mixed fp8 x fp4 operand order:
// positions 16 L + s + 4 e (e = 0..3) form one 4-byte word (see the file
// comment), four words per piece per lane. ss[t * Gp + g] = (2 / sc_g, T_g).
// store = false computes without writing.
__device__ __forceinline__ void rot_pieces(const RotIn &in, int Gp, int m, int g, int L, bool store, uint32_t *xa,
                                           float2 *ss) {
  RotUnit u = rot_unit(in, L);
  uint32_t *blk = xa + static_cast<size_t>(m * Gp + g) * (kSetBytes / 4);
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    float a[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = u.v[s4 + 4 * e] * u.c;
    // word (kq_a, w) of the A layout that holds positions 16 L + s4 + 4 e
    const int r = sigma(s4), kqb = L >> 1;
    const int off = (2 * (kqb & 1) + (r >> 1)) * 8 + 4 * (kqb >> 1) + 2 * (r & 1) + (L & 1);
    uint32_t w[3];
    split3(a, w);
#pragma unroll
    for (int p = 0; p < 3; ++p)
      if (store) blk[piece_offset(p) / 4 + off] = w[p];
  }
  if (store && L == 0)
    ss[m * Gp + g] = make_float2(__builtin_amdgcn_ldexpf(1.f, u.E - 7), u.first * 11.313708498984761f);
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

// Groups padded to whole batches of the code width.
inline int batch_groups(int bits) {
  return bits == 2 ? MxBatch<2>::GB : bits == 3 ? MxBatch<3>::GB : bits == 4 ? MxBatch<4>::GB : MxBatch<8>::GB;
}
inline int padded_groups(int G, int bits) {
  const int gb = batch_groups(bits);
  return (G + gb - 1) / gb * gb;
}

inline MxShape make_shape(int M, int K, int N, int bits, int grid, int block) {
  MxShape sh;
  const int gb = batch_groups(bits);
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

}  // namespace mx
}  // namespace lbq
