// Matrix-core dequant-GEMM for five to sixteen tokens and 2-bit RTN codes:
// y = x' W'^T with W' = s (q - z) per 128-group (Qwen3-8B BPDQ model card,
// group-wise scale and zero), on v_mfma_scale_f32_16x16x128_f8f6f4 with the
// codes as the fp4 B operand (a 2-bit code in the two low bits of an e2m1
// nibble is exactly q / 2) and the activations as three e4m3 pieces.
//
// Why: from five tokens on, the fp16 GEMM's decode (two VALU operations per
// weight pair into round(s q)) takes longer than the MFMAs it feeds. Here a
// 32-code word column costs ten bit operations, as in the matrix-core GEMV,
// and one decoded B operand serves all sixteen tokens.
//
// Two launches:
//  * rotate_pieces_kernel: x' = R x per (token, group) as in the GEMV's
//    prologue (a power-of-two scale puts the group's largest magnitude in
//    [128, 256); three e4m3 pieces h + l + l2, each the rounding of what the
//    previous ones left). It writes the pieces of each 16-token tile and
//    group as one 6 KB block in the order the GEMM's LDS reads want, the
//    group's scale as an E8M0 byte per token, the zero-point sums T_g
//    (Sylvester's H_128 has column sums 128, 0, 0, ..., so T_g = sqrt(128)
//    s_0 x_0) as fp16 (high, low) pairs of T/16, and clears the split-K
//    counters.
//  * gemm_mx_kernel: a workgroup of four waves owns 64 NB rows and one K
//    slice of at most eight groups; wave w owns NB blocks of 16 rows. Every
//    load of the slice goes out at once: its pieces (6 KB per group) global ->
//    LDS (global_load_lds), each wave's code vectors straight into registers
//    by buffer loads (per step of two groups, the 64 bytes of 2-bit planes of
//    each row; a 4x4 lane transpose hands lane (j, kq) word column kq of both
//    planes of both groups). Step st then waits for its own loads only
//    (loads complete in issue order) and passes one barrier. A step's
//    contraction takes about a tenth of a load's round trip, so a ring
//    refilled step by step would wait at every step; short slices and a grid
//    of one round (at most two workgroups per compute unit) pay that round
//    trip once. The scale/zero words and scale bytes also reach LDS by copies:
//    a store of loaded registers to LDS would make the compiler wait for every
//    load in flight.
//    Per group and row block: three MFMAs, piece p of the sixteen tokens as
//    the A rows, the token's E8M0 scale as the A scale (so the product is
//    sum x' q, no per-token rescale), then y += s * acc (four FMAs). The
//    zero-point term -s z T_g is one fp16 MFMA per 16 groups at the end of
//    the slice, as in the fp16 GEMM.
// Split-K: each workgroup writes its fp32 partial tile to the workspace; the
// last of the S workgroups of a tile to arrive (an atomic counter the rotation
// launch cleared) sums the S partials in slice order and writes y, so the
// result does not depend on arrival order. No workgroup ever waits on another.
#include "device.h"
#include "gemm_common.h"
#include "kernels.h"
#include "mx_core.h"

#include <algorithm>

namespace lbq {

namespace {

using namespace mx;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileTokens = 16;
constexpr int kPieceVecs = 3 * 4 * 2 * 16;      // 16-byte vectors of one (token tile, group): 6 KB
constexpr int kStepVecs = 2 * kPieceVecs;       // one step: two groups
constexpr int kCopies = kStepVecs / kThreads;   // global -> LDS copies per wave per step
static_assert(kCopies * kThreads == kStepVecs, "copies");
constexpr int kMaxSliceGroups = 8;              // groups per K slice (all staged at once)
constexpr int kMaxSteps = kMaxSliceGroups / 2;

// Piece layout of one (token tile, group), in 16-byte vectors:
// [piece p][32-byte column kq][half h][token i]. Lane (i, kq) of the MFMA's A
// operand reads vectors (p, kq, 0, i) and (p, kq, 1, i): the sixteen lanes of
// one ds_read_b128 pass read 256 contiguous bytes (no bank conflict). Byte b
// of column kq is element b of lane group kq of the mixed fp8 x fp4 operand.
__host__ __device__ constexpr int piece_vec(int p, int kq, int h, int i) { return ((p * 4 + kq) * 2 + h) * 16 + i; }

// ------------------------------------------------------------------ rotation

// One (token, group) unit per eight lanes, 32 units per workgroup; tokens past
// M (up to the tile's end) are rotated zeros.
__global__ void __launch_bounds__(256) rotate_pieces_kernel(const uint16_t *__restrict__ x,
                                                            const int8_t *__restrict__ signs,
                                                            uint32_t *__restrict__ pieces,
                                                            uint8_t *__restrict__ scales, uint32_t *__restrict__ tz,
                                                            int M, int Mp, int K, int Gp,
                                                            uint32_t *__restrict__ counters, int n_counters) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n_counters; i += gridDim.x * 256) counters[i] = 0;
  const int G = K / kGroup;
  const int tid = static_cast<int>(threadIdx.x);
  const long unit = static_cast<long>(blockIdx.x) * 32 + rot_unit_of(tid);
  const int L = rot_lane_of(tid);
  const bool ok = unit < static_cast<long>(Mp) * G;   // the unit's eight lanes agree
  const int m = ok ? static_cast<int>(unit / G) : 0, g = ok ? static_cast<int>(unit - static_cast<long>(m) * G) : 0;
  // buffer loads: rows past M and lanes without a unit load zeros (every lane
  // takes part in the DPP exchanges of the rotation)
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(x), 0, M * K * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(signs), 0, K, kBufferFlags);
  const RotUnit u = rot_unit(rot_load(xrs, srs, K, m, g, L, ok), L);
  if (!ok) return;
  const int mt = m / kTileTokens, i = m - mt * kTileTokens;
  uint32_t *blk = pieces + (static_cast<long>(mt) * G + g) * (kPieceVecs * 4);
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    float a[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = u.v[s4 + 4 * e] * u.c;
    // word off (0..31) of the 128-byte piece holds positions 16 L + s4 + 4 e
    // (the matrix-core GEMV's element order)
    const int r = sigma(s4), kqb = L >> 1;
    const int off = (2 * (kqb & 1) + (r >> 1)) * 8 + 4 * (kqb >> 1) + 2 * (r & 1) + (L & 1);
    uint32_t w[3];
    split3(a, w);
#pragma unroll
    for (int p = 0; p < 3; ++p) blk[piece_vec(p, off >> 3, (off >> 2) & 1, i) * 4 + (off & 3)] = w[p];
  }
  if (L != 0) return;
  // A scale: pieces times 2^(E - 7) are x' times 2 (the fp4 B value is q / 2)
  scales[((static_cast<long>(mt) * (G / 4) + g / 4) * kTileTokens + i) * 4 + (g & 3)] =
      static_cast<uint8_t>(min(max(120 + u.E, 0), 254));
  if (m >= M) return;
  uint32_t *row = tz + static_cast<long>(m) * Gp;
  const float t16 = u.first * (11.313708498984761f * 0.0625f);   // T_g / 16
  const uint32_t th = f32_to_f16_bits(t16);
  const uint32_t tl = f32_to_f16_bits(t16 - f16_bits_to_f32(th));
  row[g] = th | (tl << 16);
  if (g == G - 1)
    for (int gz = G; gz < Gp; ++gz) row[gz] = 0;
}

// ------------------------------------------------------------------ GEMM

struct MxGemmArgs {
  const uint4 *pieces;      // [Mt][G][kPieceVecs]
  const uint32_t *scales;   // [Mt][G / 4][16] (four E8M0 bytes: groups 4c .. 4c + 3 of token i)
  const uint4 *tz;          // [M][Gp / 4] of 4 u32: (T/16 high, T/16 low) fp16 per (token, group)
  const uint4 *planes;      // [N][G][2] 16-byte plane vectors
  const uint32_t *meta;     // [N][G] (fp16 s, fp16 z)
  uint16_t *y;              // [M][N]
  float *part;              // split-K partial tiles (S > 1)
  uint32_t *counters;       // split-K arrival counters, one per tile, zero on entry
  int M, K, N, S, Gp;
};

// Wait until this wave's loads of step st (of kMaxSteps = 4, L loads each,
// followed by T more) have landed: loads complete in issue order. st is a
// constant once the step loop is unrolled.
template <int L, int T>
__device__ __forceinline__ void wait_step(int st) {
  static_assert(kMaxSteps == 4, "one case per step");
  switch (st) {
    case 0: wait_vm_lds<3 * L + T>(); break;
    case 1: wait_vm_lds<2 * L + T>(); break;
    case 2: wait_vm_lds<L + T>(); break;
    default: wait_vm_lds<T>(); break;
  }
}

// Groups [g0, g1) of split `split`: whole 4-group words, so the staged scale
// bytes and scale/zero vectors of a slice start on a word.
__device__ __forceinline__ int slice_start(int split, int G, int S) {
  return 4 * static_cast<int>((static_cast<long>(split) * (G / 4)) / S);
}

template <int NB>
__global__ void __launch_bounds__(kThreads) gemm_mx_kernel(MxGemmArgs a) {
  // the slice's pieces, one LDS object per step: the compiler then tells a
  // read of one step's pieces from the copies still in flight into the others
  __shared__ __attribute__((aligned(16))) uint4 xs0[kStepVecs];
  __shared__ __attribute__((aligned(16))) uint4 xs1[kStepVecs];
  __shared__ __attribute__((aligned(16))) uint4 xs2[kStepVecs];
  __shared__ __attribute__((aligned(16))) uint4 xs3[kStepVecs];
  static_assert(kMaxSteps == 4, "one LDS object per step");
  uint4 *const xs[kMaxSteps] = {xs0, xs1, xs2, xs3};
  constexpr int kRowsWG = kWaves * 16 * NB;
  // scale/zero words of the workgroup's rows over the slice, row r at words
  // kMS r .. kMS r + 7 (the lanes of a 16-row block read at most 2-way banked)
  constexpr int kMS = kMaxSliceGroups;
  constexpr int kMetaVecs = kRowsWG * (kMaxSliceGroups / 4);   // 16-byte vectors staged
  constexpr int kMetaIters = (kMetaVecs + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) uint32_t msm[kMetaIters * kThreads * 4];
  __shared__ uint32_t ssm[kThreads];   // scale words: [word of 4 groups][token] in the first 32

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane & 15, kq = lane >> 4;
  const int G = a.K / kGroup;
  const int split = blockIdx.x;
  const int tile_id = blockIdx.z * gridDim.y + blockIdx.y;
  const int mtile = blockIdx.z;
  const int m0 = mtile * kTileTokens;
  const int row0 = blockIdx.y * kRowsWG + wave * 16 * NB + j;   // the lane's row of block 0
  const int g0 = slice_start(split, G, a.S), g1 = slice_start(split + 1, G, a.S);
  const int nq = (g1 - g0) / 4;    // 4-group words of the slice (1 or 2)
  const int nst = (g1 - g0) / 2;   // steps of two groups (2 or 4)

  const __amdgpu_buffer_rsrc_t prs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4 *>(a.planes), 0, a.N * G * 32, kBufferFlags);

  // Every load of the slice goes out at once, in this order: the scale/zero
  // words and scale bytes (global -> LDS, no register round trip), each step's
  // pieces and code vectors, the zero-point sums.
  {
    const uint32_t *mbase = a.meta + static_cast<size_t>(blockIdx.y) * kRowsWG * G + g0;
#pragma unroll
    for (int it = 0; it < kMetaIters; ++it) {
      const int i = static_cast<int>(threadIdx.x) + it * kThreads;
      // vector v of local row r; rows past N and words past the slice copy a
      // valid vector that is never read
      const int r = min(i / (kMaxSliceGroups / 4), kRowsWG - 1), v = i % (kMaxSliceGroups / 4);
      const int rr = min(r, a.N - 1 - static_cast<int>(blockIdx.y) * kRowsWG), vv = v < nq ? v : 0;
      copy16_to_lds(mbase + static_cast<size_t>(rr) * G + 4 * vv, msm + 4 * (it * kThreads + 64 * wave));
    }
    const int i = min(static_cast<int>(threadIdx.x), nq * kTileTokens - 1);
    copy4_to_lds(a.scales + (static_cast<size_t>(mtile) * (G / 4) + g0 / 4) * kTileTokens + i, ssm + 64 * wave);
  }
  // Step-major loads: for each step its pieces (global -> LDS; wave w copies
  // vectors [kCopies 64 w, kCopies 64 (w + 1)) of the step, the slice's groups
  // being contiguous in the piece array) and this lane's code vectors (16
  // bytes at offset 16 kq of its row's two groups: planes 0, 1 of the first
  // group at kq = 0, 1, of the second at 2, 3). Steps past the slice repeat
  // its last step's pieces and load zero codes, so every wave issues the same
  // count and each step can wait for its own loads alone.
  constexpr int kStepLoads = kCopies + NB;
  uint4 bv[kMaxSteps][NB];
  __builtin_amdgcn_sched_barrier(0);   // the waits below count loads in issue order
  {
    const uint4 *src = a.pieces + (static_cast<size_t>(mtile) * G + g0) * kPieceVecs + kCopies * 64 * wave + lane;
#pragma unroll
    for (int st = 0; st < kMaxSteps; ++st) {
      const int sc = min(st, nst - 1);
#pragma unroll
      for (int c = 0; c < kCopies; ++c)
        copy16_to_lds(src + sc * kStepVecs + 64 * c, xs[st] + kCopies * 64 * wave + 64 * c);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int row = row0 + nb * 16;
        const uint32_t off =
            (row < a.N && st < nst)
                ? static_cast<uint32_t>(row) * G * 32 + static_cast<uint32_t>(g0 + 2 * st) * 32 + kq * 16
                : kOutOfRange;
        bv[st][nb] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(prs, off, 0, 0));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // zero-point sums of token j over the (at most two) 16-group blocks the
  // slice touches (lane (j, kq) covers groups 16 c + 4 kq .. + 3): needed last
  constexpr int kTzLoads = 2;
  const int c0 = g0 / 16, c1 = (g1 - 1) / 16;
  const __amdgpu_buffer_rsrc_t trs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4 *>(a.tz), 0, a.M * a.Gp * 4, kBufferFlags);
  const uint32_t toff = static_cast<uint32_t>(min(m0 + j, a.M - 1) * a.Gp * 4);
  uint4 tzv[kTzLoads];
#pragma unroll
  for (int c = 0; c < kTzLoads; ++c)
    tzv[c] = __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(
                   trs, c0 + c <= c1 ? toff + static_cast<uint32_t>((16 * (c0 + c) + 4 * kq) * 4) : kOutOfRange, 0, 0));

  float4_t yacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) yacc[nb] = float4_t{0.f, 0.f, 0.f, 0.f};
  // this lane's row of block nb in the staged scale/zero words (column g - g0)
  const uint32_t *mrow = msm + (wave * 16 * NB + j) * kMS - g0;

#pragma unroll
  for (int st = 0; st < kMaxSteps; ++st) {
    // this wave's loads of step st have landed (later steps' and the sums may
    // still be in flight), and after the barrier every other wave's copies too
    __builtin_amdgcn_sched_barrier(0);   // no work of this step moves above its wait
    wait_step<kStepLoads, kTzLoads>(st);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (st >= nst) break;
    const int g = g0 + 2 * st;
    const uint4 *slot = xs[st];
    // A scale bytes of token j for groups g, g + 1 (g - g0 = 2 st: bytes 0, 1 or 2, 3)
    const uint32_t sw = ssm[(st >> 1) * kTileTokens + j] >> (16 * (st & 1));
    uint32_t w[NB][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      w[nb][0] = bv[st][nb].x;
      w[nb][1] = bv[st][nb].y;
      w[nb][2] = bv[st][nb].z;
      w[nb][3] = bv[st][nb].w;
      transpose4(w[nb][0], w[nb][1], w[nb][2], w[nb][3]);
    }
    // all MFMAs of the step first (eight independent chains at NB = 4), then
    // the scalings that read their results
    v4f_t acc[2][NB];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      v8i_t av[3];
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const uint4 lo = slot[u * kPieceVecs + piece_vec(p, kq, 0, j)];
        const uint4 hi = slot[u * kPieceVecs + piece_vec(p, kq, 1, j)];
        av[p] = v8i_t{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
                      static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
      }
      const int sa = static_cast<int>((sw >> (8 * u)) & 0xFFu);
      v8i_t bop[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        uint32_t lo4[4];
        fp4_from_pair(w[nb][2 * u], w[nb][2 * u + 1], lo4);
        bop[nb] = v8i_t{static_cast<int>(lo4[0]), static_cast<int>(lo4[1]), static_cast<int>(lo4[2]),
                        static_cast<int>(lo4[3]), 0, 0, 0, 0};
        acc[u][nb] = v4f_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[u][nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av[p], bop[nb], acc[u][nb], 0, 4, 0, sa, 0, 127);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float sc = f16_bits_to_f32(mrow[nb * 16 * kMS + g + u] & 0xFFFFu);
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[nb][r] = fmaf(sc, acc[u][nb][r], yacc[nb][r]);
      }
  }

  // zero-point term of the slice: K = (group, high/low) over 16 groups per MFMA
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (c0 + c > c1) break;
    const half8_t za = __builtin_bit_cast(half8_t, tzv[c]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      uint32_t b[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int g = 16 * (c0 + c) + 4 * kq + e;
        const half2_t sz = __builtin_bit_cast(half2_t, (g >= g0 && g < g1) ? mrow[nb * 16 * kMS + g] : 0u);
        const _Float16 v = static_cast<_Float16>(-16.0f) * (sz[0] * sz[1]);
        b[e] = __builtin_bit_cast(uint32_t, half2_t{v, v});
      }
      const half8_t bop = __builtin_bit_cast(half8_t, make_uint4(b[0], b[1], b[2], b[3]));
      yacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(za, bop, yacc[nb], 0, 0, 0);
    }
  }
  wait_vm_lds<0>();   // no copy into LDS may outlive the workgroup

  if (a.S > 1) {
    // publish this slice's partial tile; the last slice to arrive sums them all
    constexpr int kTileFloats = NB * 4 * kThreads;
    float *mine = a.part + (static_cast<size_t>(tile_id) * a.S + split) * kTileFloats + threadIdx.x;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) store_coherent(mine + (nb * 4 + r) * kThreads, yacc[nb][r]);
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
    for (int nb = 0; nb < NB; ++nb) yacc[nb] = float4_t{0.f, 0.f, 0.f, 0.f};
    for (int s2 = 0; s2 < a.S; ++s2) {
      float *src = a.part + (static_cast<size_t>(tile_id) * a.S + s2) * kTileFloats + threadIdx.x;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[nb][r] += load_coherent(src + (nb * 4 + r) * kThreads);
    }
  }

  // D layout: lane holds tokens 4 kq + r (r = 0..3), row j of block nb
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int row = row0 + nb * 16;
    if (row < a.N) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = m0 + kq * 4 + r;
        if (tok < a.M) a.y[static_cast<size_t>(tok) * a.N + row] = f32_to_f16_bits(yacc[nb][r]);
      }
    }
  }
}

}  // namespace

bool gemm_mx_supported(int M, int K, int N, int bits) {
  // 2-bit codes; whole 4-group words (K a multiple of 512); 32-bit buffer offsets
  return bits == 2 && M > 0 && K % 512 == 0 && static_cast<long long>(N) * (K / kGroup) * 32 < (1ll << 31);
}

GemmPlan gemm_mx_plan(int M, int K, int N) {
  // K slices of at most eight groups (each workgroup stages its slice's pieces
  // at once); the fewest row blocks per wave (1, 2, 4) that keep the grid
  // within two workgroups per compute unit, so the grid runs in one round.
  GemmPlan p;
  p.mt = 1;
  p.kw = 1;
  const int G4 = K / kGroup / 4;
  p.m_tiles = (M + kTileTokens - 1) / kTileTokens;
  p.S = (G4 + kMaxSliceGroups / 4 - 1) / (kMaxSliceGroups / 4);
  for (p.nb = 1; p.nb < 4; p.nb *= 2) {
    const long wgs = static_cast<long>((N + 64 * p.nb - 1) / (64 * p.nb)) * p.m_tiles * p.S;
    if (wgs <= 512) break;
  }
  p.n_tiles = (N + 64 * p.nb - 1) / (64 * p.nb);
  return p;
}

size_t gemm_mx_act_bytes(int M, int K) {
  const size_t mt = static_cast<size_t>((M + kTileTokens - 1) / kTileTokens);
  const size_t G = static_cast<size_t>(K / kGroup);
  const size_t pieces = mt * G * kPieceVecs * 16;
  const size_t scales = mt * G * kTileTokens;   // one byte per (token slot, group)
  return ((pieces + 255) / 256) * 256 + ((scales + 255) / 256) * 256;
}

hipError_t launch_gemm_mx(const GemmPlan &p, const void *planes, const void *meta, const uint16_t *x,
                          const int8_t *signs, void *act, uint32_t *tz, uint16_t *y, int M, int K, int N,
                          void *scratch, hipStream_t s, hipEvent_t between) {
  if (M <= 0) return hipSuccess;
  if (!gemm_mx_supported(M, K, N, 2) || (p.nb != 1 && p.nb != 2 && p.nb != 4) || p.mt != 1 || p.S < 1)
    return hipErrorInvalidValue;
  const int G = K / kGroup;
  if ((G / 4 + p.S - 1) / p.S > kMaxSliceGroups / 4 || p.S > G / 4) return hipErrorInvalidValue;
  const int Mt = (M + kTileTokens - 1) / kTileTokens, Mp = Mt * kTileTokens;
  if (static_cast<long long>(M) * K * 2 >= (1ll << 31)) return hipErrorInvalidValue;
  uint8_t *act8 = static_cast<uint8_t *>(act);
  uint32_t *pieces = reinterpret_cast<uint32_t *>(act8);
  const size_t piece_bytes = ((static_cast<size_t>(Mt) * G * kPieceVecs * 16 + 255) / 256) * 256;
  uint8_t *scales = act8 + piece_bytes;
  uint32_t *counters = gemm_counter_ptr(p, scratch);
  const int n_counters = gemm_counters(p);
  const int Gp = gemm_tz_stride(K);
  const long units = static_cast<long>(Mp) * G;
  const long nblk = std::max<long>((units + 31) / 32, (n_counters + 255) / 256);
  hipLaunchKernelGGL(rotate_pieces_kernel, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, s, x, signs, pieces,
                     scales, tz, M, Mp, K, Gp, counters, n_counters);
  if (between && hipEventRecord(between, s) != hipSuccess) return hipErrorUnknown;
  MxGemmArgs a;
  a.pieces = reinterpret_cast<const uint4 *>(pieces);
  a.scales = reinterpret_cast<const uint32_t *>(scales);
  a.tz = reinterpret_cast<const uint4 *>(tz);
  a.planes = static_cast<const uint4 *>(planes);
  a.meta = static_cast<const uint32_t *>(meta);
  a.y = y;
  a.part = static_cast<float *>(scratch);
  a.counters = counters;
  a.M = M;
  a.K = K;
  a.N = N;
  a.S = p.S;
  a.Gp = Gp;
  const dim3 grid(static_cast<unsigned>(p.S), static_cast<unsigned>(p.n_tiles), static_cast<unsigned>(p.m_tiles));
  if (p.nb == 1) hipLaunchKernelGGL(gemm_mx_kernel<1>, grid, dim3(kThreads), 0, s, a);
  else if (p.nb == 2) hipLaunchKernelGGL(gemm_mx_kernel<2>, grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(gemm_mx_kernel<4>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace lbq
