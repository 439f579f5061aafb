// Product-VQ dequant-GEMV for one to four tokens on the matrix cores, activation
// rotation fused into the prologue (product-VQ over fp8-grid codebook values:
// Laguna-S-2.1 gridbook model card, opening paragraph and format list).
//
// v_mfma_scale_f32_16x16x128_f8f6f4 with both operands e4m3:
//  * B = codebook values. An index byte picks four e4m3 values for four
//    consecutive weights: one 32-bit word of the B operand, read from a table
//    in LDS (32 copies of the 1 KB codebook, one per lane of an LDS pass).
//    Lane (j, kq) of a group takes the index bytes 4 kq .. 4 kq + 3
//    and 16 + 4 kq .. 16 + 4 kq + 3 of row j's 32 (weights 16 kq .. 16 kq + 15
//    and 64 + 16 kq .. 64 + 16 kq + 15), the word columns a 4x4 lane transpose
//    of the row's 16-byte loads hands it.
//  * A = the rotated activations as three e4m3 pieces per token (mx_core.h),
//    written in that same element order. The group's power of two 2^(8 - E)
//    is undone by the instruction's A scale (E8M0 exponent 119 + E per lane,
//    one token's group per A row), so the accumulators run across all groups
//    with no per-group arithmetic; the row scale is applied once at the end.
// Work split as in the RTN matrix-core GEMV: items of (16-row tile, batch of
// two groups) round-robin over the waves, partial sums per wave in LDS added
// in wave order at the end (repeat calls are bit-identical).
// Residual stages (idx [S][N][K/4], row scales [S][N]): a workgroup's tiles
// are walked once per stage (stage-major "virtual tiles"), each with its own
// partial sums, and y = sum over stages of the stage's row scale times them.
#include "kernels.h"
#include "mx_core.h"

namespace lbq {

namespace {

using namespace mx;

constexpr int kPvqMaxThreads = 1024;
constexpr int kGB = 2;   // groups per item: 64 index bytes of a row, 16 bytes per lane
// The codebook table in LDS is replicated: entry e of copy c at word 32 e + c,
// and lane l reads copy l & 31. The 32 lanes of one LDS pass then hit 32
// distinct banks whatever their indices (one table: random indices collide
// several ways per pass, and every weight quad is one lookup).
constexpr int kLutCopies = 32;

// Rotate one unit and write its A pieces in the product-VQ element order:
// positions 16 L + 4 w .. 16 L + 4 w + 3 are word 8 (L & 3) + 4 (L >> 2) + w of
// each piece; sx[m * Gp + g] = E8M0 exponent 119 + E of the group's A scale.
__device__ __forceinline__ void rot_pieces_pvq(const RotIn &in, int Gp, int m, int g, int L, bool store,
                                               uint32_t *xa, uint32_t *sx) {
  RotUnit u = rot_unit(in, L);
  uint32_t *blk = xa + static_cast<size_t>(m * Gp + g) * (kSetBytes / 4);
  const int off = 8 * (L & 3) + 4 * (L >> 2);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float a[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = u.v[4 * w + e] * u.c;
    uint32_t pw[3];
    split3(a, pw);
#pragma unroll
    for (int p = 0; p < 3; ++p)
      if (store) blk[piece_offset(p) / 4 + off + w] = pw[p];
  }
  if (store && L == 0) sx[m * Gp + g] = static_cast<uint32_t>(119 + u.E);
}

// x: raw activations [M][K] fp16 (M <= 4); signs: [K] int8 (+-1), 16-byte aligned.
template <int DEPTH, int ST>
__global__ void __launch_bounds__(kPvqMaxThreads) gemv_pvq_mx_kernel(const uint4 *__restrict__ idx,
                                                                  const uint16_t *__restrict__ row_scale,
                                                                  const uint32_t *__restrict__ codebook,
                                                                  const uint4 *__restrict__ x,
                                                                  const uint4 *__restrict__ signs,
                                                                  uint16_t *__restrict__ y, const MxShape sh) {
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  const int M = sh.M, K = sh.K, N = sh.N, G = sh.G, Gp = sh.Gp;
  const int VR = G * 2;                          // 16-byte index vectors per row
  const int b = static_cast<int>(blockIdx.x);
  const int ntl = sh.tq + (b < sh.tr ? 1 : 0);   // this workgroup's tiles: b + k grid, k < ntl
  const int rows = ntl * 16;
  constexpr int stages = ST;
  const int vrows = stages * rows;               // partial-sum rows: stage-major virtual tiles
  const int items = stages * ntl * sh.NB;
  const int nw = static_cast<int>(blockDim.x >> 6), nt = static_cast<int>(blockDim.x);
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));   // wave-uniform
  const int lane = static_cast<int>(threadIdx.x & 63), j = lane & 15, kq = lane >> 4;
  const uint32_t lcopy = static_cast<uint32_t>(lane) & (kLutCopies - 1);   // this lane's codebook copy

  // LDS: codebook [256][kLutCopies] words, piece sets [M][Gp], A-scale
  // exponents [M][Gp], the waves' row partial sums [nw][M][stages * rows].
  uint32_t *lut = smem;
  uint32_t *xa = smem + 256 * kLutCopies;
  uint32_t *sx = xa + M * Gp * (kSetBytes / 4);
  float *yl = reinterpret_cast<float *>(sx + M * Gp);

  const __amdgpu_buffer_rsrc_t prs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4 *>(idx), 0, stages * N * VR * 16, kBufferFlags);
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
  auto load = [&](uint4 &it) {
    const uint32_t past = lc.i < items ? 0u : kOutOfRange;
    int st = 0, tl = lc.tile;   // virtual tile -> (stage, tile)
#pragma unroll
    for (int k2 = 1; k2 < stages; ++k2) {
      const bool next = tl >= ntl;
      tl -= next ? ntl : 0;
      st += next ? 1 : 0;
    }
    const uint32_t pstep =
        static_cast<uint32_t>((tl * tstride * VR + lc.batch * kGB * 2) * 16 + st * N * VR * 16) + past;
    it = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(prs, pbase + pstep, 0, 0));
    lc.advance(sh, nw);
  };
  const int units = M * G, ustep = nt >> 3;
  const int u0 = rot_unit_of(static_cast<int>(threadIdx.x)), rL = rot_lane_of(static_cast<int>(threadIdx.x));
  const int m0 = (u0 >= G) + (u0 >= 2 * G) + (u0 >= 3 * G);
  // Order of the first loads (a compute unit's vector memory path returns data
  // in request order): every wave's activations and the codebook word go out
  // first, all waves pass one barrier that waits for no data, then the index
  // loads. Waves that rotate issue two ring slots, rotate, and issue the rest;
  // the others skip the rotation and issue every slot at once. Both branches
  // leave the same loads outstanding in the same order.
  constexpr int kEarly = DEPTH < 2 ? DEPTH : 2;
  const bool rotating = wv * 8 < units;   // wave-uniform
  uint4 ring[DEPTH];
  uint32_t cw;
  if (rotating) {
    const RotIn rin = rot_load(xrs, srs, K, min(m0, M - 1), u0 - m0 * G, rL, u0 < units);
    cw = codebook[threadIdx.x & 255];
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
    rot_pieces_pvq(rin, Gp, min(m0, M - 1), u0 - m0 * G, rL, u0 < units, xa, sx);
    for (int u = u0 + ustep; u < units; u += ustep) {
      const int m = (u >= G) + (u >= 2 * G) + (u >= 3 * G), g = u - m * G;
      rot_pieces_pvq(rot_load(xrs, srs, K, m, g, rL, true), Gp, m, g, rL, true, xa, sx);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = kEarly; d < DEPTH; ++d) {
      load(ring[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    cw = codebook[threadIdx.x & 255];
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      load(ring[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  {   // thread t writes copies [cpt (t >> 8), cpt (t >> 8) + cpt) of entry t & 255
    const int cpt = 256 * kLutCopies / nt, c0 = (static_cast<int>(threadIdx.x) >> 8) * cpt;
    uint32_t *dst = lut + (threadIdx.x & 255) * kLutCopies + c0;
    for (int c = 0; c < cpt; c += 4) *reinterpret_cast<uint4 *>(dst + c) = make_uint4(cw, cw, cw, cw);
  }
  {   // every set's zero piece, the row sums
    for (int i = static_cast<int>(threadIdx.x); i < M * G * (kPieceBytes / 16); i += nt) {
      const int q = i / (kPieceBytes / 16);
      reinterpret_cast<uint4 *>(xa + q * (kSetBytes / 4) + piece_offset(3) / 4)[i - q * (kPieceBytes / 16)] =
          make_uint4(0, 0, 0, 0);
    }
    for (int i = static_cast<int>(threadIdx.x); i < nw * M * vrows; i += nt) yl[i] = 0.f;
  }
  barrier_lds();   // the ring's index loads stay in flight

  // A operand source of this lane: row i = lane & 15 holds piece i & 3 of token
  // i >> 2; rows of tokens >= M read token 0's zero piece (any scale)
  const int ai = lane & 15, at = ai >> 2, ap = ai & 3;
  const uint32_t a_base = static_cast<uint32_t>(at < M ? at * Gp * kSetBytes + piece_offset(ap) : piece_offset(3)) +
                          kq * 32;
  const uint32_t *sxl = sx + min(at, M - 1) * Gp;   // A-scale exponents of this lane's token
  const char *lds = reinterpret_cast<const char *>(xa);   // a_base is a byte offset into the piece sets
  const bool t_ok = kq < M;
  float *ylane = yl + (wv * M + kq) * vrows + j;   // this wave's partial sums (one per tile it touches)

  v4f_t acc = {0.f, 0.f, 0.f, 0.f};
  auto process = [&](const uint4 &it) {
    const int g0 = pc.batch * kGB;
    // after the transpose, word e holds index bytes 4 (4 e + kq) .. + 3 of the
    // row's 64: words 0, 1 of the first group, 2, 3 of the second
    uint32_t w[4] = {it.x, it.y, it.z, it.w};
    transpose4(w[0], w[1], w[2], w[3]);
#pragma unroll
    for (int u = 0; u < kGB; ++u) {
      v8i_t bv;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          bv[4 * h + i] = static_cast<int>(lut[(((w[2 * u + h] >> (8 * i)) & 0xFFu) * kLutCopies) | lcopy]);
      const uint4 *ap4 = reinterpret_cast<const uint4 *>(lds + a_base + (g0 + u) * kSetBytes);
      const uint4 x0 = ap4[0], x1 = ap4[1];
      const v8i_t av = {static_cast<int>(x0.x), static_cast<int>(x0.y), static_cast<int>(x0.z),
                        static_cast<int>(x0.w), static_cast<int>(x1.x), static_cast<int>(x1.y),
                        static_cast<int>(x1.z), static_cast<int>(x1.w)};
      const int sa = static_cast<int>(sxl[g0 + u]);
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, sa, 0, 127);
    }
    // row tile done (the next item starts another tile, or this was the wave's last): add into LDS
    const int tile = pc.tile;
    pc.advance(sh, nw);
    if (pc.i >= items || pc.tile != tile) {
      if (t_ok) ylane[tile * 16] = acc[0] + acc[1] + acc[2];
      acc = v4f_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  // ring slot d holds items d, d + DEPTH, ... of the wave's sequence; every slot
  // is refilled on every pass (also past the wave's last item) so the loads stay
  // unconditional and the compiler keeps exact wait counts
  for (int i = wv; i < items; i += DEPTH * nw) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      if (d == 0 || i + d * nw < items) process(ring[d]);
      load(ring[d]);
    }
  }
  __syncthreads();
  // the waves' partials summed in wave order, times each stage's row scale,
  // stages added in order
  for (int i2 = static_cast<int>(threadIdx.x); i2 < M * rows; i2 += nt) {
    const int m = i2 / rows, r = i2 - m * rows, row = (b + (r >> 4) * sh.grid) * 16 + (r & 15);
    if (row >= N) continue;
    float out = 0.f;
    for (int st = 0; st < stages; ++st) {
      float s = 0.f;
      for (int w2 = 0; w2 < nw; ++w2) s += yl[(w2 * M + m) * vrows + st * rows + r];
      out += s * f16_bits_to_f32(row_scale[static_cast<size_t>(st) * N + row]);
    }
    y[static_cast<size_t>(m) * N + row] = f32_to_f16_bits(out);
  }
}

size_t pvq_mx_lds(int M, int G, int rows, int block, int stages) {
  return 1024 * kLutCopies + static_cast<size_t>(M) * G * (kSetBytes + 4) +
         static_cast<size_t>(block / 64) * M * stages * rows * 4;
}

constexpr int kComputeUnits = 256;
constexpr size_t kMaxLds = 160 * 1024;

int pvq_mx_grid(int N) {
  const int T = (N + 15) / 16;
  return T < kComputeUnits ? T : kComputeUnits;
}
// one workgroup per compute unit: eight waves for up to one tile each, sixteen
// beyond (the matrix-core RTN GEMV's measured choice on the same tile counts)
int pvq_mx_block(int N) { return (N + 15) / 16 <= kComputeUnits ? 512 : kPvqMaxThreads; }

}  // namespace

bool gemv_pvq_mx_supported(int M, int K, int N, int stages) {
  // K a multiple of 512: whole items of two groups, no padding groups
  if (M < 1 || M > 4 || K < 4 * kGroup || K % (4 * kGroup) != 0 || N < 1 || stages < 1 || stages > 3) return false;
  if (static_cast<long long>(stages) * (N + 16) * (K / kGroup) * 32 >= static_cast<long long>(kOutOfRange))
    return false;
  const int grid = pvq_mx_grid(N), T = (N + 15) / 16;
  return pvq_mx_lds(M, K / kGroup, ((T + grid - 1) / grid) * 16, pvq_mx_block(N), stages) <= kMaxLds;
}

hipError_t launch_gemv_pvq_mx(const uint8_t *idx, const uint16_t *row_scale, const uint8_t *codebook,
                              const uint16_t *x, const int8_t *signs, uint16_t *y, int M, int K, int N, int stages,
                              hipStream_t s) {
  if ((reinterpret_cast<uintptr_t>(signs) & 15u) != 0 || (reinterpret_cast<uintptr_t>(x) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(codebook) & 3u) != 0 || !gemv_pvq_mx_supported(M, K, N, stages))
    return hipErrorInvalidValue;
  const int grid = pvq_mx_grid(N);
  const int block = pvq_mx_block(N);
  const MxShape sh = make_shape(M, K, N, 2, grid, block);   // batches of two groups
  const size_t lds = pvq_mx_lds(M, sh.G, (sh.tq + (sh.tr ? 1 : 0)) * 16, block, stages);
  auto kern = stages == 1 ? gemv_pvq_mx_kernel<2, 1> : stages == 2 ? gemv_pvq_mx_kernel<2, 2> : gemv_pvq_mx_kernel<2, 3>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(block), lds, s, reinterpret_cast<const uint4 *>(idx), row_scale,
                     reinterpret_cast<const uint32_t *>(codebook), reinterpret_cast<const uint4 *>(x),
                     reinterpret_cast<const uint4 *>(signs), y, sh);
  return hipGetLastError();
}

}  // namespace lbq
