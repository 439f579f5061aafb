// Internal launchers (host functions in the .hip files) used by the C ABI.
// Each returns the HIP error of its launch(es); shapes are validated by the
// caller before any of these runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lbq {

hipError_t launch_rotate(const uint16_t *x, int M, int K, const int8_t *signs, uint16_t *out, hipStream_t s);
// the same, clearing n_counters u32 counters first (the PVQ GEMM's split-K arrivals)
hipError_t launch_rotate_clear(const uint16_t *x, int M, int K, const int8_t *signs, uint16_t *out,
                               uint32_t *counters, int n_counters, hipStream_t s);

// Screened readout (readout.hip): the survivors' selection by coarse logit
// (keys: readout_key_bytes of scratch; *final_keys receives the [M][cand]
// sorted survivors inside it; the first launch also writes xr = R x, fp16
// [M][K]) and their exact logits from the nibble planes.
size_t readout_key_bytes(int M, int N, int cand);
hipError_t launch_readout_select(const uint16_t *coarse, int M, int N, int cand, uint64_t *keys,
                                 const uint64_t **final_keys, const uint16_t *x, const int8_t *signs, uint16_t *xr,
                                 int K, hipStream_t s);
hipError_t launch_readout_refine(const uint64_t *keys, const void *hi, const void *lo, const void *meta,
                                 const uint16_t *xr, int M, int K, int N, int cand, int32_t *ids, float *logits,
                                 hipStream_t s);
// Rotation into the folded slot order (u32 slot c of each 32-chunk holds
// (x'[c], x'[c+16])); with tz non-null also the RTN GEMM's per-(token, group)
// sums tz[m * gemm_tz_stride(K) + g] = (T/16 high, T/16 low) fp16, zero-padded;
// also zeroes n_counters u32 at counters. The tokens go in launches of under
// 1 GiB of activations, or of max_tokens tokens when max_tokens > 0 is lower.
hipError_t launch_rotate_folded(const uint16_t *x, int M, int K, const int8_t *signs, uint16_t *out, uint32_t *tz,
                                uint32_t *counters, int n_counters, hipStream_t s, int max_tokens = 0);

// The routed experts' SwiGLU intermediate, rotated into the folded order: row
// m of out is R (fp16(silu(h[m][0..K-1]) h[m][K..2K-1])), with the RTN GEMM's
// zero-point sums in tz (as launch_rotate_folded). h: fp32 [M][2K], M * 2K *
// 4 bytes below 2 GiB.
hipError_t launch_swiglu_rotate_folded(const float *h, int M, int K, const int8_t *signs, uint16_t *out,
                                       uint32_t *tz, hipStream_t s);

// RTN dequant-GEMV for 1 <= M <= 16 on already-rotated activations xr [M][K].
hipError_t launch_gemv_rtn(const void *planes, const void *meta, const uint16_t *xr, uint16_t *y, int M, int K,
                           int N, int bits, hipStream_t s);

// RTN dequant-GEMV on raw activations x [M][K] (1 <= M <= 4) on the matrix
// cores (fp8 activation pieces x fp4 code operands), rotation fused into the
// prologue: one launch, no workspace. x and signs must be 16-byte aligned.
// grid / block / depth <= 0 take gemv_mfma_shape's choice; non-null events
// take the kernel's own begin / end times.
bool gemv_mfma_supported(int M, int K, int N);
bool gemv_mfma_supported_8bit(int K, int N);   // the extra bound for 8-bit codes
// true when all M tokens' activation pieces fit in LDS at once (else the
// kernel runs the tokens in passes that each stream the codes again)
bool gemv_mfma_one_pass(int M, int K, int N, int bits);
void gemv_mfma_shape(int M, int K, int N, int bits, int &grid, int &block, int &depth);
hipError_t launch_gemv_mfma(const void *planes, const void *meta, const uint16_t *x, const int8_t *signs,
                            uint16_t *y, int M, int K, int N, int bits, int grid, int block, int depth,
                            hipStream_t s, hipEvent_t start = nullptr, hipEvent_t stop = nullptr);

// Product-VQ GEMV (M <= 16) on rotated activations.
hipError_t launch_gemv_pvq(const uint8_t *idx, const uint16_t *scale, const uint8_t *codebook, const uint16_t *xr,
                           uint16_t *y, int M, int K, int N, hipStream_t s);
// Product-VQ GEMV on raw activations x [M][K] (1 <= M <= 4) on the matrix
// cores (fp8 activation pieces x fp8 codebook values), rotation fused into the
// prologue: one launch, no workspace. x and signs 16-byte aligned, codebook
// 4-byte aligned.
// stages: residual product-VQ stages (idx [stages][N][K/4], row_scale [stages][N]).
bool gemv_pvq_mx_supported(int M, int K, int N, int stages);
hipError_t launch_gemv_pvq_mx(const uint8_t *idx, const uint16_t *row_scale, const uint8_t *codebook,
                              const uint16_t *x, const int8_t *signs, uint16_t *y, int M, int K, int N, int stages,
                              hipStream_t s);
// MFMA dequant-GEMMs: RTN planes on activations rotated into the folded slot
// order (launch_rotate_folded; gemm_rtn_plan, launch_gemm_rtn, with the
// rotation's tz sums) and product-VQ on activations in natural order
// (launch_rotate_clear; gemm_plan, launch_gemm_pvq). A plan fixes
// the tiling (nb row blocks of 16 per wave, mt token tiles of 16) and the
// split-K count; split-K needs gemm_scratch_bytes(plan) of scratch whose
// arrival counters (gemm_counter_ptr, gemm_counters of them) are zero when the
// GEMM starts.
struct GemmPlan {
  int nb, mt, S, n_tiles, m_tiles;
  int kw = 1;   // RTN GEMM: wave sets per workgroup (2: alternate groups, 512 threads)
};
GemmPlan gemm_plan(int M, int K, int N, int stages);
GemmPlan gemm_rtn_plan(int M, int K, int N, int bits);
// longest K slice (groups) whose scale/zero words the RTN GEMM stages in LDS,
// for nb row blocks per wave; launch_gemm_rtn rejects plans with longer slices
int gemm_rtn_meta_max_groups(int nb);
size_t gemm_scratch_bytes(const GemmPlan &p);
int gemm_counters(const GemmPlan &p);
uint32_t *gemm_counter_ptr(const GemmPlan &p, void *scratch);
int gemm_tz_stride(int K);
bool gemm_rtn_supported(int K, int N, int bits);
hipError_t launch_gemm_rtn(const GemmPlan &p, int bits, const void *planes, const void *meta, const uint16_t *xf,
                           const uint32_t *tz, uint16_t *y, int M, int K, int N, void *scratch, hipStream_t s);
// Grouped RTN GEMM over routed experts: for each tile descriptor (e, i0, cnt,
// bits) the rows of list entries i0 .. i0 + cnt - 1 (activation row of entry i:
// perm[i] / act_div, or i when act_div is 0) times expert e's weight (byte
// offsets plane_off[e] / meta_off[e] from planes / meta, width bits), fp32
// results to out[(out_perm ? perm[i] : i)][N]. Row tiles of 64 nb, token tiles
// of 16 mt entries (cnt <= 16 mt); grid over max_tiles descriptors, those past
// *n_tiles exit at once.
struct GroupedGemm {
  int nb, mt, max_tiles, K, N;
  const int32_t *tiles;      // [max_tiles] int4 descriptors
  const int32_t *n_tiles;
  const void *planes, *meta;
  const uint64_t *plane_off, *meta_off;
  const uint16_t *xf;        // folded rotated activations, rows of K
  const uint32_t *tz;        // zero-point sums, rows of gemm_tz_stride(K)
  const int32_t *perm;
  int act_div, out_perm;
  float *out;
};
hipError_t launch_gemm_rtn_grouped(const GroupedGemm &g, hipStream_t s);
// Matrix-core GEMM for 2-bit RTN codes at up to 16 tokens per token tile
// (fp4 codes x three e4m3 activation pieces): a rotation launch writes the
// pieces and scale bytes to act (gemm_mx_act_bytes(M, K) bytes), the
// zero-point sums to tz ([M][gemm_tz_stride(K)] u32) and clears the split-K
// counters in scratch, then the GEMM (a non-null `between` is recorded after
// the rotation launch).
bool gemm_mx_supported(int M, int K, int N, int bits);
GemmPlan gemm_mx_plan(int M, int K, int N);
size_t gemm_mx_act_bytes(int M, int K);
hipError_t launch_gemm_mx(const GemmPlan &p, const void *planes, const void *meta, const uint16_t *x,
                          const int8_t *signs, void *act, uint32_t *tz, uint16_t *y, int M, int K, int N,
                          void *scratch, hipStream_t s, hipEvent_t between = nullptr);
hipError_t launch_gemm_pvq(const GemmPlan &p, const void *idx, const void *row_scale, const uint8_t *codebook,
                           const uint16_t *xf, uint16_t *y, int M, int K, int N, int stages, void *scratch,
                           hipStream_t s);

// Measurement reference: read bytes (a multiple of 16) at buf once in one
// launch of grid x block threads; non-null events take the kernel's own
// begin / end times.
hipError_t launch_stream_read(const void *buf, size_t bytes, int grid, int block, uint32_t *sink, hipStream_t s,
                              hipEvent_t start, hipEvent_t stop);

hipError_t launch_unpack_rtn(const void *planes, int K, int N, int bits, uint8_t *codes, hipStream_t s);

// MoE pieces.
hipError_t launch_moe_route(const float *logits, int M, int E, int top_k, int32_t *ids, float *weights,
                            int32_t *counts, int32_t *offsets, int32_t *perm, hipStream_t s);

struct MoeArgs {
  int E, hidden, ffn, top_k, M;
  const uint8_t *bits;
  const uint64_t *gu_plane_off, *gu_meta_off, *dn_plane_off, *dn_meta_off;
  const uint8_t *planes, *meta;
  const int8_t *signs_hidden, *signs_ffn;
  const uint16_t *x;         // [M][hidden] tokens
  const uint16_t *xr;        // [M][hidden] rotated tokens (VALU expert kernels; folded for the grouped GEMMs)
  float *h;                  // [M*top_k][2*ffn] gate|up results (matrix-core expert kernels and grouped GEMMs)
  const int32_t *offsets;    // [E+1]
  const int32_t *perm;       // [M*top_k]
  const float *weights;      // [M][top_k]
  uint16_t *act;             // [M*top_k][ffn] SwiGLU output by assignment index (rotated for the VALU kernels)
  float *out;                // [M*top_k][hidden] expert outputs, by assignment index
  uint16_t *y;               // [M][hidden]
};
// Rotation (VALU path), expert linears and the weighted combine.
hipError_t launch_moe_experts(const MoeArgs &a, hipStream_t s);
// Many tokens per expert: the expert linears as grouped MFMA GEMMs over the
// expert-sorted assignment list (after the router): tile descriptors, the
// tokens rotated once (xr, folded, sums in tz_hidden), gate|up into h (fp32,
// list order), SwiGLU + ffn rotation into act (folded, sums in tz_ffn), down
// into out (by assignment index), the combine.
struct MoePrefill {
  int32_t *tiles;        // [moe_prefill_max_tiles] int4
  int32_t *n_tiles;
  uint32_t *tz_hidden;   // [M][gemm_tz_stride(hidden)]
  uint32_t *tz_ffn;      // [M * top_k][gemm_tz_stride(ffn)]
};
int moe_prefill_tile_tokens(int M, int E, int top_k);
int moe_prefill_max_tiles(int M, int E, int top_k);
bool moe_prefill_supported(int hidden, int ffn, long assignments);
hipError_t launch_moe_prefill(const MoeArgs &a, const MoePrefill &p, hipStream_t s);
// Expert linears on the matrix cores (gate|up, SwiGLU, down; rotations fused).
bool moe_mx_supported(int hidden, int ffn, const int8_t *signs_hidden, const int8_t *signs_ffn);
hipError_t launch_moe_mx(const MoeArgs &a, hipStream_t s);
// Dynamic LDS the expert kernels need (must stay within 64 KB).
size_t moe_gateup_lds(int hidden);
size_t moe_down_lds(int ffn);
constexpr int kMoeMaxExperts = 1024;
constexpr int kMoeMaxAssignments = 1 << 20;
constexpr int kMoeMaxTopK = 32;

}  // namespace lbq
