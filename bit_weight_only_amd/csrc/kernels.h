// Internal launchers (host functions in the .hip files) used by the C ABI.
// Each returns the HIP error of its launch(es); shapes are validated by the
// caller before any of these runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lbq {

hipError_t launch_rotate(const uint16_t *x, int M, int K, const int8_t *signs, uint16_t *out, hipStream_t s);
// Rotation into the folded slot order (u32 slot c of each 32-chunk holds
// (x'[c], x'[c+16])); with tz non-null also the RTN GEMM's per-(token, group)
// sums tz[m * gemm_tz_stride(K) + g] = (T/16 high, T/16 low) fp16, zero-padded;
// also zeroes n_counters u32 at counters.
hipError_t launch_rotate_folded(const uint16_t *x, int M, int K, const int8_t *signs, uint16_t *out, uint32_t *tz,
                                uint32_t *counters, int n_counters, hipStream_t s);

// RTN dequant-GEMV for 1 <= M <= 16 on already-rotated activations xr [M][K].
hipError_t launch_gemv_rtn(const void *planes, const void *meta, const uint16_t *xr, uint16_t *y, int M, int K,
                           int N, int bits, hipStream_t s);

// RTN dequant-GEMV on raw activations x [M][K] (M = 1 or 2) with the rotation
// in the kernel's prologue: one launch, no workspace. signs must be 16-byte
// aligned. gemv_fold_supported says where this path is the faster one;
// lanes <= 0 picks the launch shape (gemv_fold_shape). Non-null events take
// the kernel's own begin / end times (hipExtLaunchKernel).
bool gemv_fold_supported(int M, int K);
void gemv_fold_shape(int M, int K, int N, int &lanes, int &rb, int &grid_cap);
hipError_t launch_gemv_fold(const void *planes, const void *meta, const uint16_t *x, const int8_t *signs, uint16_t *y,
                            int M, int K, int N, int bits, int lanes, int rb, int grid_cap, hipStream_t s,
                            hipEvent_t start = nullptr, hipEvent_t stop = nullptr);

// RTN dequant-GEMV on raw activations x [M][K] (1 <= M <= 4) on the matrix
// cores (fp8 activation pieces x fp4 code operands), rotation fused into the
// prologue: one launch, no workspace. x and signs must be 16-byte aligned.
// grid / block / depth <= 0 take gemv_mfma_shape's choice; non-null events
// take the kernel's own begin / end times.
bool gemv_mfma_supported(int M, int K, int N);
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
bool gemv_pvq_mx_supported(int M, int K, int N);
hipError_t launch_gemv_pvq_mx(const uint8_t *idx, const uint16_t *row_scale, const uint8_t *codebook,
                              const uint16_t *x, const int8_t *signs, uint16_t *y, int M, int K, int N,
                              hipStream_t s);
// MFMA dequant-GEMMs on activations rotated into the folded slot order
// (launch_rotate_folded): RTN planes (gemm_rtn_plan, launch_gemm_rtn, with the
// rotation's tz sums) and product-VQ (gemm_plan, launch_gemm_pvq). A plan fixes
// the tiling (nb row blocks of 16 per wave, mt token tiles of 16) and the
// split-K count; split-K needs gemm_scratch_bytes(plan) of scratch whose
// arrival counters (gemm_counter_ptr, gemm_counters of them) are zero when the
// GEMM starts.
struct GemmPlan {
  int nb, mt, S, n_tiles, m_tiles;
};
GemmPlan gemm_plan(int M, int K, int N);
GemmPlan gemm_rtn_plan(int M, int K, int N);
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
hipError_t launch_gemm_pvq(const GemmPlan &p, const void *idx, const void *row_scale, const uint8_t *codebook,
                           const uint16_t *xf, uint16_t *y, int M, int K, int N, void *scratch, hipStream_t s);

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
  const uint16_t *xr;        // [M][hidden] rotated tokens (VALU expert kernels)
  float *h;                  // [M*top_k][2*ffn] gate|up results (matrix-core expert kernels)
  const int32_t *offsets;    // [E+1]
  const int32_t *perm;       // [M*top_k]
  const float *weights;      // [M][top_k]
  uint16_t *act;             // [M*top_k][ffn] SwiGLU output by assignment index (rotated for the VALU kernels)
  float *out;                // [M*top_k][hidden] expert outputs, by assignment index
  uint16_t *y;               // [M][hidden]
};
// Rotation (VALU path), expert linears and the weighted combine.
hipError_t launch_moe_experts(const MoeArgs &a, hipStream_t s);
// Expert linears on the matrix cores (gate|up, SwiGLU, down; rotations fused).
bool moe_mx_supported(int hidden, int ffn, const int8_t *signs_hidden, const int8_t *signs_ffn);
hipError_t launch_moe_mx(const MoeArgs &a, hipStream_t s);
// Dynamic LDS the expert kernels need (must stay within 64 KB).
size_t moe_gateup_lds(int hidden);
size_t moe_down_lds(int ffn);
constexpr int kMoeMaxExperts = 1024;
constexpr int kMoeMaxAssignments = 8192;
constexpr int kMoeMaxTopK = 32;

}  // namespace lbq
