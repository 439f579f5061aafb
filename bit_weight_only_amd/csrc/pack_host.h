// Host-side packing routines (pack.cpp) used by the C ABI in api.hip.
#pragma once
#include <stdint.h>

#include "../../include/lbq.h"

namespace lbq {

uint16_t f64_to_f16_rne(double x);
double f16_to_f64(uint16_t h);
double e4m3_to_f64(uint8_t b);

// Rotation of one row of K values in place, per 128-block (signs, radix-2
// butterflies, sqrt(2)/16), float64.
void rotate_row(double *v, const int8_t *signs, int K);
// Scale and zero of one 128-group whose values sit at u[i * stride]: the
// zero-inclusive range rule, s as fp16 (degenerate 0 -> 1), z = rint(-mn / s).
// false when s >= 128 (the RTN GEMM's fp16 decode constants).
bool group_scale(const double *u, int stride, int bits, uint16_t &s16, double &s, double &z);
// Bit-planes of one group's 128 codes and its (s, z) fp16 pair.
void store_group(const uint8_t q[128], int bits, uint16_t s16, uint16_t z16, uint32_t *planes, uint16_t *meta);

// RTN bit-plane packing of W [N][K] (fp32, host) into planes [N][K/128][bits][4]
// and meta [N][K/128][2] fp16 bit patterns (scale, zero).
lbq_status pack_rtn(const float *W, int K, int N, int bits, const int8_t *signs, uint32_t *planes,
                    uint16_t *meta);

// Product-VQ packing of W [N][K] into idx [stages][N][K/4] and fp16 row
// scales [stages][N]: stage t encodes the residual the earlier stages left.
lbq_status pack_pvq(const float *W, int K, int N, const int8_t *signs, const uint8_t *codebook,
                    uint8_t *idx, uint16_t *scale, int stages);

// GPTQ: the upper Cholesky factor U of (R H R^T + damp mean(diag) I)^-1 of a
// host Hessian H [K][K] (original basis), and packing with error feedback
// through U (gptq.cpp).
lbq_status gptq_factor(const double *H, int K, const int8_t *signs, double damp, double *U);
lbq_status pack_gptq(const float *W, int K, int N, int bits, const int8_t *signs, const double *U,
                     uint32_t *planes, uint16_t *meta);

// Nibble split of 8-bit planes and meta: planes 4..7 / 0..3 of every group to
// hi / lo ([N][G][4][4] u32 each), and the high nibbles' (16 s, (z - 7.5) / 16).
lbq_status split_nibbles(const uint32_t *planes8, const uint16_t *meta8, int K, int N, uint32_t *hi, uint32_t *lo,
                         uint16_t *hi_meta);

}  // namespace lbq
