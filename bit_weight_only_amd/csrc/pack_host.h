// Host-side packing routines (pack.cpp) used by the C ABI in api.hip.
#pragma once
#include <stdint.h>

#include "../../include/lbq.h"

namespace lbq {

uint16_t f64_to_f16_rne(double x);
double f16_to_f64(uint16_t h);
double e4m3_to_f64(uint8_t b);

// RTN bit-plane packing of W [N][K] (fp32, host) into planes [N][K/128][bits][4]
// and meta [N][K/128][2] fp16 bit patterns (scale, zero).
lbq_status pack_rtn(const float *W, int K, int N, int bits, const int8_t *signs, uint32_t *planes,
                    uint16_t *meta);

// Product-VQ packing of W [N][K] into idx [N][K/4] and fp16 row scales [N].
lbq_status pack_pvq(const float *W, int K, int N, const int8_t *signs, const uint8_t *codebook,
                    uint8_t *idx, uint16_t *scale);

}  // namespace lbq
