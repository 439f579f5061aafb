// Offline weight packing on the host: rotation, group-128 RTN or product-VQ
// encode, bit-plane scatter. Plain C++ (no HIP): float64 arithmetic, one
// thread per slice of rows.
//
// Steps follow the packed formats documented in include/lbq.h:
//   rotation per 128-block: signs, radix-2 butterflies (half-widths 1..64,
//   (a, b) -> (a + b, a - b)), then c = sqrt(2)/16 (LLaDA2.2-mini Orin Nano
//   model card: weights quantized in a Hadamard-rotated basis, rotation signs
//   stored; Pingala-8 model card, "What this is": random Hadamard rotation);
//   group-128 asymmetric codes with fp16 scale and zero (LLaDA2.2-mini card,
//   "Routed Experts" row);
//   bit-planes in 32-bit words (Qwen3-8B BPDQ model card, opening paragraph);
//   product-VQ over fp8-grid codebook values (Laguna-S-2.1 gridbook card,
//   opening paragraph).
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "../../include/lbq.h"
#include "pack_host.h"

namespace {

constexpr int kGroup = 128;

inline double rotation_scale() { return std::sqrt(2.0) / 16.0; }

}  // namespace

namespace lbq {

// Rotate one row of K values in place, per 128-block.
void rotate_row(double *v, const int8_t *signs, int K) {
  const double c = rotation_scale();
  for (int b = 0; b < K; b += kGroup) {
    double *u = v + b;
    for (int i = 0; i < kGroup; ++i) u[i] *= static_cast<double>(signs[b + i]);
    for (int h = 1; h < kGroup; h <<= 1) {
      for (int i = 0; i < kGroup; i += 2 * h) {
        for (int j = i; j < i + h; ++j) {
          const double a = u[j], bb = u[j + h];
          u[j] = a + bb;
          u[j + h] = a - bb;
        }
      }
    }
    for (int i = 0; i < kGroup; ++i) u[i] *= c;
  }
}

}  // namespace lbq

namespace {

using lbq::rotate_row;

// Run fn(row_begin, row_end) over [0, N) on all hardware threads.
template <class F>
void parallel_rows(int N, F fn) {
  unsigned nt = std::max(1u, std::thread::hardware_concurrency());
  nt = std::min<unsigned>(nt, 64u);
  if (N < 64) nt = 1;
  if (nt <= 1) {
    fn(0, N);
    return;
  }
  std::vector<std::thread> th;
  const int chunk = (N + static_cast<int>(nt) - 1) / static_cast<int>(nt);
  for (unsigned t = 0; t < nt; ++t) {
    const int r0 = static_cast<int>(t) * chunk;
    const int r1 = std::min(N, r0 + chunk);
    if (r0 >= r1) break;
    th.emplace_back(fn, r0, r1);
  }
  for (auto &t : th) t.join();
}

}  // namespace

namespace lbq {

uint16_t f64_to_f16_rne(double x) {
  uint64_t b;
  std::memcpy(&b, &x, 8);
  const uint16_t sign = static_cast<uint16_t>((b >> 48) & 0x8000u);
  const int exp = static_cast<int>((b >> 52) & 0x7FF);
  const uint64_t mant = b & 0xFFFFFFFFFFFFFull;
  if (exp == 0x7FF) return sign | 0x7C00u | (mant ? 0x200u : 0u);
  if (exp == 0) return sign;  // |x| < 2^-1022 rounds to zero
  int e = exp - 1023;
  const uint64_t sig = mant | (1ull << 52);  // |x| = sig * 2^(e - 52)
  if (e >= 16) return sign | 0x7C00u;
  const bool normal = e >= -14;
  const int shift = normal ? 42 : 42 + (-14 - e);
  if (shift > 63) return sign;
  uint64_t q = sig >> shift;
  const uint64_t rem = sig & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  uint32_t h;
  if (normal) {
    if (q == 2048) {
      q = 1024;
      ++e;
    }
    if (e >= 16) return sign | 0x7C00u;
    h = (static_cast<uint32_t>(e + 15) << 10) | static_cast<uint32_t>(q - 1024);
  } else {
    h = static_cast<uint32_t>(q);  // q == 1024 encodes the smallest normal
  }
  return static_cast<uint16_t>(sign | h);
}

double f16_to_f64(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 0x1F;
  const int m = h & 0x3FF;
  double v;
  if (e == 0) v = std::ldexp(static_cast<double>(m), -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp(1.0 + m / 1024.0, e - 15);
  return sign ? -v : v;
}

double e4m3_to_f64(uint8_t b) {
  const int sign = b >> 7;
  const int e = (b >> 3) & 0xF;
  const int m = b & 7;
  double v;
  if (e == 15 && m == 7) v = NAN;
  else if (e == 0) v = std::ldexp(m / 8.0, -6);
  else v = std::ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -v : v;
}

void store_group(const uint8_t q[128], int bits, uint16_t s16, uint16_t z16, uint32_t *planes, uint16_t *meta) {
  for (int p = 0; p < bits; ++p) {
    for (int w4 = 0; w4 < 4; ++w4) {
      uint32_t word = 0;
      for (int j = 0; j < 32; ++j) word |= static_cast<uint32_t>((q[32 * w4 + j] >> p) & 1u) << j;
      planes[p * 4 + w4] = word;
    }
  }
  meta[0] = s16;
  meta[1] = z16;
}

bool group_scale(const double *u, int stride, int bits, uint16_t &s16, double &s, double &z) {
  double mn = 0.0, mx = 0.0;
  for (int i = 0; i < kGroup; ++i) {
    const double v = u[static_cast<size_t>(i) * stride];
    if (v < mn) mn = v;
    if (v > mx) mx = v;
  }
  const double L = static_cast<double>((1 << bits) - 1);
  s16 = f64_to_f16_rne((mx - mn) / L);
  // the MFMA GEMM's fp16 decode constants (-64 s, -16 s z; -256 s and
  // -16 s z with z up to 255 at 8 bits) must stay finite: s < 128, at 8 bits s < 16
  if ((s16 & 0x7FFFu) >= (bits == 8 ? 0x4C00u : 0x5800u)) return false;
  if (s16 == 0) s16 = 0x3C00u;                     // degenerate group: scale 1
  s = f16_to_f64(s16);
  z = std::rint(-mn / s) + 0.0;
  return true;
}

lbq_status pack_rtn(const float *W, int K, int N, int bits, const int8_t *signs, uint32_t *planes,
                    uint16_t *meta) {
  const int G = K / kGroup;
  const double L = static_cast<double>((1 << bits) - 1);
  std::atomic<int> err{0};
  parallel_rows(N, [&](int r0, int r1) {
    std::vector<double> v(K);
    for (int n = r0; n < r1 && !err.load(std::memory_order_relaxed); ++n) {
      const float *w = W + static_cast<size_t>(n) * K;
      for (int k = 0; k < K; ++k) {
        if (!std::isfinite(w[k])) {
          err = LBQ_ERR_RANGE;
          return;
        }
        v[k] = static_cast<double>(w[k]);
      }
      rotate_row(v.data(), signs, K);
      for (int g = 0; g < G; ++g) {
        const double *u = v.data() + g * kGroup;
        uint16_t s16;
        double s, z;
        // the GEMM's decode needs finite -64 s and -16 s z in fp16: s < 128
        if (!group_scale(u, 1, bits, s16, s, z)) {
          err = LBQ_ERR_RANGE;
          return;
        }
        uint8_t q[kGroup];
        for (int i = 0; i < kGroup; ++i) {
          double c = std::rint(u[i] / s) + z;
          c = std::min(std::max(c, 0.0), L);
          q[i] = static_cast<uint8_t>(c);
        }
        store_group(q, bits, s16, f64_to_f16_rne(z), planes + (static_cast<size_t>(n) * G + g) * bits * 4,
                    meta + (static_cast<size_t>(n) * G + g) * 2);
      }
    }
  });
  return static_cast<lbq_status>(err.load());
}

lbq_status pack_pvq(const float *W, int K, int N, const int8_t *signs, const uint8_t *codebook,
                    uint8_t *idx, uint16_t *scale, int stages) {
  double cb[256][4];
  double sum_c = 0.0;
  for (int j = 0; j < 256; ++j) {
    for (int d = 0; d < 4; ++d) {
      cb[j][d] = e4m3_to_f64(codebook[4 * j + d]);
      if (!std::isfinite(cb[j][d])) return LBQ_ERR_RANGE;
      sum_c += cb[j][d] * cb[j][d];
    }
  }
  if (!(sum_c > 0.0)) return LBQ_ERR_RANGE;
  std::atomic<int> err{0};
  parallel_rows(N, [&](int r0, int r1) {
    std::vector<double> v(K);
    for (int n = r0; n < r1 && !err.load(std::memory_order_relaxed); ++n) {
      const float *w = W + static_cast<size_t>(n) * K;
      for (int k = 0; k < K; ++k) {
        if (!std::isfinite(w[k])) {
          err = LBQ_ERR_RANGE;
          return;
        }
        v[k] = static_cast<double>(w[k]);
      }
      rotate_row(v.data(), signs, K);
      // stage t encodes what stages 0..t-1 left in v (residual product-VQ)
      for (int t = 0; t < stages; ++t) {
      double sum_w = 0.0;
      for (int k = 0; k < K; ++k) sum_w += v[k] * v[k];
      const double ratio = std::sqrt(sum_w / K) / std::sqrt(sum_c / 1024.0);
      uint16_t s16 = f64_to_f16_rne(ratio);
      if ((s16 & 0x7FFFu) == 0x7C00u) {
        err = LBQ_ERR_RANGE;
        return;
      }
      if (s16 == 0) s16 = 0x3C00u;
      scale[static_cast<size_t>(t) * N + n] = s16;
      const double s = f16_to_f64(s16);
      uint8_t *out = idx + (static_cast<size_t>(t) * N + n) * (K / 4);
      for (int i = 0; i < K / 4; ++i) {
        const double a0 = v[4 * i] / s, a1 = v[4 * i + 1] / s, a2 = v[4 * i + 2] / s, a3 = v[4 * i + 3] / s;
        double best = INFINITY;
        int bj = 0;
        for (int j = 0; j < 256; ++j) {
          const double d0 = (a0 - cb[j][0]) * (a0 - cb[j][0]);
          const double d1 = (a1 - cb[j][1]) * (a1 - cb[j][1]);
          const double d2 = (a2 - cb[j][2]) * (a2 - cb[j][2]);
          const double d3 = (a3 - cb[j][3]) * (a3 - cb[j][3]);
          const double dist = ((d0 + d1) + d2) + d3;
          if (dist < best) {
            best = dist;
            bj = j;
          }
        }
        out[i] = static_cast<uint8_t>(bj);
        for (int d = 0; d < 4; ++d) v[4 * i + d] -= cb[bj][d] * s;
      }
      }
    }
  });
  return static_cast<lbq_status>(err.load());
}

lbq_status split_nibbles(const uint32_t *planes8, const uint16_t *meta8, int K, int N, uint32_t *hi, uint32_t *lo,
                         uint16_t *hi_meta) {
  const size_t groups = static_cast<size_t>(N) * (K / 128);
  for (size_t i = 0; i < groups; ++i) {
    // planes 0..3 of a group are the low nibble's bits, planes 4..7 the high one's
    std::memcpy(lo + i * 16, planes8 + i * 32, 64);
    std::memcpy(hi + i * 16, planes8 + i * 32 + 16, 64);
    const double s = f16_to_f64(meta8[2 * i]), z = f16_to_f64(meta8[2 * i + 1]);
    const double sh = 16.0 * s, zh = (z - 7.5) / 16.0;
    const uint16_t a = f64_to_f16_rne(sh), b = f64_to_f16_rne(zh);
    if (!std::isfinite(sh) || !std::isfinite(zh) || f16_to_f64(a) != sh || f16_to_f64(b) != zh) return LBQ_ERR_RANGE;
    hi_meta[2 * i] = a;
    hi_meta[2 * i + 1] = b;
  }
  return LBQ_OK;
}

}  // namespace lbq
