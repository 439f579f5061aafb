// GPTQ packing on the host: group-128 codes in the Hadamard-rotated basis
// with error feedback through the inverse Hessian (LLaDA2.2-mini Orin Nano
// model card, property table, "Routed Experts" row: group-128 GPTQ in a
// Hadamard-rotated basis; Qwen3.8-27B Pingala-8 model card, "What this is":
// LDLQ rounding behind a random Hadamard rotation, the same feedback). The
// packed format is the RTN one; only the code choice differs.
//
// Two steps:
//  1. gptq_factor: H' = R H R^T (the rotation applied to the rows, then to the
//     columns), plus damp * mean(diag H') on the diagonal; then U, the upper
//     Cholesky factor of H'^-1 (H'^-1 = U^T U). With H' = V V^T, V upper
//     triangular (a Cholesky factorisation taken from the last column back),
//     H'^-1 = V^-T V^-1, so U = V^-1.
//  2. pack_gptq: per row (rows are independent given U), column by column:
//     at a group's first column its scale and zero come from the columns as
//     they stand (the RTN range rule), the code q rounds w_j / s, and the
//     rounding error e = (w_j - (q - z) s) / U[j][j] is taken off every later
//     column, w_k -= e U[j][k], one column at a time.
// Float64 throughout, built without contraction of multiply-adds, so the
// second step repeats a plain column-by-column evaluation bit for bit.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <thread>
#include <vector>

#include "../../include/lbq.h"
#include "pack_host.h"

namespace {

constexpr int kGroup = 128;

unsigned n_threads() { return std::min(64u, std::max(1u, std::thread::hardware_concurrency())); }

// fn(i0, i1) over [0, n) on the host threads (serially when n is small)
template <class F>
void parallel_range(int n, int min_per_thread, F fn) {
  const unsigned nt = std::min<unsigned>(n_threads(), std::max(1, n / std::max(1, min_per_thread)));
  if (nt <= 1) {
    fn(0, n);
    return;
  }
  std::vector<std::thread> th;
  const int chunk = (n + static_cast<int>(nt) - 1) / static_cast<int>(nt);
  for (unsigned t = 0; t < nt; ++t) {
    const int a = static_cast<int>(t) * chunk, b = std::min(n, a + chunk);
    if (a >= b) break;
    th.emplace_back(fn, a, b);
  }
  for (auto &t : th) t.join();
}

// sum_i a[i] b[i] over n terms, four interleaved partial sums
inline double dot(const double *a, const double *b, int n) {
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  int i = 0;
  for (; i + 4 <= n; i += 4) {
    s0 += a[i] * b[i];
    s1 += a[i + 1] * b[i + 1];
    s2 += a[i + 2] * b[i + 2];
    s3 += a[i + 3] * b[i + 3];
  }
  for (; i < n; ++i) s0 += a[i] * b[i];
  return (s0 + s1) + (s2 + s3);
}

}  // namespace

namespace lbq {

lbq_status gptq_factor(const double *H, int K, const int8_t *signs, double damp, double *U) {
  const size_t KK = static_cast<size_t>(K) * K;
  std::vector<double> a(H, H + KK);
  for (size_t i = 0; i < KK; ++i)
    if (!std::isfinite(a[i])) return LBQ_ERR_RANGE;
  // rows: H R^T; transpose; rows again: R H R^T (H' is symmetric)
  parallel_range(K, 64, [&](int r0, int r1) {
    for (int r = r0; r < r1; ++r) rotate_row(a.data() + static_cast<size_t>(r) * K, signs, K);
  });
  std::vector<double> b(KK);
  for (int i = 0; i < K; ++i)
    for (int j = 0; j < K; ++j) b[static_cast<size_t>(j) * K + i] = a[static_cast<size_t>(i) * K + j];
  parallel_range(K, 64, [&](int r0, int r1) {
    for (int r = r0; r < r1; ++r) rotate_row(b.data() + static_cast<size_t>(r) * K, signs, K);
  });
  double tr = 0.0;
  for (int i = 0; i < K; ++i) tr += b[static_cast<size_t>(i) * K + i];
  const double d = damp * (tr / K);
  if (!(d > 0.0) || !std::isfinite(d)) return LBQ_ERR_RANGE;
  for (int i = 0; i < K; ++i) b[static_cast<size_t>(i) * K + i] += d;
  // H' = V V^T, V upper triangular: column j from the last back,
  //   V[j][j] = sqrt(H'[j][j] - sum_{k>j} V[j][k]^2),
  //   V[i][j] = (H'[i][j] - sum_{k>j} V[i][k] V[j][k]) / V[j][j]  (i < j).
  // V is kept in a (row i holds V[i][*]); only the upper triangle is written.
  std::fill(a.begin(), a.end(), 0.0);
  for (int j = K - 1; j >= 0; --j) {
    double *vj = a.data() + static_cast<size_t>(j) * K;
    const double djj = b[static_cast<size_t>(j) * K + j] - dot(vj + j + 1, vj + j + 1, K - 1 - j);
    if (!(djj > 0.0)) return LBQ_ERR_RANGE;
    const double vjj = std::sqrt(djj);
    vj[j] = vjj;
    parallel_range(j, 256, [&](int i0, int i1) {
      for (int i = i0; i < i1; ++i) {
        double *vi = a.data() + static_cast<size_t>(i) * K;
        vi[j] = (b[static_cast<size_t>(i) * K + j] - dot(vi + j + 1, vj + j + 1, K - 1 - j)) / vjj;
      }
    });
  }
  // U = V^-1 (upper triangular), one column c at a time: U[c][c] = 1 / V[c][c],
  // U[i][c] = -(sum_{k=i+1..c} V[i][k] U[k][c]) / V[i][i] for i < c. Column c
  // is built in ut (row c of U^T) so every sum runs over contiguous memory.
  std::vector<double> ut(KK, 0.0);
  parallel_range(K, 16, [&](int c0, int c1) {
    for (int c = c0; c < c1; ++c) {
      double *col = ut.data() + static_cast<size_t>(c) * K;
      col[c] = 1.0 / a[static_cast<size_t>(c) * K + c];
      for (int i = c - 1; i >= 0; --i) {
        const double *vi = a.data() + static_cast<size_t>(i) * K;
        col[i] = -dot(vi + i + 1, col + i + 1, c - i) / vi[i];
      }
    }
  });
  for (int i = 0; i < K; ++i)
    for (int c = 0; c < K; ++c) U[static_cast<size_t>(i) * K + c] = c >= i ? ut[static_cast<size_t>(c) * K + i] : 0.0;
  return LBQ_OK;
}

lbq_status pack_gptq(const float *W, int K, int N, int bits, const int8_t *signs, const double *U,
                     uint32_t *planes, uint16_t *meta) {
  const int G = K / kGroup;
  const double L = static_cast<double>((1 << bits) - 1);
  for (int j = 0; j < K; ++j)
    if (!(U[static_cast<size_t>(j) * K + j] > 0.0) || !std::isfinite(U[static_cast<size_t>(j) * K + j]))
      return LBQ_ERR_RANGE;
  constexpr int RB = 16;   // rows per block: each row of U is read once per block
  const int n_blocks = (N + RB - 1) / RB;
  std::atomic<int> err{0};
  std::atomic<int> next{0};
  const unsigned nt = std::min<unsigned>(n_threads(), static_cast<unsigned>(n_blocks));
  auto worker = [&]() {
    std::vector<double> w(static_cast<size_t>(RB) * K);
    std::vector<uint8_t> q(static_cast<size_t>(RB) * K);
    double s[RB], z[RB], e[RB];
    std::vector<uint16_t> sg(static_cast<size_t>(RB) * G), zg(static_cast<size_t>(RB) * G);
    for (int blk = next++; blk < n_blocks && !err.load(std::memory_order_relaxed); blk = next++) {
      const int r0 = blk * RB, nr = std::min(RB, N - r0);
      for (int r = 0; r < nr; ++r) {
        const float *src = W + static_cast<size_t>(r0 + r) * K;
        double *dst = w.data() + static_cast<size_t>(r) * K;
        for (int k = 0; k < K; ++k) {
          if (!std::isfinite(src[k])) {
            err = LBQ_ERR_RANGE;
            return;
          }
          dst[k] = static_cast<double>(src[k]);
        }
        rotate_row(dst, signs, K);
      }
      for (int j = 0; j < K; ++j) {
        const int g = j / kGroup;
        if (j % kGroup == 0) {
          for (int r = 0; r < nr; ++r) {
            uint16_t sb;
            if (!group_scale(w.data() + static_cast<size_t>(r) * K + j, 1, bits, sb, s[r], z[r])) {
              err = LBQ_ERR_RANGE;
              return;
            }
            sg[static_cast<size_t>(r) * G + g] = sb;
            zg[static_cast<size_t>(r) * G + g] = f64_to_f16_rne(z[r]);
          }
        }
        const double *uj = U + static_cast<size_t>(j) * K;
        const double ujj = uj[j];
        for (int r = 0; r < nr; ++r) {
          const double wj = w[static_cast<size_t>(r) * K + j];
          double c = std::rint(wj / s[r]) + z[r];
          c = std::min(std::max(c, 0.0), L);
          q[static_cast<size_t>(r) * K + j] = static_cast<uint8_t>(c);
          e[r] = (wj - (c - z[r]) * s[r]) / ujj;
        }
        for (int r = 0; r < nr; ++r) {
          double *wr = w.data() + static_cast<size_t>(r) * K;
          const double er = e[r];
          for (int k = j + 1; k < K; ++k) wr[k] -= er * uj[k];
        }
      }
      for (int r = 0; r < nr; ++r)
        for (int g = 0; g < G; ++g) {
          const size_t row = static_cast<size_t>(r0 + r);
          store_group(q.data() + static_cast<size_t>(r) * K + g * kGroup, bits, sg[static_cast<size_t>(r) * G + g],
                      zg[static_cast<size_t>(r) * G + g], planes + (row * G + g) * bits * 4, meta + (row * G + g) * 2);
        }
    }
  };
  std::vector<std::thread> th;
  for (unsigned t = 1; t < nt; ++t) th.emplace_back(worker);
  worker();
  for (auto &t : th) t.join();
  return static_cast<lbq_status>(err.load());
}

}  // namespace lbq
