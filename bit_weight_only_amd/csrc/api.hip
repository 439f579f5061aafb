// The C ABI (include/lbq.h): argument checks, workspace layout, path choice,
// and kernel launches on the caller's stream. No allocation, no global state.
#include <hip/hip_runtime.h>

#include <cstring>

#include "../../include/lbq.h"
#include "kernels.h"
#include "pack_host.h"

using namespace lbq;

namespace {

constexpr size_t kAlign = 256;

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline lbq_status hip_status(hipError_t e) { return e == hipSuccess ? LBQ_OK : LBQ_ERR_HIP; }

lbq_status check_weight(const lbq_weight *w) {
  if (!w || !w->planes || !w->meta || !w->signs) return LBQ_ERR_NULL;
  if (w->format == LBQ_FMT_RTN_PLANES) {
    if (w->bits < 2 || w->bits > 4) return LBQ_ERR_BITS;
  } else if (w->format == LBQ_FMT_PVQ_4x8) {
    if (!w->codebook) return LBQ_ERR_NULL;
    if (w->bits != 2) return LBQ_ERR_BITS;
  } else {
    return LBQ_ERR_FORMAT;
  }
  if (w->K <= 0 || w->K % 128 != 0 || w->N <= 0) return LBQ_ERR_SHAPE;
  if (!aligned16(w->planes) || !aligned16(w->meta)) return LBQ_ERR_ALIGN;
  return LBQ_OK;
}

GemmPlan linear_gemm_plan(const lbq_weight *w, int M) {
  return w->format == LBQ_FMT_RTN_PLANES ? gemm_rtn_plan(M, w->K, w->N) : gemm_plan(M, w->K, w->N);
}

size_t tz_bytes(const lbq_weight *w, int M) {
  return w->format == LBQ_FMT_RTN_PLANES ? round_up(static_cast<size_t>(M) * gemm_tz_stride(w->K) * 4, kAlign) : 0;
}

size_t linear_ws_bytes(const lbq_weight *w, int M) {
  // the rotated activations, the RTN GEMM's per-(token, group) sums, then the
  // GEMM's split-K partial tiles and counters
  return round_up(static_cast<size_t>(M) * w->K * 2, kAlign) + tz_bytes(w, M) +
         gemm_scratch_bytes(linear_gemm_plan(w, M));
}

lbq_status forward_impl(const lbq_weight *w, const uint16_t *x, int32_t M, uint16_t *y, void *ws, size_t ws_bytes,
                        int32_t path, void *stream, hipEvent_t ev0, hipEvent_t ev1) {
  lbq_status st = check_weight(w);
  if (st != LBQ_OK) return st;
  if (M < 0) return LBQ_ERR_SHAPE;
  if (path < LBQ_PATH_AUTO || path > LBQ_PATH_GEMM) return LBQ_ERR_SHAPE;
  if (path == LBQ_PATH_GEMV && M > 16) return LBQ_ERR_SHAPE;
  if (M == 0) return LBQ_OK;
  if (!x || !y || !ws) return LBQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(ws)) return LBQ_ERR_ALIGN;
  if (ws_bytes < linear_ws_bytes(w, M)) return LBQ_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // up to four tokens share one matrix-core GEMV pass; from there on the MFMA GEMM
  const bool gemv = (path == LBQ_PATH_GEMV) || (path == LBQ_PATH_AUTO && M <= 4);
  // One to four tokens: rotation fused into the matrix-core decoder, one launch.
  if (w->format == LBQ_FMT_RTN_PLANES && gemv && gemv_mfma_supported(M, w->K, w->N) && aligned16(w->signs))
    return hip_status(launch_gemv_mfma(w->planes, w->meta, x, w->signs, y, M, w->K, w->N, w->bits, 0, 0, 0, s, ev0,
                                       ev1));
  if (w->format == LBQ_FMT_PVQ_4x8 && gemv && gemv_pvq_mx_supported(M, w->K, w->N) && aligned16(w->signs) &&
      (reinterpret_cast<uintptr_t>(w->codebook) & 3u) == 0) {
    if (ev0 && hipEventRecord(ev0, s) != hipSuccess) return LBQ_ERR_HIP;
    if (launch_gemv_pvq_mx(static_cast<const uint8_t *>(w->planes), static_cast<const uint16_t *>(w->meta),
                           static_cast<const uint8_t *>(w->codebook), x, w->signs, y, M, w->K, w->N, s) != hipSuccess)
      return LBQ_ERR_HIP;
    return (ev1 && hipEventRecord(ev1, s) != hipSuccess) ? LBQ_ERR_HIP : LBQ_OK;
  }
  uint16_t *xr = static_cast<uint16_t *>(ws);
  if (!gemv) {
    // MFMA GEMM: rotation into the folded order (with the RTN zero-point sums,
    // clearing the split-K counters), then the GEMM
    const bool rtn = w->format == LBQ_FMT_RTN_PLANES;
    if (rtn && !gemm_rtn_supported(w->K, w->N, w->bits)) return LBQ_ERR_SHAPE;
    const GemmPlan gp = linear_gemm_plan(w, M);
    uint8_t *after_x = static_cast<uint8_t *>(ws) + round_up(static_cast<size_t>(M) * w->K * 2, kAlign);
    uint32_t *tz = rtn ? reinterpret_cast<uint32_t *>(after_x) : nullptr;
    void *scratch = after_x + tz_bytes(w, M);
    if (launch_rotate_folded(x, M, w->K, w->signs, xr, tz, gemm_counter_ptr(gp, scratch), gemm_counters(gp), s) !=
        hipSuccess)
      return LBQ_ERR_HIP;
    if (ev0 && hipEventRecord(ev0, s) != hipSuccess) return LBQ_ERR_HIP;
    const hipError_t ge =
        rtn ? launch_gemm_rtn(gp, w->bits, w->planes, w->meta, xr, tz, y, M, w->K, w->N, scratch, s)
            : launch_gemm_pvq(gp, w->planes, w->meta, static_cast<const uint8_t *>(w->codebook), xr, y, M, w->K, w->N,
                              scratch, s);
    if (ge != hipSuccess) return LBQ_ERR_HIP;
    return (ev1 && hipEventRecord(ev1, s) != hipSuccess) ? LBQ_ERR_HIP : LBQ_OK;
  }
  hipError_t e = launch_rotate(x, M, w->K, w->signs, xr, s);
  if (e != hipSuccess) return LBQ_ERR_HIP;
  if (ev0 && hipEventRecord(ev0, s) != hipSuccess) return LBQ_ERR_HIP;
  if (w->format == LBQ_FMT_RTN_PLANES)
    e = launch_gemv_rtn(w->planes, w->meta, xr, y, M, w->K, w->N, w->bits, s);
  else
    e = launch_gemv_pvq(static_cast<const uint8_t *>(w->planes), static_cast<const uint16_t *>(w->meta),
                        static_cast<const uint8_t *>(w->codebook), xr, y, M, w->K, w->N, s);
  if (e != hipSuccess) return LBQ_ERR_HIP;
  return (ev1 && hipEventRecord(ev1, s) != hipSuccess) ? LBQ_ERR_HIP : LBQ_OK;
}

}  // namespace

extern "C" {

const char *lbq_status_string(lbq_status s) {
  switch (s) {
    case LBQ_OK: return "ok";
    case LBQ_ERR_NULL: return "required pointer is NULL";
    case LBQ_ERR_SHAPE: return "invalid shape";
    case LBQ_ERR_BITS: return "unsupported code width";
    case LBQ_ERR_ALIGN: return "pointer not 16-byte aligned";
    case LBQ_ERR_WORKSPACE: return "workspace too small";
    case LBQ_ERR_RANGE: return "value not representable in the packed format";
    case LBQ_ERR_HIP: return "HIP launch error";
    case LBQ_ERR_FORMAT: return "unknown or unsupported format";
  }
  return "unknown status";
}

lbq_status lbq_packed_bytes(int32_t K, int32_t N, int32_t bits, int32_t format, size_t *plane_bytes,
                            size_t *meta_bytes) {
  if (!plane_bytes || !meta_bytes) return LBQ_ERR_NULL;
  if (format == LBQ_FMT_RTN_PLANES) {
    if (bits < 2 || bits > 4) return LBQ_ERR_BITS;
  } else if (format == LBQ_FMT_PVQ_4x8) {
    if (bits != 2) return LBQ_ERR_BITS;
  } else {
    return LBQ_ERR_FORMAT;
  }
  if (K <= 0 || K % 128 != 0 || N <= 0) return LBQ_ERR_SHAPE;
  if (format == LBQ_FMT_RTN_PLANES) {
    *plane_bytes = static_cast<size_t>(N) * K / 8 * bits;
    *meta_bytes = static_cast<size_t>(N) * (K / 128) * 4;
  } else {
    *plane_bytes = static_cast<size_t>(N) * (K / 4);
    *meta_bytes = static_cast<size_t>(N) * 2;
  }
  return LBQ_OK;
}

lbq_status lbq_pack(const float *W, int32_t K, int32_t N, int32_t bits, int32_t format, const int8_t *signs,
                    const uint8_t *codebook, void *planes_out, void *meta_out) {
  if (!W || !signs || !planes_out || !meta_out) return LBQ_ERR_NULL;
  size_t pb, mb;
  lbq_status st = lbq_packed_bytes(K, N, bits, format, &pb, &mb);
  if (st != LBQ_OK) return st;
  for (int k = 0; k < K; ++k)
    if (signs[k] != 1 && signs[k] != -1) return LBQ_ERR_RANGE;
  if (format == LBQ_FMT_RTN_PLANES)
    return pack_rtn(W, K, N, bits, signs, static_cast<uint32_t *>(planes_out), static_cast<uint16_t *>(meta_out));
  if (!codebook) return LBQ_ERR_NULL;
  return pack_pvq(W, K, N, signs, codebook, static_cast<uint8_t *>(planes_out), static_cast<uint16_t *>(meta_out));
}

lbq_status lbq_linear_workspace(const lbq_weight *w, int32_t M, size_t *bytes) {
  if (!bytes) return LBQ_ERR_NULL;
  lbq_status st = check_weight(w);
  if (st != LBQ_OK) return st;
  if (M < 0) return LBQ_ERR_SHAPE;
  *bytes = linear_ws_bytes(w, M);
  return LBQ_OK;
}

lbq_status lbq_linear_forward_path(const lbq_weight *w, const uint16_t *x, int32_t M, uint16_t *y, void *ws,
                                   size_t ws_bytes, int32_t path, void *stream) {
  return forward_impl(w, x, M, y, ws, ws_bytes, path, stream, nullptr, nullptr);
}

lbq_status lbq_linear_forward_timed(const lbq_weight *w, const uint16_t *x, int32_t M, uint16_t *y, void *ws,
                                    size_t ws_bytes, void *stream, void *start_event, void *stop_event) {
  return forward_impl(w, x, M, y, ws, ws_bytes, LBQ_PATH_AUTO, stream, static_cast<hipEvent_t>(start_event),
                      static_cast<hipEvent_t>(stop_event));
}

lbq_status lbq_linear_forward(const lbq_weight *w, const uint16_t *x, int32_t M, uint16_t *y, void *ws,
                              size_t ws_bytes, void *stream) {
  return lbq_linear_forward_path(w, x, M, y, ws, ws_bytes, LBQ_PATH_AUTO, stream);
}

lbq_status lbq_unpack_codes(const lbq_weight *w, uint8_t *codes, void *stream) {
  lbq_status st = check_weight(w);
  if (st != LBQ_OK) return st;
  if (!codes) return LBQ_ERR_NULL;
  if (!aligned16(codes)) return LBQ_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (w->format == LBQ_FMT_RTN_PLANES)
    return hip_status(launch_unpack_rtn(w->planes, w->K, w->N, w->bits, codes, s));
  return hip_status(hipMemcpyAsync(codes, w->planes, static_cast<size_t>(w->N) * (w->K / 4),
                                   hipMemcpyDeviceToDevice, s));
}

lbq_status lbq_rotate(const uint16_t *x, int32_t M, int32_t K, const int8_t *signs, uint16_t *out, void *stream) {
  if (M < 0 || K <= 0 || K % 128 != 0) return LBQ_ERR_SHAPE;
  if (M == 0) return LBQ_OK;
  if (!x || !signs || !out) return LBQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(out)) return LBQ_ERR_ALIGN;
  return hip_status(launch_rotate(x, M, K, signs, out, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------- MoE

namespace {

struct MoeLayout {
  size_t xr, ids, weights, counts, offsets, perm, act, out, h, total;
};

MoeLayout moe_layout(const lbq_moe *m, int M) {
  MoeLayout L{};
  const size_t mk = static_cast<size_t>(M) * m->top_k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes, kAlign);
    return at;
  };
  L.xr = take(static_cast<size_t>(M) * m->hidden * 2);
  L.ids = take(mk * 4);
  L.weights = take(mk * 4);
  L.counts = take(static_cast<size_t>(m->E) * 4);
  L.offsets = take(static_cast<size_t>(m->E + 1) * 4);
  L.perm = take(mk * 4);
  L.act = take(mk * m->ffn * 2);
  L.out = take(mk * m->hidden * 4);
  L.h = take(mk * m->ffn * 2 * 4);
  L.total = off;
  return L;
}

lbq_status check_moe(const lbq_moe *m, int M) {
  if (!m || !m->bits || !m->gu_plane_off || !m->gu_meta_off || !m->dn_plane_off || !m->dn_meta_off || !m->planes ||
      !m->meta || !m->signs_hidden || !m->signs_ffn)
    return LBQ_ERR_NULL;
  if (m->E <= 0 || m->E > kMoeMaxExperts) return LBQ_ERR_SHAPE;
  if (m->top_k < 1 || m->top_k > m->E || m->top_k > kMoeMaxTopK) return LBQ_ERR_SHAPE;
  if (m->hidden <= 0 || m->hidden % 128 || m->ffn <= 0 || m->ffn % 128) return LBQ_ERR_SHAPE;
  if (M < 0 || static_cast<long>(M) * m->top_k > kMoeMaxAssignments) return LBQ_ERR_SHAPE;
  if (moe_gateup_lds(m->hidden) > 64 * 1024 || moe_down_lds(m->ffn) > 64 * 1024) return LBQ_ERR_SHAPE;
  if (!aligned16(m->planes) || !aligned16(m->meta)) return LBQ_ERR_ALIGN;
  return LBQ_OK;
}

}  // namespace

extern "C" {

lbq_status lbq_moe_workspace(const lbq_moe *m, int32_t M, size_t *bytes) {
  if (!bytes) return LBQ_ERR_NULL;
  lbq_status st = check_moe(m, M);
  if (st != LBQ_OK) return st;
  *bytes = moe_layout(m, M).total;
  return LBQ_OK;
}

lbq_status lbq_moe_forward(const lbq_moe *m, const uint16_t *x, const float *logits, int32_t M, uint16_t *y,
                           void *ws, size_t ws_bytes, void *stream) {
  lbq_status st = check_moe(m, M);
  if (st != LBQ_OK) return st;
  if (M == 0) return LBQ_OK;
  if (!x || !logits || !y || !ws) return LBQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(ws)) return LBQ_ERR_ALIGN;
  const MoeLayout L = moe_layout(m, M);
  if (ws_bytes < L.total) return LBQ_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *base = static_cast<uint8_t *>(ws);
  MoeArgs a{};
  a.E = m->E;
  a.hidden = m->hidden;
  a.ffn = m->ffn;
  a.top_k = m->top_k;
  a.M = M;
  a.bits = m->bits;
  a.gu_plane_off = m->gu_plane_off;
  a.gu_meta_off = m->gu_meta_off;
  a.dn_plane_off = m->dn_plane_off;
  a.dn_meta_off = m->dn_meta_off;
  a.planes = static_cast<const uint8_t *>(m->planes);
  a.meta = static_cast<const uint8_t *>(m->meta);
  a.signs_hidden = m->signs_hidden;
  a.signs_ffn = m->signs_ffn;
  a.x = x;
  a.xr = reinterpret_cast<uint16_t *>(base + L.xr);
  a.h = reinterpret_cast<float *>(base + L.h);
  int32_t *ids = reinterpret_cast<int32_t *>(base + L.ids);
  float *wts = reinterpret_cast<float *>(base + L.weights);
  int32_t *counts = reinterpret_cast<int32_t *>(base + L.counts);
  int32_t *offsets = reinterpret_cast<int32_t *>(base + L.offsets);
  int32_t *perm = reinterpret_cast<int32_t *>(base + L.perm);
  a.offsets = offsets;
  a.perm = perm;
  a.weights = wts;
  a.act = reinterpret_cast<uint16_t *>(base + L.act);
  a.out = reinterpret_cast<float *>(base + L.out);
  a.y = y;
  if (launch_moe_route(logits, M, m->E, m->top_k, ids, wts, counts, offsets, perm, s) != hipSuccess)
    return LBQ_ERR_HIP;
  return hip_status(launch_moe_experts(a, s));
}

lbq_status lbq_moe_route(const float *logits, int32_t M, int32_t E, int32_t top_k, int32_t *ids, float *weights,
                         int32_t *counts, int32_t *offsets, int32_t *perm, void *stream) {
  if (E <= 0 || E > kMoeMaxExperts || top_k < 1 || top_k > E || top_k > kMoeMaxTopK) return LBQ_ERR_SHAPE;
  if (M < 0 || static_cast<long>(M) * top_k > kMoeMaxAssignments) return LBQ_ERR_SHAPE;
  if (!ids || !weights || !counts || !offsets || !perm || (M > 0 && !logits)) return LBQ_ERR_NULL;
  return hip_status(launch_moe_route(logits, M, E, top_k, ids, weights, counts, offsets, perm,
                                     static_cast<hipStream_t>(stream)));
}

}  // extern "C"
