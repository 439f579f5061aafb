// The C ABI (include/lbq.h): argument checks, workspace layout, path choice,
// and kernel launches on the caller's stream. No allocation, no global state.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>

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
    if ((w->bits < 2 || w->bits > 4) && w->bits != 8) return LBQ_ERR_BITS;
  } else if (w->format == LBQ_FMT_PVQ_4x8) {
    if (!w->codebook) return LBQ_ERR_NULL;
    if (w->bits != 2 && w->bits != 4 && w->bits != 6) return LBQ_ERR_BITS;   // 1, 2, 3 residual stages
  } else {
    return LBQ_ERR_FORMAT;
  }
  if (w->K <= 0 || w->K % 128 != 0 || w->N <= 0) return LBQ_ERR_SHAPE;
  if (!aligned16(w->planes) || !aligned16(w->meta)) return LBQ_ERR_ALIGN;
  return LBQ_OK;
}

GemmPlan linear_gemm_plan(const lbq_weight *w, int M) {
  return w->format == LBQ_FMT_RTN_PLANES ? gemm_rtn_plan(M, w->K, w->N, w->bits)
                                          : gemm_plan(M, w->K, w->N, w->bits / 2);
}

size_t tz_bytes(const lbq_weight *w, int M) {
  return w->format == LBQ_FMT_RTN_PLANES ? round_up(static_cast<size_t>(M) * gemm_tz_stride(w->K) * 4, kAlign) : 0;
}

// Up to 16 tokens of 2-bit RTN codes may run on the matrix-core GEMM (fp4
// codes x e4m3 activation pieces).
constexpr int kMxMaxTokens = 16;
bool mx_possible(const lbq_weight *w, int M) {
  return w->format == LBQ_FMT_RTN_PLANES && M >= 1 && M <= kMxMaxTokens && gemm_mx_supported(M, w->K, w->N, w->bits);
}

size_t act_bytes(const lbq_weight *w, int M) {
  size_t b = round_up(static_cast<size_t>(M) * w->K * 2, kAlign);
  if (mx_possible(w, M)) b = std::max(b, round_up(gemm_mx_act_bytes(M, w->K), kAlign));
  return b;
}

size_t linear_ws_bytes(const lbq_weight *w, int M) {
  // the rotated activations (or the matrix-core GEMM's pieces and scale bytes),
  // the RTN GEMMs' per-(token, group) sums, then the GEMM's split-K partial
  // tiles and counters (the larger of the two GEMMs' plans)
  size_t scratch = gemm_scratch_bytes(linear_gemm_plan(w, M));
  if (mx_possible(w, M)) scratch = std::max(scratch, gemm_scratch_bytes(gemm_mx_plan(M, w->K, w->N)));
  return act_bytes(w, M) + tz_bytes(w, M) + scratch;
}

lbq_status forward_impl(const lbq_weight *w, const uint16_t *x, int32_t M, uint16_t *y, void *ws, size_t ws_bytes,
                        int32_t path, void *stream, hipEvent_t ev0, hipEvent_t ev1) {
  lbq_status st = check_weight(w);
  if (st != LBQ_OK) return st;
  if (M < 0) return LBQ_ERR_SHAPE;
  // test flag: the GEMM's rotation in launches of at most three tokens
  const int rot_tokens = (path & LBQ_PATH_SPLIT_ROTATION) ? 3 : 0;
  path &= ~LBQ_PATH_SPLIT_ROTATION;
  if (path < LBQ_PATH_AUTO || path > LBQ_PATH_GEMM_MX) return LBQ_ERR_SHAPE;
  if ((path == LBQ_PATH_GEMV || path == LBQ_PATH_GEMM_MX) && M > 16) return LBQ_ERR_SHAPE;
  if (M == 0) return LBQ_OK;
  if (path == LBQ_PATH_GEMM_MX && !mx_possible(w, M)) return LBQ_ERR_SHAPE;
  if (!x || !y || !ws) return LBQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(ws)) return LBQ_ERR_ALIGN;
  if (path == LBQ_PATH_GEMM_MX && !aligned16(w->signs)) return LBQ_ERR_ALIGN;
  if (ws_bytes < linear_ws_bytes(w, M)) return LBQ_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The matrix-core GEMM for five to sixteen tokens of 2-bit codes, on request
  // only: per launch it beat the fp16 GEMM on the smaller dense-stack shapes at
  // 16 tokens (4096 -> 6144 8.8 -> 8.4 us, 4096 -> 4096 8.6 -> 7.4 us) but not
  // on the larger ones (4096 -> 28672 15.9 -> 18.9 us, 14336 -> 4096 12.6 ->
  // 16.5 us), and its rotation launch costs about 0.8 us more, so the stack as
  // a whole measured no faster (57.5 against 56.3 us per layer)
  if (path == LBQ_PATH_GEMM_MX) {
    const GemmPlan gp = gemm_mx_plan(M, w->K, w->N);
    uint8_t *tz = static_cast<uint8_t *>(ws) + act_bytes(w, M);
    void *scratch = tz + tz_bytes(w, M);
    if (launch_gemm_mx(gp, w->planes, w->meta, x, w->signs, ws, reinterpret_cast<uint32_t *>(tz), y, M, w->K, w->N,
                       scratch, s, ev0) != hipSuccess)
      return LBQ_ERR_HIP;
    return (ev1 && hipEventRecord(ev1, s) != hipSuccess) ? LBQ_ERR_HIP : LBQ_OK;
  }
  // up to four tokens share one matrix-core GEMV pass; from there on the MFMA
  // GEMM, and also where the GEMV would need a second pass over the codes (three
  // or four tokens on long rows: 14336 -> 4096 at four tokens 17.4 -> 15.0 us)
  bool gemv = (path == LBQ_PATH_GEMV) ||
              (path == LBQ_PATH_AUTO && M <= 4 &&
               (w->format != LBQ_FMT_RTN_PLANES || !gemv_mfma_supported(M, w->K, w->N) ||
                gemv_mfma_one_pass(M, w->K, w->N, w->bits)));
  // One to four tokens: rotation fused into the matrix-core decoder, one launch.
  if (w->format == LBQ_FMT_RTN_PLANES && gemv && gemv_mfma_supported(M, w->K, w->N) && aligned16(w->signs) &&
      (w->bits != 8 || gemv_mfma_supported_8bit(w->K, w->N)))
    return hip_status(launch_gemv_mfma(w->planes, w->meta, x, w->signs, y, M, w->K, w->N, w->bits, 0, 0, 0, s, ev0,
                                       ev1));
  const int stages = w->format == LBQ_FMT_PVQ_4x8 ? w->bits / 2 : 1;
  if (w->format == LBQ_FMT_PVQ_4x8 && gemv && gemv_pvq_mx_supported(M, w->K, w->N, stages) && aligned16(w->signs) &&
      (reinterpret_cast<uintptr_t>(w->codebook) & 3u) == 0) {
    if (ev0 && hipEventRecord(ev0, s) != hipSuccess) return LBQ_ERR_HIP;
    if (launch_gemv_pvq_mx(static_cast<const uint8_t *>(w->planes), static_cast<const uint16_t *>(w->meta),
                           static_cast<const uint8_t *>(w->codebook), x, w->signs, y, M, w->K, w->N, stages,
                           s) != hipSuccess)
      return LBQ_ERR_HIP;
    return (ev1 && hipEventRecord(ev1, s) != hipSuccess) ? LBQ_ERR_HIP : LBQ_OK;
  }
  uint16_t *xr = static_cast<uint16_t *>(ws);
  // 8-bit codes and residual product-VQ stages run on the matrix-core GEMV or
  // the MFMA GEMM only
  if (gemv && ((w->format == LBQ_FMT_RTN_PLANES && w->bits == 8) || stages > 1)) {
    if (path == LBQ_PATH_GEMV) return LBQ_ERR_SHAPE;
    gemv = false;
  }
  if (!gemv) {
    // MFMA GEMM: a rotation launch (clearing the split-K counters; for RTN the
    // folded order with the zero-point sums), then the GEMM
    const bool rtn = w->format == LBQ_FMT_RTN_PLANES;
    if (rtn && !gemm_rtn_supported(w->K, w->N, w->bits)) return LBQ_ERR_SHAPE;
    const GemmPlan gp = linear_gemm_plan(w, M);
    uint8_t *after_x = static_cast<uint8_t *>(ws) + act_bytes(w, M);
    uint32_t *tz = rtn ? reinterpret_cast<uint32_t *>(after_x) : nullptr;
    void *scratch = after_x + tz_bytes(w, M);
    // (the RTN GEMM takes the folded slot order, the product-VQ GEMM natural order)
    const hipError_t re =
        rtn ? launch_rotate_folded(x, M, w->K, w->signs, xr, tz, gemm_counter_ptr(gp, scratch), gemm_counters(gp), s,
                                   rot_tokens)
            : launch_rotate_clear(x, M, w->K, w->signs, xr, gemm_counter_ptr(gp, scratch), gemm_counters(gp), s);
    if (re != hipSuccess) return LBQ_ERR_HIP;
    if (ev0 && hipEventRecord(ev0, s) != hipSuccess) return LBQ_ERR_HIP;
    const hipError_t ge =
        rtn ? launch_gemm_rtn(gp, w->bits, w->planes, w->meta, xr, tz, y, M, w->K, w->N, scratch, s)
            : launch_gemm_pvq(gp, w->planes, w->meta, static_cast<const uint8_t *>(w->codebook), xr, y, M, w->K, w->N,
                              stages, scratch, s);
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
    if ((bits < 2 || bits > 4) && bits != 8) return LBQ_ERR_BITS;
  } else if (format == LBQ_FMT_PVQ_4x8) {
    if (bits != 2 && bits != 4 && bits != 6) return LBQ_ERR_BITS;
  } else {
    return LBQ_ERR_FORMAT;
  }
  if (K <= 0 || K % 128 != 0 || N <= 0) return LBQ_ERR_SHAPE;
  if (format == LBQ_FMT_RTN_PLANES) {
    *plane_bytes = static_cast<size_t>(N) * K / 8 * bits;
    *meta_bytes = static_cast<size_t>(N) * (K / 128) * 4;
  } else {   // bits / 2 residual stages of indices and row scales
    *plane_bytes = static_cast<size_t>(bits / 2) * N * (K / 4);
    *meta_bytes = static_cast<size_t>(bits / 2) * N * 2;
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
  return pack_pvq(W, K, N, signs, codebook, static_cast<uint8_t *>(planes_out), static_cast<uint16_t *>(meta_out),
                  bits / 2);
}

lbq_status lbq_gptq_factor(const double *H, int32_t K, const int8_t *signs, double damp, double *U) {
  if (!H || !signs || !U) return LBQ_ERR_NULL;
  if (K <= 0 || K % 128 != 0) return LBQ_ERR_SHAPE;
  if (!(damp > 0.0)) return LBQ_ERR_RANGE;
  for (int k = 0; k < K; ++k)
    if (signs[k] != 1 && signs[k] != -1) return LBQ_ERR_RANGE;
  return gptq_factor(H, K, signs, damp, U);
}

lbq_status lbq_pack_gptq(const float *W, int32_t K, int32_t N, int32_t bits, const int8_t *signs, const double *U,
                         void *planes_out, void *meta_out) {
  if (!W || !signs || !U || !planes_out || !meta_out) return LBQ_ERR_NULL;
  size_t pb, mb;
  lbq_status st = lbq_packed_bytes(K, N, bits, LBQ_FMT_RTN_PLANES, &pb, &mb);
  if (st != LBQ_OK) return st;
  for (int k = 0; k < K; ++k)
    if (signs[k] != 1 && signs[k] != -1) return LBQ_ERR_RANGE;
  return pack_gptq(W, K, N, bits, signs, U, static_cast<uint32_t *>(planes_out), static_cast<uint16_t *>(meta_out));
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

}  // extern "C"

// ---------------------------------------------------------------- no-allocation entry point

namespace {

// The workspace of lbq_linear_forward_noalloc: a file-scope device array, one
// instance per GPU at that GPU's own address, held until the process ends. In
// host code its name is only a stand-in for the symbol: kernels get the device
// address that hipGetSymbolAddress returns for the GPU in use.
constexpr size_t kScratchBytes = LBQ_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the GPU the stream runs on (the current GPU
// for the null stream), looked up once per GPU with that GPU current.
lbq_status scratch_on(hipStream_t s, void **out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return LBQ_ERR_HIP;
  int dev = cur;
  if (s != nullptr && hipStreamGetDevice(s, &dev) != hipSuccess) return LBQ_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return LBQ_ERR_HIP;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (dev != cur && hipSetDevice(dev) != hipSuccess) return LBQ_ERR_HIP;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (dev != cur && hipSetDevice(cur) != hipSuccess) return LBQ_ERR_HIP;
      if (e != hipSuccess || !p) return LBQ_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return LBQ_OK;
}

}  // namespace

extern "C" {

lbq_status lbq_linear_forward_noalloc(const lbq_weight *w, const uint16_t *x, int32_t M, uint16_t *y, void *stream) {
  lbq_status st = check_weight(w);
  if (st != LBQ_OK) return st;
  if (M < 0) return LBQ_ERR_SHAPE;
  if (M == 0) return LBQ_OK;
  if (linear_ws_bytes(w, M) > kScratchBytes) return LBQ_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void *ws = nullptr;
  st = scratch_on(s, &ws);
  if (st != LBQ_OK) return st;
  // the rotation launch clears the split-K counters the GEMM finds in the
  // array (with a kernel, so the call can be captured in a graph)
  return forward_impl(w, x, M, y, ws, kScratchBytes, LBQ_PATH_AUTO, stream, nullptr, nullptr);
}

lbq_status lbq_unpack_codes(const lbq_weight *w, uint8_t *codes, void *stream) {
  lbq_status st = check_weight(w);
  if (st != LBQ_OK) return st;
  if (!codes) return LBQ_ERR_NULL;
  if (!aligned16(codes)) return LBQ_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (w->format == LBQ_FMT_RTN_PLANES)
    return hip_status(launch_unpack_rtn(w->planes, w->K, w->N, w->bits, codes, s));
  return hip_status(hipMemcpyAsync(codes, w->planes, static_cast<size_t>(w->bits / 2) * w->N * (w->K / 4),
                                   hipMemcpyDeviceToDevice, s));
}

lbq_status lbq_stream_read(const void *buf, size_t bytes, int32_t grid, int32_t block, uint32_t *sink,
                           void *stream, void *start_event, void *stop_event) {
  if (!sink || (bytes > 0 && !buf)) return LBQ_ERR_NULL;
  if (bytes % 16 != 0 || bytes / 16 >= (static_cast<size_t>(1) << 32)) return LBQ_ERR_SHAPE;
  if (grid < 1 || block < 64 || block > 1024 || block % 64 != 0) return LBQ_ERR_SHAPE;
  if (bytes > 0 && !aligned16(buf)) return LBQ_ERR_ALIGN;
  return hip_status(launch_stream_read(buf, bytes, grid, block, sink, static_cast<hipStream_t>(stream),
                                       static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)));
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
  size_t xr, ids, weights, counts, offsets, perm, act, out, h, tz_h, tz_f, tiles, n_tiles, total;
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
  L.tz_h = take(static_cast<size_t>(M) * gemm_tz_stride(m->hidden) * 4);
  L.tz_f = take(mk * gemm_tz_stride(m->ffn) * 4);
  L.tiles = take(static_cast<size_t>(moe_prefill_max_tiles(M, m->E, m->top_k)) * 16);
  L.n_tiles = take(4);
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

lbq_status lbq_split_nibbles(const void *planes8, const void *meta8, int32_t K, int32_t N, void *hi_planes,
                             void *lo_planes, void *hi_meta) {
  if (!planes8 || !meta8 || !hi_planes || !lo_planes || !hi_meta) return LBQ_ERR_NULL;
  if (K <= 0 || K % 128 != 0 || N <= 0) return LBQ_ERR_SHAPE;
  return split_nibbles(static_cast<const uint32_t *>(planes8), static_cast<const uint16_t *>(meta8), K, N,
                       static_cast<uint32_t *>(hi_planes), static_cast<uint32_t *>(lo_planes),
                       static_cast<uint16_t *>(hi_meta));
}

lbq_status lbq_moe_workspace(const lbq_moe *m, int32_t M, size_t *bytes) {
  if (!bytes) return LBQ_ERR_NULL;
  lbq_status st = check_moe(m, M);
  if (st != LBQ_OK) return st;
  *bytes = moe_layout(m, M).total;
  return LBQ_OK;
}

lbq_status lbq_moe_forward_path(const lbq_moe *m, const uint16_t *x, const float *logits, int32_t M, uint16_t *y,
                                void *ws, size_t ws_bytes, int32_t path, void *stream) {
  lbq_status st = check_moe(m, M);
  if (st != LBQ_OK) return st;
  if (path < LBQ_PATH_AUTO || path > LBQ_PATH_GEMM) return LBQ_ERR_SHAPE;
  const long assignments = static_cast<long>(M) * m->top_k;
  const bool grouped_ok = moe_prefill_supported(m->hidden, m->ffn, assignments);
  if (path == LBQ_PATH_GEMM && !grouped_ok) return LBQ_ERR_SHAPE;
  // the grouped GEMMs once the experts see about four tokens each on average
  const bool grouped = path == LBQ_PATH_GEMM || (path == LBQ_PATH_AUTO && grouped_ok && assignments >= 4L * m->E);
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
  if (grouped) {
    MoePrefill p{};
    p.tiles = reinterpret_cast<int32_t *>(base + L.tiles);
    p.n_tiles = reinterpret_cast<int32_t *>(base + L.n_tiles);
    p.tz_hidden = reinterpret_cast<uint32_t *>(base + L.tz_h);
    p.tz_ffn = reinterpret_cast<uint32_t *>(base + L.tz_f);
    return hip_status(launch_moe_prefill(a, p, s));
  }
  return hip_status(launch_moe_experts(a, s));
}

lbq_status lbq_moe_forward(const lbq_moe *m, const uint16_t *x, const float *logits, int32_t M, uint16_t *y,
                           void *ws, size_t ws_bytes, void *stream) {
  return lbq_moe_forward_path(m, x, logits, M, y, ws, ws_bytes, LBQ_PATH_AUTO, stream);
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

// ---------------------------------------------------------------- screened readout

namespace {

lbq_status check_readout(const lbq_readout *r, int M, int cand) {
  if (!r || !r->hi_planes || !r->lo_planes || !r->hi_meta || !r->meta || !r->signs) return LBQ_ERR_NULL;
  if (r->K <= 0 || r->K % 128 != 0 || r->N <= 0) return LBQ_ERR_SHAPE;
  if (M < 0 || M > 65535 || cand < 1 || cand > 64) return LBQ_ERR_SHAPE;
  if (!aligned16(r->hi_planes) || !aligned16(r->lo_planes) || !aligned16(r->hi_meta) || !aligned16(r->meta))
    return LBQ_ERR_ALIGN;
  return LBQ_OK;
}

// the high nibbles as a 4-bit weight of the library's own format
lbq_weight readout_hi_weight(const lbq_readout *r) {
  lbq_weight w{};
  w.K = r->K;
  w.N = r->N;
  w.bits = 4;
  w.format = LBQ_FMT_RTN_PLANES;
  w.planes = r->hi_planes;
  w.meta = r->hi_meta;
  w.codebook = nullptr;
  w.signs = r->signs;
  return w;
}

// workspace: the coarse linear's own workspace, the fp16 rotated activations
// of the exact step, the survivors' keys
size_t readout_ws_bytes(const lbq_readout *r, int M, int cand) {
  const lbq_weight w = readout_hi_weight(r);
  return round_up(linear_ws_bytes(&w, M), kAlign) + round_up(static_cast<size_t>(M) * r->K * 2, kAlign) +
         readout_key_bytes(M, r->N, cand);
}

}  // namespace

extern "C" {

lbq_status lbq_readout_workspace(const lbq_readout *r, int32_t M, int32_t cand, size_t *bytes) {
  if (!bytes) return LBQ_ERR_NULL;
  const lbq_status st = check_readout(r, M, cand);
  if (st != LBQ_OK) return st;
  *bytes = readout_ws_bytes(r, M, cand);
  return LBQ_OK;
}

lbq_status lbq_readout_screened(const lbq_readout *r, const uint16_t *x, int32_t M, int32_t cand, uint16_t *coarse,
                                int32_t *ids, float *logits, void *ws, size_t ws_bytes, void *stream) {
  lbq_status st = check_readout(r, M, cand);
  if (st != LBQ_OK) return st;
  if (M == 0) return LBQ_OK;
  if (!x || !coarse || !ids || !logits || !ws) return LBQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(coarse) || !aligned16(ws)) return LBQ_ERR_ALIGN;
  if (ws_bytes < readout_ws_bytes(r, M, cand)) return LBQ_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const lbq_weight w = readout_hi_weight(r);
  const size_t lin = round_up(linear_ws_bytes(&w, M), kAlign);
  uint8_t *base = static_cast<uint8_t *>(ws);
  uint16_t *xr = reinterpret_cast<uint16_t *>(base + lin);
  uint64_t *keys = reinterpret_cast<uint64_t *>(base + lin + round_up(static_cast<size_t>(M) * r->K * 2, kAlign));
  // 1. coarse logits of every row from the high nibbles
  st = forward_impl(&w, x, M, coarse, ws, lin, LBQ_PATH_AUTO, stream, nullptr, nullptr);
  if (st != LBQ_OK) return st;
  // 2. the survivors per token, 3. their exact logits
  const uint64_t *fin = nullptr;
  if (launch_readout_select(coarse, M, r->N, cand, keys, &fin, x, r->signs, xr, r->K, s) != hipSuccess)
    return LBQ_ERR_HIP;
  return hip_status(launch_readout_refine(fin, r->hi_planes, r->lo_planes, r->meta, xr, M, r->K, r->N, cand, ids,
                                          logits, s));
}

}  // extern "C"
