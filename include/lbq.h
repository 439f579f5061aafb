/*
 * lbq.h - low-bit weight-only quantized linear layers for AMD MI355X (gfx950).
 *
 * The operation. A linear layer y = x W^T whose weight W (N outputs x K
 * inputs) is stored in a Hadamard-rotated basis as low-bit codes and decoded
 * inside the matmul:
 *   - every 128-block of the K axis is rotated by R_j = c * H_128 * diag(s_j),
 *     c = 1/sqrt(128), with a stored random +-1 sign vector s (rotation signs
 *     are stored with the small tensors and weights are quantized "in a
 *     Hadamard-rotated basis": LLaDA2.2-mini Orin Nano model card, property
 *     table and file list; "random Hadamard rotation": Qwen3.8-27B Pingala-8
 *     model card, "What this is");
 *   - the rotated weight W' = W R^T is held either as group-128 2/3/4-bit
 *     codes with an fp16 scale and zero per group (the LLaDA2.2-mini card's
 *     "Routed Experts" row: group-128 codes, mixed 2/3/4-bit per expert),
 *     packed as bit-planes in 32-bit words (Qwen3-8B 2-bit BPDQ model card,
 *     opening paragraph), or as product-VQ indices into a small codebook whose
 *     values sit on the fp8 e4m3 grid (Laguna-S-2.1 gridbook model card,
 *     opening paragraph);
 *   - since R is orthogonal, y = (x R^T)(W R^T)^T: the forward pass rotates
 *     the activations once per token (fp16 out) and contracts them against the
 *     decoded codes with fp32 accumulation; y is written as fp16.
 * A routed-expert MoE block (top-k router, per-expert SwiGLU FFN at each
 * expert's own code width; Laguna-S-2.1 card: routed experts top-k; LLaDA2.2-
 * mini card: per-expert widths) runs on the same decoders.
 *
 * Conventions for every entry point.
 *   - Plain C ABI. Pointers are device pointers unless marked "host".
 *     Streams are hipStream_t passed as void* (NULL = the null stream).
 *   - Ownership: the caller allocates and frees every buffer, including the
 *     workspace. The library keeps no state between calls and never
 *     allocates; forward calls are re-entrant and only enqueue work on the
 *     given stream (they never synchronise).
 *   - Errors: a non-zero lbq_status is returned before anything is launched.
 *     A launch failure reported by HIP maps to LBQ_ERR_HIP. Nothing throws.
 *   - Alignment: planes, meta, x, y and workspace pointers must be 16-byte
 *     aligned (LBQ_ERR_ALIGN otherwise).
 *   - K must be a positive multiple of 128 (LBQ_ERR_SHAPE otherwise); M = 0
 *     is a valid no-op.
 *
 * Packed formats (byte-exact; little-endian):
 *   LBQ_FMT_RTN_PLANES, bits b in {2,3,4}, G = K/128:
 *     planes: uint32 [N][G][b][4]. Bit j of word w of plane p holds bit p of
 *             code q[n][128 g + 32 w + j]. plane_bytes = N*K*b/8.
 *     meta:   [N][G] pairs of IEEE fp16 (scale s, zero z), s at the lower
 *             address. meta_bytes = 4*N*G.
 *     Decoded rotated weight: W'[n][k] = (q[n][k] - z[n][g]) * s[n][g].
 *   LBQ_FMT_PVQ_4x8 (2 bits per weight):
 *     planes: uint8 idx [N][K/4]; byte i holds the codebook index of weights
 *             4i..4i+3 (byte 2v+h is half h of 8-weight vector v).
 *     meta:   fp16 row scale [N].
 *     codebook: 256 entries x 4 fp8 e4m3 (OCP "fn") bytes, row-major.
 *     Decoded rotated weight: W'[n][4i+d] = s[n] * C[idx[n][i]][d].
 */
#ifndef LBQ_H
#define LBQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LBQ_OK = 0,
  LBQ_ERR_NULL = -1,       /* a required pointer is NULL */
  LBQ_ERR_SHAPE = -2,      /* K not a positive multiple of 128, N <= 0, M < 0, top_k outside [1, E], ... */
  LBQ_ERR_BITS = -3,       /* bits outside {2,3,4} (RTN) or != 2 (PVQ) */
  LBQ_ERR_ALIGN = -4,      /* a pointer that must be 16-byte aligned is not */
  LBQ_ERR_WORKSPACE = -5,  /* workspace smaller than the *_workspace query returned */
  LBQ_ERR_RANGE = -6,      /* packing: non-finite weight or an RTN group scale of 128 or more */
  LBQ_ERR_HIP = -7,        /* a HIP launch reported an error */
  LBQ_ERR_FORMAT = -8      /* unknown format, or a format the entry point does not take */
} lbq_status;

typedef enum {
  LBQ_FMT_RTN_PLANES = 0,
  LBQ_FMT_PVQ_4x8 = 1
} lbq_format;

/* Kernel path for lbq_linear_forward_path. AUTO picks the GEMV for M <= 4 and
 * the MFMA GEMM above (measured crossover); forcing the GEMV needs M <= 16. */
typedef enum {
  LBQ_PATH_AUTO = 0,
  LBQ_PATH_GEMV = 1,
  LBQ_PATH_GEMM = 2
} lbq_path;

/* A packed weight: a plain view of caller-owned device buffers. */
typedef struct {
  int32_t K, N, bits, format;
  const void *planes;    /* RTN: uint32 [N][K/128][bits][4]; PVQ: uint8 [N][K/4] */
  const void *meta;      /* RTN: fp16 pairs [N][K/128][2]; PVQ: fp16 [N] */
  const void *codebook;  /* PVQ: 256x4 e4m3 bytes; RTN: ignored (may be NULL) */
  const int8_t *signs;   /* [K] rotation signs, each +1 or -1 */
} lbq_weight;

/* A routed-expert MoE block of E experts, each a SwiGLU FFN:
 *   gate|up: RTN weight K = hidden, N = 2*ffn (rows 0..ffn-1 gate, ffn..2ffn-1 up)
 *   down:    RTN weight K = ffn,    N = hidden
 * Expert e uses code width bits[e] for both of its weights. All experts share
 * the hidden-space signs (gate|up input) and the ffn-space signs (down input).
 * Expert e's buffers start at planes + *_plane_off[e] and meta + *_meta_off[e]
 * (byte offsets, each 16-byte aligned). hidden and ffn are multiples of 128. */
typedef struct {
  int32_t E, hidden, ffn, top_k;
  const uint8_t *bits;            /* [E] in {2,3,4} */
  const uint64_t *gu_plane_off;   /* [E] */
  const uint64_t *gu_meta_off;    /* [E] */
  const uint64_t *dn_plane_off;   /* [E] */
  const uint64_t *dn_meta_off;    /* [E] */
  const void *planes;             /* base of all expert code planes */
  const void *meta;               /* base of all expert scale/zero pairs */
  const int8_t *signs_hidden;     /* [hidden] */
  const int8_t *signs_ffn;        /* [ffn] */
} lbq_moe;

/* Text for a status code (static storage). */
const char *lbq_status_string(lbq_status s);

/* Byte sizes of the packed buffers of one K x N weight (host query). */
lbq_status lbq_packed_bytes(int32_t K, int32_t N, int32_t bits, int32_t format,
                            size_t *plane_bytes, size_t *meta_bytes);

/* Offline packing on the host (threaded, float64 arithmetic):
 *   W: host fp32 [N][K] row-major (PyTorch Linear layout, y = x W^T).
 *   signs: host int8 [K] of +-1.  codebook: host [256][4] e4m3 bytes (PVQ only).
 *   planes_out / meta_out: host buffers of lbq_packed_bytes' sizes.
 * RTN (bits 2/3/4): rotate each row per 128-block (signs, radix-2 butterflies,
 * then c), then per group mn = min(0, min w'), mx = max(0, max w'),
 * s = fp16_rne((mx - mn) / (2^b - 1)) (0 -> 1), z = rint(-mn / s),
 * q = clamp(rint(w' / s) + z, 0, 2^b - 1), and scatter q into bit-planes.
 * PVQ (bits 2): rotate, s_n = fp16_rne(rms(w'_n) / rms(C)) (0 -> 1), and per
 * 4-weight half the nearest codebook entry to w'/s_n (squared distance,
 * ties to the lower index).
 * Returns LBQ_ERR_RANGE for non-finite W, a PVQ scale that overflows fp16, or
 * an RTN scale s >= 128 (the MFMA GEMM's decode holds -64 s and -16 s z in
 * fp16; a group would need a weight range of 128 (2^b - 1) to reach it). */
lbq_status lbq_pack(const float *W, int32_t K, int32_t N, int32_t bits, int32_t format,
                    const int8_t *signs, const uint8_t *codebook,
                    void *planes_out, void *meta_out);

/* Workspace bytes lbq_linear_forward needs for M tokens (host query). */
lbq_status lbq_linear_workspace(const lbq_weight *w, int32_t M, size_t *bytes);

/* y[M][N] (fp16) = x[M][K] (fp16) W_hat^T, W_hat the weight w decodes to.
 * The activation rotation runs either inside the GEMV's prologue (RTN codes,
 * signs 16-byte aligned: one to four tokens on the matrix cores when K is a
 * multiple of 512, else one or two tokens on rows of up to 8192 / 4096 inputs)
 * or as its own launch into the workspace, followed by the dequant-GEMV
 * (M <= 4) or the MFMA dequant-GEMM (M >= 5). Accumulation is fp32; the
 * GEMM rounds each decoded RTN weight s q to fp16 (the zero-point term s z
 * sum_k x'_k is added separately). The RTN GEMM needs N*K*b/8 < 2^31 - 4096
 * (LBQ_ERR_SHAPE otherwise). The result of a call does not depend on timing:
 * repeat calls give identical bits. */
lbq_status lbq_linear_forward(const lbq_weight *w, const uint16_t *x, int32_t M,
                              uint16_t *y, void *ws, size_t ws_bytes, void *stream);

/* lbq_linear_forward with an explicit kernel path (lbq_path). */
lbq_status lbq_linear_forward_path(const lbq_weight *w, const uint16_t *x, int32_t M,
                                   uint16_t *y, void *ws, size_t ws_bytes, int32_t path,
                                   void *stream);

/* lbq_linear_forward (AUTO path) with the main kernel's duration bracketed by
 * two caller-owned HIP events (hipEvent_t created with timing enabled; either
 * may be NULL). For the single-token GEMV with the rotation in its prologue
 * the events take that kernel's own begin and end times (hipExtLaunchKernel);
 * on the other paths they are recorded on the stream right before and after
 * the GEMV / GEMM launch (after the separate rotation launch). For measuring
 * the kernel; the result is the one lbq_linear_forward gives. */
lbq_status lbq_linear_forward_timed(const lbq_weight *w, const uint16_t *x, int32_t M,
                                    uint16_t *y, void *ws, size_t ws_bytes, void *stream,
                                    void *start_event, void *stop_event);

/* Workspace bytes lbq_moe_forward needs for M tokens (host query). */
lbq_status lbq_moe_workspace(const lbq_moe *m, int32_t M, size_t *bytes);

/* Routed-expert MoE block: per token t, the top_k experts by logit (ties to the
 * lower id) with softmax weights over the selected logits; for each selected
 * expert e: h = x_t W_gu(e)^T, a = silu(h[:ffn]) * h[ffn:], o = a W_dn(e)^T;
 * y_t = sum_j w_tj o_tj, summed in fp32 in slot order, written fp16.
 *   x: fp16 [M][hidden]; logits: fp32 [M][E]; y: fp16 [M][hidden]. */
lbq_status lbq_moe_forward(const lbq_moe *m, const uint16_t *x, const float *logits, int32_t M,
                           uint16_t *y, void *ws, size_t ws_bytes, void *stream);

/* Router pass alone (the first step of lbq_moe_forward), for inspection:
 *   ids int32 [M][top_k], weights fp32 [M][top_k], counts int32 [E],
 *   offsets int32 [E+1] (exclusive prefix sum of counts), perm int32 [M*top_k]
 *   = assignment indices t*top_k + j grouped by expert in offset order and, within
 *   one expert, in increasing t*top_k + j. */
lbq_status lbq_moe_route(const float *logits, int32_t M, int32_t E, int32_t top_k,
                         int32_t *ids, float *weights, int32_t *counts, int32_t *offsets,
                         int32_t *perm, void *stream);

/* Codes as the GPU decoders see them: RTN writes uint8 codes [N][K] produced by
 * the kernels' own plane-merge routine; PVQ copies the uint8 indices [N][K/4]. */
lbq_status lbq_unpack_codes(const lbq_weight *w, uint8_t *codes, void *stream);

/* out[M][K] (fp16) = R x for each token row (fp32 butterflies, fp16 out). */
lbq_status lbq_rotate(const uint16_t *x, int32_t M, int32_t K, const int8_t *signs,
                      uint16_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LBQ_H */
