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
 *     "Routed Experts" row: group-128 codes, mixed 2/3/4-bit per expert), or
 *     8-bit codes of the same form (its "Non-Expert Path" and "Readout &
 *     Embeddings" rows),
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
 *   LBQ_FMT_RTN_PLANES, bits b in {2,3,4,8}, G = K/128:
 *     planes: uint32 [N][G][b][4]. Bit j of word w of plane p holds bit p of
 *             code q[n][128 g + 32 w + j]. plane_bytes = N*K*b/8.
 *     meta:   [N][G] pairs of IEEE fp16 (scale s, zero z), s at the lower
 *             address. meta_bytes = 4*N*G.
 *     Decoded rotated weight: W'[n][k] = (q[n][k] - z[n][g]) * s[n][g].
 *   LBQ_FMT_PVQ_4x8, bits b in {2,4,6} = 2 per residual stage, S = b/2:
 *     planes: uint8 idx [S][N][K/4]; byte i of a row holds the codebook index
 *             of weights 4i..4i+3 (byte 2v+h is half h of 8-weight vector v).
 *     meta:   fp16 row scales [S][N].
 *     codebook: 256 entries x 4 fp8 e4m3 (OCP "fn") bytes, row-major, shared by
 *             every stage (values on the e4m3 grid, or on the NVFP4 e2m1 grid
 *             held as e4m3 bytes).
 *     Decoded rotated weight: W'[n][4i+d] = sum_t s_t[n] * C[idx_t[n][i]][d].
 *     (Laguna-S-2.1 card: product-VQ over 8-weight vectors with fp8- or
 *     NVFP4-grid codebooks; three stages carry the 48 index bits per vector of
 *     its 6.0-bpw FP8-CB rung.)
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
  LBQ_ERR_BITS = -3,       /* bits outside {2,3,4,8} (RTN) or {2,4,6} (PVQ) */
  LBQ_ERR_ALIGN = -4,      /* a pointer that must be 16-byte aligned is not */
  LBQ_ERR_WORKSPACE = -5,  /* workspace smaller than the *_workspace query returned */
  LBQ_ERR_RANGE = -6,      /* packing: non-finite weight or an RTN group scale out of range */
  LBQ_ERR_HIP = -7,        /* a HIP launch reported an error */
  LBQ_ERR_FORMAT = -8      /* unknown format, or a format the entry point does not take */
} lbq_status;

typedef enum {
  LBQ_FMT_RTN_PLANES = 0,
  LBQ_FMT_PVQ_4x8 = 1
} lbq_format;

/* Kernel path for lbq_linear_forward_path. AUTO picks the GEMV for M <= 4 and
 * the MFMA GEMM above (measured crossover), and the GEMM also where the RTN
 * matrix-core GEMV would run its tokens in two passes over the codes (three or
 * four tokens on long rows); forcing the GEMV needs M <= 16.
 * LBQ_PATH_GEMM_MX (2-bit RTN codes, M <= 16, K a multiple of 512,
 * 16-byte-aligned signs) runs the matrix-core GEMM: fp4 codes times three e4m3
 * pieces per rotated activation (about twelve significant bits, as in the
 * matrix-core GEMV), the scale applied in fp32 per group. AUTO does not take
 * it (it measured no faster end to end than the fp16 GEMM); forcing it
 * elsewhere returns LBQ_ERR_SHAPE (LBQ_ERR_ALIGN for unaligned signs).
 * LBQ_PATH_SPLIT_ROTATION may be OR-ed into any of them (for tests): the
 * GEMM's separate rotation launch then goes in launches of at most three
 * tokens each, the split it otherwise makes only past 1 GiB of activations. */
typedef enum {
  LBQ_PATH_AUTO = 0,
  LBQ_PATH_GEMV = 1,
  LBQ_PATH_GEMM = 2,
  LBQ_PATH_GEMM_MX = 3,
  LBQ_PATH_SPLIT_ROTATION = 0x100
} lbq_path;

/* A packed weight: a plain view of caller-owned device buffers. */
typedef struct {
  int32_t K, N, bits, format;
  const void *planes;    /* RTN: uint32 [N][K/128][bits][4]; PVQ: uint8 [bits/2][N][K/4] */
  const void *meta;      /* RTN: fp16 pairs [N][K/128][2]; PVQ: fp16 [bits/2][N] */
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

/* Text for a status code (static storage; never NULL, unknown codes give
 * "unknown status"). */
const char *lbq_status_string(lbq_status s);

/* Byte sizes of the packed buffers of one K x N weight (host query; nothing
 * is launched). RTN: planes N*K*bits/8, meta 4*N*K/128 (the bit-plane layout
 * above: Qwen3-8B BPDQ card, opening paragraph; the fp16 scale and zero per
 * 128-group: LLaDA2.2-mini card, "Routed Experts" row). PVQ: indices N*K/4,
 * row scales 2*N (Laguna-S-2.1 card, opening paragraph: two 8-bit indices per
 * 8-weight vector). Errors: LBQ_ERR_NULL (an output pointer), LBQ_ERR_BITS,
 * LBQ_ERR_FORMAT, LBQ_ERR_SHAPE. */
lbq_status lbq_packed_bytes(int32_t K, int32_t N, int32_t bits, int32_t format,
                            size_t *plane_bytes, size_t *meta_bytes);

/* Offline packing on the host (threaded, float64 arithmetic). The method
 * quantizes each weight in a Hadamard-rotated basis with group-128 codes and
 * stores the rotation signs beside it (LLaDA2.2-mini card, property table,
 * "Routed Experts" row, and its file list), as bit-planes (Qwen3-8B BPDQ card,
 * opening paragraph) or as product-VQ indices into an fp8-valued codebook
 * (Laguna-S-2.1 card, opening paragraph). All buffers are host memory owned by
 * the caller; nothing is launched.
 *   W: host fp32 [N][K] row-major (PyTorch Linear layout, y = x W^T).
 *   signs: host int8 [K] of +-1.  codebook: host [256][4] e4m3 bytes (PVQ only).
 *   planes_out / meta_out: host buffers of lbq_packed_bytes' sizes.
 * RTN (bits 2/3/4/8): rotate each row per 128-block (signs, radix-2 butterflies,
 * then c), then per group mn = min(0, min w'), mx = max(0, max w'),
 * s = fp16_rne((mx - mn) / (2^b - 1)) (0 -> 1), z = rint(-mn / s),
 * q = clamp(rint(w' / s) + z, 0, 2^b - 1), and scatter q into bit-planes.
 * PVQ (bits 2/4/6): rotate, s_n = fp16_rne(rms(w'_n) / rms(C)) (0 -> 1), and per
 * 4-weight half the nearest codebook entry to w'/s_n (squared distance,
 * ties to the lower index); each further stage does the same on what the
 * earlier stages left (w' minus their decode), with its own row scale.
 * Returns LBQ_ERR_RANGE for non-finite W, a PVQ scale that overflows fp16, or
 * an RTN scale s >= 128 at 2/3/4 bits or s >= 16 at 8 bits (the MFMA GEMM's
 * decode holds -64 s (-256 s at 8 bits) and -16 s z in fp16; a group would
 * need a weight range of 128 (2^b - 1), or 16 * 255, to reach it). */
lbq_status lbq_pack(const float *W, int32_t K, int32_t N, int32_t bits, int32_t format,
                    const int8_t *signs, const uint8_t *codebook,
                    void *planes_out, void *meta_out);

/* GPTQ, step 1 (host, offline): the factor the error feedback of
 * lbq_pack_gptq runs through. The weights are quantized with group-128 GPTQ in
 * the Hadamard-rotated basis (LLaDA2.2-mini card, property table, "Routed
 * Experts" row; Qwen3.8-27B Pingala-8 card, "What this is": LDLQ rounding
 * behind a random Hadamard rotation).
 *   H: host float64 [K][K], symmetric positive semi-definite proxy Hessian of
 *      the layer input in the original basis (e.g. X^T X / n of calibration
 *      activations X [n][K]).
 *   signs: host int8 [K] of +-1 (the weight's rotation signs).
 *   damp: > 0; damp * mean(diag H') is added to the diagonal of H'.
 *   U: host float64 [K][K] out: the upper Cholesky factor of H'^-1
 *      (H'^-1 = U^T U), H' = R H R^T + damping; zeros below the diagonal.
 * O(K^3) on the host threads. Errors: LBQ_ERR_NULL, LBQ_ERR_SHAPE (K not a
 * positive multiple of 128), LBQ_ERR_RANGE (signs not +-1, non-finite H, a
 * zero diagonal mean, or H' not positive definite after damping). */
lbq_status lbq_gptq_factor(const double *H, int32_t K, const int8_t *signs, double damp, double *U);

/* GPTQ, step 2 (host, offline): pack W [N][K] (host fp32, as lbq_pack) into
 * the RTN bit-plane format (same planes / meta layout and sizes), choosing the
 * codes with error feedback through U (from lbq_gptq_factor): rotate each row;
 * then for each column j in order, at the first column of each 128-group the
 * group's scale and zero from its current values (the lbq_pack RTN rule),
 * q = clamp(rint(w_j / s) + z, 0, 2^b - 1), e = (w_j - (q - z) s) / U[j][j],
 * and w_k -= e U[j][k] for every later column k. Float64; the result depends
 * only on (W, signs, U, bits). Errors as lbq_pack (RTN), plus LBQ_ERR_RANGE
 * for a non-positive diagonal of U. */
lbq_status lbq_pack_gptq(const float *W, int32_t K, int32_t N, int32_t bits, const int8_t *signs,
                         const double *U, void *planes_out, void *meta_out);

/* Workspace bytes lbq_linear_forward needs for M tokens on any path (host
 * query; the rotated activations, or for 2-bit codes at M <= 16 the larger
 * e4m3 pieces of LBQ_PATH_GEMM_MX, the GEMM's zero-point sums and its split-K
 * partial tiles and counters). Errors as lbq_linear_forward's argument
 * checks. */
lbq_status lbq_linear_workspace(const lbq_weight *w, int32_t M, size_t *bytes);

/* y[M][N] (fp16) = x[M][K] (fp16) W_hat^T, W_hat the weight w decodes to:
 * the weight stays packed and is decoded inside the matmul (Qwen3-8B BPDQ
 * card, opening paragraph: bit-planes kept packed for the whole run;
 * Laguna-S-2.1 card, opening paragraph: codebook decode at matmul time), the
 * activations are rotated into the weight's basis (Qwen3.8-27B Pingala-8 card,
 * "What this is": random Hadamard rotation).
 *   x: fp16 [M][K], y: fp16 [M][N], row-major, device, 16-byte aligned;
 *   ws: device workspace of lbq_linear_workspace(w, M) bytes or more.
 * Paths (AUTO):
 *   - M <= 4, K a multiple of 512, signs 16-byte aligned (PVQ: codebook 4-byte
 *     aligned): one launch, the matrix-core GEMV with the rotation in its
 *     prologue (nothing is written to ws), unless for RTN codes the tokens'
 *     activation pieces do not all fit in LDS at once (three or four tokens on
 *     long rows): then the MFMA GEMM as for M >= 5;
 *   - other M <= 4: a rotation launch into ws, then the staged VALU GEMV
 *     (8-bit codes and multi-stage PVQ: the MFMA GEMM instead; a forced GEMV
 *     that the matrix-core GEMV cannot take returns LBQ_ERR_SHAPE for them);
 *   - M >= 5: a rotation launch into ws (for RTN in the GEMM's folded
 *     order, with the zero-point sums), then the MFMA dequant-GEMM.
 * Accumulation is fp32; the fp16 GEMM rounds each decoded RTN weight s q to fp16
 * (the zero-point term s z sum_k x'_k is added separately), and each decoded
 * multi-stage PVQ weight to one fp16 value in units of stage 1's row scale. The RTN GEMM needs
 * N*K*b/8 < 2^31 - 4096 (LBQ_ERR_SHAPE otherwise). The result of a call does
 * not depend on timing: repeat calls give identical bits. Errors are returned
 * before any launch: LBQ_ERR_NULL, _SHAPE, _BITS, _ALIGN, _FORMAT, _WORKSPACE;
 * LBQ_ERR_HIP if a launch fails. */
lbq_status lbq_linear_forward(const lbq_weight *w, const uint16_t *x, int32_t M,
                              uint16_t *y, void *ws, size_t ws_bytes, void *stream);

/* lbq_linear_forward with an explicit kernel path (lbq_path, optionally with
 * LBQ_PATH_SPLIT_ROTATION): LBQ_PATH_GEMV (M <= 16, LBQ_ERR_SHAPE above),
 * LBQ_PATH_GEMM (any M) or LBQ_PATH_GEMM_MX (2-bit RTN, M <= 16, K a multiple
 * of 512; LBQ_ERR_SHAPE otherwise: a rotation launch writing the e4m3 pieces,
 * a power-of-two scale per (token, group) and the zero-point sums into ws,
 * then the matrix-core GEMM). The same operation and arguments; for tests that
 * reach every kernel at shapes AUTO would send elsewhere. */
lbq_status lbq_linear_forward_path(const lbq_weight *w, const uint16_t *x, int32_t M,
                                   uint16_t *y, void *ws, size_t ws_bytes, int32_t path,
                                   void *stream);

/* lbq_linear_forward (AUTO path) with the main kernel's duration bracketed by
 * two caller-owned HIP events (hipEvent_t created with timing enabled; either
 * may be NULL), for measuring the decode kernel against the bytes it moves
 * (Laguna-S-2.1 card, "Reading it honestly": decode speed tracks bytes). For
 * the RTN matrix-core GEMV (rotation in its prologue) the events take that
 * kernel's own begin and end times (hipExtLaunchKernel); on the other paths
 * they are recorded on the stream right before and after the GEMV / GEMM
 * launch (after the separate rotation launch). The result is the one
 * lbq_linear_forward gives. */
lbq_status lbq_linear_forward_timed(const lbq_weight *w, const uint16_t *x, int32_t M,
                                    uint16_t *y, void *ws, size_t ws_bytes, void *stream,
                                    void *start_event, void *stop_event);

/* Bytes of the device scratch array behind lbq_linear_forward_noalloc. */
#define LBQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* lbq_linear_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same operation, arguments and result as lbq_linear_forward
 * with the AUTO path, but with the library's own scratch in place of the
 * caller's workspace. The scratch is a static device array of
 * LBQ_NOALLOC_SCRATCH_BYTES per GPU (each GPU the library runs on holds it
 * from its first use until the process ends); the call allocates nothing and
 * returns LBQ_ERR_WORKSPACE, before any launch, when lbq_linear_workspace(w, M)
 * exceeds it. Every call on one GPU shares that GPU's array, which keeps the
 * last call's contents (the calls clear what must start at zero themselves):
 * calls that overlap in time on one GPU (other streams, other host threads)
 * race on it and give wrong results. The stream's GPU is the one used (the
 * current GPU for the null stream). */
lbq_status lbq_linear_forward_noalloc(const lbq_weight *w, const uint16_t *x, int32_t M,
                                      uint16_t *y, void *stream);

/* Workspace bytes lbq_moe_forward needs for M tokens (host query): router
 * outputs, the per-assignment intermediates and expert outputs. */
lbq_status lbq_moe_workspace(const lbq_moe *m, int32_t M, size_t *bytes);

/* Routed-expert MoE block (Laguna-S-2.1 card, base-model line: routed experts
 * chosen top-k per token; LLaDA2.2-mini card, "Routed Experts" row: each expert
 * at its own 2/3/4-bit width, group-128 codes in the rotated basis): per
 * token t, the top_k experts by logit (ties to the lower id) with softmax
 * weights over the selected logits; for each selected expert e:
 * h = x_t W_gu(e)^T, a = silu(h[:ffn]) * h[ffn:], o = a W_dn(e)^T;
 * y_t = sum_j w_tj o_tj, summed in fp32 in slot order, written fp16.
 *   x: fp16 [M][hidden]; logits: fp32 [M][E]; y: fp16 [M][hidden] (device,
 *   16-byte aligned); ws: lbq_moe_workspace(m, M) bytes.
 * Limits: E <= 1024, top_k <= 32, M * top_k <= 2^20 (LBQ_ERR_SHAPE). Errors
 * as lbq_linear_forward. */
lbq_status lbq_moe_forward(const lbq_moe *m, const uint16_t *x, const float *logits, int32_t M,
                           uint16_t *y, void *ws, size_t ws_bytes, void *stream);

/* lbq_moe_forward with an explicit path for the expert linears: LBQ_PATH_GEMV
 * (the matrix-core expert GEMVs, tokens of an expert in chunks of four) or
 * LBQ_PATH_GEMM (grouped MFMA dequant-GEMMs over the expert-sorted assignment
 * list, with the codes decoded inside the mainloop rather than expanded to a
 * dense copy first: the prefill gap the Laguna-S-2.1 card names in "Reading it
 * honestly"). AUTO takes the GEMMs once M * top_k >= 4 E (about four tokens per
 * expert). The GEMM path needs hidden and ffn of at most 5120 and
 * M * top_k * ffn * 8 below 2^31 (LBQ_ERR_SHAPE otherwise). Same operation,
 * arguments and errors as lbq_moe_forward. */
lbq_status lbq_moe_forward_path(const lbq_moe *m, const uint16_t *x, const float *logits, int32_t M,
                                uint16_t *y, void *ws, size_t ws_bytes, int32_t path, void *stream);

/* Router pass alone (the first step of lbq_moe_forward; Laguna-S-2.1 card,
 * base-model line: 256 routed experts, top-k per token), for inspection:
 *   ids int32 [M][top_k], weights fp32 [M][top_k], counts int32 [E],
 *   offsets int32 [E+1] (exclusive prefix sum of counts), perm int32 [M*top_k]
 *   = assignment indices t*top_k + j grouped by expert in offset order and, within
 *   one expert, in increasing t*top_k + j. */
lbq_status lbq_moe_route(const float *logits, int32_t M, int32_t E, int32_t top_k,
                         int32_t *ids, float *weights, int32_t *counts, int32_t *offsets,
                         int32_t *perm, void *stream);

/* Codes as the GPU decoders see them, for the bit-exact read-back check
 * (Qwen3.8-27B Pingala-8 card, "Results": the packed file read back tensor by
 * tensor against freshly regenerated data with zero mismatches): RTN writes
 * uint8 codes [N][K] produced by the kernels' own plane-merge routine; PVQ
 * copies the uint8 indices [bits/2][N][K/4]. codes: device, 16-byte aligned. */
lbq_status lbq_unpack_codes(const lbq_weight *w, uint8_t *codes, void *stream);

/* out[M][K] (fp16) = R x for each token row, R = blockdiag(c H_128 diag(s))
 * (Qwen3.8-27B Pingala-8 card, "What this is": random Hadamard rotation;
 * LLaDA2.2-mini card, file list: stored rotation signs); fp32 butterflies,
 * fp16 out. x, out: device [M][K], 16-byte aligned; signs: device [K]. */
lbq_status lbq_rotate(const uint16_t *x, int32_t M, int32_t K, const int8_t *signs,
                      uint16_t *out, void *stream);

/* Nibble-split planes of an 8-bit weight, for the screened readout (host,
 * offline). The readout keeps its 8-bit codes and the same codes split into
 * high and low nibble planes (LLaDA2.2-mini card, property table, "Readout &
 * Embeddings" row, and its file list). With q = 16 hi + lo:
 *   planes8: host uint32 [N][K/128][8][4] and meta8: host fp16 pairs
 *     [N][K/128][2] (s, z), as lbq_pack writes them at 8 bits;
 *   hi_planes / lo_planes: host uint32 [N][K/128][4][4] out: planes 4..7 and
 *     0..3, i.e. the 4-bit plane sets of hi and lo;
 *   hi_meta: host fp16 pairs [N][K/128][2] out: (16 s, (z - 7.5) / 16), which
 *     make hi_planes a 4-bit weight whose decode s (16 hi + 7.5 - z) takes
 *     each high nibble at the middle of the 16 codes it spans.
 * Errors: LBQ_ERR_NULL, LBQ_ERR_SHAPE (K not a positive multiple of 128, N <= 0),
 * LBQ_ERR_RANGE (a scale or zero whose high-nibble form is not exact in fp16:
 * outside what lbq_pack writes at 8 bits). */
lbq_status lbq_split_nibbles(const void *planes8, const void *meta8, int32_t K, int32_t N,
                             void *hi_planes, void *lo_planes, void *hi_meta);

/* A readout weight in nibble-split form (device views, 16-byte aligned):
 * hi_planes, lo_planes and hi_meta as lbq_split_nibbles writes them, meta the
 * 8-bit (s, z) pairs, signs [K] +-1. */
typedef struct {
  int32_t K, N;
  const void *hi_planes, *lo_planes, *hi_meta, *meta;
  const int8_t *signs;
} lbq_readout;

/* Workspace bytes of lbq_readout_screened for M tokens and cand survivors
 * (host query). Errors as lbq_readout_screened's argument checks. */
lbq_status lbq_readout_workspace(const lbq_readout *r, int32_t M, int32_t cand, size_t *bytes);

/* Screened readout (the LLaDA2.2-mini card's screened readout over the
 * nibble-split planes of its 8-bit lm_head). Per token t:
 *   1. coarse[t][n] (fp16, every row n) = x_t W_hi^T, W_hi the 4-bit weight
 *      (hi_planes, hi_meta): half the bytes of the 8-bit weight, by the
 *      lbq_linear_forward path for M tokens;
 *   2. the cand rows with the largest coarse logits, larger first, ties to the
 *      lower row (decided on the fp16 values of step 1);
 *   3. their exact logits from both nibbles, q = 16 hi + lo with the 8-bit
 *      (s, z), against the fp16-rotated x_t, fp32 accumulation.
 *   x: fp16 [M][K]; coarse: fp16 [M][N] out; ids: int32 [M][cand] out (rows,
 *   in step 2's order; -1 past the N-th when cand > N); logits: fp32
 *   [M][cand] out (0 for -1 ids). 1 <= cand <= 64, M <= 65535.
 * Errors as lbq_linear_forward, plus LBQ_ERR_SHAPE for cand or M out of range. */
lbq_status lbq_readout_screened(const lbq_readout *r, const uint16_t *x, int32_t M, int32_t cand,
                                uint16_t *coarse, int32_t *ids, float *logits, void *ws, size_t ws_bytes,
                                void *stream);

/* Measurement reference, not part of the layer: one launch of grid x block
 * threads (block a multiple of 64, at most 1024) that reads bytes (a multiple
 * of 16, below 64 GiB) at buf (device, 16-byte aligned) once, as a plain
 * streaming read. Its duration for a GEMV launch's byte count is the floor
 * that launch faces before any decode work, the figure a decode kernel that
 * tracks bytes moved (Laguna-S-2.1 card, "Reading it honestly") is compared
 * with beside the HBM peak. sink: device u32 it may write. Optional events as
 * in lbq_linear_forward_timed (the kernel's own begin and end). bytes = 0 is
 * an empty launch (the launch floor). */
lbq_status lbq_stream_read(const void *buf, size_t bytes, int32_t grid, int32_t block, uint32_t *sink,
                           void *stream, void *start_event, void *stop_event);

#ifdef __cplusplus
}
#endif

#endif /* LBQ_H */
