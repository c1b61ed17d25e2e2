/*
 * nvq.h -- C ABI of libnvq.so: NVFP4 quantization, residual-channel selection,
 * W4A4 MoE grouped GEMM with residual compensation and asymmetric W4A16 QAT
 * GEMMs on AMD Instinct MI355X (gfx950).
 *
 * Method sources (cited by page and section; the pages print no equations):
 *  - QUADS explainer ("QUADS: Stabilizing NVFP4 Reinforcement Learning for MoE
 *    via QUantization-error Alignment across Dual Sides", gist.science):
 *      §1   NVFP4 W4A4 GEMMs, E2M1 grid with 8 magnitudes per sign;
 *      §2.1 weights take the same quantize-dequantize path on both sides,
 *           activations are quantized online;
 *      §2.2-A asymmetric W4A16 QAT: fake-quantized NVFP4 weights, BF16
 *           activations in the trainer forward;
 *      §2.2-B residual activation compensation: the channels with the largest
 *           quantization residual get a correction added to the W4A4 output.
 *  - TRACE post ("TRACE : un entraînement conscient de la quantification guidé
 *    par le rollout ...", sns.style), "Fonctionnement, côté ingénierie" and
 *    "L'idée centrale de TRACE": block-scaled FP4, the trainer takes its
 *    rounding from the rollout's recorded quantization (codes and scales).
 *  - NVFP4 layout the pages leave open: 16-element blocks along K, one E4M3
 *    (OCP FP8 "FN") scale per block, one fp32 scale per tensor
 *    s_t = amax / (6 * 448), E2M1 elements (OCP MX v1.0), round to nearest,
 *    ties to even, two codes per byte with the even element in the low nibble.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers, row-major, owned by the caller.
 *    The library allocates nothing; scratch memory is the caller's workspace
 *    `ws` of `ws_bytes` bytes (size it with the matching *_workspace_bytes
 *    query; 256-byte aligned).
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *    work on it; none synchronizes the host.  Calls that share a workspace
 *    must be ordered on one stream.
 *  - Checks the host can make (shapes, null pointers, 16-byte alignment of
 *    vector-loaded tensors, workspace size) return a negative NVQ_E* code and
 *    enqueue nothing.  A HIP launch failure returns NVQ_EHIP.
 *  - Conditions only the device sees set bits of a status word kept in the
 *    workspace (NVQ_STATUS_*), read with nvq_device_status().
 *  - bf16 tensors are passed as uint16_t bit patterns.
 *  - Empty inputs: a tensor whose row (or token) count is 0 may be passed as
 *    NULL.  The outputs that are not empty are still written as the
 *    definitions give them: nvfp4_quantize with rows == 0 writes
 *    s_t = fl32(amax / 2688) with the amax of nothing taken as 0 (or
 *    amax_in) and chan_score = 0; nvq_moe_permute with T == 0 writes all-zero
 *    expert offsets; the WGRAD mode of qat_fakequant_gemm_w4a16 writes dw = 0
 *    (leaves it with accumulate) for experts without rows.
 */
#ifndef NVQ_H
#define NVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum nvq_status {
  NVQ_OK = 0,
  NVQ_EINVAL = -1,       /* null pointer or bad enum/value */
  NVQ_ESHAPE = -2,       /* shape not supported (K % 16, k > K, ...) */
  NVQ_EALIGN = -3,       /* a vector-loaded tensor is not 16-byte aligned */
  NVQ_EWORKSPACE = -4,   /* workspace missing or too small */
  NVQ_EHIP = -5,         /* a HIP runtime call failed */
  NVQ_EUNSUPPORTED = -6  /* valid request this build does not implement */
};

enum nvq_dtype { NVQ_F32 = 0, NVQ_BF16 = 1 };

/* device status bits (nvq_device_status) */
enum {
  NVQ_STATUS_NONFINITE = 1u << 0, /* a quantized input held Inf or NaN */
  NVQ_STATUS_BAD_EXPERT = 1u << 1 /* a top-k expert id was outside [0, E) */
};

const char* nvq_status_string(int status);

/* Reads the status word of workspace `ws` after `stream` drains (this call
 * synchronizes the stream).  *flags receives NVQ_STATUS_* bits. */
int nvq_device_status(const void* ws, void* stream, uint32_t* flags);

/* ------------------------------------------------------------------------ */
/* NVFP4 quantization (QUADS §1, §2.1; TRACE "Fonctionnement").
 *
 * x        [batch, rows, K] of dtype x_dtype (NVQ_F32 or NVQ_BF16), 16-byte
 *          aligned; K % 16 == 0; 1 <= batch <= 65535.  Row r of item b starts
 *          at element (b * rows + r) * ldx: ldx >= K is the row stride in
 *          elements (0 means K, a dense tensor) and ldx * element size must be
 *          a multiple of 16 bytes (NVQ_EALIGN otherwise; ldx < K: NVQ_ESHAPE).
 *          Outputs are always dense.
 * amax_in  nullable device [batch] fp32: replaces amax_t = max|x| of each
 *          batch item (e.g. to requantize with a known scale).
 * codes    [batch, rows, K/2]  E2M1 codes, even element in the low nibble.
 * scales   [batch, rows, K/16] E4M3 block-scale codes (never 0x7F).
 * tensor_scale [batch] fp32 s_t = fl32(amax_t / 2688).
 * chan_score   nullable [K] fp32 (only with batch == 1): per-channel residual
 *          score, the sum of |x - dequant(q(x))| over rows in a fixed order
 *          (16-row sequential sub-chunk sums, summed in order within 128-row
 *          chunks, chunks summed in order; every sum fp32).
 * Decisions are exact: each scale is the E4M3 value nearest the real quotient
 * amax_b / (6 s_t) (ties to even, saturating at 448) and each code the E2M1
 * value nearest |x| / (s_b s_t) (ties to even, saturating at 6).
 * Each batch item is one tensor with its own s_t (stacked expert weights).
 * A non-finite input sets NVQ_STATUS_NONFINITE.
 */
size_t nvfp4_quantize_workspace_bytes(int64_t batch, int64_t rows, int64_t K);
int nvfp4_quantize(const void* x, int x_dtype, int64_t batch, int64_t rows, int64_t K,
                   int64_t ldx, const float* amax_in, uint8_t* codes, uint8_t* scales,
                   float* tensor_scale, float* chan_score, void* ws, size_t ws_bytes,
                   void* stream);

/* Allocation-free variant of nvfp4_quantize, for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments, results
 * and host-side errors as nvfp4_quantize, without ws / ws_bytes: the scratch
 * memory (status word, amax partials, residual chunk partials) is a static
 * array inside the library, NVQ_QUANTIZE_NOALLOC_SCRATCH_BYTES on every GPU
 * the library runs on, held until the process ends.  A call whose scratch
 * need (nvfp4_quantize_workspace_bytes(batch, rows, K)) exceeds it returns
 * NVQ_EWORKSPACE and launches nothing.  The first call on a device looks up
 * that device's array (hipGetSymbolAddress); no call allocates.  Every call on
 * one GPU shares the array: calls that may overlap on one GPU (other streams,
 * other host threads) race and must be ordered by the caller.  The device
 * status word lives in the shared array and is not reported to the caller;
 * use nvfp4_quantize when NVQ_STATUS_NONFINITE must be read. */
#define NVQ_QUANTIZE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int nvfp4_quantize_noalloc(const void* x, int x_dtype, int64_t batch, int64_t rows, int64_t K,
                           int64_t ldx, const float* amax_in, uint8_t* codes, uint8_t* scales,
                           float* tensor_scale, float* chan_score, void* stream);

/* NVFP4 dequantization: y = sign * fl32(fl32(G * s_b) * s_t), written as fp32
 * (y_dtype NVQ_F32) or rounded to nearest-even bf16 (NVQ_BF16).  This is the
 * quantize-dequantize image both sides use for the weights (QUADS §2.1).
 * codes [batch, rows, K/2] (8-byte aligned), scales [batch, rows, K/16],
 * tensor_scale [batch], y [batch, rows, K] (16-byte aligned); K % 16 == 0,
 * 1 <= batch <= 65535.  No rows: nothing is written.  Errors (NVQ_EINVAL,
 * NVQ_ESHAPE, NVQ_EALIGN) launch nothing. */
int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                     int64_t batch, int64_t rows, int64_t K, void* y, int y_dtype, void* stream);

/* ------------------------------------------------------------------------ */
/* Rollout-guided rounding (TRACE post: "L'idée centrale de TRACE" -- the
 * rollout's quantization guides the trainer's rounding and the cache keeps
 * only the mantissa and the scale factors; "Fonctionnement, côté ingénierie"
 * -- each value rounds to the grid point above or below, the discrete choice
 * both sides must share).
 *
 * The guidance record of a quantized tensor is one bit per element, bits
 * [batch, rows, K/8] u8 (element c of a row in bit c % 8 of byte c / 8), kept
 * with the rollout's block scales and tensor scale: 0.1875 byte per element
 * against 0.5625 for codes + scales.
 *   NVQ_GUIDE_MANTISSA   the mantissa bit (index & 1) of the rollout's code;
 *   NVQ_GUIDE_DIRECTION  1 when the rollout's magnitude G s_b s_t lies strictly
 *                        above |x| (rounded up), else 0.
 */
enum { NVQ_GUIDE_MANTISSA = 0, NVQ_GUIDE_DIRECTION = 1 };

/* Writes the guidance record `bits` of the NVFP4 record (codes [batch, rows,
 * K/2], scales [batch, rows, K/16], tensor_scale [batch]) of x.  Mantissa mode
 * reads only the codes (x, scales, tensor_scale may be NULL); direction mode
 * reads x [batch, rows, K] (x_dtype NVQ_F32 or NVQ_BF16, 16-byte aligned), the
 * value that was quantized.  K % 16 == 0, 1 <= batch <= 65535; codes 8-byte
 * and bits 2-byte aligned.  Device pointers, caller-owned; asynchronous on stream.  Errors
 * (NVQ_EINVAL, NVQ_ESHAPE, NVQ_EALIGN) launch nothing. */
int nvfp4_guidance_record(const void* x, int x_dtype, const uint8_t* codes, const uint8_t* scales,
                          const float* tensor_scale, int64_t batch, int64_t rows, int64_t K,
                          int mode, uint8_t* bits, void* stream);

/* Rebuilds NVFP4 codes [batch, rows, K/2] for master values w [batch, rows, K]
 * (w_dtype NVQ_F32 or NVQ_BF16, e.g. weights the trainer has updated since the
 * rollout quantized them) from a guidance record: the rollout's scales
 * [batch, rows, K/16] and tensor_scale [batch] are reused unchanged, and for
 * each element, with lo / hi the indices of the grid points G s_b s_t at or
 * below / at or above |w| (hi = 7 beyond the grid):
 *   mantissa:  of a = min(lo, 6) and a + 1, the one whose mantissa bit is the
 *              recorded bit (adjacent E2M1 points differ in that bit);
 *   direction: recorded 1 -> hi, 0 -> lo.
 * The sign is signbit(w); a zero block or tensor scale gives magnitude 0.
 * Decisions are exact.  With w equal to the quantized tensor this gives back
 * the rollout's codes.  ws is nullable (else 256-byte aligned, >= 256 bytes):
 * a non-finite w sets NVQ_STATUS_NONFINITE in its status word (that element's
 * code is then unspecified).  K % 16 == 0, 1 <= batch <= 65535; w 16-byte,
 * codes 8-byte, bits 2-byte aligned.
 * Errors (NVQ_EINVAL, NVQ_ESHAPE, NVQ_EALIGN, NVQ_EWORKSPACE) launch nothing. */
int nvfp4_guided_quantize(const void* w, int w_dtype, int64_t batch, int64_t rows, int64_t K,
                          const uint8_t* bits, const uint8_t* scales, const float* tensor_scale,
                          int mode, uint8_t* codes, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Residual-channel selection (QUADS §2.2-B).
 *
 * Selects the k channels with the largest residual score (ties to the lower
 * channel index) and writes them in rank order to idx_out [k] (int32).
 * x [rows, K] (row stride ldx >= K elements, 0 means K) is the tensor whose
 * NVFP4 record (codes [rows, K/2], scales [rows, K/16], tensor_scale [1],
 * dense) is given; it is read only to recompute scores or residuals.
 * scores_in  nullable [K]: the chan_score of nvfp4_quantize.  When NULL the
 *            score is recomputed from x and its NVFP4 record (codes, scales,
 *            tensor_scale), in the same order as nvfp4_quantize.
 * scores_out nullable [K]: receives the score used.
 * resid_out  nullable [rows, k] bf16: the compensation operand
 *            bf16(fl32(x - dequant(q(x))))[:, idx_out].
 * 0 <= k <= K; k == 0 writes nothing to idx_out/resid_out.  k <= 1024 takes
 * any K (radix select); k > 1024 needs K <= 8192, else NVQ_EUNSUPPORTED.
 * Scores compare as numbers (-0 equals +0); they must not be NaN.
 */
size_t residual_topk_workspace_bytes(int64_t rows, int64_t K, int32_t k);
int residual_topk_channels(const void* x, int x_dtype, int64_t rows, int64_t K, int64_t ldx,
                           const uint8_t* codes, const uint8_t* scales,
                           const float* tensor_scale, const float* scores_in, float* scores_out,
                           int32_t k, int32_t* idx_out, uint16_t* resid_out, void* ws,
                           size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* MoE routing glue (TRACE "Fonctionnement": the router's discrete expert
 * choice).  Per token: the topk largest of E fp32 logits, descending, ties
 * to the lower expert id; weights = softmax over the chosen logits.
 * logits [T, E] fp32; ids [T, topk] int32; weights [T, topk] fp32.
 * Requires 1 <= topk <= E <= 1024. */
int nvq_moe_route(const float* logits, int64_t T, int64_t E, int64_t topk, int32_t* ids,
                  float* weights, void* stream);

/* Token-expert pairs p = t*topk + j sorted stably by expert (histogram,
 * exclusive scan, stable scatter).  ids [T, topk]; sorted_pair [P];
 * expert_offsets [E+1] (rows of expert e are [off[e], off[e+1])); pos [P]
 * the inverse map (sorted position of pair p).  An id outside [0, E) sets
 * NVQ_STATUS_BAD_EXPERT and that pair is dropped. */
size_t nvq_moe_permute_workspace_bytes(int64_t T, int64_t topk, int64_t E);
int nvq_moe_permute(const int32_t* ids, int64_t T, int64_t topk, int64_t E,
                    int32_t* sorted_pair, int32_t* expert_offsets, int32_t* pos, void* ws,
                    size_t ws_bytes, void* stream);

/* out[t, n] = bf16( sum_j w[t, j] * y[pos[t*topk + j], n] ), j ascending, fp32
 * accumulation.  y [P, N] bf16 in sorted-pair order; a pair the permutation
 * dropped (pos < 0) is left out of the sum.  N % 8 == 0.
 * out_amax: nullable device fp32 word (4-byte aligned) that receives max |out|
 * over the stored bf16 values (0 for no tokens); the call clears it first.
 * When out is the next layer's input (QUADS §2.1: activations are quantized
 * online at every forward), passing it as amax_in to nvfp4_quantize replaces
 * that call's amax pass with an identical result.  Calls sharing the word
 * must be ordered on one stream. */
int nvq_moe_combine(const uint16_t* y, const int32_t* pos, const float* weights, int64_t T,
                    int64_t topk, int64_t N, uint16_t* out, float* out_amax, void* stream);

/* ------------------------------------------------------------------------ */
/* Chained backward of the MoE layer's glue (QUADS §2.2-A: the trainer's
 * backward with the identity straight-through estimator runs through the
 * layer's SwiGLU and expert combine; its GEMMs are qat_fakequant_gemm_w4a16).
 * All tensors bf16 unless stated, row-major, 16-byte aligned device pointers,
 * caller-owned; asynchronous on stream; errors (NVQ_EINVAL, NVQ_ESHAPE,
 * NVQ_EALIGN) launch nothing.  Zero rows (tokens) do nothing. */

/* h [rows, I] = bf16(silu(g) u) with g = y1[:, :I], u = y1[:, I:], y1
 * [rows, 2I] of dtype y1_dtype (NVQ_F32 or NVQ_BF16), silu(g) = g / (1 +
 * exp(-g)), evaluated in fp32 with the hardware exp and reciprocal (the
 * result is rounded to bf16).  I % 8 == 0. */
int nvq_swiglu_forward(const void* y1, int y1_dtype, int64_t rows, int64_t I, uint16_t* h,
                       void* stream);

/* dy1 [rows, 2I] = (dh u s (1 + g (1 - s)), dh g s), s = 1 / (1 + exp(-g)):
 * the gradient of h = silu(g) u with respect to the gate and up
 * pre-activations y1 (layout and dtype as above), given dh [rows, I].  fp32
 * arithmetic, bf16 result.  I % 8 == 0. */
int nvq_swiglu_backward(const void* y1, int y1_dtype, const uint16_t* dh, int64_t rows, int64_t I,
                        uint16_t* dy1, void* stream);

/* Backward of nvq_moe_combine (out[t] = sum_j w[t,j] y[pos[t,j]]):
 *   dy[pos[t,j], :] = bf16(fl32(w[t,j] dout[t, :]))   dy [P, N] sorted-pair order
 *   dw[t, j]       = sum_n dout[t,n] y[pos[t,j], n]   fp32 (nullable; y is read
 *                    only for it)
 * dout [T, N]; pos [T, topk] the permutation's inverse map (pairs with pos < 0
 * are skipped, their dw is 0); weights [T, topk] fp32.  N % 8 == 0.  The token
 * gradient of the gate/up input, sum_j dx_pairs[pos[t,j]], is nvq_moe_combine
 * with unit weights. */
int nvq_moe_combine_backward(const uint16_t* dout, const uint16_t* y, const int32_t* pos,
                             const float* weights, int64_t T, int64_t topk, int64_t N,
                             uint16_t* dy, float* dw, void* stream);

/* ------------------------------------------------------------------------ */
/* W4A4 MoE grouped GEMM with residual compensation (QUADS §1, §2.2-B).
 *
 * For every sorted row p of expert e (off[e] <= p < off[e+1]) and t = a_row[p]:
 *   Y[p, n] = s_tA s_tW sum_c G_A[t,c] s_bA[t,c] G_W[e,n,c] s_bW[e,n,c]
 *           + s_tW sum_j resid[t, j] G_W[e,n,idx_j] s_bW[e,n,idx_j]
 * i.e. deq(qA) deq(qW_e)^T plus the bf16 residual of the selected channels
 * times the dequantized weight columns.  fp32 accumulation.
 * Epilogue NVQ_EPI_NONE writes Y (bf16 [rows, N] and/or fp32 [rows, N]);
 * NVQ_EPI_SWIGLU writes h = bf16(silu(Y[:, :N/2]) * Y[:, N/2:]) [rows, N/2]
 * (out_f32, if given, still receives the full pre-activation Y).
 * Path NVQ_GEMM_DEQ16 (what NVQ_GEMM_AUTO selects) dequantizes each NVFP4 tile
 * exactly to fp16 and feeds fp16 MFMA, in 128-row tiles; NVQ_GEMM_DEQ16_WIDE
 * is the same arithmetic in 256-row tiles with both operands dequantized once
 * per workgroup (an evaluated alternative; slower here).  NVQ_GEMM_FP8_BLOCK
 * runs one FP8 MFMA per
 * 16-element block on the raw E2M1 magnitudes and applies both block scales to
 * the block product in fp32 (the evaluated alternative; same result to
 * rounding, slower).  K % 128 == 0; k % 8 == 0. */
enum { NVQ_EPI_NONE = 0, NVQ_EPI_SWIGLU = 1 };
enum { NVQ_GEMM_AUTO = 0, NVQ_GEMM_DEQ16 = 1, NVQ_GEMM_FP8_BLOCK = 2, NVQ_GEMM_DEQ16_WIDE = 3 };

typedef struct nvq_moe_gemm_args {
  size_t struct_size;            /* sizeof(nvq_moe_gemm_args) */
  int64_t rows;                  /* P: sorted rows */
  int64_t K, N, E;
  int64_t a_rows;                /* rows of the A record (tokens) */
  const int32_t* a_row;          /* [rows] A row of each sorted row; NULL = identity */
  const int32_t* expert_offsets; /* [E+1] */
  const uint8_t* a_codes;        /* [a_rows, K/2] */
  const uint8_t* a_scales;       /* [a_rows, K/16] */
  const float* a_tensor_scale;   /* [1] */
  const uint16_t* a_resid;       /* [a_rows, k] bf16 compensation operand (k > 0) */
  const int32_t* comp_idx;       /* [k] selected channels */
  int32_t k;                     /* multiple of 8; 0 disables the compensation */
  const uint8_t* w_codes;        /* [E, N, K/2] */
  const uint8_t* w_scales;       /* [E, N, K/16] */
  const float* w_tensor_scale;   /* [E] */
  int32_t epilogue;
  int32_t path;
  uint16_t* out_bf16;            /* [rows, N] or [rows, N/2] (SWIGLU); nullable if out_f32 */
  float* out_f32;                /* [rows, N] fp32 pre-epilogue; nullable */
  void* ws;
  size_t ws_bytes;
  int32_t a_row_div;             /* > 0: A row of sorted row p is a_row[p] / a_row_div
                                    (pass sorted pair ids with topk); 0: a_row[p] */
  /* Optional, read only when struct_size covers them: the channel-major copy of
   * the weight record made by nvfp4_channel_major.  When both are set the
   * compensation columns are gathered from it (the k selected channels are k
   * contiguous rows there) instead of from every row of w_codes. */
  const uint8_t* w_codes_cm;     /* [E, K, N/2] or NULL */
  const uint8_t* w_scales_cm;    /* [E, K/16, N] or NULL */
  /* Optional, read only when struct_size covers it: with NVQ_EPI_SWIGLU, a
   * device fp32 word (4-byte aligned) that receives max |h| over every row
   * the call writes, taken on the stored bf16 values (the call clears it
   * first; 0 for no rows).  Passed as amax_in to nvfp4_quantize of h, it
   * replaces that call's own amax pass with an identical result (a maximum
   * does not depend on order).  NULL: not computed.  NVQ_EINVAL with another
   * epilogue.  Calls sharing the word must be ordered on one stream. */
  float* h_amax;
  /* Optional, read only when struct_size covers them: the layer's combine
   * fused into this call (NVQ_EPI_NONE, path DEQ16 or AUTO; out_bf16 needed):
   * comb_out[t, n] = bf16( sum_j comb_weights[t, j] * out_bf16[comb_pos[t*topk
   * + j], n] ), j ascending, fp32 -- the same values as nvq_moe_combine on this
   * call's bf16 output, bit for bit (QUADS §2.2-B asks for the correction in
   * fused kernels).  comb_pair [rows] is the sorted pair id of each row (token
   * = pair / comb_topk), comb_pos [comb_T, comb_topk] the permutation's inverse
   * map (pos < 0: dropped pair), comb_weights [comb_T, comb_topk].  Each output
   * row piece is written by the last workgroup to finish a row of that token
   * (arrival counters in the workspace; moe_gemm_workspace_bytes_comb).
   * comb_out NULL: no combine. */
  const int32_t* comb_pair;
  const int32_t* comb_pos;
  const float* comb_weights;
  int64_t comb_T;
  int32_t comb_topk;
  uint16_t* comb_out;
} nvq_moe_gemm_args;

/* Channel-major copy of an NVFP4 weight record (same codes and scales, other
 * layout), for the compensation gather of moe_grouped_gemm_w4a4_comp: the
 * correction multiplies the residual by the weight columns of the selected
 * channels (QUADS §2.2-B), and in the row-major record one column touches
 * every weight row.  Built once per weight version (the rollout's weights are
 * static between syncs).
 *   codes  [batch, N, K/2] (even element in the low nibble) -> codes_cm [batch, K, N/2]
 *          (row n even in the low nibble)
 *   scales [batch, N, K/16]                                -> scales_cm [batch, K/16, N]
 * N % 16 == 0, K % 16 == 0, 1 <= batch <= 65535; codes and codes_cm 8-byte
 * aligned.  Device pointers, caller-owned, no overlap; asynchronous on stream.
 * Errors: NVQ_EINVAL (null pointer), NVQ_ESHAPE, NVQ_EALIGN; nothing is
 * launched then. */
int nvfp4_channel_major(const uint8_t* codes, const uint8_t* scales, int64_t batch, int64_t N,
                        int64_t K, uint8_t* codes_cm, uint8_t* scales_cm, void* stream);

/* Workspace: tile table plus the packed compensation weights [E, N, k16] bf16;
 * the _comb variant also holds the fused combine's arrival counters (T tokens). */
size_t moe_gemm_workspace_bytes(int64_t rows, int64_t E, int64_t N, int32_t k);
size_t moe_gemm_workspace_bytes_comb(int64_t rows, int64_t E, int64_t N, int32_t k, int64_t T);
int moe_grouped_gemm_w4a4_comp(const nvq_moe_gemm_args* args, void* stream);

/* ------------------------------------------------------------------------ */
/* Asymmetric W4A16 QAT grouped GEMMs (QUADS §2.2-A; TRACE "L'idée centrale"):
 * the weight is the dequantized NVFP4 record W^_e = deq(codes, scales, s_t)
 * taken as-is from the rollout (its rounding is reused, not recomputed);
 * activations stay bf16.  Identity straight-through gradient.
 *   FWD   y[p, n]  = sum_c x[a_row[p], c] W^_e[n, c]        -> [rows, N]
 *   DGRAD dx[p, c] = sum_n dy[p, n] W^_e[n, c]              -> [rows, K]
 *   WGRAD dw[e, n, c] (+)= sum_{p of e} dy[p, n] x[a_row[p], c]  -> [E, N, K] fp32
 * fp32 accumulation. */
enum { NVQ_QAT_FWD = 0, NVQ_QAT_DGRAD = 1, NVQ_QAT_WGRAD = 2 };

typedef struct nvq_qat_gemm_args {
  size_t struct_size;            /* sizeof(nvq_qat_gemm_args) */
  int32_t mode;
  int32_t accumulate;            /* WGRAD: 1 adds to dw, 0 overwrites */
  int64_t rows, K, N, E;
  int64_t x_rows;
  const int32_t* a_row;          /* [rows] row of x for each sorted row; NULL = identity */
  const int32_t* expert_offsets; /* [E+1] */
  const uint16_t* x;             /* [x_rows, K] bf16 (FWD, WGRAD) */
  const uint16_t* dy;            /* [rows, N] bf16 (DGRAD, WGRAD) */
  const uint8_t* w_codes;        /* [E, N, K/2] */
  const uint8_t* w_scales;       /* [E, N, K/16] */
  const float* w_tensor_scale;   /* [E] */
  uint16_t* out_bf16;            /* FWD y / DGRAD dx, nullable if out_f32 */
  float* out_f32;                /* FWD y / DGRAD dx fp32, nullable */
  float* dw;                     /* WGRAD [E, N, K] */
  void* ws;
  size_t ws_bytes;
} nvq_qat_gemm_args;

size_t qat_gemm_workspace_bytes(int64_t rows, int64_t E);
int qat_fakequant_gemm_w4a16(const nvq_qat_gemm_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVQ_H */
