/*
 * bsq.h -- block-scaled quantized linear layer (fp8r / nvfp4) on AMD gfx950.
 *
 * Computes bf16 Y = X W^T for a linear layer whose weights are stored in one
 * of two block-scaled formats, as the "BFL (fp8r / nvfp4)" page of the
 * diffusers quantization docs defines them (scheme list):
 *
 *   fp8r  : W is E4M3 [N][K] with one fp32 scale per row (output channel);
 *           activations are quantized to E4M3 per row (token) at run time.
 *   nvfp4 : W is E2M1 packed two per byte [N][K/2] with an E4M3 scale for
 *           every 16 consecutive elements of a row [N][K/16], an fp32 global
 *           scale (weight_scale_2) and a calibrated fp32 activation scale
 *           (input_scale) used to quantize activations to nvfp4 at run time.
 *
 * The same page's "Kernels" section pairs an fp8 GEMM with row-wise scales
 * (fp8r), runtime nvfp4 activation quantization before an fp4 GEMM (nvfp4),
 * and a fallback that dequantizes the weights to the compute dtype (bf16)
 * and runs a plain linear with unquantized activations.
 *
 * Conventions for every entry point:
 *  - bf16 tensors are passed as uint16_t bit patterns. Every data pointer is
 *    a DEVICE pointer (including the fp32 scalars global_scale, w_scale2 and
 *    input_scale); the caller owns all memory. The library never allocates,
 *    frees or synchronizes; work is enqueued on `stream` (NULL = default
 *    stream) and the call returns once it is enqueued.
 *  - Matrices are row-major. ldx / ldy are leading dimensions in elements;
 *    all other operands are dense ([rows][cols] with no padding).
 *  - Shapes: M, N >= 0 (0 means nothing to do and returns BSQ_OK without
 *    touching any pointer); K > 0 and K % 32 == 0; ldx >= K with ldx a
 *    multiple of 8; ldy >= N. M, N <= 2^30 and K <= 2^20.
 *  - Alignment: every data pointer 16-byte aligned, except fp32 scale
 *    vectors and scalars (4-byte) and E4M3 block-scale arrays (4-byte).
 *  - Outputs must not alias inputs.
 *  - Errors: arguments are validated on the host, in full, before any HIP
 *    call; a failed validation returns its status and enqueues nothing.
 *    BSQ_ERR_DEVICE means the current device is not gfx950 (or there is
 *    none); BSQ_ERR_HIP means a launch failed (bsq_last_hip_error() gives
 *    the HIP message for the calling thread). No exception crosses the ABI.
 *  - Determinism: the same inputs produce the same output bits; there are
 *    no atomics in any reduction.
 *  - Rounding: every fp32 step is IEEE round-to-nearest-even, with no
 *    flush-to-zero; E4M3 / E2M1 encodings round to nearest with ties to the
 *    even code, saturate at +-448 / +-6 and keep the sign of zero.
 */
#ifndef BSQ_H
#define BSQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSQ_ABI_VERSION 3

typedef enum {
  BSQ_OK = 0,
  BSQ_ERR_NULL = 1,      /* a required pointer is NULL */
  BSQ_ERR_SHAPE = 2,     /* bad M/N/K/ld, or K % 32 != 0 */
  BSQ_ERR_ALIGN = 3,     /* a pointer is not aligned as required */
  BSQ_ERR_WORKSPACE = 4, /* workspace NULL or smaller than bsq_gemm_workspace_bytes() */
  BSQ_ERR_DEVICE = 5,    /* no device, or the current device is not gfx950 */
  BSQ_ERR_HIP = 6,       /* a HIP launch failed */
  BSQ_ERR_ARG = 7        /* an invalid enum or flag value */
} bsq_status;

typedef enum { BSQ_FMT_FP8R = 1, BSQ_FMT_NVFP4 = 2 } bsq_format;

/* Keep activations in bf16 and dequantize only the weights inside the GEMM
 * (the fallback's arithmetic: "BFL (fp8r / nvfp4)", last paragraph of
 * "Kernels"), without rounding the weights to bf16 first. */
#define BSQ_WEIGHT_ONLY 0x1u

int bsq_abi_version(void);
const char* bsq_status_string(bsq_status s);
/* Message of the last HIP error seen by this thread ("" if none). */
const char* bsq_last_hip_error(void);

/*
 * Per-row E4M3 quantization ("BFL (fp8r / nvfp4)", fp8r bullet: activations
 * are quantized to E4M3 per row at run time). For each row m of X:
 *   a = max_k |x|, d = fp32(a / 448), r = fp32(1 / d),
 *   xq[m][k] = E4M3(fp32(x[m][k] * r)), x_scale[m] = d
 * (a zero row gives d = 0 and signed-zero codes). Dequantized value:
 * e4m3(xq) * d. Applied to a weight matrix W [N][K] this produces the fp8r
 * weight and its per-row weight_scale.
 *   x       [M][ldx] bf16        xq      [M][K] E4M3 codes
 *   x_scale [M] fp32
 */
bsq_status bsq_quantize_act_fp8r(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                 uint8_t* xq, float* x_scale, hipStream_t stream);

/*
 * nvfp4 quantization with a given global scale g = *global_scale
 * ("BFL (fp8r / nvfp4)", nvfp4 bullet and "Kernels" table: activations are
 * quantized to nvfp4 at run time with the calibrated input_scale):
 *   G = fp32(1 / g); per 16-element block b of a row:
 *   a_b = max |x|, sf_b = E4M3(fp32(fp32(a_b / 6) * G)),
 *   r_b = sf_b == 0 ? 0 : fp32(G / e4m3(sf_b)), q = E2M1(fp32(x * r_b)).
 * Dequantized value: e2m1(q) * e4m3(sf_b) * g. Values beyond the calibrated
 * range saturate. g must be a positive normal fp32 with 1/g finite.
 * Applied to W with g = weight_scale_2 it produces the nvfp4 weight tensors.
 *   x        [M][ldx] bf16
 *   xq       [M][K/2] packed E2M1, element 2j in the low nibble of byte j
 *   x_bscale [M][K/16] E4M3 block scales
 */
bsq_status bsq_quantize_act_nvfp4(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                  const float* global_scale, uint8_t* xq, uint8_t* x_bscale,
                                  hipStream_t stream);

/*
 * Calibrate an nvfp4 global scale: *out_scale = fp32(amax(X) / (6 * 448)),
 * or 1.0 when X is all zeros, so that the tensor maximum maps onto the
 * largest nvfp4 magnitude (the calibrated input_scale / weight_scale_2 of
 * the nvfp4 bullet). Needs a workspace of bsq_calibrate_workspace_bytes(M, K)
 * bytes (4-byte aligned). M must be > 0.
 */
size_t bsq_calibrate_workspace_bytes(int64_t M, int64_t K);
bsq_status bsq_calibrate_global_scale(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                      float* out_scale, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* Workspace the GEMM entry points need (quantized activations):
 *   fp8r:  M*K + 4*M bytes, nvfp4: M*K/2 + M*K/16 bytes (each part padded
 *   to 256 bytes); 0 with BSQ_WEIGHT_ONLY. The workspace pointer of
 *   bsq_gemm_fp8r and bsq_gemm_nvfp4 must be 256-byte aligned (BSQ_ERR_ALIGN
 *   otherwise; torch's and hipMalloc's allocations are); it may be NULL when
 *   the size is 0. */
size_t bsq_gemm_workspace_bytes(bsq_format f, int64_t M, int64_t N, int64_t K, uint32_t flags);

/*
 * fp8r linear ("BFL (fp8r / nvfp4)", fp8r bullet and "Kernels" table: fp8
 * GEMM with row-wise scales). Default (W8A8): quantizes X per row into the
 * workspace (as bsq_quantize_act_fp8r), then
 *   y[m][n] = bf16( (sum_k e4m3(xq[m][k]) * e4m3(w[n][k])) * sx[m] * w_scale[n] )
 * with fp32 accumulation. With BSQ_WEIGHT_ONLY (W8A16):
 *   y[m][n] = bf16( (sum_k x[m][k] * e4m3(w[n][k])) * w_scale[n] ).
 *   x [M][ldx] bf16, w [N][K] E4M3, w_scale [N] fp32, y [M][ldy] bf16
 */
bsq_status bsq_gemm_fp8r(const uint16_t* x, int64_t ldx, const uint8_t* w, const float* w_scale,
                         uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, uint32_t flags,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * bsq_gemm_fp8r for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, kernels and output bits as bsq_gemm_fp8r, without the
 * workspace arguments. The quantized activations go to a scratch array that
 * the library holds on each GPU it runs on, of BSQ_NOALLOC_MAX_BYTES (64 MiB),
 * until the process ends; a shape whose workspace (bsq_gemm_workspace_bytes)
 * exceeds it returns BSQ_ERR_WORKSPACE and enqueues nothing. Calls no hipMalloc / hipFree.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap on
 * one GPU (other streams, other host threads) race and must be ordered by
 * the caller. With BSQ_WEIGHT_ONLY no scratch is used.
 */
#define BSQ_NOALLOC_MAX_BYTES ((size_t)64 << 20)
bsq_status bsq_gemm_fp8r_noalloc(const uint16_t* x, int64_t ldx, const uint8_t* w, const float* w_scale,
                                 uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, uint32_t flags,
                                 hipStream_t stream);

/*
 * nvfp4 linear ("BFL (fp8r / nvfp4)", nvfp4 bullet and "Kernels" table).
 * Default (W4A4): quantizes X to nvfp4 with *input_scale into the workspace
 * (as bsq_quantize_act_nvfp4), then
 *   y[m][n] = bf16( (sum_k xh[m][k] * wh[n][k]) * (*input_scale) * (*w_scale2) )
 * with xh = e2m1 * e4m3(block scale) (exact) for both operands and fp32
 * accumulation. With BSQ_WEIGHT_ONLY (W4A16, input_scale may be NULL):
 *   y[m][n] = bf16( (sum_k x[m][k] * wh[n][k]) * (*w_scale2) ).
 *   x [M][ldx] bf16, w [N][K/2] packed E2M1, w_bscale [N][K/16] E4M3,
 *   w_scale2 [1] fp32, input_scale [1] fp32, y [M][ldy] bf16
 */
bsq_status bsq_gemm_nvfp4(const uint16_t* x, int64_t ldx, const uint8_t* w, const uint8_t* w_bscale,
                          const float* w_scale2, const float* input_scale, uint16_t* y, int64_t ldy,
                          int64_t M, int64_t N, int64_t K, uint32_t flags, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * The same two GEMMs on activations that are already quantized (laid out as
 * bsq_quantize_act_fp8r / bsq_quantize_act_nvfp4 write them), for callers
 * that quantize X elsewhere -- e.g. once for several linears sharing an
 * input. Arithmetic, layouts and rounding are those of the W8A8 and W4A4
 * paths above; no workspace is needed.
 *   bsq_gemm_fp8r_q : xq [M][K] E4M3, x_scale [M] fp32 (16-byte aligned xq)
 *   bsq_gemm_nvfp4_q: xq [M][K/2] packed E2M1, x_bscale [M][K/16] E4M3,
 *                     input_scale [1] fp32
 */
bsq_status bsq_gemm_fp8r_q(const uint8_t* xq, const float* x_scale, const uint8_t* w, const float* w_scale,
                           uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t stream);
bsq_status bsq_gemm_nvfp4_q(const uint8_t* xq, const uint8_t* x_bscale, const float* input_scale,
                            const uint8_t* w, const uint8_t* w_bscale, const float* w_scale2, uint16_t* y,
                            int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * Grouped launch: several independent pre-quantized linears of one scheme in
 * one kernel launch (the four linears of a joint transformer block -- qkv,
 * proj, MLP up and down -- whose 28 blocks the FLUX 3 Image Klein release
 * page, section one, describes; each linear's arithmetic is that of the
 * "BFL (fp8r / nvfp4)" scheme list and "Kernels" table, as above). One grid
 * holds every problem's work, longest K first, so one problem's last round
 * overlaps the next problem's first instead of leaving compute units idle
 * between launches, and each launch's fixed cost is paid once:
 *  - problems that alone would run on the tiled kernels (several hundred
 *    tokens and more) share one grid of them when the group fills the 256
 *    compute units (at least one round of 128 x 128 tiles two to a unit --
 *    half a round for nvfp4 -- or two rounds of 256 x 192 / 256 x 256
 *    tiles); each y is
 *    then, bit for bit, what bsq_gemm_fp8r_q (format BSQ_FMT_FP8R) or
 *    bsq_gemm_nvfp4_q (BSQ_FMT_NVFP4) returns for its operands;
 *  - a group of at most 64 tokens in which some problem alone would take the
 *    few-token kernels runs as one grid of the few-token kernels, with one
 *    workgroup shape (waves splitting K, activation blocks) for the whole
 *    group: each y holds the same products summed over K in that shape's
 *    order -- bit for bit the single call's where the single call runs the
 *    same shape on the few-token kernels, otherwise (another shape, or the
 *    tiled kernels alone) within the GEMM tolerance of it;
 *  - anything else (fp8r with K % 128 != 0, nvfp4 with K % 256 != 0, fewer
 *    tiles, 65 or more tokens on mixed routes) runs one launch per problem,
 *    in the order given, with the single calls' results.
 * Every grouped call is deterministic: the same group gives the same bits.
 *   problems : host array of `count` descriptors (read during the call only);
 *              count 0 is a no-op, 1 <= count <= BSQ_MAX_GROUP otherwise
 *   per problem, with the layouts and alignment of the two entry points:
 *     xq       fp8r [M][K] E4M3 | nvfp4 [M][K/2] packed E2M1
 *     x_scale  fp8r fp32 [M] row scales | nvfp4 E4M3 [M][K/16] block scales
 *     input_scale  nvfp4 [1] fp32 | fp8r NULL
 *     w        fp8r [N][K] E4M3 | nvfp4 [N][K/2]
 *     w_scale  fp8r fp32 [N] | nvfp4 E4M3 [N][K/16]
 *     w_scale2 nvfp4 [1] fp32 | fp8r NULL
 *     y [M][ldy] bf16; problems with M == 0 or N == 0 are skipped.
 * No output may alias another problem's output or any input. Errors:
 * BSQ_ERR_ARG for an unknown format, count < 0 or count > BSQ_MAX_GROUP, or a
 * non-NULL input_scale / w_scale2 with fp8r; otherwise the statuses of the
 * two entry points. Every problem is validated before anything is enqueued.
 */
#define BSQ_MAX_GROUP 8
typedef struct {
  const uint8_t* xq;
  const void* x_scale;
  const float* input_scale;
  const uint8_t* w;
  const void* w_scale;
  const float* w_scale2;
  uint16_t* y;
  int64_t ldy;
  int64_t M, N, K;
} bsq_gemm_problem;
bsq_status bsq_gemm_grouped_q(bsq_format format, const bsq_gemm_problem* problems, int count, hipStream_t stream);

/*
 * Grouped launch of weight-only linears (BSQ_WEIGHT_ONLY: bf16 activations
 * times the dequantized weights, the fallback's arithmetic of the "BFL (fp8r /
 * nvfp4)" page, last paragraph of "Kernels"). Problem i's y is what
 * bsq_gemm_fp8r (format BSQ_FMT_FP8R) or bsq_gemm_nvfp4 (BSQ_FMT_NVFP4) with
 * BSQ_WEIGHT_ONLY returns for it. A group whose problems all take the
 * few-token route alone runs as one grid of the few-token kernels, with one
 * workgroup shape for the group (bit for bit the single call's where that call
 * runs the same shape, otherwise within the GEMM tolerance of it); any other
 * group runs one launch per problem, in the order given, with the single
 * calls' results. Deterministic.
 *   problems : host array of `count` descriptors (read during the call only);
 *              count 0 is a no-op, 1 <= count <= BSQ_MAX_GROUP otherwise
 *   per problem: x [M][ldx] bf16 (ldx >= K, ldx % 8 == 0); w, w_scale as
 *     bsq_gemm_fp8r (E4M3 [N][K], fp32 [N]; w_scale2 NULL) or bsq_gemm_nvfp4
 *     (packed E2M1 [N][K/2], E4M3 [N][K/16], w_scale2 [1] fp32); y [M][ldy];
 *     problems with M == 0 or N == 0 are skipped.
 * Errors: BSQ_ERR_ARG for an unknown format, count < 0 or count >
 * BSQ_MAX_GROUP, or a non-NULL w_scale2 with fp8r; otherwise the statuses of
 * the two entry points. Every problem is validated before anything is enqueued.
 */
typedef struct {
  const uint16_t* x;
  int64_t ldx;
  const uint8_t* w;
  const void* w_scale;
  const float* w_scale2;
  uint16_t* y;
  int64_t ldy;
  int64_t M, N, K;
} bsq_weight_only_problem;
bsq_status bsq_gemm_grouped_weight_only(bsq_format format, const bsq_weight_only_problem* problems, int count,
                                        hipStream_t stream);

/*
 * W4A4 linear whose output is also handed to the next quantized linear in
 * nvfp4 ("BFL (fp8r / nvfp4)": every quantized linear quantizes its input at
 * run time; here the producing GEMM does it in its epilogue, where the
 * 16-element blocks -- along this N, the next linear's K -- lie inside one
 * output tile). Y is the bsq_gemm_nvfp4_q result; yq / y_bscale are exactly
 * what bsq_quantize_act_nvfp4(Y, y_scale) returns for that bf16 Y:
 *   xq, x_bscale, input_scale, w, w_bscale, w_scale2: as bsq_gemm_nvfp4_q
 *   y_scale   [1] fp32: global scale of Y's encoding (the next input_scale)
 *   yq        [M][N/2] packed E2M1 (16-byte aligned), y_bscale [M][N/16] E4M3
 *   y         [M][ldy] bf16, or NULL to skip writing the bf16 output
 * Requires N % 32 == 0 (BSQ_ERR_SHAPE otherwise). Shapes that the fused
 * kernels do not cover (K % 256 != 0 beyond the few-token range) run the
 * GEMM and then the quantizer; with y == NULL they need a workspace of
 * bsq_gemm_nvfp4_quantize_y_workspace_bytes(M, N, K, 0) bytes (16-byte
 * aligned, 0 for every other shape); the query with with_y != 0 returns 0.
 */
size_t bsq_gemm_nvfp4_quantize_y_workspace_bytes(int64_t M, int64_t N, int64_t K, int with_y);
bsq_status bsq_gemm_nvfp4_q_quantize_y(const uint8_t* xq, const uint8_t* x_bscale, const float* input_scale,
                                       const uint8_t* w, const uint8_t* w_bscale, const float* w_scale2,
                                       const float* y_scale, uint8_t* yq, uint8_t* y_bscale, uint16_t* y,
                                       int64_t ldy, int64_t M, int64_t N, int64_t K, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/*
 * Quantized-output linears in either format ("BFL (fp8r / nvfp4)": every
 * quantized linear quantizes its input at run time -- fp8r per row to E4M3,
 * nvfp4 per 16-block with its calibrated input_scale; here the producing GEMM
 * hands the next linear its input already encoded):
 *   bsq_gemm_fp8r_q_quantize_y       : the W8A8 linear of bsq_gemm_fp8r_q,
 *   bsq_gemm_nvfp4_q_quantize_y_fp8r : the W4A4 linear of bsq_gemm_nvfp4_q,
 * whose bf16 output Y (bit for bit that entry point's) is also returned
 * encoded for the next linear, exactly as the activation quantizers encode
 * that Y:
 *   out_format BSQ_FMT_NVFP4: y_global [1] fp32 = the next linear's
 *     input_scale; yq [M][N/2] packed E2M1; yq_scale uint8 [M][N/16] E4M3
 *     (= bsq_quantize_act_nvfp4(Y, y_global));
 *   out_format BSQ_FMT_FP8R: y_global must be NULL; yq [M][N] E4M3;
 *     yq_scale fp32 [M] row scales (= bsq_quantize_act_fp8r(Y)).
 * (bsq_gemm_nvfp4_q_quantize_y above is the W4A4 producer with nvfp4 output.)
 * The nvfp4 blocks lie inside an output tile and are encoded in the GEMM's
 * epilogue. An fp8r row scale needs the whole row: the epilogue records each
 * row's maximum over every 64-column segment of its tile, and one pass then
 * takes each row's maximum of those (exact, so the result does not depend on
 * the order) and encodes Y. Few-token shapes (and W4A4 with K % 256 != 0) run
 * the GEMM and then the quantizer.
 *   y [M][ldy] bf16 (ldy % 8 == 0), or NULL to skip writing it; yq 16-byte
 *   aligned; N % 32 == 0 (BSQ_ERR_SHAPE otherwise).
 * Workspace: bsq_gemm_quantize_y_workspace_bytes(out_format, M, N, y != NULL)
 * bytes, 256-byte aligned (NULL when 0): a bf16 Y when y is NULL, and for
 * fp8r output the fp32 row maxima [M][ceil(N/64)].
 */
size_t bsq_gemm_quantize_y_workspace_bytes(bsq_format out_format, int64_t M, int64_t N, int with_y);
bsq_status bsq_gemm_fp8r_q_quantize_y(const uint8_t* xq, const float* x_scale, const uint8_t* w, const float* w_scale,
                                      bsq_format out_format, const float* y_global, uint8_t* yq, void* yq_scale,
                                      uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);
bsq_status bsq_gemm_nvfp4_q_quantize_y_fp8r(const uint8_t* xq, const uint8_t* x_bscale, const float* input_scale,
                                            const uint8_t* w, const uint8_t* w_bscale, const float* w_scale2,
                                            uint8_t* yq, float* y_rowscale, uint16_t* y, int64_t ldy, int64_t M,
                                            int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                                            hipStream_t stream);

/*
 * Weight-only linears (the BSQ_WEIGHT_ONLY semantics of bsq_gemm_nvfp4 and
 * bsq_gemm_fp8r: bf16 activations, W4A16 or W8A16) whose output is also
 * handed to the next quantized linear, encoded exactly as the activation
 * quantizers encode that bf16 Y ("BFL (fp8r / nvfp4)": every quantized linear
 * quantizes its input at run time; a weight-only producer can feed one):
 *   w_format BSQ_FMT_NVFP4: w [N][K/2] packed E2M1, w_scale = E4M3 block
 *     scales uint8 [N][K/16], w_scale2 [1] fp32 (K % 64 == 0 for the fused
 *     tiled route; other K run the GEMM, then the quantizer);
 *   w_format BSQ_FMT_FP8R: w [N][K] E4M3, w_scale = fp32 row scales [N],
 *     w_scale2 must be NULL;
 *   x [M][ldx] bf16 (ldx % 8 == 0);
 *   out_format, y_global, yq, yq_scale, y, ldy, workspace: as
 *     bsq_gemm_fp8r_q_quantize_y (same workspace query,
 *     bsq_gemm_quantize_y_workspace_bytes).
 * Y is, bit for bit, what bsq_gemm_nvfp4 / bsq_gemm_fp8r with
 * BSQ_WEIGHT_ONLY return. On the tiled route the nvfp4 blocks are encoded in
 * the GEMM's epilogue and an fp8r encoding takes the epilogue's row maxima and
 * one pass; few-token and decode-GEMM shapes run the GEMM and then the
 * quantizer. Errors: BSQ_ERR_ARG for an unknown format or a w_scale2 with fp8r
 * weights, otherwise as bsq_gemm_fp8r_q_quantize_y.
 */
bsq_status bsq_gemm_weight_only_quantize_y(bsq_format w_format, const uint16_t* x, int64_t ldx, const uint8_t* w,
                                           const void* w_scale, const float* w_scale2, bsq_format out_format,
                                           const float* y_global, uint8_t* yq, void* yq_scale, uint16_t* y,
                                           int64_t ldy, int64_t M, int64_t N, int64_t K, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream);

/*
 * Low-rank adapter (LoRA) side path on the quantized linear. "FLUX 3 Image
 * Klein vs Qwen-Image-2.1" (model overview) and the FLUX 3 Image Klein
 * open-source release page (section three, speed figures): the quantized
 * model can run with a LoRA attached, at about 5 % more generation time. The
 * pages give no arithmetic; these entry points compute the standard adapter
 *   y = linear(x) + s * (x A^T) B^T
 * where linear(x) is exactly what bsq_gemm_fp8r / bsq_gemm_nvfp4 compute for
 * the same arguments and flags, the adapter reads the unquantized bf16 x,
 *   lora_a [rank][K] bf16 (down projection), lora_b [N][rank] bf16 (up
 *   projection), 1 <= rank <= 128, lora_scale s a finite fp32 host value
 *   (alpha / rank times the adapter's strength).
 * Arithmetic: T = bf16(s * sum_k x[m][k] a[j][k]) (fp32 accumulation), then
 *   y[m][n] = bf16( base_acc[m][n] * (the linear's scales) + sum_j T[m][j] b[n][j] )
 * with the adapter sum accumulated in fp32 onto the scaled base accumulator,
 * so the output is rounded once. T is the only other rounding. On the tiled
 * W4A4 path (K % 256 == 0 beyond the few-token range) the output scale
 * alpha = input_scale * w_scale2 is folded into T instead: T = bf16(s / alpha
 * * sum ...) is accumulated with the base and the sum scaled by alpha, which
 * requires alpha to be a positive normal fp32 number (calibrated scales are).
 * Workspace: bsq_lora_workspace_bytes(f, M, N, K, rank, flags) bytes,
 * 256-byte aligned: the linear's workspace, T [M][rank], and for shapes where
 * the down projection splits K over workgroups its fp32 partial products.
 * Extra shape rules: ldx < 2^24; M * rank and N * rank below 2^29.
 * BSQ_ERR_ARG for a non-finite lora_scale; lora_a / lora_b 16-byte aligned.
 */
size_t bsq_lora_workspace_bytes(bsq_format f, int64_t M, int64_t N, int64_t K, int64_t rank, uint32_t flags);
bsq_status bsq_gemm_fp8r_lora(const uint16_t* x, int64_t ldx, const uint8_t* w, const float* w_scale,
                              const uint16_t* lora_a, const uint16_t* lora_b, int64_t rank, float lora_scale,
                              uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, uint32_t flags,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);
bsq_status bsq_gemm_nvfp4_lora(const uint16_t* x, int64_t ldx, const uint8_t* w, const uint8_t* w_bscale,
                               const float* w_scale2, const float* input_scale, const uint16_t* lora_a,
                               const uint16_t* lora_b, int64_t rank, float lora_scale, uint16_t* y, int64_t ldy,
                               int64_t M, int64_t N, int64_t K, uint32_t flags, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);
/*
 * The adapter's down projection alone, as the entry points above compute it:
 *   t[m][j] = bf16( s * sum_k x[m][k] a[j][k] ),  t [M][rank] bf16 (16-byte aligned)
 * x [M][ldx] bf16 (rules as for the quantizers, plus ldx < 2^24), lora_a and
 * rank as above. Workspace: bsq_lora_down_workspace_bytes(M, K, rank) bytes,
 * 16-byte aligned (0, and workspace may be NULL, when K is not split).
 */
size_t bsq_lora_down_workspace_bytes(int64_t M, int64_t K, int64_t rank);
bsq_status bsq_lora_down(const uint16_t* x, int64_t ldx, const uint16_t* lora_a, int64_t M, int64_t K,
                         int64_t rank, float lora_scale, uint16_t* t, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * Fallback dequantization to bf16 ("BFL (fp8r / nvfp4)", last paragraph of
 * "Kernels": on other devices the weights are dequantized to the compute
 * dtype every forward and the layer runs as a regular linear):
 *   nvfp4: w_bf16[n][k] = bf16( fp32( (e2m1 * e4m3(sf)) * (*w_scale2) ) )
 *          (w_scale is the [N][K/16] E4M3 block-scale array)
 *   fp8r:  w_bf16[n][k] = bf16( fp32( e4m3(w) * w_scale[n] ) )
 *          (w_scale is the [N] fp32 row-scale vector; w_scale2 must be NULL)
 * Bit-exact: every step is one rounding as written.
 */
bsq_status bsq_dequant_to_bf16(bsq_format f, const uint8_t* w, const void* w_scale,
                               const float* w_scale2, int64_t N, int64_t K, uint16_t* w_bf16,
                               hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BSQ_H */
