/*
 * w4a4.h -- C ABI of the MI355X (gfx950) quantized-linear library.
 *
 * The library implements the deployment path of a low-bit linear layer as
 * the pages on world-action / vision-language-action quantization describe
 * it: per-channel smoothing, a block-64 Walsh-Hadamard rotation, dynamic
 * per-token 4-bit (or 8-bit, or NVFP4) activation quantization, a W4A4 (or
 * W8A8, or NVFP4) GEMM with a dequantising epilogue, and an optional 16-bit
 * low-rank or kept-channel branch added to the output.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every array pointer is a DEVICE pointer (memory from hipMalloc or a
 *    PyTorch CUDA/HIP tensor) unless stated otherwise.  The caller owns every
 *    buffer; the library never allocates, frees or keeps a pointer after it
 *    returns.
 *  - Every call is asynchronous on ``stream`` (a hipStream_t; NULL = the
 *    null stream).  Device-side faults surface at the caller's next
 *    synchronisation.
 *  - Return value: W4A4_OK (0) or a negative w4a4_status.  All argument
 *    checks run on the host before anything is launched; on error nothing
 *    is launched and no output is written.  w4a4_last_error() returns a
 *    thread-local message describing the last failure.
 *  - Row-major storage with an explicit row stride ("ld", in elements) for
 *    floating-point inputs/outputs.  Quantized codes are dense row-major.
 *  - M == 0 or N == 0 is a valid no-op.
 *  - NaN / Inf in inputs give unspecified (but memory-safe) results.
 *
 * Packed layouts (produced by quantize_act / pack_weights, consumed by the
 * linear entry points):
 *  - INT4 : R x K/2 bytes, row-major; byte j of a row holds code 2j in its
 *           low nibble and code 2j+1 in its high nibble, two's complement
 *           (-8..7).  scales: fp32[R], one step per row.
 *  - INT8 : R x K bytes (int8 codes).  scales: fp32[R].
 *  - W4A8 activations (quantize_act with W4A4_FMT_W4A8): the INT8
 *           quantization, R x K bytes, with every aligned group of 8 codes
 *           k0..k0+7 stored as k0, k0+2, k0+4, k0+6, k0+1, k0+3, k0+5, k0+7
 *           (the order in which INT4 weight codes unpack to bytes, so the
 *           matrix cores take both operands without reordering).
 *           scales: fp32[R].  W4A8 weights are INT4.
 *  - FP8  : R x K bytes of OCP E4M3 (E4M3FN) codes, zero encoded +0.
 *           scales: fp32[R], step = fp32(amax/448).
 *  - NVFP4: R x K/2 bytes of E2M1 nibbles (same nibble order; sign bit 3,
 *           exponent bits 2..1 with bias 1, mantissa bit 0).  scales:
 *           R x K/16 bytes of OCP E4M3 (E4M3FN, bias 7, max 448), one per 16
 *           consecutive K elements.  quantize_act and pack_weights write
 *           non-negative scales; the GEMM reads a byte with the sign bit
 *           set as the negated value, as the format defines it (0x7F and
 *           0xFF, NaN in E4M3FN, are never written and give NaN outputs).
 *           The fp32 tensor scale g travels in the
 *           w4a4_qdesc (quantize / pack) and in ``alpha`` (linear).
 */
#ifndef W4A4_H
#define W4A4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A4_ABI_VERSION 3
#define W4A4_MAX_BRANCH 128 /* largest branch width (rank or kept channels) */
#define W4A4_LOWRANK_MAX_PARTS 4 /* hi/lo pairs a branch ``a`` operand may hold (ra = 2 P r) */

typedef enum w4a4_status {
  W4A4_OK = 0,
  W4A4_ERR_INVALID_ARG = -1,       /* null pointer, negative size, bad stride */
  W4A4_ERR_UNSUPPORTED_SHAPE = -2, /* K not a multiple of the required block */
  W4A4_ERR_MISALIGNED = -3,        /* pointer / row stride not 16-byte aligned */
  W4A4_ERR_UNSUPPORTED_FORMAT = -4,/* format / dtype / option combination */
  W4A4_ERR_WORKSPACE = -5,         /* workspace given but smaller than required */
  W4A4_ERR_LAUNCH_FAILED = -6      /* HIP launch error (see w4a4_last_error) */
} w4a4_status;

/* Code formats. */
enum { W4A4_FMT_INT4 = 0, W4A4_FMT_INT8 = 1, W4A4_FMT_NVFP4 = 2, W4A4_FMT_W4A8 = 3, W4A4_FMT_FP8 = 4 };
/* W4A4_FMT_W4A8 names the pairing of INT8 activation codes with INT4 weight
 * codes: quantize_act writes the activations in the W4A8 layout, the
 * weights come from pack_weights with W4A4_FMT_INT4 (pack_weights rejects
 * W4A4_FMT_W4A8), and w4a8_linear / w4a4_workspace_size take the pair. */
/* Element types of float inputs / outputs.  I32 = raw integer accumulators. */
enum { W4A4_DT_F32 = 0, W4A4_DT_BF16 = 1, W4A4_DT_I32 = 2 };
/* Order of the two transforms applied before quantization. */
enum { W4A4_ORDER_SMOOTH_THEN_ROTATE = 0, W4A4_ORDER_ROTATE_THEN_SMOOTH = 1 };
/* 16-bit branch kinds. */
enum { W4A4_BRANCH_NONE = 0, W4A4_BRANCH_BF16 = 1 };

/* Quantizer descriptor.
 *  fmt          W4A4_FMT_*.
 *  fwht_block   0 (no rotation) or 64 (block Walsh-Hadamard, FoldQuantVLA
 *               contribution 2: FWHT with block size 64).  The rotation is
 *               the Sylvester-ordered Hadamard scaled by 1/8, evaluated in
 *               fp32 with butterfly stages 1, 2, 4, 8, 16, 32.
 *  order        W4A4_ORDER_*: smoothing then rotation (FoldQuantVLA's order)
 *               or rotation then smoothing (QuantWAMs Eq. 1 order, A R S^-1).
 *  tensor_scale NVFP4 only: the fp32 per-tensor scale g (> 0, finite).
 */
typedef struct w4a4_qdesc {
  int32_t fmt;
  int32_t fwht_block;
  int32_t order;
  float tensor_scale;
} w4a4_qdesc;

/* 16-bit branch fused into the linear epilogue (Q-WAM abstract: a 16-bit
 * low-rank branch next to the 4-bit complement; QuantWAMs sec. 4.2: BF16
 * bypass of kept channels).  Adds  sum_j a[m, j] * b[n, j mod r]  for
 * j < ra to every output, in fp32 after the dequantised main product.
 *  A kept-channel branch assumes the quantized operands were made with
 *  smoothing factors 0 on those channels and smoothing before the rotation
 *  (see quantize_act_gather).
 *  a   bf16, M x ra, row stride lda (elements).  For a rank-r factor product
 *      (x L1) L2 it holds the hi and lo bf16 halves of x L1 (ra = 2r, as
 *      produced by w4a4_lowrank_project), or P such pairs whose sum is
 *      x L1 (ra = 2 P r); for kept channels it holds x[:, idx] (ra = r).
 *  b   bf16, N x r, row stride ldb: L2 transposed, or W[:, idx].
 *  r   8..W4A4_MAX_BRANCH, a multiple of 8; ra is r or 2 P r with
 *      1 <= P <= W4A4_LOWRANK_MAX_PARTS.
 */
typedef struct w4a4_branch {
  int32_t kind;
  int32_t r;
  int32_t ra;
  int32_t reserved;
  const void* a;
  int64_t lda;
  const void* b;
  int64_t ldb;
} w4a4_branch;

/* quantize_act -- runtime activation quantizer.
 * FoldQuantVLA contribution 2 (channel scaling, FWHT-64, dynamic per-token
 * quantization without timestep tables) and contribution 4 (INT4
 * activations); QuantWAMs sec. 3.1 Eq. 1 (the quantizer receives A R S^-1).
 *
 *  x          M x K activations, x_dtype BF16 or F32, row stride ldx >= K.
 *  inv_smooth fp32[K] per-channel factors multiplied into x (1/s), or NULL.
 *  q          format, rotation, order; NVFP4 needs q->tensor_scale.
 *  codes      output, packed layout of q->fmt (R = M).
 *  scales     output: fp32[M] steps (INT4/INT8; step = fp32(amax/7) or
 *             fp32(amax/127), codes = clamp(rne(fp32(y/step)))), fp32[M]
 *             (FP8; step = fp32(amax/448), codes = E4M3 rne of
 *             fp32(y/step)) or M x K/16 E4M3 bytes (NVFP4).
 * Shape rules: K % 16 == 0; K % 64 == 0 when fwht_block == 64.
 * Alignment: x, codes 16-byte aligned; ldx * elem_size % 16 == 0.
 */
int quantize_act(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                 const float* inv_smooth, const w4a4_qdesc* q,
                 void* codes, void* scales, void* stream);

/* quantize_act_gather -- quantize_act that also writes the BF16 bypass
 * operand of kept channels, xo[m, j] = x[m, idx[j]] (exact), from the same
 * pass over x, so the 16-bit branch costs no second read of x (QuantWAMs
 * sec. 3.1 / 4.2: the kept channels travel on a BF16 path next to the
 * quantized ones).  Arguments as quantize_act, plus:
 *  idx  int32[r] channel indices, 1 <= r <= W4A4_MAX_BRANCH; an index
 *       outside [0, K) gives 0.
 *  xo   bf16 M x r, row stride ldo >= r: the w4a4_branch ``a`` operand
 *       (ra = r).
 * x must be BF16.  Same result as quantize_act followed by
 * w4a4_lowrank_project with idx.  Kept channels leave the quantized path
 * through smoothing factors of 0, which removes raw channels only when
 * smoothing precedes the rotation: q->order must be
 * W4A4_ORDER_SMOOTH_THEN_ROTATE (else W4A4_ERR_UNSUPPORTED_FORMAT). */
int quantize_act_gather(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                        const float* inv_smooth, const w4a4_qdesc* q, void* codes, void* scales,
                        const int32_t* idx, int64_t r, void* xo, int64_t ldo, void* stream);

/* quantize_act_lowrank -- quantize_act that also writes the low-rank branch
 * operand (Q-WAM abstract: a 16-bit low-rank branch x L1 L2 beside the
 * 4-bit complement); the workgroup that quantizes a group of rows also
 * projects them, so x comes from HBM once (the projection's read of the
 * same rows is served from cache).  Arguments as quantize_act, plus:
 *  l1t  bf16 r x K, row stride K, 16-byte aligned: L1 transposed.
 *  r    16 or 32.
 *  out  bf16 M x ldo (ldo >= 2r): T = x L1 evaluated in fp32 (exact bf16
 *       products, fp32 sums) and written as hi = bf16(T) in columns [0, r)
 *       and lo = bf16(T - hi) in [r, 2r): the w4a4_branch ``a`` operand
 *       (ra = 2r), as w4a4_lowrank_project writes it.
 * x must be BF16; K a multiple of 64, at most 4096 (a row is held in one
 * wave's registers); other shapes are W4A4_ERR_UNSUPPORTED_SHAPE (use quantize_act and
 * w4a4_lowrank_project).
 * Codes and scales are those quantize_act writes. */
int quantize_act_lowrank(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                         const float* inv_smooth, const w4a4_qdesc* q, void* codes, void* scales,
                         const void* l1t, int64_t r, void* out, int64_t ldo, void* stream);

/* quantize_act_project -- quantize_act and w4a4_lowrank_project (low-rank
 * form) in one launch (Q-WAM abstract: the 16-bit low-rank branch x L1 L2
 * beside the 4-bit complement).  Some workgroups quantize rows, the others
 * compute tiles of T = x L1; both read x (the second read mostly from
 * cache), and codes, scales and out are bit-identical to those of the two
 * separate calls.  Arguments as quantize_act, plus:
 *  l1t  bf16 r x K, row stride K, 16-byte aligned: L1 transposed.
 *  r    1 .. W4A4_MAX_BRANCH.
 *  out  bf16 M x ldo (ldo >= 2r): hi = bf16(T) in columns [0, r), lo =
 *       bf16(T - hi) in [r, 2r), as w4a4_lowrank_project writes them.
 * x must be BF16 (else W4A4_ERR_UNSUPPORTED_FORMAT); K a multiple of 16
 * (64 with the rotation) and at most 5120 (one wave per row), else
 * W4A4_ERR_UNSUPPORTED_SHAPE (use the two calls). */
int quantize_act_project(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                         const float* inv_smooth, const w4a4_qdesc* q, void* codes, void* scales,
                         const void* l1t, int64_t r, void* out, int64_t ldo, void* stream);

/* pack_weights -- offline weight packing with the inverse transform folded
 * in (FoldQuantVLA contribution 1: every activation transform is undone
 * inside the weight that consumes it; QuantWAMs sec. 3.3, after Eq. 14: the
 * rotation shared by a layer group lives in its weights).  Same arithmetic as
 * quantize_act on the N rows of W (one scale per output channel), with the
 * smoothing factors s multiplied instead of 1/s.
 *  w       N x K weights (BF16 or F32), row stride ldw.
 *  smooth  fp32[K] factors s, or NULL.
 *  codes / scales as quantize_act with R = N.
 */
int pack_weights(const void* w, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw,
                 const float* smooth, const w4a4_qdesc* q,
                 void* codes, void* scales, void* stream);

/* pack_weights_gptq -- pack_weights with GPTQ-style rounding instead of
 * round-to-nearest (QuantWAMs sec. 3.3: the error feedback of GPTQ is weighted by
 * the layer's activation second moments, per-column scores at most decide
 * the order in which GPTQ visits the columns, and the Hadamard transform,
 * shared by every context, is folded into W before rounding).  The
 * rows are transformed as in pack_weights and keep its per-row steps; the
 * columns are then rounded in the order perm (NULL: natural), each
 * column's error over u[t][t] updating every later column v by
 * w -= err * u[t][v] in float64 (one product, one subtraction, in t
 * order).
 *  q        fmt INT4 or INT8 (W4A8 weights are INT4).
 *  u        device float64 K x K, row-major: the upper Cholesky factor of
 *           (Sigma + lambda I)^-1 with Sigma, the activation second moments
 *           in the quantizer's transformed space, in processing order
 *           (calibration data; only the upper triangle is read, u[t][t] > 0).
 *  perm     device int32[K], a permutation, or NULL.
 *  workspace device scratch of at least w4a4_gptq_workspace_size(N, K)
 *           bytes, 256-byte aligned (required).
 * Shape rules: as pack_weights, and K % 32 == 0.  Offline: many launches,
 * not for the hot path. */
int pack_weights_gptq(const void* w, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw,
                      const float* smooth, const w4a4_qdesc* q, const double* u,
                      const int32_t* perm, void* codes, void* scales,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace pack_weights_gptq needs for N x K weights. */
size_t w4a4_gptq_workspace_size(int64_t N, int64_t K);

/* w4a4_linear -- y = alpha * dequant(A_codes . W_codes^T) (+ branch).
 * FoldQuantVLA contribution 4 (W4A4 projections) and overview (integer
 * GEMMs with per-token / per-channel scales); QuantWAMs sec. 4.2 (NVFP4
 * W4A4 kernels, BF16 bypass).
 *  fmt      W4A4_FMT_INT4: exact int32 accumulation of int4 x int4, then
 *           y = fp32(fp32(acc) * a_scales[m]) * w_scales[n] * alpha.
 *           W4A4_FMT_NVFP4: sum of E2M1*E4M3 products (exact operands,
 *           fp32 accumulation), times alpha = fp32(g_a * g_w).
 *  a_codes / a_scales   M rows (M <= 2^28) from quantize_act; w_codes /
 *           w_scales N rows from pack_weights (same fmt, same K; K a
 *           multiple of 64, at most 65536).
 *  br       NULL or a w4a4_branch (kind NONE or BF16).
 *  y        M x N output, y_dtype F32 or BF16 (round to nearest even) with
 *           row stride N <= ldy <= 2^22 elements; y_dtype I32 writes the raw integer
 *           accumulators (INT formats, no branch, alpha ignored).
 *  workspace / workspace_bytes  optional device scratch (NULL / 0 for
 *           none).  Few-token shapes (M <= 64) whose unsplit grid would be
 *           small (few output channels, long K) split K over workgroups
 *           when it is given: int32 partial tiles go to the workspace and a
 *           second kernel adds them (exact) and runs the epilogue.  Size
 *           from w4a4_workspace_size; no initialisation needed; contents
 *           are overwritten.  Calls sharing one workspace must be ordered
 *           on one stream.  A non-NULL workspace smaller than required is
 *           W4A4_ERR_WORKSPACE.
 * Shape rules: K % 64 == 0.  Alignment: codes 16-byte aligned.
 */
int w4a4_linear(const void* a_codes, const void* a_scales,
                const void* w_codes, const void* w_scales,
                int64_t M, int64_t N, int64_t K, int32_t fmt, float alpha,
                const w4a4_branch* br, void* y, int32_t y_dtype, int64_t ldy,
                void* workspace, size_t workspace_bytes, void* stream);

/* w4a4_linear_noalloc -- w4a4_linear for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  Same arguments and results as the
 * linear entry point of fmt (W4A4_FMT_INT4 / NVFP4: w4a4_linear, INT8:
 * w8a8_linear, W4A8: w4a8_linear, FP8: fp8_linear) given a workspace of
 * w4a4_workspace_size bytes, but without a workspace argument: when the
 * few-token plan splits K, the int32 partial tiles go to a static device
 * buffer of W4A4_NOALLOC_SCRATCH_BYTES that the library owns, one per GPU,
 * held until the process ends.  It calls no allocator.  Every call on a GPU
 * shares that GPU's buffer: calls that can overlap on one GPU (unordered
 * streams, concurrent host threads) race and must not be issued; calls
 * ordered on one stream are fine.  No initialisation is needed (partials
 * are fully written before they are read).  A plan needing more than the
 * buffer is W4A4_ERR_WORKSPACE with nothing launched (no shape the linear
 * entry points accept needs more). */
#define W4A4_NOALLOC_SCRATCH_BYTES (4u << 20)
int w4a4_linear_noalloc(const void* a_codes, const void* a_scales,
                        const void* w_codes, const void* w_scales,
                        int64_t M, int64_t N, int64_t K, int32_t fmt, float alpha,
                        const w4a4_branch* br, void* y, int32_t y_dtype, int64_t ldy,
                        void* stream);

/* w8a8_linear -- INT8 W8A8 sibling (FoldQuantVLA contribution 3: INT8 at
 * o_proj / down_proj).  Same arguments and semantics as w4a4_linear with
 * W4A4_FMT_INT8 codes (exact int32 accumulation). */
int w8a8_linear(const void* a_codes, const void* a_scales,
                const void* w_codes, const void* w_scales,
                int64_t M, int64_t N, int64_t K, float alpha,
                const w4a4_branch* br, void* y, int32_t y_dtype, int64_t ldy,
                void* workspace, size_t workspace_bytes, void* stream);

/* w4a8_linear -- W4A8: INT8 activation codes x INT4 weight codes, the GEMM
 * of the denoising steps whose activations stay at 8 bits while the weights
 * keep their 4-bit codes (QuantWAMs, Experimental Details, quantization
 * configuration; sec. 4.4.3, fixed-intervention rollout scheduling).
 *  a_codes / a_scales   M rows from quantize_act with W4A4_FMT_W4A8
 *           (int8 M x K in the W4A8 layout, fp32[M]).
 *  w_codes / w_scales   N rows from pack_weights with W4A4_FMT_INT4
 *           (packed int4 N x K/2, fp32[N]).
 *  Exact int32 accumulation of int8 x int4 products, then
 *  y = fp32(fp32(acc) * a_scales[m]) * w_scales[n] * alpha, as for INT4.
 *  br, y, y_dtype (I32 = raw accumulators), ldy, workspace and the shape
 *  and alignment rules are those of w4a4_linear; size a workspace with
 *  w4a4_workspace_size(M, N, K, W4A4_FMT_W4A8). */
int w4a8_linear(const void* a_codes, const void* a_scales,
                const void* w_codes, const void* w_scales,
                int64_t M, int64_t N, int64_t K, float alpha,
                const w4a4_branch* br, void* y, int32_t y_dtype, int64_t ldy,
                void* workspace, size_t workspace_bytes, void* stream);

/* fp8_linear -- FP8 W8A8 (QuantWAMs sec. 4.2: upgraded layers run FP8
 * W8A8 kernels).  a_codes / w_codes: OCP E4M3 codes from quantize_act /
 * pack_weights with W4A4_FMT_FP8, fp32 steps per row.  The products of the
 * codes' values are exact and accumulate in fp32 (order unspecified), then
 * y = fp32(fp32(acc * a_scales[m]) * w_scales[n]) * alpha.  br, y (F32 or
 * BF16; no I32), ldy, workspace and the shape and alignment rules are those
 * of w4a4_linear; size a workspace with w4a4_workspace_size(M, N, K,
 * W4A4_FMT_FP8). */
int fp8_linear(const void* a_codes, const void* a_scales,
               const void* w_codes, const void* w_scales,
               int64_t M, int64_t N, int64_t K, float alpha,
               const w4a4_branch* br, void* y, int32_t y_dtype, int64_t ldy,
               void* workspace, size_t workspace_bytes, void* stream);

/* lowrank_add -- standalone 16-bit branch, y += (x L1) L2 or
 * y += x[:, idx] W_idx^T (Q-WAM abstract: 16-bit low-rank branch as a dense
 * product; QuantWAMs sec. 3.1 / 4.2: kept channels on a BF16 path).
 *  x    M x K activations, row stride ldx; x_dtype must be W4A4_DT_BF16
 *       (anything else is W4A4_ERR_UNSUPPORTED_FORMAT).
 *  l1t  bf16 r x K (row stride K, 16-byte aligned): L1 transposed, one
 *       K-contiguous row per rank component, for the low-rank form; NULL
 *       when idx is given.
 *  idx  int32[r] channel indices (0 <= idx < K) for the kept-channel form,
 *       or NULL.  Exactly one of l1 / idx is non-NULL.
 *  lw   bf16 N x r, row stride ldlw: L2 transposed, or W[:, idx].
 *  y    M x N, F32 or BF16, row stride ldy; read, added to, written back.
 *  Accumulation: x L1 in fp32, then the rank-r product in fp32, added to
 *  y in fp32, one rounding to y_dtype.
 */
int lowrank_add(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                const void* l1t, const int32_t* idx, const void* lw, int64_t ldlw,
                int64_t r, int64_t N, void* y, int32_t y_dtype, int64_t ldy,
                void* stream);

/* w4a4_lowrank_project -- first half of the branch, producing the
 * w4a4_branch ``a`` operand.  For l1t != NULL (L1 transposed, bf16 r x K):
 * t = x L1 in fp32, written as bf16 hi = bf16(t) and lo = bf16(t - hi) in
 * columns [0, r) and [r, 2r) of out (the branch's ra = 2r).  For
 * idx != NULL, out = x[:, idx] (M x r, exact).
 *  x M x K, x_dtype W4A4_DT_BF16 (else W4A4_ERR_UNSUPPORTED_FORMAT), row
 *  stride ldx <= 2^26 elements, K <= 2^24; out bf16 with row stride
 *  ldo >= w4a4_lowrank_width(M, K, l1t ? r : -r). */
int w4a4_lowrank_project(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                         const void* l1t, const int32_t* idx, int64_t r,
                         void* out, int64_t ldo, void* stream);

/* w4a4_lowrank_width -- columns w4a4_lowrank_project needs in its output:
 * 2r for a rank-r projection (r > 0), or |r| for a gather of |r| kept
 * channels (r < 0); M and K do not change it.  Host-only, no device
 * access. */
int64_t w4a4_lowrank_width(int64_t M, int64_t K, int64_t r);

/* w4a4_transform_amax -- max |transform(x)| over a whole R x K tensor,
 * written to amax_out (device fp32[1]).  The calibration statistic of the
 * static NVFP4 tensor scale g = amax / (6 * 448) (QuantWAMs sec. 4.2:
 * statistics are collected after both transforms).  ``scale`` is 1/s for
 * activations and s for weights; q->fmt is ignored. */
int w4a4_transform_amax(const void* x, int32_t x_dtype, int64_t R, int64_t K, int64_t ldx,
                        const float* scale, const w4a4_qdesc* q, float* amax_out,
                        void* stream);

/* w4a4_linear_plan -- which kernel the linear entry points run for
 * (M, N, K, fmt), without launching anything (host only, no device access).
 * fmt is W4A4_FMT_INT4 (also for w4a4_linear), INT8 (w8a8_linear), NVFP4,
 * W4A8 (w4a8_linear) or FP8 (fp8_linear); with_workspace says whether a
 * workspace of w4a4_workspace_size bytes will be passed.  Writes
 * plan[0] = W4A4_PLAN_* kernel family, plan[1] x plan[2] = rows x columns of
 * one workgroup's output tile, plan[3] = K splits (1 = one kernel).
 * Returns W4A4_OK, or a negative status for shapes / formats the linear
 * entry points would reject (no kernel exists for the combination). */
enum { W4A4_PLAN_DECODE = 1, W4A4_PLAN_DECODE_SPLIT = 2, W4A4_PLAN_TILE = 3, W4A4_PLAN_NVFP4_SHARED = 4 };
int w4a4_linear_plan(int64_t M, int64_t N, int64_t K, int32_t fmt, int32_t with_workspace, int32_t* plan);

/* Bytes of workspace w4a4_linear / w8a8_linear / w4a8_linear / fp8_linear
 * use for (M, N, K, fmt); 0 when the shape runs without one. */
size_t w4a4_workspace_size(int64_t M, int64_t N, int64_t K, int32_t fmt);

const char* w4a4_status_string(int status);
const char* w4a4_last_error(void);
int w4a4_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* W4A4_H */
