// C ABI of the quantized-linear library: host-side argument checks and
// dispatch to the gfx950 kernels.  Every check runs before any launch, so
// a rejected call launches nothing and writes nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/w4a4.h"
#include "launch.h"

static_assert(w4a4::kNoAllocScratchBytes == W4A4_NOALLOC_SCRATCH_BYTES, "one size for the static split-K buffer");

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() { return W4A4_OK; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(W4A4_ERR_LAUNCH_FAILED, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

size_t dt_size(int32_t dt) { return dt == W4A4_DT_BF16 ? 2 : 4; }

// Shared checks of quantize_act / pack_weights / transform_amax.
int check_quant(const char* fn, const void* x, int32_t dt, int64_t R, int64_t K, int64_t ldx,
                const float* scale, const w4a4_qdesc* q, bool need_outputs, const void* codes,
                const void* scales) {
  if (!q) return fail(W4A4_ERR_INVALID_ARG, "%s: q is NULL", fn);
  if (R < 0 || K <= 0) return fail(W4A4_ERR_INVALID_ARG, "%s: bad sizes R=%lld K=%lld", fn, (long long)R, (long long)K);
  if (dt != W4A4_DT_F32 && dt != W4A4_DT_BF16)
    return fail(W4A4_ERR_UNSUPPORTED_FORMAT, "%s: input dtype %d not F32/BF16", fn, dt);
  if (q->fmt != W4A4_FMT_INT4 && q->fmt != W4A4_FMT_INT8 && q->fmt != W4A4_FMT_NVFP4 &&
      q->fmt != W4A4_FMT_W4A8 && q->fmt != W4A4_FMT_FP8)
    return fail(W4A4_ERR_UNSUPPORTED_FORMAT, "%s: unknown fmt %d", fn, q->fmt);
  if (q->fwht_block != 0 && q->fwht_block != 64)
    return fail(W4A4_ERR_UNSUPPORTED_FORMAT, "%s: fwht_block must be 0 or 64", fn);
  if (q->order != W4A4_ORDER_SMOOTH_THEN_ROTATE && q->order != W4A4_ORDER_ROTATE_THEN_SMOOTH)
    return fail(W4A4_ERR_UNSUPPORTED_FORMAT, "%s: unknown order %d", fn, q->order);
  if (need_outputs && q->fmt == W4A4_FMT_NVFP4 &&
      !(std::isfinite(q->tensor_scale) && q->tensor_scale > 0.f))
    return fail(W4A4_ERR_INVALID_ARG, "%s: NVFP4 tensor_scale must be finite and > 0", fn);
  if (K % 16 != 0) return fail(W4A4_ERR_UNSUPPORTED_SHAPE, "%s: K=%lld not a multiple of 16", fn, (long long)K);
  if (q->fwht_block == 64 && K % 64 != 0)
    return fail(W4A4_ERR_UNSUPPORTED_SHAPE, "%s: K=%lld not a multiple of the rotation block 64", fn, (long long)K);
  if (K > w4a4::quant_max_k())
    return fail(W4A4_ERR_UNSUPPORTED_SHAPE, "%s: K=%lld above %lld", fn, (long long)K, (long long)w4a4::quant_max_k());
  if (ldx < K) return fail(W4A4_ERR_INVALID_ARG, "%s: ldx < K", fn);
  if (R == 0) return ok();
  if (!x) return fail(W4A4_ERR_INVALID_ARG, "%s: x is NULL", fn);
  if (need_outputs && (!codes || !scales)) return fail(W4A4_ERR_INVALID_ARG, "%s: output pointer is NULL", fn);
  if (!aligned(x, 16) || (ldx * (int64_t)dt_size(dt)) % 16 != 0)
    return fail(W4A4_ERR_MISALIGNED, "%s: x / ldx not 16-byte aligned", fn);
  if (scale && !aligned(scale, 16)) return fail(W4A4_ERR_MISALIGNED, "%s: scale vector not 16-byte aligned", fn);
  if (need_outputs) {
    if (!aligned(codes, 16)) return fail(W4A4_ERR_MISALIGNED, "%s: codes not 16-byte aligned", fn);
    if (q->fmt != W4A4_FMT_NVFP4 && !aligned(scales, 4))
      return fail(W4A4_ERR_MISALIGNED, "%s: scales not 4-byte aligned", fn);
  }
  return ok();
}

int run_quant(const char* fn, const void* x, int32_t dt, int64_t R, int64_t K, int64_t ldx,
              const float* scale, const w4a4_qdesc* q, void* codes, void* scales, void* stream,
              const int32_t* gidx = nullptr, int64_t gr = 0, void* gout = nullptr, int64_t ldg = 0) {
  int st = check_quant(fn, x, dt, R, K, ldx, scale, q, true, codes, scales);
  if (st != W4A4_OK || R == 0) return st;
  // quantizer modes: 0 int4, 1 int8, 2 nvfp4, 4 W4A8 int8, 5 fp8
  const int mode = q->fmt == W4A4_FMT_W4A8 ? 4 : (q->fmt == W4A4_FMT_FP8 ? 5 : q->fmt);
  hipError_t e = w4a4::launch_quantize(mode, dt == W4A4_DT_BF16, x, R, K, ldx, scale, q->tensor_scale,
                                       q->fwht_block, q->order, codes, scales, nullptr,
                                       (hipStream_t)stream, gidx, (int)gr, gout, ldg);
  return launch_status(e, fn);
}

int check_branch(const char* fn, const w4a4_branch* br, int64_t M, int64_t N) {
  if (!br || br->kind == W4A4_BRANCH_NONE) return ok();
  if (br->kind != W4A4_BRANCH_BF16) return fail(W4A4_ERR_UNSUPPORTED_FORMAT, "%s: unknown branch kind %d", fn, br->kind);
  if (br->r <= 0 || br->r > W4A4_MAX_BRANCH || br->r % 8 != 0)
    return fail(W4A4_ERR_INVALID_ARG, "%s: branch r=%d must be a multiple of 8 in [8, %d]", fn, br->r, W4A4_MAX_BRANCH);
  if (br->ra != br->r && !(br->ra % (2 * br->r) == 0 && br->ra / (2 * br->r) <= W4A4_LOWRANK_MAX_PARTS))
    return fail(W4A4_ERR_INVALID_ARG, "%s: branch ra must be r or 2 p r with p <= %d", fn, W4A4_LOWRANK_MAX_PARTS);
  if (br->lda < br->ra || br->ldb < br->r || br->lda % 8 != 0 || br->ldb % 8 != 0)
    return fail(W4A4_ERR_INVALID_ARG, "%s: branch strides must be >= width and multiples of 8", fn);
  if (M > 0 && N > 0) {
    if (!br->a || !br->b) return fail(W4A4_ERR_INVALID_ARG, "%s: branch operand is NULL", fn);
    if (!aligned(br->a, 16) || !aligned(br->b, 16))
      return fail(W4A4_ERR_MISALIGNED, "%s: branch operands not 16-byte aligned", fn);
  }
  return ok();
}

int run_linear(const char* fn, int fmt, const void* a_codes, const void* a_scales, const void* w_codes,
               const void* w_scales, int64_t M, int64_t N, int64_t K, float alpha, const w4a4_branch* br,
               void* y, int32_t y_dtype, int64_t ldy, void* workspace, size_t ws_bytes, void* stream,
               bool check_only = false) {
  if (M < 0 || N < 0 || K <= 0) return fail(W4A4_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (K % 64 != 0) return fail(W4A4_ERR_UNSUPPORTED_SHAPE, "%s: K=%lld not a multiple of 64", fn, (long long)K);
  if (K > 65536) return fail(W4A4_ERR_UNSUPPORTED_SHAPE, "%s: K=%lld above 65536", fn, (long long)K);
  if (M > INT32_MAX || N > INT32_MAX) return fail(W4A4_ERR_UNSUPPORTED_SHAPE, "%s: M/N too large", fn);
  // per-row scales are addressed with 32-bit byte offsets
  if (M > (1LL << 28)) return fail(W4A4_ERR_UNSUPPORTED_SHAPE, "%s: M=%lld above 2^28", fn, (long long)M);
  if (y_dtype != W4A4_DT_F32 && y_dtype != W4A4_DT_BF16 && y_dtype != W4A4_DT_I32)
    return fail(W4A4_ERR_UNSUPPORTED_FORMAT, "%s: y dtype %d", fn, y_dtype);
  const bool has_br = br && br->kind != W4A4_BRANCH_NONE;
  if (y_dtype == W4A4_DT_I32 && (fmt == W4A4_FMT_NVFP4 || fmt == W4A4_FMT_FP8 || has_br))
    return fail(W4A4_ERR_UNSUPPORTED_FORMAT, "%s: I32 output needs an integer format and no branch", fn);
  if (!std::isfinite(alpha)) return fail(W4A4_ERR_INVALID_ARG, "%s: alpha not finite", fn);
  int st = check_branch(fn, br, M, N);
  if (st != W4A4_OK) return st;
  if (ldy < N) return fail(W4A4_ERR_INVALID_ARG, "%s: ldy < N", fn);
  if (ldy > (1LL << 22)) return fail(W4A4_ERR_UNSUPPORTED_SHAPE, "%s: ldy above 2^22 elements", fn);
  if (M == 0 || N == 0) return ok();
  if (!a_codes || !a_scales || !w_codes || !w_scales || !y)
    return fail(W4A4_ERR_INVALID_ARG, "%s: NULL operand", fn);
  if (!aligned(a_codes, 16) || !aligned(w_codes, 16))
    return fail(W4A4_ERR_MISALIGNED, "%s: codes not 16-byte aligned", fn);
  if (!aligned(a_scales, 4) || !aligned(w_scales, 4) || !aligned(y, dt_size(y_dtype)))
    return fail(W4A4_ERR_MISALIGNED, "%s: scales / y misaligned", fn);
  if (M > 64 || fmt == W4A4_FMT_NVFP4) {
    int bm = 0, bn = 0;
    if (w4a4::wide_plan(fmt, M, N, K, &bm, &bn) < 0)
      return fail(W4A4_ERR_UNSUPPORTED_SHAPE, "%s: no many-token kernel for fmt %d at %lldx%lldx%lld", fn, fmt,
                  (long long)M, (long long)N, (long long)K);
  }
  if (check_only) return ok();

  w4a4::GemmArgs g{};
  g.a = (const uint8_t*)a_codes;
  g.sa = a_scales;
  g.w = (const uint8_t*)w_codes;
  g.sw = w_scales;
  g.M = (int)M; g.N = (int)N; g.K = (int)K;
  g.alpha = alpha;
  if (has_br) {
    g.br.a = (const uint16_t*)br->a; g.br.lda = br->lda;
    g.br.b = (const uint16_t*)br->b; g.br.ldb = br->ldb;
    g.br.r = br->r; g.br.ra = br->ra;
  }
  g.y = y; g.y_dtype = y_dtype; g.ldy = ldy;
  hipError_t e;
  if (fmt == W4A4_FMT_NVFP4) {
    e = w4a4::launch_gemm_wide(2, g, (hipStream_t)stream);
  } else {
    const size_t need = w4a4::gemm_int_workspace(fmt, M, N, K);
    if (workspace && ws_bytes < need)
      return fail(W4A4_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need);
    if (workspace && !aligned(workspace, 16))
      return fail(W4A4_ERR_MISALIGNED, "%s: workspace not 16-byte aligned", fn);
    e = w4a4::launch_gemm_int(fmt, g, workspace, ws_bytes, (hipStream_t)stream);
  }
  return launch_status(e, fn);
}

}  // namespace

extern "C" {

int quantize_act(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx, const float* inv_smooth,
                 const w4a4_qdesc* q, void* codes, void* scales, void* stream) {
  return run_quant("quantize_act", x, x_dtype, M, K, ldx, inv_smooth, q, codes, scales, stream);
}

int pack_weights_gptq(const void* w, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw, const float* smooth,
                      const w4a4_qdesc* q, const double* u, const int32_t* perm, void* codes, void* scales,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "pack_weights_gptq";
  int st = check_quant(fn, w, w_dtype, N, K, ldw, smooth, q, true, codes, scales);
  if (st != W4A4_OK) return st;
  if (q->fmt != W4A4_FMT_INT4 && q->fmt != W4A4_FMT_INT8)
    return fail(W4A4_ERR_UNSUPPORTED_FORMAT, "%s: GPTQ rounding is for INT4 / INT8 codes", fn);
  if (K % 32 != 0) return fail(W4A4_ERR_UNSUPPORTED_SHAPE, "%s: K=%lld not a multiple of 32", fn, (long long)K);
  if (N == 0) return ok();
  if (N > INT32_MAX / 2 || K > (1 << 20)) return fail(W4A4_ERR_UNSUPPORTED_SHAPE, "%s: too large", fn);
  if (!u) return fail(W4A4_ERR_INVALID_ARG, "%s: u is NULL", fn);
  if (!aligned(u, 8) || (perm && !aligned(perm, 4))) return fail(W4A4_ERR_MISALIGNED, "%s: u / perm misaligned", fn);
  const size_t need = w4a4::gptq_workspace(N, K);
  if (!workspace || workspace_bytes < need)
    return fail(W4A4_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(W4A4_ERR_MISALIGNED, "%s: workspace not 256-byte aligned", fn);
  hipError_t e = w4a4::launch_gptq(q->fmt == W4A4_FMT_INT4 ? 7 : 127, w_dtype == W4A4_DT_BF16, w, N, K, ldw, smooth,
                                   q->fwht_block, q->order, u, perm, codes, (float*)scales, workspace,
                                   (hipStream_t)stream);
  return launch_status(e, fn);
}

size_t w4a4_gptq_workspace_size(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return 0;
  return w4a4::gptq_workspace(N, K);
}

int quantize_act_gather(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx, const float* inv_smooth,
                        const w4a4_qdesc* q, void* codes, void* scales, const int32_t* idx, int64_t r, void* xo,
                        int64_t ldo, void* stream) {
  const char* fn = "quantize_act_gather";
  if (x_dtype != W4A4_DT_BF16) return fail(W4A4_ERR_UNSUPPORTED_FORMAT, "%s: x must be BF16", fn);
  if (q && q->order != W4A4_ORDER_SMOOTH_THEN_ROTATE)
    return fail(W4A4_ERR_UNSUPPORTED_FORMAT,
                "%s: kept channels need smoothing before the rotation (order SMOOTH_THEN_ROTATE)", fn);
  if (r <= 0 || r > W4A4_MAX_BRANCH)
    return fail(W4A4_ERR_INVALID_ARG, "%s: r=%lld outside [1, %d]", fn, (long long)r, W4A4_MAX_BRANCH);
  if (ldo < r) return fail(W4A4_ERR_INVALID_ARG, "%s: ldo < r", fn);
  if (M > 0) {
    if (!idx || !xo) return fail(W4A4_ERR_INVALID_ARG, "%s: idx / xo is NULL", fn);
    if (!aligned(idx, 4) || !aligned(xo, 2)) return fail(W4A4_ERR_MISALIGNED, "%s: idx / xo misaligned", fn);
  }
  return run_quant(fn, x, x_dtype, M, K, ldx, inv_smooth, q, codes, scales, stream, idx, r, xo, ldo);
}

int quantize_act_lowrank(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx, const float* inv_smooth,
                         const w4a4_qdesc* q, void* codes, void* scales, const void* l1t, int64_t r, void* out,
                         int64_t ldo, void* stream) {
  const char* fn = "quantize_act_lowrank";
  if (x_dtype != W4A4_DT_BF16) return fail(W4A4_ERR_UNSUPPORTED_FORMAT, "%s: x must be BF16", fn);
  if (r != 16 && r != 32) return fail(W4A4_ERR_INVALID_ARG, "%s: r=%lld must be 16 or 32", fn, (long long)r);
  if (ldo < 2 * r) return fail(W4A4_ERR_INVALID_ARG, "%s: ldo < 2r", fn);
  if (!w4a4::quant_lowrank_fits(K, r))
    return fail(W4A4_ERR_UNSUPPORTED_SHAPE,
                "%s: K=%lld with r=%lld: K must be a multiple of 64, at most 4096", fn,
                (long long)K, (long long)r);
  int st = check_quant(fn, x, x_dtype, M, K, ldx, inv_smooth, q, true, codes, scales);
  if (st != W4A4_OK || M == 0) return st;
  if (!l1t || !out) return fail(W4A4_ERR_INVALID_ARG, "%s: l1t / out is NULL", fn);
  if (!aligned(l1t, 16) || !aligned(out, 2)) return fail(W4A4_ERR_MISALIGNED, "%s: l1t / out misaligned", fn);
  const int mode = q->fmt == W4A4_FMT_W4A8 ? 4 : (q->fmt == W4A4_FMT_FP8 ? 5 : q->fmt);
  hipError_t e = w4a4::launch_quantize_lowrank(mode, x, M, K, ldx, inv_smooth, q->tensor_scale, q->fwht_block,
                                               q->order, codes, scales, (const uint16_t*)l1t, (int)r,
                                               (uint16_t*)out, ldo, (hipStream_t)stream);
  return launch_status(e, fn);
}

static int check_lowrank(const char* fn, const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                         const void* l1t, const int32_t* idx, int64_t r);

int quantize_act_project(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx, const float* inv_smooth,
                         const w4a4_qdesc* q, void* codes, void* scales, const void* l1t, int64_t r, void* out,
                         int64_t ldo, void* stream) {
  const char* fn = "quantize_act_project";
  int st = check_lowrank(fn, x, x_dtype, M, K, ldx, l1t, nullptr, r);
  if (st != W4A4_OK) return st;
  if (!l1t) return fail(W4A4_ERR_INVALID_ARG, "%s: l1t is NULL", fn);
  if (ldo < 2 * r) return fail(W4A4_ERR_INVALID_ARG, "%s: ldo < 2r", fn);
  if (!w4a4::quant_project_fits(K, r))
    return fail(W4A4_ERR_UNSUPPORTED_SHAPE, "%s: K=%lld above 5120 (one wave per row)", fn, (long long)K);
  st = check_quant(fn, x, x_dtype, M, K, ldx, inv_smooth, q, true, codes, scales);
  if (st != W4A4_OK || M == 0) return st;
  if (!out || !aligned(out, 2)) return fail(W4A4_ERR_INVALID_ARG, "%s: out NULL or misaligned", fn);
  const int mode = q->fmt == W4A4_FMT_W4A8 ? 4 : (q->fmt == W4A4_FMT_FP8 ? 5 : q->fmt);
  hipError_t e = w4a4::launch_quantize_project(mode, x, M, K, ldx, inv_smooth, q->tensor_scale, q->fwht_block,
                                               q->order, codes, scales, (const uint16_t*)l1t, (int)r,
                                               (uint16_t*)out, ldo, (hipStream_t)stream);
  return launch_status(e, fn);
}

int pack_weights(const void* w, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw, const float* smooth,
                 const w4a4_qdesc* q, void* codes, void* scales, void* stream) {
  if (q && q->fmt == W4A4_FMT_W4A8)
    return fail(W4A4_ERR_UNSUPPORTED_FORMAT, "pack_weights: W4A8 weights are packed with W4A4_FMT_INT4");
  return run_quant("pack_weights", w, w_dtype, N, K, ldw, smooth, q, codes, scales, stream);
}

int w4a4_linear_noalloc(const void* a_codes, const void* a_scales, const void* w_codes, const void* w_scales,
                        int64_t M, int64_t N, int64_t K, int32_t fmt, float alpha, const w4a4_branch* br, void* y,
                        int32_t y_dtype, int64_t ldy, void* stream) {
  const char* fn = "w4a4_linear_noalloc";
  if (fmt != W4A4_FMT_INT4 && fmt != W4A4_FMT_INT8 && fmt != W4A4_FMT_NVFP4 && fmt != W4A4_FMT_W4A8 &&
      fmt != W4A4_FMT_FP8)
    return fail(W4A4_ERR_UNSUPPORTED_FORMAT, "%s: unknown fmt %d", fn, fmt);
  // every argument check first, so a rejected call touches no device
  int st = run_linear(fn, fmt, a_codes, a_scales, w_codes, w_scales, M, N, K, alpha, br, y, y_dtype, ldy, nullptr,
                      0, stream, true);
  if (st != W4A4_OK) return st;
  const size_t need = (fmt != W4A4_FMT_NVFP4 && M > 0 && N > 0) ? w4a4::gemm_int_workspace(fmt, M, N, K) : 0;
  if (need > w4a4::kNoAllocScratchBytes)
    return fail(W4A4_ERR_WORKSPACE, "%s: the split plan needs %zu bytes, above the %zu-byte static buffer", fn, need,
                w4a4::kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0 && M > 0 && N > 0) {
    hipError_t e = w4a4::noalloc_scratch(&ws);
    if (e != hipSuccess) return launch_status(e, fn);
  }
  return run_linear(fn, fmt, a_codes, a_scales, w_codes, w_scales, M, N, K, alpha, br, y, y_dtype, ldy, ws,
                    ws ? w4a4::kNoAllocScratchBytes : 0, stream);
}

int w4a4_linear(const void* a_codes, const void* a_scales, const void* w_codes, const void* w_scales,
                int64_t M, int64_t N, int64_t K, int32_t fmt, float alpha, const w4a4_branch* br, void* y,
                int32_t y_dtype, int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
  if (fmt != W4A4_FMT_INT4 && fmt != W4A4_FMT_NVFP4)
    return fail(W4A4_ERR_UNSUPPORTED_FORMAT, "w4a4_linear: fmt %d is not INT4 or NVFP4", fmt);
  return run_linear("w4a4_linear", fmt, a_codes, a_scales, w_codes, w_scales, M, N, K, alpha, br, y, y_dtype,
                    ldy, workspace, workspace_bytes, stream);
}

int w8a8_linear(const void* a_codes, const void* a_scales, const void* w_codes, const void* w_scales,
                int64_t M, int64_t N, int64_t K, float alpha, const w4a4_branch* br, void* y, int32_t y_dtype,
                int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
  return run_linear("w8a8_linear", W4A4_FMT_INT8, a_codes, a_scales, w_codes, w_scales, M, N, K, alpha, br, y,
                    y_dtype, ldy, workspace, workspace_bytes, stream);
}

int w4a8_linear(const void* a_codes, const void* a_scales, const void* w_codes, const void* w_scales,
                int64_t M, int64_t N, int64_t K, float alpha, const w4a4_branch* br, void* y, int32_t y_dtype,
                int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
  return run_linear("w4a8_linear", W4A4_FMT_W4A8, a_codes, a_scales, w_codes, w_scales, M, N, K, alpha, br, y,
                    y_dtype, ldy, workspace, workspace_bytes, stream);
}

int fp8_linear(const void* a_codes, const void* a_scales, const void* w_codes, const void* w_scales,
               int64_t M, int64_t N, int64_t K, float alpha, const w4a4_branch* br, void* y, int32_t y_dtype,
               int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
  return run_linear("fp8_linear", W4A4_FMT_FP8, a_codes, a_scales, w_codes, w_scales, M, N, K, alpha, br, y,
                    y_dtype, ldy, workspace, workspace_bytes, stream);
}

static int check_lowrank(const char* fn, const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                         const void* l1t, const int32_t* idx, int64_t r) {
  if (x_dtype != W4A4_DT_BF16)
    return fail(W4A4_ERR_UNSUPPORTED_FORMAT, "%s: x dtype %d: the 16-bit branch takes BF16 activations", fn, x_dtype);
  if (M < 0 || K <= 0) return fail(W4A4_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (r <= 0 || r > W4A4_MAX_BRANCH) return fail(W4A4_ERR_INVALID_ARG, "%s: r=%lld outside [1, %d]", fn, (long long)r, W4A4_MAX_BRANCH);
  if ((l1t == nullptr) == (idx == nullptr)) return fail(W4A4_ERR_INVALID_ARG, "%s: exactly one of l1t / idx", fn);
  if (K % 8 != 0) return fail(W4A4_ERR_UNSUPPORTED_SHAPE, "%s: K not a multiple of 8", fn);
  if (K > (1LL << 24) || ldx > (1LL << 26))   // byte offsets of 16 rows (or r <= 128 rows of L1) fit 32 bits
    return fail(W4A4_ERR_UNSUPPORTED_SHAPE, "%s: K above 2^24 or ldx above 2^26", fn);
  if (ldx < K) return fail(W4A4_ERR_INVALID_ARG, "%s: ldx < K", fn);
  if (M > 0) {
    if (!x) return fail(W4A4_ERR_INVALID_ARG, "%s: x is NULL", fn);
    if (!aligned(x, 16) || ldx % 8 != 0) return fail(W4A4_ERR_MISALIGNED, "%s: x / ldx not 16-byte aligned", fn);
    if (idx && !aligned(idx, 4)) return fail(W4A4_ERR_MISALIGNED, "%s: idx misaligned", fn);
    if (l1t && !aligned(l1t, 16)) return fail(W4A4_ERR_MISALIGNED, "%s: l1t not 16-byte aligned", fn);
  }
  return ok();
}

int lowrank_add(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx, const void* l1t,
                const int32_t* idx, const void* lw, int64_t ldlw, int64_t r, int64_t N, void* y, int32_t y_dtype,
                int64_t ldy, void* stream) {
  const char* fn = "lowrank_add";
  int st = check_lowrank(fn, x, x_dtype, M, K, ldx, l1t, idx, r);
  if (st != W4A4_OK) return st;
  if (N < 0) return fail(W4A4_ERR_INVALID_ARG, "%s: N < 0", fn);
  if (y_dtype != W4A4_DT_F32 && y_dtype != W4A4_DT_BF16)
    return fail(W4A4_ERR_UNSUPPORTED_FORMAT, "%s: y dtype %d", fn, y_dtype);
  if (ldlw < r || ldy < N) return fail(W4A4_ERR_INVALID_ARG, "%s: ldlw < r or ldy < N", fn);
  if (M == 0 || N == 0) return ok();
  if (!lw || !y) return fail(W4A4_ERR_INVALID_ARG, "%s: NULL operand", fn);
  if (!aligned(lw, 2) || !aligned(y, dt_size(y_dtype))) return fail(W4A4_ERR_MISALIGNED, "%s: lw / y misaligned", fn);
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return fail(W4A4_ERR_UNSUPPORTED_SHAPE, "%s: too large", fn);
  hipError_t e = w4a4::launch_lowrank_add((const uint16_t*)x, M, K, ldx, (const uint16_t*)l1t, idx, (int)r,
                                          (const uint16_t*)lw, ldlw, N, y, y_dtype, ldy, (hipStream_t)stream);
  return launch_status(e, fn);
}

int64_t w4a4_lowrank_width(int64_t M, int64_t K, int64_t r) {
  (void)M;
  (void)K;
  return r < 0 ? -r : 2 * r;   // gather: |r| kept channels; projection: the hi/lo pair
}

int w4a4_lowrank_project(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx, const void* l1t,
                         const int32_t* idx, int64_t r, void* out, int64_t ldo, void* stream) {
  const char* fn = "w4a4_lowrank_project";
  int st = check_lowrank(fn, x, x_dtype, M, K, ldx, l1t, idx, r);
  if (st != W4A4_OK) return st;
  if (ldo < w4a4_lowrank_width(M, K, l1t ? r : -r)) return fail(W4A4_ERR_INVALID_ARG, "%s: ldo too small", fn);
  if (M == 0) return ok();
  if (!out || !aligned(out, 2)) return fail(W4A4_ERR_INVALID_ARG, "%s: out NULL or misaligned", fn);
  if (M > INT32_MAX || K > INT32_MAX) return fail(W4A4_ERR_UNSUPPORTED_SHAPE, "%s: too large", fn);
  hipError_t e = w4a4::launch_lowrank_project((const uint16_t*)x, M, K, ldx, (const uint16_t*)l1t, idx, (int)r,
                                              (uint16_t*)out, ldo, (hipStream_t)stream);
  return launch_status(e, fn);
}

int w4a4_transform_amax(const void* x, int32_t x_dtype, int64_t R, int64_t K, int64_t ldx, const float* scale,
                        const w4a4_qdesc* q, float* amax_out, void* stream) {
  const char* fn = "w4a4_transform_amax";
  int st = check_quant(fn, x, x_dtype, R, K, ldx, scale, q, false, nullptr, nullptr);
  if (st != W4A4_OK) return st;
  if (!amax_out || !aligned(amax_out, 4)) return fail(W4A4_ERR_INVALID_ARG, "%s: amax_out NULL or misaligned", fn);
  hipError_t e = w4a4::launch_quantize(3, x_dtype == W4A4_DT_BF16, x, R, K, ldx, scale, 1.f, q->fwht_block,
                                       q->order, nullptr, nullptr, amax_out, (hipStream_t)stream);
  return launch_status(e, fn);
}

int w4a4_linear_plan(int64_t M, int64_t N, int64_t K, int32_t fmt, int32_t with_workspace, int32_t* plan) {
  const char* fn = "w4a4_linear_plan";
  if (!plan) return fail(W4A4_ERR_INVALID_ARG, "%s: plan is NULL", fn);
  if (M <= 0 || N <= 0 || K <= 0) return fail(W4A4_ERR_INVALID_ARG, "%s: sizes must be positive", fn);
  if (K % 64 != 0 || K > 65536 || M > INT32_MAX || N > INT32_MAX)
    return fail(W4A4_ERR_UNSUPPORTED_SHAPE, "%s: unsupported shape", fn);
  if (fmt != W4A4_FMT_INT4 && fmt != W4A4_FMT_INT8 && fmt != W4A4_FMT_NVFP4 && fmt != W4A4_FMT_W4A8 &&
      fmt != W4A4_FMT_FP8)
    return fail(W4A4_ERR_UNSUPPORTED_FORMAT, "%s: unknown fmt %d", fn, fmt);
  if (M <= 64 && fmt != W4A4_FMT_NVFP4) {
    int rows = 0, cols = 0;
    const int splits = w4a4::decode_shape(fmt, M, N, K, with_workspace != 0, &rows, &cols);
    plan[0] = splits > 1 ? W4A4_PLAN_DECODE_SPLIT : W4A4_PLAN_DECODE;
    plan[1] = rows;
    plan[2] = cols;
    plan[3] = splits;
    return ok();
  }
  int bm = 0, bn = 0;
  const int cfg = w4a4::wide_plan(fmt, M, N, K, &bm, &bn);
  if (cfg < 0) return fail(W4A4_ERR_UNSUPPORTED_SHAPE, "%s: no many-token kernel for fmt %d", fn, fmt);
  plan[0] = (fmt == W4A4_FMT_NVFP4 && cfg == 0) ? W4A4_PLAN_NVFP4_SHARED : W4A4_PLAN_TILE;
  plan[1] = bm;
  plan[2] = bn;
  plan[3] = 1;
  return ok();
}

size_t w4a4_workspace_size(int64_t M, int64_t N, int64_t K, int32_t fmt) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 64 != 0) return 0;
  if (fmt != W4A4_FMT_INT4 && fmt != W4A4_FMT_INT8 && fmt != W4A4_FMT_W4A8 && fmt != W4A4_FMT_FP8) return 0;
  return w4a4::gemm_int_workspace(fmt, M, N, K);
}

const char* w4a4_status_string(int status) {
  switch (status) {
    case W4A4_OK: return "ok";
    case W4A4_ERR_INVALID_ARG: return "invalid argument";
    case W4A4_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case W4A4_ERR_MISALIGNED: return "misaligned pointer or stride";
    case W4A4_ERR_UNSUPPORTED_FORMAT: return "unsupported format";
    case W4A4_ERR_WORKSPACE: return "workspace too small";
    case W4A4_ERR_LAUNCH_FAILED: return "kernel launch failed";
    default: return "unknown status";
  }
}

const char* w4a4_last_error(void) { return g_last_error.c_str(); }

int w4a4_abi_version(void) { return W4A4_ABI_VERSION; }

}  // extern "C"
