// Internal launchers behind the C ABI (host side, C++ linkage).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4a4 {

// quantize.hip -------------------------------------------------------------
// mode: 0 int4, 1 int8, 2 nvfp4, 3 transform-amax only, 4 int8 in the W4A8 order
// (each aligned group of 8 codes stored even-K codes first, then odd-K codes),
// 5 fp8 (OCP E4M3, step amax/448).
// gidx / gr / gout / ldg: optional kept-channel gather from the same pass
// (bf16 input): gout[m * ldg + j] = x[m, gidx[j]] for j < gr <= 128.
hipError_t launch_quantize(int mode, bool bf16in, const void* x, int64_t R, int64_t K,
                           int64_t ldx, const float* scale, float g, int rot, int order,
                           void* codes, void* scales, float* amax_out, hipStream_t st,
                           const int32_t* gidx = nullptr, int gr = 0, void* gout = nullptr,
                           int64_t ldg = 0);
int64_t quant_max_k();
// quantize_act fused with the low-rank projection T = x L1 (bf16 input):
// out[m, j] = bf16(T), out[m, r + j] = bf16(T - bf16(T)) for j < r.
// Shapes: quant_lowrank_fits(K, r) (r 16 or 32, K % 64 == 0, K <= 4096).
hipError_t launch_quantize_lowrank(int mode, const void* x, int64_t R, int64_t K, int64_t ldx, const float* scale,
                                   float g, int rot, int order, void* codes, void* scales, const uint16_t* l1t, int r,
                                   uint16_t* out, int64_t ldo, hipStream_t st);
// quantize_act and the low-rank projection in one launch (bf16 input):
// codes / scales as launch_quantize, out as launch_lowrank_project.
// Shapes: quant_project_fits(K, r) (K % 16 == 0, K <= 5120, 1 <= r <= 128).
hipError_t launch_quantize_project(int mode, const void* x, int64_t R, int64_t K, int64_t ldx, const float* scale,
                                   float g, int rot, int order, void* codes, void* scales, const uint16_t* l1t, int r,
                                   uint16_t* out, int64_t ldo, hipStream_t st);
bool quant_project_fits(int64_t K, int64_t r);
int64_t quant_lowrank_max_k();
int quant_lowrank_max_r();
bool quant_lowrank_fits(int64_t K, int64_t r);

// gemm_int.hip / gemm_nvfp4.hip --------------------------------------------
struct BranchArgs {
  const uint16_t* a;  // bf16 M x ra
  int64_t lda;
  const uint16_t* b;  // bf16 N x r
  int64_t ldb;
  int r;
  int ra;
};

struct GemmArgs {
  const uint8_t* a;      // codes, M rows
  const void* sa;        // fp32[M] or E4M3 M x K/16
  const uint8_t* w;      // codes, N rows
  const void* sw;
  int M, N, K;
  float alpha;
  BranchArgs br;         // br.r == 0: no branch
  void* y;
  int y_dtype;           // 0 f32, 1 bf16, 2 i32
  int64_t ldy;
};

// fmt: 0 int4, 1 int8, 3 int8 activations x int4 weights (W4A8), 4 fp8 (E4M3).
// workspace may be null (no split-K).
hipError_t launch_gemm_int(int fmt, GemmArgs g, void* workspace, size_t ws_bytes, hipStream_t st);
size_t gemm_int_workspace(int fmt, int64_t M, int64_t N, int64_t K);

// Size of the library-owned split-K buffer (one per GPU) behind
// w4a4_linear_noalloc, and its device address on the current device
// (looked up once per device; never allocates).
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
hipError_t noalloc_scratch(void** ptr);

// gemm_wide.hip: many-token kernel with packed operands in LDS, fmt 0 int4, 1 int8, 2 nvfp4, 3 W4A8,
// 4 fp8
hipError_t launch_gemm_wide(int fmt, GemmArgs g, hipStream_t st);
// The many-token tile the launcher picks for (fmt, M, N, K): its
// configuration index (>= 0, tile bm x bn), or -1 when no kernel exists.
int wide_plan(int fmt, int64_t M, int64_t N, int64_t K, int* bm, int* bn);
// Few-token plan (M <= 64): the number of K splits (1 = one kernel, no
// reduction) and the rows x columns of one workgroup's output tile.
int decode_shape(int fmt, int64_t M, int64_t N, int64_t K, bool with_workspace, int* rows, int* cols);

// gptq.hip --------------------------------------------------------------------
// GPTQ-style rounding at pack time: codes (int4 packed if qmax == 7, else
// int8) and the per-row steps of N rows; u fp64 K x K (processing order),
// perm int32[K] or null; workspace of gptq_workspace(N, K) bytes.
size_t gptq_workspace(int64_t N, int64_t K);
hipError_t launch_gptq(int qmax, bool bf16in, const void* x, int64_t N, int64_t K, int64_t ldx, const float* smooth,
                       int rot, int order, const double* u, const int32_t* perm, void* codes, float* scales,
                       void* workspace, hipStream_t st);

// branch.hip ----------------------------------------------------------------
hipError_t launch_lowrank_project(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                  const uint16_t* l1t, const int32_t* idx, int r,
                                  uint16_t* out, int64_t ldo, hipStream_t st);
hipError_t launch_lowrank_add(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                              const uint16_t* l1t, const int32_t* idx, int r, const uint16_t* lw,
                              int64_t ldlw, int64_t N, void* y, int y_dtype, int64_t ldy,
                              hipStream_t st);

}  // namespace w4a4
