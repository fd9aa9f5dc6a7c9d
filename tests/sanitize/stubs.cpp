// Host-only stand-ins for the launchers behind the C ABI, for a sanitizer
// build of the argument checks (abi.cpp) without device code.  Each one
// counts that it was reached and launches nothing; the plan queries answer
// like a small fixed plan.
#include <hip/hip_runtime.h>

#include "../../w4a4_post_quantized_channel_amd/csrc/launch.h"

int g_launches = 0;

const char* hipGetErrorString(hipError_t) { return "stub"; }

namespace w4a4 {
hipError_t launch_quantize(int, bool, const void*, int64_t, int64_t, int64_t, const float*, float, int, int, void*,
                           void*, float*, hipStream_t, const int32_t*, int, void*, int64_t) {
  ++g_launches;
  return hipSuccess;
}
int64_t quant_max_k() { return 8LL * 64 * 16 * 4; }
hipError_t launch_quantize_lowrank(int, const void*, int64_t, int64_t, int64_t, const float*, float, int, int, void*,
                                   void*, const uint16_t*, int, uint16_t*, int64_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
int64_t quant_lowrank_max_k() { return 4096; }
int quant_lowrank_max_r() { return 32; }
bool quant_lowrank_fits(int64_t K, int64_t r) { return K % 64 == 0 && K <= 4096 && (r == 16 || r == 32); }
hipError_t launch_quantize_project(int, const void*, int64_t, int64_t, int64_t, const float*, float, int, int, void*,
                                   void*, const uint16_t*, int, uint16_t*, int64_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
bool quant_project_fits(int64_t K, int64_t r) { return K % 16 == 0 && K <= 5 * 1024 && r >= 1 && r <= 128; }
hipError_t launch_gemm_int(int, GemmArgs, void*, size_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
size_t gemm_int_workspace(int, int64_t M, int64_t N, int64_t K) { return M <= 64 && N < 1024 && K >= 4096 ? 1 << 20 : 0; }
hipError_t launch_gemm_wide(int, GemmArgs, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
int wide_plan(int fmt, int64_t, int64_t, int64_t, int* bm, int* bn) {
  *bm = 128;
  *bn = 256;
  return fmt >= 0 && fmt <= 4 ? 1 : -1;
}
int decode_shape(int, int64_t, int64_t, int64_t, bool, int* rows, int* cols) {
  *rows = 32;
  *cols = 16;
  return 1;
}
hipError_t noalloc_scratch(void** ptr) {
  static unsigned char buf[256];
  *ptr = buf;
  return hipSuccess;
}
size_t gptq_workspace(int64_t N, int64_t K) { return (size_t)N * K * 13; }
hipError_t launch_gptq(int, bool, const void*, int64_t, int64_t, int64_t, const float*, int, int, const double*,
                       const int32_t*, void*, float*, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_lowrank_project(const uint16_t*, int64_t, int64_t, int64_t, const uint16_t*, const int32_t*, int,
                                  uint16_t*, int64_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_lowrank_add(const uint16_t*, int64_t, int64_t, int64_t, const uint16_t*, const int32_t*, int,
                              const uint16_t*, int64_t, int64_t, void*, int, int64_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
}  // namespace w4a4
