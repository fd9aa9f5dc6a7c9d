// Drives every C-ABI entry point with rejected and accepted arguments under
// AddressSanitizer and UndefinedBehaviorSanitizer (host code only): a
// rejected call returns its status and reaches no launcher, an accepted one
// reaches it, and every error message is a bounded, terminated string.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/w4a4.h"

extern int g_launches;
static int g_failures = 0;

#define EXPECT(call, want_status, want_launch)                                                          \
  do {                                                                                                  \
    const int before = g_launches;                                                                     \
    const int st = (call);                                                                             \
    const int launched = g_launches - before;                                                          \
    const char* msg = w4a4_last_error();                                                               \
    if (st != (want_status) || (launched > 0) != (want_launch) || std::strlen(msg) >= 512) {           \
      std::printf("FAIL line %d: status %d (want %d) launched %d msg '%s'\n", __LINE__, st, (want_status), \
                  launched, msg);                                                                      \
      ++g_failures;                                                                                    \
    }                                                                                                  \
  } while (0)

int main() {
  void* P = reinterpret_cast<void*>(uintptr_t(0x100000));     // aligned stand-in pointers: never dereferenced
  void* Q = reinterpret_cast<void*>(uintptr_t(0x200000));
  void* MIS = reinterpret_cast<void*>(uintptr_t(0x100004));
  w4a4_qdesc q{W4A4_FMT_INT4, 64, W4A4_ORDER_SMOOTH_THEN_ROTATE, 1.0f};
  w4a4_qdesc qbad{9, 64, 0, 1.0f}, qrot{W4A4_FMT_INT4, 32, 0, 1.0f}, qnv{W4A4_FMT_NVFP4, 64, 0, 0.0f};
  w4a4_qdesc qord{W4A4_FMT_INT4, 64, W4A4_ORDER_ROTATE_THEN_SMOOTH, 1.0f};

  // quantize_act
  EXPECT(quantize_act(P, W4A4_DT_BF16, 64, 2048, 2048, nullptr, &q, Q, Q, nullptr), W4A4_OK, true);
  EXPECT(quantize_act(P, W4A4_DT_BF16, 0, 2048, 2048, nullptr, &q, nullptr, nullptr, nullptr), W4A4_OK, false);
  EXPECT(quantize_act(P, W4A4_DT_BF16, 64, 2048, 2048, nullptr, nullptr, Q, Q, nullptr), W4A4_ERR_INVALID_ARG, false);
  EXPECT(quantize_act(P, W4A4_DT_BF16, -1, 2048, 2048, nullptr, &q, Q, Q, nullptr), W4A4_ERR_INVALID_ARG, false);
  EXPECT(quantize_act(P, 7, 64, 2048, 2048, nullptr, &q, Q, Q, nullptr), W4A4_ERR_UNSUPPORTED_FORMAT, false);
  EXPECT(quantize_act(P, W4A4_DT_BF16, 64, 2048, 2048, nullptr, &qbad, Q, Q, nullptr), W4A4_ERR_UNSUPPORTED_FORMAT, false);
  EXPECT(quantize_act(P, W4A4_DT_BF16, 64, 2048, 2048, nullptr, &qrot, Q, Q, nullptr), W4A4_ERR_UNSUPPORTED_FORMAT, false);
  EXPECT(quantize_act(P, W4A4_DT_BF16, 64, 2048, 2048, nullptr, &qnv, Q, Q, nullptr), W4A4_ERR_INVALID_ARG, false);
  EXPECT(quantize_act(P, W4A4_DT_BF16, 64, 2040, 2040, nullptr, &q, Q, Q, nullptr), W4A4_ERR_UNSUPPORTED_SHAPE, false);
  EXPECT(quantize_act(P, W4A4_DT_BF16, 64, 1LL << 40, 1LL << 40, nullptr, &q, Q, Q, nullptr), W4A4_ERR_UNSUPPORTED_SHAPE, false);
  EXPECT(quantize_act(MIS, W4A4_DT_BF16, 64, 2048, 2048, nullptr, &q, Q, Q, nullptr), W4A4_ERR_MISALIGNED, false);
  EXPECT(quantize_act(P, W4A4_DT_BF16, 64, 2048, 100, nullptr, &q, Q, Q, nullptr), W4A4_ERR_INVALID_ARG, false);
  EXPECT(quantize_act(nullptr, W4A4_DT_BF16, 64, 2048, 2048, nullptr, &q, Q, Q, nullptr), W4A4_ERR_INVALID_ARG, false);
  // gather, low-rank and GPTQ variants
  int32_t* idx = reinterpret_cast<int32_t*>(Q);
  EXPECT(quantize_act_gather(P, W4A4_DT_BF16, 64, 2048, 2048, nullptr, &q, Q, Q, idx, 64, Q, 64, nullptr), W4A4_OK, true);
  EXPECT(quantize_act_gather(P, W4A4_DT_BF16, 64, 2048, 2048, nullptr, &qord, Q, Q, idx, 64, Q, 64, nullptr),
         W4A4_ERR_UNSUPPORTED_FORMAT, false);
  EXPECT(quantize_act_gather(P, W4A4_DT_BF16, 64, 2048, 2048, nullptr, &q, Q, Q, idx, 500, Q, 500, nullptr),
         W4A4_ERR_INVALID_ARG, false);
  EXPECT(quantize_act_lowrank(P, W4A4_DT_BF16, 64, 3072, 3072, nullptr, &q, Q, Q, P, 32, Q, 64, nullptr), W4A4_OK, true);
  EXPECT(quantize_act_lowrank(P, W4A4_DT_F32, 64, 3072, 3072, nullptr, &q, Q, Q, P, 32, Q, 64, nullptr),
         W4A4_ERR_UNSUPPORTED_FORMAT, false);
  EXPECT(quantize_act_lowrank(P, W4A4_DT_BF16, 64, 8192, 8192, nullptr, &q, Q, Q, P, 32, Q, 64, nullptr),
         W4A4_ERR_UNSUPPORTED_SHAPE, false);
  EXPECT(quantize_act_project(P, W4A4_DT_BF16, 64, 3072, 3072, nullptr, &q, Q, Q, P, 32, Q, 64, nullptr), W4A4_OK, true);
  EXPECT(quantize_act_project(P, W4A4_DT_F32, 64, 3072, 3072, nullptr, &q, Q, Q, P, 32, Q, 64, nullptr),
         W4A4_ERR_UNSUPPORTED_FORMAT, false);
  EXPECT(quantize_act_project(P, W4A4_DT_BF16, 64, 8192, 8192, nullptr, &q, Q, Q, P, 32, Q, 64, nullptr),
         W4A4_ERR_UNSUPPORTED_SHAPE, false);
  EXPECT(quantize_act_project(P, W4A4_DT_BF16, 64, 3072, 3072, nullptr, &q, Q, Q, P, 32, Q, 63, nullptr),
         W4A4_ERR_INVALID_ARG, false);
  EXPECT(quantize_act_project(P, W4A4_DT_BF16, 64, 3072, 3072, nullptr, &q, Q, Q, nullptr, 32, Q, 64, nullptr),
         W4A4_ERR_INVALID_ARG, false);
  EXPECT(pack_weights_gptq(P, W4A4_DT_BF16, 64, 256, 256, nullptr, &q, reinterpret_cast<double*>(P), nullptr, Q, Q,
                           Q, w4a4_gptq_workspace_size(64, 256), nullptr), W4A4_OK, true);
  EXPECT(pack_weights_gptq(P, W4A4_DT_BF16, 64, 256, 256, nullptr, &q, reinterpret_cast<double*>(P), nullptr, Q, Q,
                           Q, 10, nullptr), W4A4_ERR_WORKSPACE, false);
  // linear entry points
  EXPECT(w4a4_linear(P, Q, P, Q, 64, 2048, 2048, W4A4_FMT_INT4, 1.0f, nullptr, Q, W4A4_DT_BF16, 2048, nullptr, 0,
                     nullptr), W4A4_OK, true);
  EXPECT(w4a4_linear(P, Q, P, Q, 64, 2048, 2048, W4A4_FMT_INT8, 1.0f, nullptr, Q, W4A4_DT_BF16, 2048, nullptr, 0,
                     nullptr), W4A4_ERR_UNSUPPORTED_FORMAT, false);
  EXPECT(w8a8_linear(P, Q, P, Q, 64, 2048, 8190, 1.0f, nullptr, Q, W4A4_DT_BF16, 2048, nullptr, 0, nullptr),
         W4A4_ERR_UNSUPPORTED_SHAPE, false);
  EXPECT(w8a8_linear(P, Q, P, Q, 64, 2048, 8192, 1.0f / 0.0f, nullptr, Q, W4A4_DT_BF16, 2048, nullptr, 0, nullptr),
         W4A4_ERR_INVALID_ARG, false);
  EXPECT(fp8_linear(P, Q, P, Q, 64, 2048, 8192, 1.0f, nullptr, Q, W4A4_DT_I32, 2048, nullptr, 0, nullptr),
         W4A4_ERR_UNSUPPORTED_FORMAT, false);
  EXPECT(w4a8_linear(P, Q, MIS, Q, 64, 2048, 8192, 1.0f, nullptr, Q, W4A4_DT_BF16, 2048, nullptr, 0, nullptr),
         W4A4_ERR_MISALIGNED, false);
  EXPECT(w8a8_linear(P, Q, P, Q, 64, 512, 8192, 1.0f, nullptr, Q, W4A4_DT_BF16, 512, Q, 16, nullptr),
         W4A4_ERR_WORKSPACE, false);
  w4a4_branch br{W4A4_BRANCH_BF16, 32, 64, 0, P, 64, Q, 32};
  EXPECT(w4a4_linear(P, Q, P, Q, 1024, 3072, 3072, W4A4_FMT_INT4, 1.0f, &br, Q, W4A4_DT_BF16, 3072, nullptr, 0,
                     nullptr), W4A4_OK, true);
  br.ra = 48;
  EXPECT(w4a4_linear(P, Q, P, Q, 1024, 3072, 3072, W4A4_FMT_INT4, 1.0f, &br, Q, W4A4_DT_BF16, 3072, nullptr, 0,
                     nullptr), W4A4_ERR_INVALID_ARG, false);
  EXPECT(w4a4_linear_noalloc(P, Q, P, Q, 64, 512, 8192, W4A4_FMT_INT8, 1.0f, nullptr, Q, W4A4_DT_BF16, 512, nullptr),
         W4A4_OK, true);
  EXPECT(w4a4_linear_noalloc(P, Q, P, Q, 64, 512, 8192, 11, 1.0f, nullptr, Q, W4A4_DT_BF16, 512, nullptr),
         W4A4_ERR_UNSUPPORTED_FORMAT, false);
  // branch calls and helpers
  EXPECT(lowrank_add(P, W4A4_DT_BF16, 64, 256, 256, P, nullptr, Q, 32, 32, 128, Q, W4A4_DT_BF16, 128, nullptr),
         W4A4_OK, true);
  EXPECT(lowrank_add(P, W4A4_DT_F32, 64, 256, 256, P, nullptr, Q, 32, 32, 128, Q, W4A4_DT_BF16, 128, nullptr),
         W4A4_ERR_UNSUPPORTED_FORMAT, false);
  EXPECT(w4a4_lowrank_project(P, W4A4_DT_BF16, 64, 256, 256, nullptr, nullptr, 8, Q, 16, nullptr),
         W4A4_ERR_INVALID_ARG, false);
  int32_t plan[4];
  EXPECT(w4a4_linear_plan(64, 2048, 2048, W4A4_FMT_INT4, 1, plan), W4A4_OK, false);
  EXPECT(w4a4_linear_plan(64, 2048, 2040, W4A4_FMT_INT4, 1, plan), W4A4_ERR_UNSUPPORTED_SHAPE, false);
  for (int s = -8; s <= 1; ++s)
    if (std::strlen(w4a4_status_string(s)) == 0) ++g_failures;
  if (w4a4_abi_version() != W4A4_ABI_VERSION) ++g_failures;
  std::printf("%s: %d failures\n", g_failures ? "FAILED" : "ok", g_failures);
  return g_failures ? 1 : 0;
}
