// Shared epilogue pieces of the GEMM kernels: the 16-bit branch as extra
// bf16 MFMA steps on the fp32 accumulators, and the output store.
#pragma once
#include "device_common.h"
#include "launch.h"

namespace w4a4 {

// 16 consecutive bytes (8 bf16) of row `row`, starting at element k, or
// zeros when the row or the chunk is out of range.
__device__ __forceinline__ v8bf load_bf16x8(const uint16_t* base, int64_t ld, int row, int nrows,
                                            int k, int klen) {
  uint4 d = make_uint4(0, 0, 0, 0);
  if (row < nrows && k < klen) d = *reinterpret_cast<const uint4*>(base + (int64_t)row * ld + k);
  return __builtin_bit_cast(v8bf, d);
}

// acc[i][j] (16x16 fp32 MFMA tiles, lane holds rows 4*(lane/16)+0..3 of
// column lane%16) += A_br[rows, :ra] . B_br[cols, (k mod r)]^T.
// m_base / n_base: first row / column of this wave's tile.
template <int TI, int TJ>
__device__ __forceinline__ void branch_mfma(v4f (&acc)[TI][TJ], const BranchArgs& br, int M, int N,
                                            int m_base, int n_base, int lane) {
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  for (int kk = 0; kk < br.ra; kk += 32) {
    const int ka = kk + lk;
    const int kb = ka % br.r;
    v8bf af[TI], bfr[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) af[i] = load_bf16x8(br.a, br.lda, m_base + i * 16 + lr, M, ka, br.ra);
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      bfr[j] = load_bf16x8(br.b, br.ldb, n_base + j * 16 + lr, N, kb, ka < br.ra ? br.r : 0);
    }
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  }
}

// Store one fp32 value (f32 or bf16 output).
__device__ __forceinline__ void store_out(void* y, int y_dtype, int64_t ldy, int m, int n, float v) {
  if (y_dtype == 0) {
    reinterpret_cast<float*>(y)[(int64_t)m * ldy + n] = v;
  } else {
    reinterpret_cast<uint16_t*>(y)[(int64_t)m * ldy + n] = (uint16_t)f32_to_bf16_bits(v);
  }
}

}  // namespace w4a4
