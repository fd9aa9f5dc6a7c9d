// 16-bit branch kernels for gfx950: the rank-r product (x L1) L2 of the
// Q-WAM abstract's Action-Subspace Protection (a 16-bit low-rank branch
// beside the 4-bit complement, both dense products) and the kept-channel
// product x[:, idx] W[:, idx]^T of the QuantWAMs BF16 bypass (sec. 3.1
// top-K mask, sec. 4.2).
//
//  * project: t = x L1 (fp32, v_mfma_f32_16x16x32_bf16 with L1 given
//    transposed so both operands are K-contiguous), one 16 x 16 tile of t
//    per workgroup with K split over its eight waves and summed in LDS,
//    written as the bf16 hi/lo pair the GEMM epilogue consumes; or the
//    gather x[:, idx].
//  * lowrank_add: the same projection kept in fp32 in LDS, then
//    y[m, n] += sum_j t[m, j] lw[n, j] on the vector ALUs, one rounding to
//    the output type.
#include "device_common.h"
#include "launch.h"
#include "lds_dma.h"
#include "project_body.h"

namespace w4a4 {

constexpr int kRows = 16;

// Partial t[16 x r] over this wave's K range, r <= 128 (TJ = r/16 tiles).
// l1t is L1 transposed (r rows of K), so both operands are K-contiguous.
// Result left in `part` as 16x16 MFMA accumulators.
template <int TJ>
__device__ __forceinline__ void project_tile(const uint16_t* x, int64_t ldx, int M, int K,
                                             const uint16_t* l1t, int r, int m0, int k_begin,
                                             int k_end, int lane, v4f (&part)[TJ]) {
  const int lr = lane & 15, lq = lane >> 4;
#pragma unroll
  for (int j = 0; j < TJ; ++j) part[j] = v4f{0.f, 0.f, 0.f, 0.f};
  const int m = m0 + lr;
  for (int k = k_begin; k < k_end; k += 32) {
    const int kc = k + lq * 8;
    uint4 d = make_uint4(0, 0, 0, 0);
    if (m < M && kc < K) d = *reinterpret_cast<const uint4*>(x + (int64_t)m * ldx + kc);
    const v8bf af = __builtin_bit_cast(v8bf, d);
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int col = j * 16 + lr;
      uint4 bd = make_uint4(0, 0, 0, 0);
      if (col < r && kc < K) bd = *reinterpret_cast<const uint4*>(l1t + (int64_t)col * K + kc);
      part[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(v8bf, bd), part[j], 0, 0, 0);
    }
  }
}

// t (16 x r, fp32) into LDS: sum of the four waves' partials.
template <int TJ>
__device__ void project_block(const uint16_t* x, int64_t ldx, int M, int K, const uint16_t* l1t,
                              const int32_t* idx, int r, int m0, float* sT /*[4][16][128]*/) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  if (l1t) {
    const int kq = ((K + 127) / 128) * 32;  // K range per wave, multiple of 32
    v4f part[TJ];
    project_tile<TJ>(x, ldx, M, K, l1t, r, m0, wave * kq, min(K, (wave + 1) * kq), lane, part);
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) sT[(wave * 16 + lq * 4 + q) * 128 + j * 16 + lr] = part[j][q];
    __syncthreads();
    for (int e = tid; e < 16 * r; e += 256) {
      const int row = e / r, col = e % r;
      sT[row * 128 + col] = sT[row * 128 + col] + sT[(16 + row) * 128 + col] +
                            sT[(32 + row) * 128 + col] + sT[(48 + row) * 128 + col];
    }
    __syncthreads();
  } else {
    for (int e = tid; e < 16 * r; e += 256) {
      const int row = e / r, col = e % r;
      const int m = m0 + row;
      const int c = idx[col];
      sT[row * 128 + col] = (m < M && c >= 0 && c < K) ? bf16_bits_to_f32(x[(int64_t)m * ldx + c]) : 0.f;
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(64 * kProjWaves) project_kernel(const uint16_t* x, int64_t ldx, int M, int K,
                                                                 const uint16_t* l1t, int r, uint16_t* out,
                                                                 int64_t ldo) {
  __shared__ __attribute__((aligned(16))) uint8_t area[kProjLdsBytes];
  project_block(x, ldx, M, K, l1t, r, out, ldo, blockIdx.x * kProjRows, blockIdx.y * 16, area);
}

// Gather of kept channels: out[m, j] = x[m, idx[j]] (exact).
__global__ void __launch_bounds__(256) gather_kernel(const uint16_t* x, int64_t ldx, int M, int K,
                                                     const int32_t* idx, int r, uint16_t* out, int64_t ldo) {
  const int64_t total = (int64_t)M * r;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t m = e / r;
    const int j = (int)(e - m * r);
    const int c = idx[j];
    out[m * ldo + j] = (c >= 0 && c < K) ? x[m * ldx + c] : (uint16_t)0;
  }
}

template <int TJ>
__global__ void __launch_bounds__(256) lowrank_add_kernel(const uint16_t* x, int64_t ldx, int M, int K,
                                                          const uint16_t* l1t, const int32_t* idx, int r,
                                                          const uint16_t* lw, int64_t ldlw, int N,
                                                          void* y, int y_dtype, int64_t ldy) {
  __shared__ float sT[64 * 128];
  const int m0 = blockIdx.x * kRows;
  project_block<TJ>(x, ldx, M, K, l1t, idx, r, m0, sT);
  const int rows = min(kRows, M - m0);
  for (int n = blockIdx.y * 256 + threadIdx.x; n < N; n += gridDim.y * 256) {
    float acc[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i) acc[i] = 0.f;
    for (int j = 0; j < r; ++j) {
      const float b = bf16_bits_to_f32(lw[(int64_t)n * ldlw + j]);
#pragma unroll
      for (int i = 0; i < kRows; ++i) acc[i] = acc[i] + sT[i * 128 + j] * b;
    }
    for (int i = 0; i < rows; ++i) {
      const int64_t o = (int64_t)(m0 + i) * ldy + n;
      if (y_dtype == 0) {
        float* yp = reinterpret_cast<float*>(y);
        yp[o] = yp[o] + acc[i];
      } else {
        uint16_t* yp = reinterpret_cast<uint16_t*>(y);
        yp[o] = (uint16_t)f32_to_bf16_bits(bf16_bits_to_f32(yp[o]) + acc[i]);
      }
    }
  }
}

#define W4A4_TJ_SWITCH(r, CALL) \
  switch ((r + 15) / 16) {      \
    case 1: CALL(1); break;     \
    case 2: CALL(2); break;     \
    case 3: CALL(3); break;     \
    case 4: CALL(4); break;     \
    case 5: CALL(5); break;     \
    case 6: CALL(6); break;     \
    case 7: CALL(7); break;     \
    case 8: CALL(8); break;     \
    default: return hipErrorInvalidValue; \
  }

hipError_t launch_lowrank_project(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                  const uint16_t* l1t, const int32_t* idx, int r, uint16_t* out,
                                  int64_t ldo, hipStream_t st) {
  if (!l1t) {
    int64_t blocks = (M * r + 255) / 256;
    blocks = blocks > 2048 ? 2048 : (blocks < 1 ? 1 : blocks);
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, ldx, (int)M, (int)K, idx, r,
                       out, ldo);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((M + kRows - 1) / kRows), (unsigned)((r + 15) / 16));
  hipLaunchKernelGGL(project_kernel, grid, dim3(64 * kProjWaves), 0, st, x, ldx, (int)M, (int)K, l1t, r, out, ldo);
  return hipGetLastError();
}

hipError_t launch_lowrank_add(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* l1t,
                              const int32_t* idx, int r, const uint16_t* lw, int64_t ldlw, int64_t N,
                              void* y, int y_dtype, int64_t ldy, hipStream_t st) {
  const int64_t mb = (M + kRows - 1) / kRows;
  int64_t nb = (N + 255) / 256;
  // keep roughly >= 1024 blocks of work without re-projecting too often
  if (nb > 4) nb = mb >= 256 ? 1 : (nb < 8 ? nb : 8);
  dim3 grid((unsigned)mb, (unsigned)nb);
#define W4A4_ADD(T)                                                                                  \
  hipLaunchKernelGGL((lowrank_add_kernel<T>), grid, dim3(256), 0, st, x, ldx, (int)M, (int)K, l1t, idx, r, \
                     lw, ldlw, (int)N, y, y_dtype, ldy)
  W4A4_TJ_SWITCH(r, W4A4_ADD)
#undef W4A4_ADD
  return hipGetLastError();
}

}  // namespace w4a4
