// GPTQ-style weight rounding at pack time, for gfx950 (QuantWAMs sec. 3.3:
// GPTQ compensation governed by the layer's activation second moments,
// column scores only as an ordering inside GPTQ, the common rotation fused
// into the weights).
//
// Input: the transformed weight rows y (fp32, from the quantizer's
// transform), their round-to-nearest steps, the processing order perm and
// u, the upper Cholesky factor (fp64, processing order) of the damped
// inverse second-moment matrix.  Column t of the processing order is
// rounded from its current value; its error over u[t][t] updates every later
// column v by w -= err * u[t][v].  Every update is one fp64 product and one
// fp64 subtraction, applied to each element in t order, so the codes match
// a plain sequential evaluation bit for bit whatever the blocking.
//
//  * load: W[n][t] = y[n][perm[t]] as fp64.
//  * block (kGB columns from t0): one thread per row holds the block's
//    columns in registers and rounds them in order with the in-block
//    updates (the block's rows of u in LDS); it writes the codes (int8, in
//    original column order) and the block's errors.
//  * trail: every later column takes the block's kGB updates in order; a
//    workgroup keeps the block's rows of u for its 64 columns in LDS and
//    walks 64 rows.
//  * pack: int8 codes -> int4 nibbles (low nibble = even column) or bytes.
#include "device_common.h"
#include "launch.h"

namespace w4a4 {

constexpr int kGB = 32;        // columns per block
constexpr int kGCols = 64;     // trailing columns per workgroup
constexpr int kGRows = 64;     // rows per trailing workgroup

__global__ void __launch_bounds__(256) gptq_load_kernel(const float* y, const int32_t* perm, int N, int K,
                                                        double* W) {
  const int64_t total = (int64_t)N * K;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t n = e / K;
    const int t = (int)(e - n * K);
    const int c = perm ? perm[t] : t;
    W[e] = (double)y[n * K + c];
  }
}

template <int QMAX>
__global__ void __launch_bounds__(256) gptq_block_kernel(double* W, const float* step, const double* u,
                                                         const int32_t* perm, int N, int K, int t0,
                                                         int8_t* q8, double* err) {
  __shared__ double su[kGB][kGB];   // u[t0 + k][t0 + j]
  for (int e = threadIdx.x; e < kGB * kGB; e += 256) {
    const int k = e / kGB, j = e % kGB;
    su[k][j] = u[(int64_t)(t0 + k) * K + t0 + j];
  }
  __syncthreads();
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  double w[kGB];
  double* wr = W + (int64_t)n * K + t0;
#pragma unroll
  for (int j = 0; j < kGB; ++j) w[j] = wr[j];
  const double s = (double)step[n];
  double* er = err + (int64_t)n * kGB;
  int8_t* qr = q8 + (int64_t)n * K;
#pragma unroll
  for (int k = 0; k < kGB; ++k) {
    double q = 0.0;
    if (s > 0.0) q = __builtin_fmin(__builtin_fmax(__builtin_rint(w[k] / s), (double)(-QMAX - 1)), (double)QMAX);
    const double qs = q * s;            // exact: |q| <= 128 and s is an fp32 value
    const double e = (w[k] - qs) / su[k][k];
#pragma unroll
    for (int j = k + 1; j < kGB; ++j) {
      const double d = e * su[k][j];
      w[j] = w[j] - d;
    }
    er[k] = e;
    qr[perm ? perm[t0 + k] : t0 + k] = (int8_t)(int)q;
    // keep each column's reads of u with its own updates (hoisting the
    // whole triangle's reads overflows the registers)
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Columns [t1, K): W[n][t] -= err[n][k] * u[t0 + k][t] for k = 0 .. kGB - 1 in order.
__global__ void __launch_bounds__(256) gptq_trail_kernel(double* W, const double* u, const double* err, int N,
                                                         int K, int t0, int t1) {
  __shared__ double su[kGB][kGCols];
  __shared__ double se[4][kGB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = t1 + blockIdx.x * kGCols + lane;
  for (int e = threadIdx.x; e < kGB * kGCols; e += 256) {
    const int k = e / kGCols, c = e % kGCols;
    const int tc = t1 + blockIdx.x * kGCols + c;
    su[k][c] = tc < K ? u[(int64_t)(t0 + k) * K + tc] : 0.0;
  }
  __syncthreads();
  const int n0 = blockIdx.y * kGRows;
  for (int r = wave; r < kGRows; r += 4) {   // wave-uniform
    const int n = n0 + r;
    if (n >= N) break;
    if (lane < kGB) se[wave][lane] = err[(int64_t)n * kGB + lane];
    __builtin_amdgcn_wave_barrier();
    if (t < K) {
      double w = W[(int64_t)n * K + t];
#pragma unroll
      for (int k = 0; k < kGB; ++k) {
        const double d = se[wave][k] * su[k][lane];
        w = w - d;
      }
      W[(int64_t)n * K + t] = w;
    }
    __builtin_amdgcn_wave_barrier();   // se[wave] is rewritten for the next row
  }
}

__global__ void __launch_bounds__(256) gptq_pack_kernel(const int8_t* q8, int N, int K, bool int4, uint8_t* codes) {
  const int64_t per_row = int4 ? K / 2 : K;
  const int64_t total = (int64_t)N * per_row;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t n = e / per_row, b = e - n * per_row;
    if (int4) {
      const int8_t lo = q8[n * K + 2 * b], hi = q8[n * K + 2 * b + 1];
      codes[e] = (uint8_t)((lo & 0xF) | ((hi & 0xF) << 4));
    } else {
      codes[e] = (uint8_t)q8[n * K + b];
    }
  }
}

size_t gptq_workspace(int64_t N, int64_t K) {
  const size_t y = (size_t)N * K * 4, w = (size_t)N * K * 8, q = (size_t)N * K, e = (size_t)N * kGB * 8;
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  return up(y) + up(w) + up(q) + up(e);
}

hipError_t launch_gptq(int qmax, bool bf16in, const void* x, int64_t N, int64_t K, int64_t ldx, const float* smooth,
                       int rot, int order, const double* u, const int32_t* perm, void* codes, float* scales,
                       void* workspace, hipStream_t st) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  float* y = reinterpret_cast<float*>(ws);
  double* W = reinterpret_cast<double*>(ws + up((size_t)N * K * 4));
  int8_t* q8 = reinterpret_cast<int8_t*>(ws + up((size_t)N * K * 4) + up((size_t)N * K * 8));
  double* err = reinterpret_cast<double*>(ws + up((size_t)N * K * 4) + up((size_t)N * K * 8) + up((size_t)N * K));
  // transformed rows and round-to-nearest steps (quantizer modes 6 / 7)
  hipError_t e = launch_quantize(qmax == 7 ? 6 : 7, bf16in, x, N, K, ldx, smooth, 1.0f, rot, order, y, scales,
                                 nullptr, st);
  if (e != hipSuccess) return e;
  const int64_t total = N * K;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(gptq_load_kernel, dim3((unsigned)blocks), dim3(256), 0, st, y, perm, (int)N, (int)K, W);
  const dim3 bgrid((unsigned)((N + 255) / 256));
  for (int t0 = 0; t0 < K; t0 += kGB) {
    if (qmax == 7)
      hipLaunchKernelGGL((gptq_block_kernel<7>), bgrid, dim3(256), 0, st, W, scales, u, perm, (int)N, (int)K, t0,
                         q8, err);
    else
      hipLaunchKernelGGL((gptq_block_kernel<127>), bgrid, dim3(256), 0, st, W, scales, u, perm, (int)N, (int)K,
                         t0, q8, err);
    const int t1 = t0 + kGB;
    if (t1 < K) {
      const dim3 tgrid((unsigned)((K - t1 + kGCols - 1) / kGCols), (unsigned)((N + kGRows - 1) / kGRows));
      hipLaunchKernelGGL(gptq_trail_kernel, tgrid, dim3(256), 0, st, W, u, err, (int)N, (int)K, t0, t1);
    }
  }
  hipLaunchKernelGGL(gptq_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, st, q8, (int)N, (int)K, qmax == 7,
                     (uint8_t*)codes);
  return hipGetLastError();
}

}  // namespace w4a4
