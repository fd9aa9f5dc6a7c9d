// Integer GEMM with dequantising epilogue for gfx950: W4A4 (int4 codes) and
// W8A8 (int8 codes) on the int8 matrix cores, exact int32 accumulation.
//
// FoldQuantVLA overview / contributions 3-4: integer GEMMs with per-token
// activation and per-channel weight scales, W4A4 projections and INT8 W8A8
// projections.  y[m, n] = fp32(fp32(acc) * sa[m]) * sw[n] * alpha, then the
// optional bf16 branch (Q-WAM 16-bit low-rank branch / QuantWAMs BF16
// bypass) on the same fp32 accumulators.
//
// Design.  C = A . W^T with both operands K-contiguous.  A workgroup tile
// BM x BN is split over four waves; each wave owns (WM/16) x (WN/16) tiles
// of v_mfma_i32_16x16x64_i8.  K advances 128 elements per step through a
// double-buffered LDS stage (16-byte global loads, one barrier per step).
// int4 codes stay packed in HBM and LDS (half the bytes of int8) and are
// widened in registers: for a packed dword d, (d << 4) & 0xF0F0F0F0 holds
// the even-index codes and d & 0xF0F0F0F0 the odd-index codes, each as the
// exact signed byte 16*q.  Both operands get the same lane permutation, so
// the MFMA returns exactly 256 * sum(qa * qw); the epilogue shifts right
// by 8.  Split-K (few output tiles, long K) adds int32 partials with
// device-scope atomics into a workspace; the last workgroup of a tile
// (arrival counter) reads the totals with atomic exchange (leaving the
// workspace zeroed for the next call) and runs the epilogue, so the result
// is bit-identical to the unsplit sum.
#include "device_common.h"
#include "epilogue.h"
#include "launch.h"

namespace w4a4 {

constexpr int kBK = 128;  // K elements per main-loop step

template <bool INT4, int BM, int BN, int WM, int WN>
struct IntTile {
  static constexpr int RB = INT4 ? kBK / 2 : kBK;   // bytes per row per step
  static constexpr int PITCH = RB + 16;             // padded LDS row pitch
  static constexpr int TI = WM / 16, TJ = WN / 16;
  static constexpr int WAVES_N = BN / WN;
  static_assert((BM / WM) * (BN / WN) == 4, "four waves per workgroup");
  static constexpr int CH_A = BM * RB / 16;         // 16-byte chunks per stage
  static constexpr int CH_B = BN * RB / 16;
  static constexpr int LA = (CH_A + 255) / 256;
  static constexpr int LB = (CH_B + 255) / 256;
};

template <bool INT4, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(256) gemm_int_kernel(GemmArgs g) {
  using T = IntTile<INT4, BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * T::PITCH];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * T::PITCH];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int wm0 = (wave / T::WAVES_N) * WM, wn0 = (wave % T::WAVES_N) * WN;
  const int64_t rowbytes = INT4 ? (g.K >> 1) : g.K;
  const int nk_total = (g.K + kBK - 1) / kBK;
  const int per = (nk_total + g.splits - 1) / g.splits;
  const int ks0 = blockIdx.z * per;
  const int ks1 = min(nk_total, ks0 + per);

  v4i acc[T::TI][T::TJ];
#pragma unroll
  for (int i = 0; i < T::TI; ++i)
#pragma unroll
    for (int j = 0; j < T::TJ; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  uint4 ra[T::LA], rb[T::LB];
  auto gload = [&](int ks) {
    const int64_t kb0 = (int64_t)ks * T::RB;
#pragma unroll
    for (int t = 0; t < T::LA; ++t) {
      const int c = tid + t * 256;
      const int r = c / (T::RB / 16), col = (c % (T::RB / 16)) * 16;
      uint4 d = make_uint4(0, 0, 0, 0);
      if (c < T::CH_A && m0 + r < g.M && kb0 + col < rowbytes)
        d = *reinterpret_cast<const uint4*>(g.a + (int64_t)(m0 + r) * rowbytes + kb0 + col);
      ra[t] = d;
    }
#pragma unroll
    for (int t = 0; t < T::LB; ++t) {
      const int c = tid + t * 256;
      const int r = c / (T::RB / 16), col = (c % (T::RB / 16)) * 16;
      uint4 d = make_uint4(0, 0, 0, 0);
      if (c < T::CH_B && n0 + r < g.N && kb0 + col < rowbytes)
        d = *reinterpret_cast<const uint4*>(g.w + (int64_t)(n0 + r) * rowbytes + kb0 + col);
      rb[t] = d;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int t = 0; t < T::LA; ++t) {
      const int c = tid + t * 256;
      if (c < T::CH_A) {
        const int r = c / (T::RB / 16), col = (c % (T::RB / 16)) * 16;
        *reinterpret_cast<uint4*>(&sA[buf][r * T::PITCH + col]) = ra[t];
      }
    }
#pragma unroll
    for (int t = 0; t < T::LB; ++t) {
      const int c = tid + t * 256;
      if (c < T::CH_B) {
        const int r = c / (T::RB / 16), col = (c % (T::RB / 16)) * 16;
        *reinterpret_cast<uint4*>(&sB[buf][r * T::PITCH + col]) = rb[t];
      }
    }
  };

  const int lr = lane & 15, lq = lane >> 4;
  if (ks0 < ks1) {
    gload(ks0);
    sstore(0);
    __syncthreads();
    for (int ks = ks0; ks < ks1; ++ks) {
      const int buf = (ks - ks0) & 1;
      if (ks + 1 < ks1) gload(ks + 1);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {  // two 64-deep MFMA steps per stage
        v4i af[T::TI], bfr[T::TJ];
        if constexpr (INT4) {
#pragma unroll
          for (int i = 0; i < T::TI; ++i) {
            const uint2 d = *reinterpret_cast<const uint2*>(
                &sA[buf][(wm0 + i * 16 + lr) * T::PITCH + sub * 32 + lq * 8]);
            af[i] = v4i{(int)((d.x << 4) & 0xF0F0F0F0u), (int)(d.x & 0xF0F0F0F0u),
                        (int)((d.y << 4) & 0xF0F0F0F0u), (int)(d.y & 0xF0F0F0F0u)};
          }
#pragma unroll
          for (int j = 0; j < T::TJ; ++j) {
            const uint2 d = *reinterpret_cast<const uint2*>(
                &sB[buf][(wn0 + j * 16 + lr) * T::PITCH + sub * 32 + lq * 8]);
            bfr[j] = v4i{(int)((d.x << 4) & 0xF0F0F0F0u), (int)(d.x & 0xF0F0F0F0u),
                         (int)((d.y << 4) & 0xF0F0F0F0u), (int)(d.y & 0xF0F0F0F0u)};
          }
        } else {
#pragma unroll
          for (int i = 0; i < T::TI; ++i)
            af[i] = *reinterpret_cast<const v4i*>(
                &sA[buf][(wm0 + i * 16 + lr) * T::PITCH + sub * 64 + lq * 16]);
#pragma unroll
          for (int j = 0; j < T::TJ; ++j)
            bfr[j] = *reinterpret_cast<const v4i*>(
                &sB[buf][(wn0 + j * 16 + lr) * T::PITCH + sub * 64 + lq * 16]);
        }
#pragma unroll
        for (int i = 0; i < T::TI; ++i)
#pragma unroll
          for (int j = 0; j < T::TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (ks + 1 < ks1) sstore(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- split-K reduction --------------------------------------------------
  if (g.splits > 1) {
#pragma unroll
    for (int i = 0; i < T::TI; ++i)
#pragma unroll
      for (int j = 0; j < T::TJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm0 + i * 16 + lq * 4 + r, n = n0 + wn0 + j * 16 + lr;
          if (m < g.M && n < g.N) atomicAdd(&g.ws[(int64_t)m * g.N + n], acc[i][j][r]);
        }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const uint32_t tile = blockIdx.y * gridDim.x + blockIdx.x;
      const uint32_t prev = atomicAdd(&g.counters[tile], 1u);
      const int last = prev == (uint32_t)(g.splits - 1);
      if (last) g.counters[tile] = 0u;
      s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
#pragma unroll
    for (int i = 0; i < T::TI; ++i)
#pragma unroll
      for (int j = 0; j < T::TJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm0 + i * 16 + lq * 4 + r, n = n0 + wn0 + j * 16 + lr;
          acc[i][j][r] = (m < g.M && n < g.N) ? atomicExch(&g.ws[(int64_t)m * g.N + n], 0) : 0;
        }
  }

  // ---- epilogue -----------------------------------------------------------
  if (g.y_dtype == 2) {
#pragma unroll
    for (int i = 0; i < T::TI; ++i)
#pragma unroll
      for (int j = 0; j < T::TJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm0 + i * 16 + lq * 4 + r, n = n0 + wn0 + j * 16 + lr;
          const int v = INT4 ? (acc[i][j][r] >> 8) : acc[i][j][r];
          if (m < g.M && n < g.N) reinterpret_cast<int32_t*>(g.y)[(int64_t)m * g.ldy + n] = v;
        }
    return;
  }
  const float* sa = reinterpret_cast<const float*>(g.sa);
  const float* sw = reinterpret_cast<const float*>(g.sw);
  v4f accf[T::TI][T::TJ];
#pragma unroll
  for (int i = 0; i < T::TI; ++i)
#pragma unroll
    for (int j = 0; j < T::TJ; ++j) {
      const int n = n0 + wn0 + j * 16 + lr;
      const float swn = n < g.N ? sw[n] : 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm0 + i * 16 + lq * 4 + r;
        const float sam = m < g.M ? sa[m] : 0.f;
        const int q = INT4 ? (acc[i][j][r] >> 8) : acc[i][j][r];
        float v = (float)q * sam;
        v = v * swn;
        accf[i][j][r] = v * g.alpha;
      }
    }
  if (g.br.r > 0) branch_mfma<T::TI, T::TJ>(accf, g.br, g.M, g.N, m0 + wm0, n0 + wn0, lane);
#pragma unroll
  for (int i = 0; i < T::TI; ++i)
#pragma unroll
    for (int j = 0; j < T::TJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm0 + i * 16 + lq * 4 + r, n = n0 + wn0 + j * 16 + lr;
        if (m < g.M && n < g.N) store_out(g.y, g.y_dtype, g.ldy, m, n, accf[i][j][r]);
      }
}

// ---------------------------------------------------------------------------
// Host-side configuration
// ---------------------------------------------------------------------------
struct IntCfg {
  int bm, bn;
};

static IntCfg pick_cfg(int64_t M, int64_t N) {
  if (M <= 64) return {64, 64};
  return {128, 128};
}

static int pick_splits(int64_t M, int64_t N, int64_t K, IntCfg c) {
  const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
  const int64_t nk = (K + kBK - 1) / kBK;
  int s = 1;
  // Aim for about two workgroups per CU (256 CUs) while each split keeps
  // at least two K steps.
  while (tiles * s * 2 <= 512 && nk / (s * 2) >= 2) s *= 2;
  const int64_t per = (nk + s - 1) / s;
  return (int)((nk + per - 1) / per);
}

size_t gemm_int_workspace(int fmt, int64_t M, int64_t N, int64_t K) {
  (void)fmt;
  IntCfg c = pick_cfg(M, N);
  if (pick_splits(M, N, K, c) <= 1) return 0;
  const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
  return (size_t)(M * N * 4 + ((tiles * 4 + 255) / 256) * 256);
}

int gemm_int_splits(int fmt, int64_t M, int64_t N, int64_t K, size_t ws_bytes) {
  IntCfg c = pick_cfg(M, N);
  const size_t need = gemm_int_workspace(fmt, M, N, K);
  if (need == 0 || ws_bytes < need) return 1;
  return pick_splits(M, N, K, c);
}

hipError_t launch_gemm_int(int fmt, GemmArgs g, hipStream_t st) {
  IntCfg c = pick_cfg(g.M, g.N);
  dim3 grid((g.N + c.bn - 1) / c.bn, (g.M + c.bm - 1) / c.bm, g.splits);
  const bool int4 = fmt == 0;
  if (c.bm == 64) {
    if (int4) hipLaunchKernelGGL((gemm_int_kernel<true, 64, 64, 32, 32>), grid, dim3(256), 0, st, g);
    else hipLaunchKernelGGL((gemm_int_kernel<false, 64, 64, 32, 32>), grid, dim3(256), 0, st, g);
  } else {
    if (int4) hipLaunchKernelGGL((gemm_int_kernel<true, 128, 128, 64, 64>), grid, dim3(256), 0, st, g);
    else hipLaunchKernelGGL((gemm_int_kernel<false, 128, 128, 64, 64>), grid, dim3(256), 0, st, g);
  }
  return hipGetLastError();
}

}  // namespace w4a4
