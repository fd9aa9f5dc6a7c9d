// NVFP4 W4A4 GEMM for gfx950 (LatentQuant abstract / QuantWAMs sec. 4.2:
// NVFP4 W4A4 kernels; the element format is E2M1 with one E4M3 scale per
// 16 consecutive K elements and an fp32 tensor scale per operand).
//
// gfx950's block-scaled fp4 matrix instructions take power-of-two (E8M0)
// scales per 32 elements, which cannot carry an E4M3 scale per 16.  Every
// product value(c) * value(e) of an E2M1 code and an E4M3 scale has at most
// 6 significant bits and lies in [2^-10, 2688], so it is exact in fp16 (and
// bf16).  The kernel therefore widens both operands exactly to 16-bit in
// registers (codes and scales stay packed in HBM and LDS: 0.5625 bytes per
// element) and runs the 16-bit matrix instruction with fp32 accumulation;
// alpha = fp32(g_a * g_w) multiplies the result.  Tiling and the LDS stage follow
// the integer kernel: BM x BN tile over four waves, 128 K elements per
// stage, double-buffered LDS, one barrier per stage.
#include "device_common.h"
#include "epilogue.h"
#include "launch.h"

namespace w4a4 {

constexpr int kFBK = 128;

// fp32 bit pattern of an E2M1 nibble's value.
__device__ __forceinline__ uint32_t e2m1_f32_bits(uint32_t n) {
  const uint32_t e = (n >> 1) & 3u, m = n & 1u;
  const uint32_t mag = e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3F000000u : 0u);
  return ((n & 8u) << 28) | mag;
}

// Eight E2M1 codes (one dword, low nibble first) times one E4M3 scale S.
//
// HW path (fp16 operands): v_cvt_scalef32_pk_f16_fp4 multiplies by the
// power of two 2^floor(log2 S) only (it reads the scale as an exponent), so
// the kernel follows it with an exact packed fp16 multiply by the rest of
// S, S / 2^floor(log2 S) in [1, 2) with at most four significant bits.
// Every product value(c) * S has at most 6 significant bits and lies in
// [2^-10, 2688]: exact in fp16.  SW path (bf16 operands): decode each
// nibble to fp32, multiply by S (exact), keep the upper half of the fp32
// pattern (exact bf16).
template <bool HW>
struct Widen;

template <>
struct Widen<true> {
  typedef v8h type;
  static __device__ __forceinline__ v8h run(uint32_t d, float S) {
    S = S > 0.f ? S : 1.0f;  // a zero block scale only ever carries zero codes
    const float mant = __uint_as_float((__float_as_uint(S) & 0x007FFFFFu) | 0x3F800000u);
    const _Float16 mh = (_Float16)mant;
    const v2h m2 = v2h{mh, mh};
    v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, S, 0) * m2;
    v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, S, 1) * m2;
    v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, S, 2) * m2;
    v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, S, 3) * m2;
    return v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  }
  static __device__ __forceinline__ v4f mfma(v8h a, v8h b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Widen<false> {
  typedef v8bf type;
  static __device__ __forceinline__ v8bf run(uint32_t d, float S) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(e2m1_f32_bits((d >> (8 * i)) & 0xFu)) * S;
      const float hi = __uint_as_float(e2m1_f32_bits((d >> (8 * i + 4)) & 0xFu)) * S;
      w[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
    }
    return __builtin_bit_cast(v8bf, make_uint4(w[0], w[1], w[2], w[3]));
  }
  static __device__ __forceinline__ v4f mfma(v8bf a, v8bf b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <int BM, int BN, int WM, int WN, bool HW>
__global__ void __launch_bounds__(256) gemm_nvfp4_kernel(GemmArgs g) {
  constexpr int RB = kFBK / 2, PITCH = RB + 16, SB = kFBK / 16;  // 64 B codes, 8 B scales
  constexpr int TI = WM / 16, TJ = WN / 16, WAVES_N = BN / WN;
  static_assert((BM / WM) * (BN / WN) == 4, "four waves per workgroup");
  constexpr int CH_A = BM * RB / 16, CH_B = BN * RB / 16;
  constexpr int LA = (CH_A + 255) / 256, LB = (CH_B + 255) / 256;
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * PITCH];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * PITCH];
  __shared__ __attribute__((aligned(16))) uint32_t sAs[2][BM * 2];
  __shared__ __attribute__((aligned(16))) uint32_t sBs[2][BN * 2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int wm0 = (wave / WAVES_N) * WM, wn0 = (wave % WAVES_N) * WN;
  const int64_t rowbytes = g.K >> 1, srow = g.K >> 4;
  const int nk = (g.K + kFBK - 1) / kFBK;
  const uint8_t* sa8 = reinterpret_cast<const uint8_t*>(g.sa);
  const uint8_t* sw8 = reinterpret_cast<const uint8_t*>(g.sw);

  v4f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  uint4 ra[LA], rb[LB];
  uint2 rsa = make_uint2(0, 0), rsb = make_uint2(0, 0);
  auto scale_pair = [&](const uint8_t* base, int row, int nrows, int64_t s0) -> uint2 {
    uint2 v = make_uint2(0, 0);
    if (row < nrows) {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(base + (int64_t)row * srow + s0);
      if (s0 < srow) v.x = p[0];
      if (s0 + 4 < srow) v.y = p[1];
    }
    return v;
  };
  auto gload = [&](int ks) {
    const int64_t kb0 = (int64_t)ks * RB;
#pragma unroll
    for (int t = 0; t < LA; ++t) {
      const int c = tid + t * 256, r = c / (RB / 16), col = (c % (RB / 16)) * 16;
      uint4 d = make_uint4(0, 0, 0, 0);
      if (c < CH_A && m0 + r < g.M && kb0 + col < rowbytes)
        d = *reinterpret_cast<const uint4*>(g.a + (int64_t)(m0 + r) * rowbytes + kb0 + col);
      ra[t] = d;
    }
#pragma unroll
    for (int t = 0; t < LB; ++t) {
      const int c = tid + t * 256, r = c / (RB / 16), col = (c % (RB / 16)) * 16;
      uint4 d = make_uint4(0, 0, 0, 0);
      if (c < CH_B && n0 + r < g.N && kb0 + col < rowbytes)
        d = *reinterpret_cast<const uint4*>(g.w + (int64_t)(n0 + r) * rowbytes + kb0 + col);
      rb[t] = d;
    }
    const int64_t s0 = (int64_t)ks * SB;
    if (tid < BM) rsa = scale_pair(sa8, m0 + tid, g.M, s0);
    if (tid < BN) rsb = scale_pair(sw8, n0 + tid, g.N, s0);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int t = 0; t < LA; ++t) {
      const int c = tid + t * 256;
      if (c < CH_A) {
        const int r = c / (RB / 16), col = (c % (RB / 16)) * 16;
        *reinterpret_cast<uint4*>(&sA[buf][r * PITCH + col]) = ra[t];
      }
    }
#pragma unroll
    for (int t = 0; t < LB; ++t) {
      const int c = tid + t * 256;
      if (c < CH_B) {
        const int r = c / (RB / 16), col = (c % (RB / 16)) * 16;
        *reinterpret_cast<uint4*>(&sB[buf][r * PITCH + col]) = rb[t];
      }
    }
    if (tid < BM) *reinterpret_cast<uint2*>(&sAs[buf][tid * 2]) = rsa;
    if (tid < BN) *reinterpret_cast<uint2*>(&sBs[buf][tid * 2]) = rsb;
  };

  const int lr = lane & 15, lq = lane >> 4;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nk) gload(ks + 1);
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {  // four 32-deep MFMA steps per stage
      typename Widen<HW>::type af[TI], bfr[TJ];
      const int sidx = sub * 2 + (lq >> 1);  // scale byte of this lane's 8 elements
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int r = wm0 + i * 16 + lr;
        const uint32_t d = *reinterpret_cast<const uint32_t*>(&sA[buf][r * PITCH + sub * 16 + lq * 4]);
        const uint32_t sc = (sAs[buf][r * 2 + (sidx >> 2)] >> (8 * (sidx & 3))) & 0xFFu;
        af[i] = Widen<HW>::run(d, e4m3_to_f32(sc));
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int r = wn0 + j * 16 + lr;
        const uint32_t d = *reinterpret_cast<const uint32_t*>(&sB[buf][r * PITCH + sub * 16 + lq * 4]);
        const uint32_t sc = (sBs[buf][r * 2 + (sidx >> 2)] >> (8 * (sidx & 3))) & 0xFFu;
        bfr[j] = Widen<HW>::run(d, e4m3_to_f32(sc));
      }
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = Widen<HW>::mfma(af[i], bfr[j], acc[i][j]);
    }
    if (ks + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = acc[i][j][r] * g.alpha;
  if (g.br.r > 0) branch_mfma<TI, TJ>(acc, g.br, g.M, g.N, m0 + wm0, n0 + wn0, lane);
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm0 + i * 16 + lq * 4 + r, n = n0 + wn0 + j * 16 + lr;
        if (m < g.M && n < g.N) store_out(g.y, g.y_dtype, g.ldy, m, n, acc[i][j][r]);
      }
}

#ifndef W4A4_FP4_HW_CVT
#define W4A4_FP4_HW_CVT 1
#endif

size_t gemm_nvfp4_workspace(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_gemm_nvfp4(GemmArgs g, hipStream_t st) {
  if (g.M <= 64) {
    dim3 grid((g.N + 63) / 64, (g.M + 63) / 64, 1);
    hipLaunchKernelGGL((gemm_nvfp4_kernel<64, 64, 32, 32, W4A4_FP4_HW_CVT>), grid, dim3(256), 0, st, g);
  } else {
    dim3 grid((g.N + 127) / 128, (g.M + 127) / 128, 1);
    hipLaunchKernelGGL((gemm_nvfp4_kernel<128, 128, 64, 64, W4A4_FP4_HW_CVT>), grid, dim3(256), 0, st, g);
  }
  return hipGetLastError();
}

}  // namespace w4a4
