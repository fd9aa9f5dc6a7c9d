// NVFP4 W4A4 GEMM for gfx950 (LatentQuant abstract / QuantWAMs sec. 4.2:
// NVFP4 W4A4 kernels; the element format is E2M1 with one E4M3 scale per
// 16 consecutive K elements and an fp32 tensor scale per operand).
//
// gfx950's block-scaled fp4 matrix instructions take power-of-two (E8M0)
// scales per 32 elements, which cannot carry an E4M3 scale per 16.  Every
// product value(c) * value(e) of an E2M1 code and an E4M3 scale has at most
// 6 significant bits and lies in [2^-10, 2688], so it is exact in fp16.
// The kernel therefore widens both operands exactly to fp16 in registers
// and runs v_mfma_f32_16x16x32_f16 with fp32 accumulation; alpha =
// fp32(g_a * g_w) multiplies the result.
//
// Widening.  v_cvt_scalef32_pk_f16_fp4 multiplies two fp4 codes by the
// power of two 2^floor(log2 S) of its fp32 scale operand only, so it is
// followed by an exact packed fp16 multiply by the rest of the scale,
// S / 2^floor(log2 S) in [1, 2) (at most four significant bits).  Codes stay
// packed in HBM and LDS (0.5 byte per element); each E4M3 scale is decoded
// once per workgroup when its stage is written to LDS, into the pair
// (fp32 S, fp16x2 mantissa), so a fragment of 8 elements costs four
// converts and four packed multiplies.
//
// Tiling: BM x BN workgroup tile over four waves (2 x 2, each BM/2 x BN/2
// as 16 x 16 MFMA tiles), 128 K elements per stage through a
// double-buffered LDS stage, one barrier per stage.  Tiles are ordered so
// that each XCD (workgroup id mod 8) walks a contiguous band of tiles and
// its L2 reuses the A and W tiles of that band.
#include "device_common.h"
#include "epilogue.h"
#include "launch.h"

namespace w4a4 {

constexpr int kFBK = 128;  // K elements per stage

// (exponent carrier, fp16x2 mantissa) of an E4M3 scale byte.
__device__ __forceinline__ uint2 scale_pair(uint32_t e) {
  float S = e4m3_to_f32(e);
  S = S > 0.f ? S : 1.0f;  // a zero block scale only ever carries zero codes
  const float mant = __uint_as_float((__float_as_uint(S) & 0x007FFFFFu) | 0x3F800000u);
  const _Float16 mh = (_Float16)mant;
  const v2h m2 = v2h{mh, mh};
  return make_uint2(__float_as_uint(S), __builtin_bit_cast(uint32_t, m2));
}

// Eight E2M1 codes (one dword, low nibble first) times their scale -> 8 fp16.
__device__ __forceinline__ v8h widen8(uint32_t d, uint2 sp) {
  const float S = __uint_as_float(sp.x);
  const v2h m2 = __builtin_bit_cast(v2h, sp.y);
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, S, 0) * m2;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, S, 1) * m2;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, S, 2) * m2;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, S, 3) * m2;
  return v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

template <int BM, int BN>
__global__ void __launch_bounds__(256, 2) gemm_nvfp4_kernel(GemmArgs g, int tiles_n) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int RB = kFBK / 2, PITCH = RB + 16;  // 64 bytes of codes per row and stage
  constexpr int SB = kFBK / 16;                   // 8 scale blocks per row and stage
  constexpr int SPITCH = SB + 2;                  // scale pairs per LDS row, padded
  constexpr int TI = WM / 16, TJ = WN / 16;
  constexpr int CH_A = BM * RB / 16, CH_B = BN * RB / 16;
  constexpr int LA = (CH_A + 255) / 256, LB = (CH_B + 255) / 256;
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * PITCH];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * PITCH];
  __shared__ __attribute__((aligned(16))) uint2 sAs[2][BM * SPITCH];
  __shared__ __attribute__((aligned(16))) uint2 sBs[2][BN * SPITCH];

  // XCD-aware tile order: workgroup id w runs on XCD w % 8; give each XCD
  // a contiguous band of the row-major tile sequence.
  const int nwg = gridDim.x;
  const int wid = blockIdx.x;
  int t = (wid % 8) * (nwg / 8) + wid / 8;
  if (nwg % 8 != 0) t = wid;  // uneven grids keep the plain order
  const int n0 = (t % tiles_n) * BN, m0 = (t / tiles_n) * BM;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
  const int64_t rowbytes = g.K >> 1, srow = g.K >> 4;
  const int nk = (g.K + kFBK - 1) / kFBK;
  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(g.a + (int64_t)m0 * rowbytes, (uint32_t)(min(BM, g.M - m0) * rowbytes));
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(g.w + (int64_t)n0 * rowbytes, (uint32_t)(min(BN, g.N - n0) * rowbytes));
  const __amdgpu_buffer_rsrc_t rsSA = make_rsrc(reinterpret_cast<const uint8_t*>(g.sa) + (int64_t)m0 * srow,
                                                (uint32_t)(min(BM, g.M - m0) * srow));
  const __amdgpu_buffer_rsrc_t rsSB = make_rsrc(reinterpret_cast<const uint8_t*>(g.sw) + (int64_t)n0 * srow,
                                                (uint32_t)(min(BN, g.N - n0) * srow));

  v4f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // staging registers: codes, and one dword (4 scale bytes) per half row
  uint4 ra[LA], rb[LB];
  uint32_t rsa = 0, rsb = 0;
  auto gload = [&](int ks) {
    const int64_t kb0 = (int64_t)ks * RB;
#pragma unroll
    for (int t2 = 0; t2 < LA; ++t2) {
      const int c = tid + t2 * 256, r = c / (RB / 16), col = (c % (RB / 16)) * 16;
      const bool ok = c < CH_A && kb0 + col < rowbytes;
      ra[t2] = buf_load16(rsA, ok ? (uint32_t)(r * rowbytes + kb0 + col) : kOOB);
    }
#pragma unroll
    for (int t2 = 0; t2 < LB; ++t2) {
      const int c = tid + t2 * 256, r = c / (RB / 16), col = (c % (RB / 16)) * 16;
      const bool ok = c < CH_B && kb0 + col < rowbytes;
      rb[t2] = buf_load16(rsB, ok ? (uint32_t)(r * rowbytes + kb0 + col) : kOOB);
    }
    const int64_t s0 = (int64_t)ks * SB;
    const int r = tid >> 1, h = (tid & 1) * 4;
    if (r < BM) rsa = buf_load4(rsSA, s0 + h < srow ? (uint32_t)(r * srow + s0 + h) : kOOB);
    if (r < BN) rsb = buf_load4(rsSB, s0 + h < srow ? (uint32_t)(r * srow + s0 + h) : kOOB);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int t2 = 0; t2 < LA; ++t2) {
      const int c = tid + t2 * 256;
      if (c < CH_A) {
        const int r = c / (RB / 16), col = (c % (RB / 16)) * 16;
        *reinterpret_cast<uint4*>(&sA[buf][r * PITCH + col]) = ra[t2];
      }
    }
#pragma unroll
    for (int t2 = 0; t2 < LB; ++t2) {
      const int c = tid + t2 * 256;
      if (c < CH_B) {
        const int r = c / (RB / 16), col = (c % (RB / 16)) * 16;
        *reinterpret_cast<uint4*>(&sB[buf][r * PITCH + col]) = rb[t2];
      }
    }
    const int r = tid >> 1, h = (tid & 1) * 4;
    if (r < BM) {
      uint4* p = reinterpret_cast<uint4*>(&sAs[buf][r * SPITCH + h]);
      const uint2 s0 = scale_pair(rsa & 0xFF), s1 = scale_pair((rsa >> 8) & 0xFF);
      const uint2 s2 = scale_pair((rsa >> 16) & 0xFF), s3 = scale_pair(rsa >> 24);
      p[0] = make_uint4(s0.x, s0.y, s1.x, s1.y);
      p[1] = make_uint4(s2.x, s2.y, s3.x, s3.y);
    }
    if (r < BN) {
      uint4* p = reinterpret_cast<uint4*>(&sBs[buf][r * SPITCH + h]);
      const uint2 s0 = scale_pair(rsb & 0xFF), s1 = scale_pair((rsb >> 8) & 0xFF);
      const uint2 s2 = scale_pair((rsb >> 16) & 0xFF), s3 = scale_pair(rsb >> 24);
      p[0] = make_uint4(s0.x, s0.y, s1.x, s1.y);
      p[1] = make_uint4(s2.x, s2.y, s3.x, s3.y);
    }
  };

  const int lr = lane & 15, lq = lane >> 4;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nk) gload(ks + 1);
    // Lane group lq owns bytes [16 lq, 16 lq + 16) of every row's 64 code
    // bytes in this stage (elements 32 lq .. 32 lq + 31, scale blocks 2 lq
    // and 2 lq + 1): one 16-byte LDS read for the codes of all four MFMA
    // steps and one for the two scale pairs.  Sub-step `sub` takes the
    // codes' dword `sub` (block 2 lq + sub / 2).  A and W use the same
    // assignment, so every MFMA step multiplies matching K elements.
    uint4 ca[TI], sa2[TI], cb[TJ], sb2[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int r = wm0 + i * 16 + lr;
      ca[i] = *reinterpret_cast<const uint4*>(&sA[buf][r * PITCH + lq * 16]);
      sa2[i] = *reinterpret_cast<const uint4*>(&sAs[buf][r * SPITCH + lq * 2]);
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int r = wn0 + j * 16 + lr;
      cb[j] = *reinterpret_cast<const uint4*>(&sB[buf][r * PITCH + lq * 16]);
      sb2[j] = *reinterpret_cast<const uint4*>(&sBs[buf][r * SPITCH + lq * 2]);
    }
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {  // four 32-deep MFMA steps per stage
      v8h af[TI], bfr[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const uint32_t d = sub == 0 ? ca[i].x : sub == 1 ? ca[i].y : sub == 2 ? ca[i].z : ca[i].w;
        af[i] = widen8(d, sub < 2 ? make_uint2(sa2[i].x, sa2[i].y) : make_uint2(sa2[i].z, sa2[i].w));
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const uint32_t d = sub == 0 ? cb[j].x : sub == 1 ? cb[j].y : sub == 2 ? cb[j].z : cb[j].w;
        bfr[j] = widen8(d, sub < 2 ? make_uint2(sb2[j].x, sb2[j].y) : make_uint2(sb2[j].z, sb2[j].w));
      }
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bfr[j], acc[i][j], 0, 0, 0);
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

hipError_t launch_gemm_nvfp4(GemmArgs g, hipStream_t st) {
  if (g.M <= 64) {
    const int tn = (g.N + 63) / 64, tm = (g.M + 63) / 64;
    hipLaunchKernelGGL((gemm_nvfp4_kernel<64, 64>), dim3(tn * tm), dim3(256), 0, st, g, tn);
  } else {
    const int tn = (g.N + 127) / 128, tm = (g.M + 127) / 128;
    hipLaunchKernelGGL((gemm_nvfp4_kernel<128, 128>), dim3(tn * tm), dim3(256), 0, st, g, tn);
  }
  return hipGetLastError();
}

}  // namespace w4a4
