// Many-token GEMM kernels for gfx950: W4A4 (int4), W8A8 (int8) and NVFP4,
// one tile kernel for all three formats.
//
// FoldQuantVLA overview / contributions 3-4 (integer GEMMs with per-token
// and per-channel scales, W4A4 and INT8 W8A8 projections); LatentQuant
// abstract and QuantWAMs sec. 4.2 (NVFP4 W4A4 kernels, BF16 bypass).
//
// Design.  The packed operands are widened once per workgroup, while a
// K stage is written to LDS, into the element type of the matrix
// instruction:
//   int4  -> signed bytes 16*q ((d << 4) & 0xF0F0F0F0 holds the even
//            codes, d & 0xF0F0F0F0 the odd ones); v_mfma_i32_16x16x64_i8
//            then returns exactly 256 * sum(qa * qw);
//   int8  -> copied;
//   NVFP4 -> exact fp16 value(c) * value(e): v_cvt_scalef32_pk_f16_fp4 by
//            the scale's power of two, then an exact packed fp16 multiply by
//            its mantissa; v_mfma_f32_16x16x32_f16 accumulates in fp32.
// Within a stage every row holds 128 bytes of widened elements; both
// operands use the same element order, so each MFMA step multiplies
// matching K elements.  The inner loop is LDS reads (16 bytes per lane per
// fragment) and MFMAs only.  Four or eight waves per workgroup (two per
// SIMD for the large tile, so one wave's MFMAs overlap the other's
// staging), each wave a tile of 16 x 16 MFMA tiles; the LDS stage is
// double-buffered, fed from a three-stage register ring (global loads run
// two stages ahead of the MFMAs; one barrier per stage).  Tiles are ordered so that each
// XCD (workgroup id mod 8) walks a contiguous band of the tile sequence,
// keeping that band's A and W tiles in its L2.
#include <type_traits>

#include "device_common.h"
#include "epilogue.h"
#include "launch.h"

namespace w4a4 {

namespace {

constexpr int kRowBytes = 128;            // widened bytes per row per stage
constexpr int kPitch = kRowBytes + 16;    // padded LDS row pitch

enum { F_INT4 = 0, F_INT8 = 1, F_NVFP4 = 2 };

template <int FMT>
struct Fmt;

// int4: 128 K elements per stage (64 packed bytes per row)
template <>
struct Fmt<F_INT4> {
  static constexpr int BK = 128;
  static constexpr int SRC_BYTES = 64;   // packed source bytes per row per stage
  typedef v4i acc_t;
};
template <>
struct Fmt<F_INT8> {
  static constexpr int BK = 128;
  static constexpr int SRC_BYTES = 128;
  typedef v4i acc_t;
};
// NVFP4: 64 K elements per stage (32 packed bytes and 4 scale bytes per row)
template <>
struct Fmt<F_NVFP4> {
  static constexpr int BK = 64;
  static constexpr int SRC_BYTES = 32;
  typedef v4f acc_t;
};

__device__ __forceinline__ uint2 fp4_scale_pair(uint32_t e) {
  // gfx950 converts OCP E4M3 in hardware (exact; code 0 gives 0.0, whose
  // codes are all zero, so its scale pair never matters)
  const float S = __builtin_amdgcn_cvt_f32_fp8((int)e, 0);
  const float mant = __uint_as_float((__float_as_uint(S) & 0x007FFFFFu) | 0x3F800000u);
  return make_uint2(__float_as_uint(S), __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(mant, mant)));
}

// 8 E2M1 codes (dword d) times scale pair -> 4 dwords of fp16
__device__ __forceinline__ uint4 fp4_widen8(uint32_t d, uint2 sp) {
  const float S = __uint_as_float(sp.x);
  const v2h m2 = __builtin_bit_cast(v2h, sp.y);
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, S, 0) * m2;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, S, 1) * m2;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, S, 2) * m2;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, S, 3) * m2;
  return make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                    __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
}

// Global -> registers -> widened LDS rows, for one operand tile of ROWS rows
// staged by NT threads.  The stage is cut into chunks of CB source bytes
// (16, or 8 where 16-byte chunks would leave threads idle), so that every
// thread stages the same number of chunks with straight-line code; chunk c
// covers row c / CPR, source bytes (c % CPR) * CB .. +CB of that row's
// stage.  StageMap holds the per-thread offsets (fixed for the kernel),
// StageRegs one stage of loaded data.
template <int FMT, int ROWS, int NT>
struct StageMap {
  static constexpr int SRC = Fmt<FMT>::SRC_BYTES;
  static constexpr int CB = (ROWS * SRC / 16) % NT == 0 ? 16 : 8;
  static constexpr int CPR = SRC / CB;                 // chunks per row
  static constexpr int CHUNKS = ROWS * CPR;
  static constexpr int PER = CHUNKS / NT;              // chunks per thread
  static constexpr int WIDEN = FMT == F_INT4 ? 2 : (FMT == F_NVFP4 ? 4 : 1);
  static_assert(CHUNKS % NT == 0 && PER > 0, "whole chunks per thread");
  uint32_t off[PER];    // source byte offset of the chunk in stage 0
  uint32_t soff[PER];   // NVFP4: scale byte offset in stage 0
  int col[PER];         // source column in bytes
  int lds[PER];         // LDS byte offset of the chunk's widened output

  __device__ __forceinline__ void init(int tid, int64_t rowbytes, int64_t srow) {
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      const int c = tid + t * NT;
      const int r = c / CPR, cc = c % CPR;
      col[t] = cc * CB;
      off[t] = (uint32_t)(r * rowbytes + cc * CB);
      soff[t] = (uint32_t)(r * srow + cc * (CB / 8));
      lds[t] = r * kPitch + cc * CB * WIDEN;
    }
  }
};

template <int FMT, int ROWS, int NT>
struct StageRegs {
  typedef StageMap<FMT, ROWS, NT> Map;
  static constexpr int CB = Map::CB;
  typedef typename std::conditional<CB == 16, uint4, uint2>::type raw_t;
  raw_t raw[Map::PER];
  uint32_t sc[Map::PER];  // NVFP4: the chunk's scale bytes (one per 16 codes)

  // Loads are issued unconditionally (offsets past the resource read as
  // zeros), so the compiler can keep exact wait counts across the loop.
  __device__ __forceinline__ void load(const Map& mp, __amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rss,
                                       int64_t rowbytes, int ks, bool valid) {
    const int64_t kb0 = (int64_t)ks * Map::SRC;
#pragma unroll
    for (int t = 0; t < Map::PER; ++t) {
      const bool ok = valid && kb0 + mp.col[t] < rowbytes;
      const int off = ok ? (int)(mp.off[t] + (uint32_t)kb0) : (int)kOOB;
      if constexpr (CB == 16)
        raw[t] = buf_load16(rs, (uint32_t)off);
      else
        raw[t] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0));
      if constexpr (FMT == F_NVFP4) {
        const int soff = ok ? (int)(mp.soff[t] + (uint32_t)(kb0 / 8)) : (int)kOOB;
        if constexpr (CB == 16)
          sc[t] = __builtin_amdgcn_raw_buffer_load_b16(rss, soff, 0, 0);
        else
          sc[t] = __builtin_amdgcn_raw_buffer_load_b8(rss, soff, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void store(const Map& mp, uint8_t* lds) const {
#pragma unroll
    for (int t = 0; t < Map::PER; ++t) {
      uint4* dst = reinterpret_cast<uint4*>(lds + mp.lds[t]);
      const raw_t d = raw[t];
      if constexpr (FMT == F_INT8) {
        *reinterpret_cast<raw_t*>(dst) = d;
      } else if constexpr (FMT == F_INT4) {
        // 8 codes per dword -> 8 bytes: the even codes of the dword, then the odd ones
        dst[0] = make_uint4((d.x << 4) & 0xF0F0F0F0u, d.x & 0xF0F0F0F0u, (d.y << 4) & 0xF0F0F0F0u,
                            d.y & 0xF0F0F0F0u);
        if constexpr (CB == 16)
          dst[1] = make_uint4((d.z << 4) & 0xF0F0F0F0u, d.z & 0xF0F0F0F0u, (d.w << 4) & 0xF0F0F0F0u,
                              d.w & 0xF0F0F0F0u);
      } else {
        // 16 codes per scale byte -> 32 bytes of fp16
        const uint2 s0 = fp4_scale_pair(sc[t] & 0xFFu);
        dst[0] = fp4_widen8(d.x, s0);
        dst[1] = fp4_widen8(d.y, s0);
        if constexpr (CB == 16) {
          const uint2 s1 = fp4_scale_pair((sc[t] >> 8) & 0xFFu);
          dst[2] = fp4_widen8(d.z, s1);
          dst[3] = fp4_widen8(d.w, s1);
        }
      }
    }
  }
};

template <int FMT>
__device__ __forceinline__ void mma(typename Fmt<FMT>::acc_t& c, uint4 a, uint4 b) {
  if constexpr (FMT == F_NVFP4)
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  else
    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, a), __builtin_bit_cast(v4i, b), c, 0, 0, 0);
}

}  // namespace

// Instruction-group pattern for one stage: global loads first, then each
// MFMA followed by its share of VALU work and one LDS access.
template <int FMT, int NMFMA>
__device__ __forceinline__ void interleave() {
  constexpr int V = FMT == F_NVFP4 ? 3 : (FMT == F_INT4 ? 1 : 0);
  __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);   // VMEM reads
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // first fragment reads
#pragma unroll
  for (int k = 0; k < NMFMA; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    if constexpr (V > 0) __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
    __builtin_amdgcn_sched_group_barrier(0x080, 1, 0);  // one LDS read or write
  }
}

template <int FMT, int BM, int BN, int WR, int WC>
__global__ void __launch_bounds__(64 * WR * WC) __attribute__((amdgpu_waves_per_eu(WR * WC / 4, WR * WC / 4)))
gemm_tile_kernel(GemmArgs g, int tiles_n) {
  constexpr int NT = 64 * WR * WC;
  constexpr int WM = BM / WR, WN = BN / WC;
  constexpr int TI = WM / 16, TJ = WN / 16;
  typedef typename Fmt<FMT>::acc_t acc_t;
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * kPitch];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * kPitch];

  const int nwg = gridDim.x, wid = blockIdx.x;
  const int t = (nwg % 8 == 0) ? (wid % 8) * (nwg / 8) + wid / 8 : wid;
  const int n0 = (t % tiles_n) * BN, m0 = (t / tiles_n) * BM;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int wm0 = (wave / WC) * WM, wn0 = (wave % WC) * WN;
  const int64_t rowbytes = FMT == F_INT8 ? g.K : (g.K >> 1);
  const int64_t srow = g.K >> 4;
  const int nk = (g.K + Fmt<FMT>::BK - 1) / Fmt<FMT>::BK;
  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(g.a + (int64_t)m0 * rowbytes, (uint32_t)(min(BM, g.M - m0) * rowbytes));
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(g.w + (int64_t)n0 * rowbytes, (uint32_t)(min(BN, g.N - n0) * rowbytes));
  __amdgpu_buffer_rsrc_t rsSA = rsA, rsSB = rsB;
  if constexpr (FMT == F_NVFP4) {
    rsSA = make_rsrc(reinterpret_cast<const uint8_t*>(g.sa) + (int64_t)m0 * srow, (uint32_t)(min(BM, g.M - m0) * srow));
    rsSB = make_rsrc(reinterpret_cast<const uint8_t*>(g.sw) + (int64_t)n0 * srow, (uint32_t)(min(BN, g.N - n0) * srow));
  }

  acc_t acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = acc_t{0, 0, 0, 0};

  // Register ring of three stages: the loads of stage s + 3 are issued at
  // the start of iteration s, and stage s + 1 is widened into LDS at its
  // end, so global loads have two iterations of MFMA work to land.  Stages
  // past the end load zeros; widening them into the idle LDS buffer is
  // harmless.  The steady-state loop has no conditional code.
  StageMap<FMT, BM, NT> mA;
  StageMap<FMT, BN, NT> mB;
  mA.init(tid, rowbytes, srow);
  mB.init(tid, rowbytes, srow);
  StageRegs<FMT, BM, NT> stA[3];
  StageRegs<FMT, BN, NT> stB[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    stA[i].load(mA, rsA, rsSA, rowbytes, i, i < nk);
    stB[i].load(mB, rsB, rsSB, rowbytes, i, i < nk);
  }
  stA[0].store(mA, sA[0]);
  stB[0].store(mB, sB[0]);
  __syncthreads();

  auto step = [&](int s, auto slot_c) {
    constexpr int i = decltype(slot_c)::value;  // s % 3
    const int buf = s & 1;
    stA[i].load(mA, rsA, rsSA, rowbytes, s + 3, s + 3 < nk);  // slot i held stage s, already in LDS
    stB[i].load(mB, rsB, rsSB, rowbytes, s + 3, s + 3 < nk);
    const uint8_t* a_base = sA[buf] + (wm0 + lr) * kPitch + lq * 16;
    const uint8_t* b_base = sB[buf] + (wn0 + lr) * kPitch + lq * 16;
#pragma unroll
    for (int sub = 0; sub < kRowBytes / 64; ++sub) {  // 64 bytes of each row per MFMA step
      uint4 af[TI], bfr[TJ];
#pragma unroll
      for (int ii = 0; ii < TI; ++ii) af[ii] = *reinterpret_cast<const uint4*>(a_base + ii * 16 * kPitch + sub * 64);
#pragma unroll
      for (int j = 0; j < TJ; ++j) bfr[j] = *reinterpret_cast<const uint4*>(b_base + j * 16 * kPitch + sub * 64);
#pragma unroll
      for (int ii = 0; ii < TI; ++ii)
#pragma unroll
        for (int j = 0; j < TJ; ++j) mma<FMT>(acc[ii][j], af[ii], bfr[j]);
    }
    constexpr int nx = (i + 1) % 3;
    stA[nx].store(mA, sA[buf ^ 1]);
    stB[nx].store(mB, sB[buf ^ 1]);
    // Schedule: the widening (VALU) and LDS writes of the next stage, and
    // the second half's fragment reads, go between this stage's MFMAs, so
    // the matrix pipe keeps running while the wave does its staging work.
    interleave<FMT, TI * TJ * (kRowBytes / 64)>();
    __syncthreads();
  };
  int ks = 0;
  for (; ks + 2 < nk; ks += 3) {
    step(ks, std::integral_constant<int, 0>());
    step(ks + 1, std::integral_constant<int, 1>());
    step(ks + 2, std::integral_constant<int, 2>());
  }
  if (ks < nk) step(ks, std::integral_constant<int, 0>());
  if (ks + 1 < nk) step(ks + 1, std::integral_constant<int, 1>());

  epilogue_tiles<FMT == F_INT4 ? 0 : (FMT == F_INT8 ? 1 : 2)>(acc, g, m0 + wm0, n0 + wn0, lane);
}

// ---------------------------------------------------------------------------
// Host dispatch: the largest tile that still gives the GPU about one
// workgroup per CU.
// ---------------------------------------------------------------------------
template <int FMT>
static hipError_t launch_tile(GemmArgs g, hipStream_t st) {
  const int64_t t_256 = ((g.M + 127) / 128) * ((g.N + 255) / 256);
  const int64_t t_128 = ((g.M + 127) / 128) * ((g.N + 127) / 128);
  if (t_256 >= 224) {  // 128 x 256 tiles, eight waves of 64 x 64
    const int tn = (g.N + 255) / 256;
    hipLaunchKernelGGL((gemm_tile_kernel<FMT, 128, 256, 2, 4>), dim3((unsigned)t_256), dim3(512), 0, st, g, tn);
  } else if (t_128 >= 160) {  // 128 x 128 tiles, four waves of 64 x 64
    const int tn = (g.N + 127) / 128;
    hipLaunchKernelGGL((gemm_tile_kernel<FMT, 128, 128, 2, 2>), dim3((unsigned)t_128), dim3(256), 0, st, g, tn);
  } else {  // 64 x 128 tiles, four waves of 32 x 64
    const int64_t t_64 = ((g.M + 63) / 64) * ((g.N + 127) / 128);
    const int tn = (g.N + 127) / 128;
    hipLaunchKernelGGL((gemm_tile_kernel<FMT, 64, 128, 2, 2>), dim3((unsigned)t_64), dim3(256), 0, st, g, tn);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_tile(int fmt, GemmArgs g, hipStream_t st) {
  if (fmt == 0) return launch_tile<F_INT4>(g, st);
  if (fmt == 1) return launch_tile<F_INT8>(g, st);
  return launch_tile<F_NVFP4>(g, st);
}

}  // namespace w4a4
