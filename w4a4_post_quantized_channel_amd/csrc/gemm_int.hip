// Integer GEMM with dequantising epilogue for gfx950: W4A4 (int4 codes) and
// W8A8 (int8 codes) on the int8 matrix cores, exact int32 accumulation.
//
// FoldQuantVLA overview / contributions 3-4: integer GEMMs with per-token
// activation and per-channel weight scales, W4A4 projections and INT8 W8A8
// projections.  y[m, n] = fp32(fp32(acc) * sa[m]) * sw[n] * alpha, then the
// optional bf16 branch (Q-WAM 16-bit low-rank branch / QuantWAMs BF16
// bypass) on the same fp32 accumulators.
//
// int4 codes stay packed in HBM (and LDS) and are widened in registers: for
// a packed dword d, (d << 4) & 0xF0F0F0F0 holds the even-index codes and
// d & 0xF0F0F0F0 the odd-index codes, each as the exact signed byte 16*q.
// Both operands get the same lane permutation, so v_mfma_i32_16x16x64_i8
// returns exactly 256 * sum(qa * qw); the epilogue shifts right by 8.
//
// This file holds the few-token path; many tokens go to gemm_wide.hip.
//  * decode kernel (<= 64 tokens, weight streaming): 16*TI token rows x
//    16*TJ output channels per workgroup of four waves, each wave on an
//    interleaved quarter of the workgroup's K range.  A wave copies its
//    operand rows into its own LDS area with buffer loads to LDS: one
//    instruction moves whole 128-byte (int8) or 64-byte (int4) row segments
//    of 8 or 16 rows, every 16-byte chunk placed at position
//    chunk XOR ring_swz(row) so that the MFMA-layout reads (ds_read_b128,
//    16 rows per instruction) spread over the LDS banks.
//    Loading the MFMA layout straight from global memory instead touches 16
//    half-used cache lines per instruction and streams the weights about a
//    third slower.  Chunks past K or past the last row fall outside the
//    buffer resource and arrive as zeros.  The four partial tiles are summed
//    in LDS.  K is split over workgroups when a workspace is given; a
//    second kernel adds the int32 partial tiles (exact) and runs the
//    epilogue.  Splits never hand off inside one kernel: on gfx950 a
//    cross-workgroup handoff needs an agent-scope fence, which writes back
//    and invalidates the XCD's L2.
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "epilogue.h"
#include "launch.h"
#include "lds_dma.h"

namespace w4a4 {

constexpr int kBK = 128;  // K elements per main-loop step

__device__ __forceinline__ v4i widen_int4(uint32_t lo, uint32_t hi) {
  return v4i{(int)((lo << 4) & 0xF0F0F0F0u), (int)(lo & 0xF0F0F0F0u), (int)((hi << 4) & 0xF0F0F0F0u),
             (int)(hi & 0xF0F0F0F0u)};
}

// ---------------------------------------------------------------------------
// Decode kernels: 16*TI token rows x 16*TJ output channels per workgroup of
// four waves.  Each wave takes an interleaved quarter of the workgroup's K
// range and issues the buffer loads of a chunk of 128-deep steps before
// their MFMAs.  With a workspace the K range is split over blockIdx.z:
// partial tiles go to the workspace and a second kernel adds them and runs
// the epilogue (the kernel boundary orders the writes; no fences).
// ---------------------------------------------------------------------------
constexpr int kDecTJ = 4;  // 64 output channels per workgroup when K is split

// Row blocks of 16 tokens per workgroup: with a split, one row tile covers
// all M <= 64 rows; without one, tiles of 32 rows (16 for M <= 32) give
// twice the workgroups of a 64-row tile.
static int decode_ti(int64_t M, bool split) {
  if (split) return M > 32 ? 4 : (M > 16 ? 2 : 1);
  return M > 32 ? 2 : 1;
}

// LDS bytes of a decode wave's ring of step slots: int4 rows are half as
// long per step, and a smaller ring measured faster there; int8 activation
// rows take a deeper ring (the register prefetch below holds one slot),
// except in K splits, whose waves run few steps: every ring slot beyond
// them is a step of zeros that still costs its copies and MFMAs.
template <bool BOTH_INT4, bool SPLIT>
constexpr int dec_ring_bytes() { return BOTH_INT4 ? 12 * 1024 : (SPLIT ? 18 * 1024 : 30 * 1024); }

// XOR swizzle of the 16-byte chunks of a ring row with CPR chunks (4: int4
// rows of 64 bytes, 8: int8 / FP8 rows of 128 bytes), a function of row
// mod 16.  gfx950 serves a 16-byte LDS read in four cycles of 16 lanes, a
// cycle taking the lanes that agree in lane bit 5 and in the parity of
// lane bits 2..4, over 64 four-byte banks.  With these functions every
// cycle of a fragment read (lane -> row lane % 16; chunk lane / 16, or
// 4 h + lane / 16, or 2 (lane / 16) + h) touches 16 distinct 16-byte bank
// groups; chunk XOR (row mod CPR) left two-way conflicts on 64-byte rows
// and on the W4A8 activation reads.
template <int CPR>
__device__ __forceinline__ int ring_swz(int row) {
  static_assert(CPR == 4 || CPR == 8, "ring row length");
  if constexpr (CPR == 4) return (row >> 2) & 2;
  else return ((row >> 1) & 1) ^ (row & 4) ^ (((row >> 3) & 1) * 6);
}

// f(integral_constant<int, J>) for J = J0 .. J1 - 1, in order.
template <int J0, int J1, typename F>
__device__ __forceinline__ void drain_ring(F&& f) {
  if constexpr (J0 < J1) {
    f(std::integral_constant<int, J0>{});
    drain_ring<J0 + 1, J1>(f);
  }
}

// Operand formats of the decode kernel: both int4, both int8, int8
// activations with int4 weights (W4A8), or both OCP E4M3 (FP8).  int4
// codes are widened to 16*q, so the MFMA sum carries a factor 256 (both
// int4) or 16 (W4A8) that the epilogue shifts out (KIND 0 / 3).  FP8
// accumulates in fp32 on the 16x16x128 fp8 matrix instruction (KIND 4).
enum { DF_I4 = 0, DF_I8 = 1, DF_W4A8 = 2, DF_F8 = 3 };
template <int DF>
struct DecFmt {
  static constexpr bool A4 = DF == DF_I4, W4 = DF == DF_I4 || DF == DF_W4A8;   // operand packed as int4
  static constexpr int SBA = A4 ? 64 : 128, SBB = W4 ? 64 : 128;   // bytes of a row per 128-element step
  static constexpr int KIND = DF == DF_I4 ? 0 : (DF == DF_I8 ? 1 : (DF == DF_W4A8 ? 3 : 4));
  typedef typename std::conditional<DF == DF_F8, v4f, v4i>::type acc_t;
  typedef typename std::conditional<DF == DF_F8, float, int>::type elem_t;
};

typedef int v8i __attribute__((ext_vector_type(8)));

// 32 bytes of fp8 codes from two 16-byte LDS chunks, as one operand.
__device__ __forceinline__ v8i lds_pair(const uint8_t* p0, const uint8_t* p1) {
  const uint4 a = *reinterpret_cast<const uint4*>(p0), b = *reinterpret_cast<const uint4*>(p1);
  return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// One 16x16x128 fp8 product (both sides in the same K order), unit scales
// (E8M0 127 = 2^0).
__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <int DF, int TI, int TJ>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_int_decode_kernel(GemmArgs g, int kwg, int32_t* part) {
  static_assert(TI == 1 || TI == 2 || TI == 4, "row blocks per workgroup");
  // every argument in scalar registers before any branch: one batch of
  // argument loads and one wait
  asm volatile("" ::"s"(g.a), "s"(g.sa), "s"(g.w), "s"(g.sw), "s"(g.M), "s"(g.N), "s"(g.K), "s"(g.alpha),
               "s"(g.br.a), "s"(g.br.lda), "s"(g.br.b), "s"(g.br.ldb), "s"(g.br.r), "s"(g.br.ra), "s"(g.y),
               "s"(g.y_dtype), "s"(g.ldy), "s"(kwg), "s"(part));
  typedef DecFmt<DF> F;
  constexpr int SBA = F::SBA, SBB = F::SBB;
  constexpr int CPRA = SBA / 16, CPRB = SBB / 16;          // 16-byte chunks per row and step
  constexpr int RPIA = 64 / CPRA, RPIB = 64 / CPRB;        // rows per copy instruction
  constexpr int NIA = 16 * TI / RPIA, NIB = 16 * TJ / RPIB;
  constexpr int PER_STEP = NIA + NIB;                      // copy instructions per step (A first)
  constexpr int AREG = 16 * TI * SBA;                      // A rows' bytes in a slot; W rows follow
  constexpr int STEP_BYTES = AREG + 16 * TJ * SBB;
  constexpr int NBUF0 = dec_ring_bytes<DF == DF_I4, TJ == kDecTJ>() / STEP_BYTES;
  constexpr int NBUF = NBUF0 > 8 ? 8 : (NBUF0 < 2 ? 2 : NBUF0);   // ring slots per wave
  constexpr int WAVE_BYTES = NBUF * STEP_BYTES;
  constexpr int RED_BYTES = 4 * TI * TJ * 1024;
  constexpr int LDS_BYTES = 4 * WAVE_BYTES > RED_BYTES ? 4 * WAVE_BYTES : RED_BYTES;
  static_assert((NBUF - 1) * PER_STEP <= 63 && NBUF <= 8, "vmcnt range");
  static_assert(AREG == NIA * 1024, "A copies fill whole instructions");
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int lr = lane & 15, lq = lane >> 4;
  const int n0 = blockIdx.x * 16 * TJ, m0 = blockIdx.y * 16 * TI;
  const int64_t rbA = F::A4 ? (g.K >> 1) : g.K, rbB = F::W4 ? (g.K >> 1) : g.K;   // row bytes
  const int kz0 = blockIdx.z * kwg, kz1 = min(g.K, kz0 + kwg);
  const v4u rsA = rsrc_words(g.a + (int64_t)m0 * rbA, (uint32_t)(min(16 * TI, g.M - m0) * rbA));
  const v4u rsB = rsrc_words(g.w + (int64_t)n0 * rbB, (uint32_t)(min(16 * TJ, g.N - n0) * rbB));
  uint8_t* const area = smem + wave * WAVE_BYTES;
  // this wave's steps: k = kz0 + 128 * (wave + 4 t), t < nsteps
  const int kw = kz0 + wave * kBK;
  const int nsteps = kw < kz1 ? (kz1 - kw + 4 * kBK - 1) / (4 * kBK) : 0;

  // Without a split this kernel runs the epilogue: its scales load now, so
  // their latency hides behind the main loop.
  EpiScales<1, TJ> es;
  if (!part && wave < TI) load_epi_scales(es, g, m0 + wave * 16, n0, lane);

  // copy instruction d: lane -> row d*RPI + lane/CPR of its operand, LDS
  // chunk position lane%CPR holding chunk position^(row mod CPR).  The
  // lane's row offset and chunk byte are fixed; a step adds its K byte
  // through the scalar offset, and a lane past K takes the out-of-range
  // offset.  Destinations are 32-bit LDS addresses from one base.
  uint32_t voff[PER_STEP], cpos[PER_STEP];
#pragma unroll
  for (int d = 0; d < PER_STEP; ++d) {
    const bool isa = d < NIA;
    const int cpr = isa ? CPRA : CPRB, rpi = isa ? RPIA : RPIB;
    const int r = (isa ? d : d - NIA) * rpi + lane / cpr;
    cpos[d] = 16u * (uint32_t)((lane % cpr) ^ (cpr == 4 ? ring_swz<4>(r) : ring_swz<8>(r)));
    voff[d] = (uint32_t)(r * (isa ? rbA : rbB)) + cpos[d];
  }
  const uint32_t area_lds = lds_addr(area);
  auto issue = [&](int t, int slot) {   // copies of step t into ring slot `slot`
    const int k = kw + t * 4 * kBK;
    const uint32_t st = area_lds + (uint32_t)(slot * STEP_BYTES);
#pragma unroll
    for (int d = 0; d < PER_STEP; ++d) {
      const bool isa = d < NIA;                   // compile-time per instruction
      const uint32_t rb = (uint32_t)(isa ? rbA : rbB);
      const uint32_t kb = (uint32_t)((isa ? F::A4 : F::W4) ? (k >> 1) : k);
      const bool ok = k < kz1 && kb + cpos[d] < rb;
      dma16_at(isa ? rsA : rsB, st + d * 1024, ok ? voff[d] : kOOB, kb);
    }
  };

  typedef typename F::acc_t acc_t;
  typedef typename F::elem_t elem_t;
  acc_t acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = acc_t{0, 0, 0, 0};

  // Fragments of one step: int8 operands take a 16-byte chunk per half
  // step (h), int4 operands one chunk for both halves.
  struct Frags {
    uint4 a[DecFmt<DF>::A4 ? 1 : 2][TI];
    uint4 b[DecFmt<DF>::W4 ? 1 : 2][TJ];
    v8i a8[TI], b8[TJ];   // FP8: both halves as one operand
  };
  // LDS reads of one step from its ring slot.  int4 rows: lane group lq
  // holds K [32 lq, 32 lq + 32) of the step as one chunk.  int8 rows: half h
  // of lane group lq is chunk 4 h + lq (both int8) or 2 lq + h (W4A8, whose
  // activation chunks hold their codes in the widened int4 order).
  auto load = [&](const uint8_t* st, Frags& f) {
    if constexpr (DF == DF_F8) {
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int R = i * 16 + lr;
        f.a8[i] = lds_pair(st + R * SBA + 16 * (lq ^ ring_swz<8>(R)), st + R * SBA + 16 * ((4 + lq) ^ ring_swz<8>(R)));
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int R = j * 16 + lr;
        f.b8[j] = lds_pair(st + AREG + R * SBB + 16 * (lq ^ ring_swz<8>(R)),
                           st + AREG + R * SBB + 16 * ((4 + lq) ^ ring_swz<8>(R)));
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int R = i * 16 + lr;
      if constexpr (F::A4) {
        f.a[0][i] = *reinterpret_cast<const uint4*>(st + R * SBA + 16 * (lq ^ ring_swz<4>(R)));
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int c = DF == DF_W4A8 ? 2 * lq + h : 4 * h + lq;
          f.a[h][i] = *reinterpret_cast<const uint4*>(st + R * SBA + 16 * (c ^ ring_swz<8>(R)));
        }
      }
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int R = j * 16 + lr;
      if constexpr (F::W4) {
        f.b[0][j] = *reinterpret_cast<const uint4*>(st + AREG + R * SBB + 16 * (lq ^ ring_swz<4>(R)));
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          f.b[h][j] = *reinterpret_cast<const uint4*>(st + AREG + R * SBB + 16 * ((4 * h + lq) ^ ring_swz<8>(R)));
      }
    }
  };
  // The MFMAs of one step (int4 chunks widened to 16 q per byte; FP8: one
  // 128-deep product of both halves).
  auto math = [&](const Frags& f) {
    if constexpr (DF == DF_F8) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = mfma_fp8(f.a8[i], f.b8[j], acc[i][j]);
      return;
    } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v4i b[TJ];
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        b[j] = F::W4 ? (h ? widen_int4(f.b[0][j].z, f.b[0][j].w) : widen_int4(f.b[0][j].x, f.b[0][j].y))
                     : __builtin_bit_cast(v4i, f.b[F::W4 ? 0 : h][j]);
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const v4i a = F::A4 ? (h ? widen_int4(f.a[0][i].z, f.a[0][i].w) : widen_int4(f.a[0][i].x, f.a[0][i].y))
                            : __builtin_bit_cast(v4i, f.a[F::A4 ? 0 : h][i]);
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[j], acc[i][j], 0, 0, 0);
      }
    }
    }
  };

  // Ring of NBUF step slots per wave: the copies of step t + NBUF - 1 are
  // issued before step t's MFMAs.  With three or more slots, step t + 1's
  // fragments are read from LDS while step t's MFMAs run on the fragments
  // read one iteration earlier (a slot is refilled two iterations after
  // its fragments were read); with two slots that would wait for the copy
  // just issued, so a step is read and multiplied in one go.  The last
  // NBUF - 1 steps drain the ring with no further copies; each drain
  // position has a fixed number of younger steps, so every wait is exact.
  // A wave with fewer than NBUF - 1 steps runs the missing ones on copies
  // past kz1, which read as zeros and add nothing: the code stays free of
  // branches around the waits.
  constexpr int LA = NBUF >= 3 ? 1 : 0;   // steps of register lookahead
#pragma unroll
  for (int p = 0; p < NBUF - 1; ++p) issue(p, p);
  Frags cur, nxt;
  int rslot = 0, wslot = NBUF - 1;   // rslot: slot of the next step to read
  if constexpr (LA == 1) {
    wait_vmcnt<(NBUF - 2) * PER_STEP>();
    asm volatile("" ::: "memory");
    load(area, cur);
    rslot = 1;
  }
  for (int t = 0; t < nsteps - (NBUF - 1); ++t) {
    issue(t + NBUF - 1, wslot);
    wslot = wslot == NBUF - 1 ? 0 : wslot + 1;
    wait_vmcnt<(NBUF - 1 - LA) * PER_STEP>();   // steps up to t + LA are in LDS
    asm volatile("" ::: "memory");
    load(area + rslot * STEP_BYTES, nxt);
    rslot = rslot == NBUF - 1 ? 0 : rslot + 1;
    if constexpr (LA == 1) {
      math(cur);
      cur = nxt;
    } else {
      math(nxt);
    }
  }
  drain_ring<0, NBUF - 1>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    if constexpr (LA == 0 || j < NBUF - 2) {
      wait_vmcnt<(NBUF - 2 - LA - j) * PER_STEP>();
      asm volatile("" ::: "memory");
      load(area + rslot * STEP_BYTES, nxt);
      rslot = rslot == NBUF - 1 ? 0 : rslot + 1;
    }
    if constexpr (LA == 1) {
      math(cur);
      cur = nxt;
    } else {
      math(nxt);
    }
  });
  __syncthreads();   // every wave is done with its copy area; LDS now holds the partial tiles
  elem_t (*red)[TI][TJ][4][64] = reinterpret_cast<elem_t (*)[TI][TJ][4][64]>(smem);

  // sum the four waves' partial tiles; wave w < TI keeps row block w
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][i][j][r][lane] = acc[i][j][r];
  __syncthreads();
  if (wave >= TI) return;
  acc_t tot[1][TJ];
#pragma unroll
  for (int j = 0; j < TJ; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      tot[0][j][r] = red[0][wave][j][r][lane] + red[1][wave][j][r][lane] + red[2][wave][j][r][lane] +
                     red[3][wave][j][r][lane];
  if (part) {  // one contiguous 1 KB block per (tile, row block, 16-column block, split)
    const int64_t tile = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      uint4* p = reinterpret_cast<uint4*>(part + (((tile * TI + wave) * TJ + j) * gridDim.z + blockIdx.z) * 256);
      p[lane] = __builtin_bit_cast(uint4, tot[0][j]);
    }
    return;
  }
  epilogue_tiles<F::KIND>(tot, g, m0 + wave * 16, n0, lane, nullptr, &es);
}

// One wave per 16 x 16 output tile (tile, row block, column block): add its
// S partial blocks (coalesced 1 KB reads, up to eight in flight; the
// epilogue's scales load alongside the first ones), then the epilogue.
template <int KIND, int TI>
__global__ void __launch_bounds__(64) gemm_int_reduce_kernel(GemmArgs g, int S, const int32_t* part) {
  constexpr int TJ = kDecTJ;
  constexpr int ZB = 8;  // partial blocks whose loads are in flight together
  const int lane = threadIdx.x;
  const int nt = (g.N + 16 * TJ - 1) / (16 * TJ);
  const int64_t blk = blockIdx.x;              // (tile * TI + rb) * TJ + j
  const int j = (int)(blk % TJ), rb = (int)((blk / TJ) % TI);
  const int64_t tile = blk / (TI * TJ);
  const int n0 = (int)(tile % nt) * 16 * TJ + j * 16, m0 = (int)(tile / nt) * 16 * TI + rb * 16;
  EpiScales<1, 1> es;
  load_epi_scales(es, g, m0, n0, lane);
  const uint4* p = reinterpret_cast<const uint4*>(part + blk * S * 256) + lane;
  typedef typename std::conditional<KIND == 4, v4f, v4i>::type acc_t;   // FP8 partials are fp32
  acc_t tot[1][1] = {{acc_t{0, 0, 0, 0}}};
  for (int z0 = 0; z0 < S; z0 += ZB) {
    uint4 v[ZB];
#pragma unroll
    for (int dz = 0; dz < ZB; ++dz)
      if (z0 + dz < S) v[dz] = p[(z0 + dz) * 64];
#pragma unroll
    for (int dz = 0; dz < ZB; ++dz)
      if (z0 + dz < S) tot[0][0] += __builtin_bit_cast(acc_t, v[dz]);
  }
  epilogue_tiles<KIND>(tot, g, m0, n0, lane, nullptr, &es);
}

// ---------------------------------------------------------------------------
// Host-side dispatch
// ---------------------------------------------------------------------------
struct DecodePlan {
  int splits;
  int kwg;
  int ti;          // row blocks per workgroup of the split kernel (one row tile)
  int64_t tiles;
  size_t ws_bytes;
};

// K is split only when the unsplit grid (16 channels x 16 or 32 rows per
// workgroup) has fewer than 128 workgroups: then about 256 workgroups
// stream the weights, each split a multiple of four 128-deep steps (one per
// wave).  Small weight matrices and short K are not split: the second
// kernel costs more than the split saves.
static DecodePlan decode_plan(int64_t M, int64_t N, int64_t K, bool int4) {
  DecodePlan p{};
  p.ti = decode_ti(M, true);
  p.tiles = (N + 16 * kDecTJ - 1) / (16 * kDecTJ);  // M <= 64: one row tile
  const int64_t unit = 4 * kBK;
  const int64_t nunits = (K + unit - 1) / unit;
  const int64_t wbytes = N * K / (int4 ? 2 : 1);
  const int ti_ns = decode_ti(M, false);
  const int64_t wg_unsplit = ((N + 15) / 16) * ((M + 16 * ti_ns - 1) / (16 * ti_ns));
  int64_t s = (wg_unsplit >= 128 || wbytes < (1 << 20) || nunits < 4) ? 1 : 256 / p.tiles;
  s = s < 1 ? 1 : (s > nunits ? nunits : s);
  const int64_t per = (nunits + s - 1) / s;
  p.kwg = (int)(per * unit);
  p.splits = (int)((nunits + per - 1) / per);
  p.ws_bytes = p.splits > 1 ? (size_t)(p.splits * p.tiles * 16 * p.ti * 16 * kDecTJ * 4) : 0;
  return p;
}

// fmt: 0 int4 x int4, 1 int8 x int8, 3 int8 activations x int4 weights
size_t gemm_int_workspace(int fmt, int64_t M, int64_t N, int64_t K) {
  return M <= 64 ? decode_plan(M, N, K, fmt == 0 || fmt == 3).ws_bytes : 0;
}

// ---------------------------------------------------------------------------
// Library-owned split-K buffer for callers that cannot allocate.  Every GPU
// holds its own copy of this array (kNoAllocScratchBytes, until the process
// ends).  In host code ``scratch`` names a host-side stand-in, never the
// device memory: its device address is looked up once per device with
// hipGetSymbolAddress (that device current) and only that address is passed
// to kernels.  The split plan needs at most 256 partial tiles of 64 x 64
// int32 (4 MiB).
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *ptr = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

int decode_shape(int fmt, int64_t M, int64_t N, int64_t K, bool with_workspace, int* rows, int* cols) {
  const DecodePlan p = decode_plan(M, N, K, fmt == 0 || fmt == 3);
  const bool split = with_workspace && p.splits > 1;
  *rows = 16 * (split ? p.ti : decode_ti(M, false));
  *cols = split ? 16 * kDecTJ : 16;
  return split ? p.splits : 1;
}

template <int DF>
static void launch_decode(const GemmArgs& g, const DecodePlan& p, int32_t* part, hipStream_t st) {
  constexpr int KIND = DecFmt<DF>::KIND;
  if (part) {
    const dim3 grid((unsigned)p.tiles, 1, p.splits);
    const dim3 rgrid((unsigned)(p.tiles * p.ti * kDecTJ));
    switch (p.ti) {
      case 1:
        hipLaunchKernelGGL((gemm_int_decode_kernel<DF, 1, kDecTJ>), grid, dim3(256), 0, st, g, p.kwg, part);
        hipLaunchKernelGGL((gemm_int_reduce_kernel<KIND, 1>), rgrid, dim3(64), 0, st, g, p.splits, part);
        break;
      case 2:
        hipLaunchKernelGGL((gemm_int_decode_kernel<DF, 2, kDecTJ>), grid, dim3(256), 0, st, g, p.kwg, part);
        hipLaunchKernelGGL((gemm_int_reduce_kernel<KIND, 2>), rgrid, dim3(64), 0, st, g, p.splits, part);
        break;
      default:
        hipLaunchKernelGGL((gemm_int_decode_kernel<DF, 4, kDecTJ>), grid, dim3(256), 0, st, g, p.kwg, part);
        hipLaunchKernelGGL((gemm_int_reduce_kernel<KIND, 4>), rgrid, dim3(64), 0, st, g, p.splits, part);
        break;
    }
    return;
  }
  // whole K per workgroup: 16 output channels and 16 or 32 rows each, for more workgroups
  const int ti = decode_ti(g.M, false);
  const dim3 grid((g.N + 15) / 16, (g.M + 16 * ti - 1) / (16 * ti), 1);
  if (ti == 1) hipLaunchKernelGGL((gemm_int_decode_kernel<DF, 1, 1>), grid, dim3(256), 0, st, g, g.K, part);
  else hipLaunchKernelGGL((gemm_int_decode_kernel<DF, 2, 1>), grid, dim3(256), 0, st, g, g.K, part);
}

hipError_t launch_gemm_int(int fmt, GemmArgs g, void* workspace, size_t ws_bytes, hipStream_t st) {
  if (g.M <= 64) {
    const DecodePlan p = decode_plan(g.M, g.N, g.K, fmt == 0 || fmt == 3);   // int4 weights
    const bool split = p.splits > 1 && workspace && ws_bytes >= p.ws_bytes;
    int32_t* part = split ? reinterpret_cast<int32_t*>(workspace) : nullptr;
    if (fmt == 0) launch_decode<DF_I4>(g, p, part, st);
    else if (fmt == 1) launch_decode<DF_I8>(g, p, part, st);
    else if (fmt == 4) launch_decode<DF_F8>(g, p, part, st);
    else launch_decode<DF_W4A8>(g, p, part, st);
    return hipGetLastError();
  }
  return launch_gemm_wide(fmt, g, st);
}

}  // namespace w4a4
