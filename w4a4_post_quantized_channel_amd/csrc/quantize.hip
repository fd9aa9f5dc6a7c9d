// Runtime quantizer for gfx950: smoothing, block-64 Walsh-Hadamard rotation
// and per-row quantization, fused in one pass over the input.
//
// FoldQuantVLA (contribution 2): channel scaling, FWHT with block 64 and
// dynamic per-token quantization.  QuantWAMs sec. 3.1 Eq. 1: the quantizer
// sees A R S^-1.  The same kernel packs weights (one row per output
// channel, multiplying by s instead of 1/s: FoldQuantVLA contribution 1).
//
// Work mapping.  A row of K elements is cut into slots of 16 consecutive
// elements; slot s of a row lives in lane (s mod 64) of the row's wave
// group, chunk s / (64 * WPR).  A 64-element Hadamard block is one quad of
// lanes: butterfly stages 1, 2, 4, 8 run inside a lane's registers, stages
// 16 and 32 across the quad (DPP quad permutes, xor 1 and xor 2).  An
// NVFP4 scale block (16 elements) is exactly one lane.  The whole row stays
// in registers, so the per-row absolute maximum needs no second HBM read.
// WPR (waves per row) is 1 for many rows, 4 or 8 for few (8 for long rows).
//
// Exactness.  Every value the quantizer decides on is the one the fp32
// definition gives: the butterflies are the same additions in the same
// order (a cross-lane stage computes own + c * partner with c = +-1, an
// exact negation, so the upper lane holds the negated sum; that sign and
// the final 1/8 are carried into the divisor, an exact power-of-two
// rescaling).  A code is taken from the one-multiply quotient
// RN(v * RN(1/D)) unless that quotient lies within a few representable
// steps of a rounding boundary of the code grid; such slots are redone with
// two Markstein corrections, q <- q + (v - D*q) * r, which give RN(v / D)
// for normal operands.  Divisors outside [2^-80, 2^100] take the plain IEEE
// division of the unscaled value.
#include "device_common.h"
#include "launch.h"
#include "lds_dma.h"
#include "project_body.h"

namespace w4a4 {

struct QuantArgs {
  const void* x;
  int64_t R;
  int K;
  int64_t ldx;          // elements
  const float* scale;   // K factors or null
  float g;              // NVFP4 tensor scale
  int rot;              // 0 or 64
  int order;            // 0 smooth->rotate, 1 rotate->smooth
  uint8_t* codes;
  void* scales;
  float* amax_out;      // transform_amax mode
  // kept-channel gather (bf16 input only): gout[row * ldg + j] = x[row, gidx[j]]
  // for j < gr (gr == 0: none); indices outside [0, K) give 0
  const int32_t* gidx;
  int gr;
  uint16_t* gout;
  int64_t ldg;
};

// MODE_INT8W: int8 codes for the W4A8 GEMM, every aligned group of 8 codes
// stored as its even-K codes then its odd-K codes (the order packed int4
// weight codes take when widened to bytes).
// MODE_FP8: OCP E4M3 codes with one step amax/448 per row.
// MODE_Y4 / MODE_Y8: no codes; the transformed row y itself (fp32, row-major
// K) and the round-to-nearest step amax/7 or amax/127 (the input of
// GPTQ-style rounding).
enum { MODE_INT4 = 0, MODE_INT8 = 1, MODE_NVFP4 = 2, MODE_AMAX = 3, MODE_INT8W = 4, MODE_FP8 = 5,
       MODE_Y4 = 6, MODE_Y8 = 7 };

constexpr float kTinyStep = 8.271806125530277e-25f;  // 2^-80

// RN(a / b) given r = RN(1 / b), for b >= 2^-80 and finite a.
__device__ __forceinline__ float div_rn(float a, float b, float r) {
  float q = a * r;
  float t = __builtin_fmaf(-b, q, a);
  q = __builtin_fmaf(t, r, q);
  t = __builtin_fmaf(-b, q, a);
  return __builtin_fmaf(t, r, q);
}

// Raw bytes of slot s (16 elements) of a row: 32 bytes (bf16) or 64 bytes
// (fp32).  Offsets past the row's resource read zeros.
template <bool BF16IN>
struct SlotRaw {
  uint4 d[BF16IN ? 2 : 4];
};

template <bool BF16IN>
__device__ __forceinline__ SlotRaw<BF16IN> load_slot(__amdgpu_buffer_rsrc_t rs, int s) {
  SlotRaw<BF16IN> r;
  constexpr int B = BF16IN ? 32 : 64;
#pragma unroll
  for (int i = 0; i < B / 16; ++i) r.d[i] = buf_load16(rs, (uint32_t)(s * B + i * 16));
  return r;
}

template <bool BF16IN>
__device__ __forceinline__ void unpack_slot(const SlotRaw<BF16IN>& r, float (&v)[16]) {
  if constexpr (BF16IN) {
    const uint32_t w[8] = {r.d[0].x, r.d[0].y, r.d[0].z, r.d[0].w, r.d[1].x, r.d[1].y, r.d[1].z, r.d[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[4 * i] = __uint_as_float(r.d[i].x);
      v[4 * i + 1] = __uint_as_float(r.d[i].y);
      v[4 * i + 2] = __uint_as_float(r.d[i].z);
      v[4 * i + 3] = __uint_as_float(r.d[i].w);
    }
  }
}

// Stages h = 1, 2, 4, 8 inside the 16 registers of one slot.
__device__ __forceinline__ void fwht16_local(float (&v)[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if ((j & h) == 0) {
        const float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
}

template <int CTRL>
__device__ __forceinline__ float quad_perm(float x) {
  // every lane of the quad is written, so no old value is needed
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Stages h = 16 (partner lane ^ 1) and 32 (lane ^ 2).  Each lane computes
// own + c * partner with c = -1 in the lane that holds the upper index, so
// that lane stores the negated difference; the returned factor is the sign
// every value of this lane now carries.
__device__ __forceinline__ float fwht16_cross(float (&v)[16], int lane) {
  const float c1 = (lane & 1) ? -1.f : 1.f;
  const float c2 = (lane & 2) ? -1.f : 1.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = __builtin_fmaf(c1, quad_perm<0xB1>(v[j]), v[j]);
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = __builtin_fmaf(c2, quad_perm<0x4E>(v[j]), v[j]);
  return c1 * c2;
}

// Maximum over the wave (exact in any order): DPP within each 16-lane row
// (quad swaps, then the half-row and row mirrors leave the row maximum in
// every lane of the row), then the four row maxima read as scalars.
__device__ __forceinline__ float wave_max(float m) {
  m = fmaxf(m, quad_perm<0xB1>(m));    // lane ^ 1
  m = fmaxf(m, quad_perm<0x4E>(m));    // lane ^ 2
  m = fmaxf(m, quad_perm<0x141>(m));   // row_half_mirror: quad q <-> 1 - q in each half row
  m = fmaxf(m, quad_perm<0x140>(m));   // row_mirror: half rows swap
  const int b = __float_as_int(m);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// Boundary screen for E2M1 quotients taken with one multiply,
// q0 = RN(v * RN(1/D)), which is within three representable steps of
// RN(v / D).  Every E2M1 rounding boundary (0.25, 0.75, 1.25, 1.75, 2.5,
// 3.5, 5) has at most three significant bits, so its low 16 bits are zero.
// If no q0 of a slot has its low 16 bits within 4 of a multiple of 2^16, no
// boundary lies between q0 and RN(v / D) and both give the same code;
// otherwise the slot is redone exactly.  Returns the minimum over the slot
// of ((bits(q0) + 4) mod 2^16).
__device__ __forceinline__ uint32_t near_boundary(const float (&q)[16]) {
  us2 mn = (us2){0xFFFF, 0xFFFF};
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    const uint32_t p = __builtin_amdgcn_perm(__float_as_uint(q[i + 1]), __float_as_uint(q[i]), 0x05040100u);
    us2 t = __builtin_bit_cast(us2, p) + (us2){4, 4};
    mn = __builtin_elementwise_min(mn, t);
  }
  return (uint32_t)__builtin_elementwise_min(mn.x, mn.y);
}

constexpr float kBig = 1.2676506002282294e30f;     // 2^100
constexpr float kMinA = 8.077935669463161e-28f;    // 2^-90: dividends at or above keep residuals normal

// One NVFP4 block of 16 transformed values y = v * fl (fl a power of two,
// possibly negative): E4M3 block scale e and the 16 E2M1 codes packed in two
// dwords (low nibble first).  stab holds (S, RN(1/S)) per E4M3 code; live
// says whether the block exists (a screened slot past the end of a row must
// not take the exact path).
__device__ __forceinline__ uint32_t nvfp4_block16(const float (&v)[16], float fl, float g, float rg, bool g_fast,
                                                  const float2* stab, bool live, uint2& codes) {
  float mv = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) mv = fmaxf(mv, __builtin_fabsf(v[i]));
  const float m = mv * __builtin_fabsf(fl);                                             // max |y| of the block
  const float sb = m >= kMinA ? div_rn(m, 6.0f, 0.16666667163372040f) : m / 6.0f;      // RN(m / 6)
  const float sv = (g_fast && sb >= kMinA) ? div_rn(sb, g, rg) : sb / g;                // RN(sb / g)
  const uint32_t e = f32_to_e4m3_sat(sv);
  const float2 SR = stab[e];
  uint32_t w[2] = {0u, 0u};
  if (SR.x > 0.f) {
    const bool fast = SR.x >= kTinyStep && SR.x <= kBig;
    const float D = SR.x / fl, rD = SR.y * fl;   // exact power-of-two rescaling
    float q[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = v[i] * rD;
    if (live && (!fast || near_boundary(q) <= 8u)) {
      if (fast) {
#pragma unroll
        for (int i = 0; i < 16; ++i) q[i] = div_rn(v[i], D, rD);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) q[i] = (v[i] * fl) / SR.x;
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t d = 0;
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, q[8 * h + 0], q[8 * h + 1], 1.0f, 0);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, q[8 * h + 2], q[8 * h + 3], 1.0f, 1);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, q[8 * h + 4], q[8 * h + 5], 1.0f, 2);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, q[8 * h + 6], q[8 * h + 7], 1.0f, 3);
      // the converter writes -0 as 0x8; the packed format uses +0
      const uint32_t mag = d & 0x77777777u;
      const uint32_t nz = (mag + 0x77777777u) & 0x88888888u;
      w[h] = mag | (d & nz);
    }
  }
  codes = make_uint2(w[0], w[1]);
  return e;
}

// Smoothing and rotation of one slot in place; returns the factor fl with
// y = v * fl (see the kernel).
// PRESC: the slot's factors were loaded beforehand (``psc``).
template <bool BF16IN, bool PRESC = false>
__device__ __forceinline__ float transform_slot(const SlotRaw<BF16IN>& raw, float (&v)[16],
                                                __amdgpu_buffer_rsrc_t rsc, bool has_scale, int rot, int order,
                                                int s, int lane, const uint4 (&psc)[4]) {
  unpack_slot<BF16IN>(raw, v);
  float sc[16];
  if (has_scale) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 u;
      if constexpr (PRESC) u = psc[i];
      else u = buf_load16(rsc, (uint32_t)(s * 64 + i * 16));
      sc[4 * i] = __uint_as_float(u.x); sc[4 * i + 1] = __uint_as_float(u.y);
      sc[4 * i + 2] = __uint_as_float(u.z); sc[4 * i + 3] = __uint_as_float(u.w);
    }
  }
  if (order == 0 && has_scale) {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = v[i] * sc[i];
  }
  float fl = 1.0f;
  if (rot) {
    fwht16_local(v);
    fl = 0.125f * fwht16_cross(v, lane);
    if (order == 1) {  // rotate, then smooth: the factor must precede the smoothing product
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = v[i] * fl;
      fl = 1.0f;
    }
  }
  if (order == 1 && has_scale) {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = v[i] * sc[i];
  }
  return fl;
}

// Per-row work of the row quantizer: transform the row held in ``raw``
// (slot (c * WPR + sub) * 64 + lane in chunk c), quantize, store codes and
// steps (or the transformed row, or the running maximum).  Waves of one row
// (WPR > 1) meet through ``red`` with block barriers.
// PRESC: the smoothing factors of every slot were loaded beforehand (psc[c]).
template <int MODE, bool BF16IN, int NC, int WPR, bool PRESC = false>
__device__ __forceinline__ void quant_row_body(const QuantArgs& a, int64_t row, const SlotRaw<BF16IN> (&raw)[NC],
                                               int lane, int wave, int sub, float* red, const float2* stab,
                                               __amdgpu_buffer_rsrc_t rsc, float rg, bool g_fast, float& tmax,
                                               const uint4 (&psc)[PRESC ? NC : 1][4]) {
  constexpr int QMAX = (MODE == MODE_INT4 || MODE == MODE_Y4) ? 7 : 127;
  constexpr bool I8 = MODE == MODE_INT8 || MODE == MODE_INT8W;
  constexpr bool YOUT = MODE == MODE_Y4 || MODE == MODE_Y8;
  constexpr bool F8 = MODE == MODE_FP8;
  constexpr float QDIV = F8 ? 448.0f : (float)QMAX;   // step = amax / QDIV
  const int nslots = a.K >> 4;
  const bool has_scale = a.scale != nullptr;
  (void)wave;
  (void)red;
  (void)stab;
  (void)rg;
  (void)g_fast;
  (void)tmax;
  // --- transform --------------------------------------------------------
  // After this, the value the definition quantizes is y = v * fl exactly
  // (fl = +-1/8 after a smoothing-then-rotation; the power-of-two factor
  // and the lane's butterfly sign are carried into the divisor instead of
  // being multiplied into every element).  Where v * fl would fall below
  // the normal range, every decision is code 0 on both readings, or the
  // slot takes the exact path, which forms y itself.
  // Integer modes need the whole row for its maximum; NVFP4 transforms
  // and quantizes one slot at a time.
  if constexpr (MODE == MODE_INT4 || I8 || F8 || YOUT || MODE == MODE_AMAX) {
    float v[NC][16];
    float fl = 1.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) fl = transform_slot<BF16IN, PRESC>(raw[c], v[c], rsc, has_scale, a.rot, a.order,
                                                                    (c * WPR + sub) * 64 + lane, lane,
                                                                    psc[PRESC ? c : 0]);
    const float afl = __builtin_fabsf(fl);
    float mv = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) mv = fmaxf(mv, __builtin_fabsf(v[c][i]));
    float m = wave_max(mv) * afl;   // = max |y| (rounding is monotone)
    if constexpr (MODE == MODE_AMAX) {
      tmax = fmaxf(tmax, m);
      return;
    } else {
      if constexpr (WPR > 1) {
        if (lane == 0) red[wave] = m;
        __syncthreads();
        m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        if constexpr (WPR == 8) m = fmaxf(m, fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7])));
        __syncthreads();
      }
      const float step = m / QDIV;   // IEEE division
      const bool fast = step >= kTinyStep && step <= kBig;
      const float rstep = fast ? 1.0f / step : 0.f;
      const float D = step / fl, rD = rstep * fl;   // exact power-of-two rescaling
      if (lane == 0 && sub == 0) reinterpret_cast<float*>(a.scales)[row] = step;
      if constexpr (YOUT) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int s = (c * WPR + sub) * 64 + lane;
          if (s >= nslots) continue;
          float4* yp = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.codes) + (size_t)row * a.K + s * 16);
#pragma unroll
          for (int k = 0; k < 4; ++k)
            yp[k] = make_float4(v[c][4 * k] * fl, v[c][4 * k + 1] * fl, v[c][4 * k + 2] * fl, v[c][4 * k + 3] * fl);
        }
        return;
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int s = (c * WPR + sub) * 64 + lane;
        // One-multiply quotients; a boundary k + 1/2 lies between t and
        // RN(v / D) only if |t - rint(t)| is within three steps of 1/2.
        float t[16], r[16], dmax = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          t[i] = v[c][i] * rD;
          r[i] = __builtin_rintf(t[i]);
          dmax = fmaxf(dmax, __builtin_fabsf(t[i] - r[i]));
        }
        constexpr float kEdge = I8 ? 0.5f - 3.0517578125e-05f : 0.5f - 1.9073486328125e-06f;
        bool near;
        if constexpr (F8) {
          // E4M3 rounding boundaries have at most five significant bits, so
          // the low 19 bits of their fp32 patterns are zero; a one-multiply
          // quotient within three steps of one has low bits within 4 of 0.
          uint32_t lo = 0xFFFFFFFFu;
#pragma unroll
          for (int i = 0; i < 16; ++i) lo = min(lo, (__float_as_uint(t[i]) + 4u) & 0x7FFFFu);
          near = lo <= 8u;
        } else {
          near = dmax >= kEdge;
        }
        if (s < nslots && (!fast || near)) {
          if (fast) {
#pragma unroll
            for (int i = 0; i < 16; ++i) t[i] = div_rn(v[c][i], D, rD);
          } else if (step > 0.f) {
#pragma unroll
            for (int i = 0; i < 16; ++i) t[i] = (v[c][i] * fl) / step;
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) t[i] = 0.f;
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) r[i] = __builtin_rintf(t[i]);
        }
        if (s >= nslots) continue;
        if constexpr (F8) {
          // |t| <= 448 up to one rounding: the clamp is the nearest value
          uint32_t w[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float a0 = __builtin_amdgcn_fmed3f(t[4 * k], -448.0f, 448.0f);
            const float a1 = __builtin_amdgcn_fmed3f(t[4 * k + 1], -448.0f, 448.0f);
            const float a2 = __builtin_amdgcn_fmed3f(t[4 * k + 2], -448.0f, 448.0f);
            const float a3 = __builtin_amdgcn_fmed3f(t[4 * k + 3], -448.0f, 448.0f);
            uint32_t d = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
            d = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, d, true);
            // the converter keeps the sign of zero; the format's zero is +0
            const uint32_t mag = d & 0x7F7F7F7Fu;
            w[k] = mag | (d & ((mag + 0x7F7F7F7Fu) & 0x80808080u));
          }
          *reinterpret_cast<uint4*>(a.codes + (size_t)row * a.K + s * 16) = make_uint4(w[0], w[1], w[2], w[3]);
          continue;
        }
        uint32_t q[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          q[i] = (uint32_t)(int)__builtin_amdgcn_fmed3f(r[i], (float)(-QMAX - 1), (float)QMAX);
        if constexpr (MODE == MODE_INT4) {
          uint32_t w0 = 0, w1 = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            w0 |= (q[i] & 0xFu) << (4 * i);
            w1 |= (q[i + 8] & 0xFu) << (4 * i);
          }
          *reinterpret_cast<uint2*>(a.codes + (size_t)row * (a.K >> 1) + s * 8) = make_uint2(w0, w1);
        } else {
          uint32_t w[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            // natural order: dword k holds codes 4k .. 4k+3; W4A8 order: dword k
            // holds the even (k even) or odd (k odd) codes of group k / 2
            const int b = MODE == MODE_INT8W ? 8 * (k >> 1) + (k & 1) : 4 * k;
            const int d = MODE == MODE_INT8W ? 2 : 1;
            w[k] = (q[b] & 0xFFu) | ((q[b + d] & 0xFFu) << 8) | ((q[b + 2 * d] & 0xFFu) << 16) |
                   ((q[b + 3 * d] & 0xFFu) << 24);
          }
          *reinterpret_cast<uint4*>(a.codes + (size_t)row * a.K + s * 16) = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
    }
  } else {  // NVFP4: one E4M3 scale per slot (16 elements)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int s = (c * WPR + sub) * 64 + lane;
      float vs[16];
      const float fl = transform_slot<BF16IN, PRESC>(raw[c], vs, rsc, has_scale, a.rot, a.order, s, lane,
                                                     psc[PRESC ? c : 0]);
      uint2 w;
      const uint32_t e = nvfp4_block16(vs, fl, a.g, rg, g_fast, stab, s < nslots, w);
      if (s < nslots) {
        *reinterpret_cast<uint2*>(a.codes + (size_t)row * (a.K >> 1) + s * 8) = w;
        reinterpret_cast<uint8_t*>(a.scales)[(size_t)row * (a.K >> 4) + s] = (uint8_t)e;
      }
    }
  }
}

template <int MODE, bool BF16IN, int NC, int WPR>
__global__ void __launch_bounds__(64 * (WPR > 4 ? WPR : 4)) quant_rows_kernel(QuantArgs a) {
  // Every argument the kernel reads goes into scalar registers before any
  // branch, so the argument loads issue as one batch with one wait (left to
  // itself the compiler fetched them in three dependent rounds).
  asm volatile("" ::"s"(a.x), "s"(a.R), "s"(a.K), "s"(a.ldx), "s"(a.scale), "s"(a.g), "s"(a.rot), "s"(a.order),
               "s"(a.codes), "s"(a.scales), "s"(a.amax_out), "s"(a.gidx), "s"(a.gr), "s"(a.gout), "s"(a.ldg));
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  static_assert(WPR == 1 || WPR == 4 || WPR == 8, "waves per row");
  constexpr int NWB = WPR > 4 ? WPR : 4;            // waves per block
  constexpr int RPB = NWB / WPR;                    // rows per block
  const int sub = WPR == 1 ? 0 : wave;              // wave index inside the row group
  const int grp = WPR == 1 ? wave : 0;              // row group inside the block
  const bool has_scale = a.scale != nullptr;
  constexpr int ESZ = BF16IN ? 2 : 4;
  __shared__ float red[NWB];
  // NVFP4: (S, RN(1/S)) for every E4M3 code e, S = fp32(value(e) * g).
  __shared__ float2 stab[MODE == MODE_NVFP4 ? 128 : 1];
  if constexpr (MODE == MODE_NVFP4) {
    for (int e = threadIdx.x; e < 128; e += blockDim.x) {
      const float S = e < 0x7F ? e4m3_to_f32((uint32_t)e) * a.g : 0.f;
      stab[e] = make_float2(S, S > 0.f ? 1.0f / S : 0.f);  // IEEE division
    }
    __syncthreads();
  }

  // Smoothing factors: loaded per slot where they are used (every row
  // reads the same K factors, so these hit in cache); past K they read 0.
  const __amdgpu_buffer_rsrc_t rsc = make_rsrc(a.scale, has_scale ? (uint32_t)(a.K * 4) : 0u);
  const float rg = MODE == MODE_NVFP4 ? 1.0f / a.g : 1.0f;   // RN(1/g), IEEE division
  const bool g_fast = a.g >= kTinyStep && a.g <= kBig;

  float tmax = 0.f;  // MODE_AMAX: running max over this wave's rows
  for (int64_t row = (int64_t)blockIdx.x * RPB + grp; row < a.R; row += (int64_t)gridDim.x * RPB) {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(reinterpret_cast<const char*>(a.x) + (size_t)row * a.ldx * ESZ, (uint32_t)(a.K * ESZ));
    SlotRaw<BF16IN> raw[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) raw[c] = load_slot<BF16IN>(rs, (c * WPR + sub) * 64 + lane);
    // Kept channels of this row, from the lines this pass is reading anyway:
    // lane j of the row's first wave copies x[row, gidx[j]] (j < gr).
    if constexpr (BF16IN) {
      if (a.gr > 0 && sub == 0) {
        const uint16_t* xr = reinterpret_cast<const uint16_t*>(a.x) + (size_t)row * a.ldx;
        for (int j = lane; j < a.gr; j += 64) {
          const int c = a.gidx[j];
          a.gout[(size_t)row * a.ldg + j] = (c >= 0 && c < a.K) ? xr[c] : (uint16_t)0;
        }
      }
    }
    const uint4 nopre[1][4] = {};
    quant_row_body<MODE, BF16IN, NC, WPR>(a, row, raw, lane, wave, sub, red, stab, rsc, rg, g_fast, tmax, nopre);
  }
  if constexpr (MODE == MODE_AMAX) {
    if (lane == 0) atomicMax(reinterpret_cast<unsigned int*>(a.amax_out), __float_as_uint(tmax));
  }
}

struct LowrankArgs {
  const uint16_t* l1t;   // r x K bf16, row stride K
  int r;
  uint16_t* out;         // M x ldo bf16: hi in [0, r), lo in [r, 2r)
  int64_t ldo;
};

// quantize_act and the low-rank projection t = x L1 in one launch (Q-WAM
// abstract: the 16-bit branch x L1 L2 beside the 4-bit complement).  The
// first nq workgroups quantize rows, eight at a time, one per wave, exactly
// as quant_rows_kernel does with one wave per row; each of the others
// computes one 16 x 16 tile of t (project_block, as project_kernel).  The
// two parts read x independently and write separate outputs, so they run
// side by side on different CUs, and both outputs are bit-identical to the
// two separate calls; one launch replaces two.
template <int MODE, int NC>
__global__ void __launch_bounds__(64 * kProjWaves) quant_project_kernel(QuantArgs a, LowrankArgs p, int nq, int mt) {
  __shared__ __attribute__((aligned(16))) uint8_t area[kProjLdsBytes];
  __shared__ float2 stab[MODE == MODE_NVFP4 ? 128 : 1];
  if ((int)blockIdx.x >= nq) {   // projection workgroup
    const int t = (int)blockIdx.x - nq;
    project_block(reinterpret_cast<const uint16_t*>(a.x), a.ldx, (int)a.R, a.K, p.l1t, p.r, p.out, p.ldo,
                  (t % mt) * kProjRows, (t / mt) * 16, area);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int RPB = kProjWaves;   // rows per workgroup, one per wave
  if constexpr (MODE == MODE_NVFP4) {
    for (int e = threadIdx.x; e < 128; e += blockDim.x) {
      const float S = e < 0x7F ? e4m3_to_f32((uint32_t)e) * a.g : 0.f;
      stab[e] = make_float2(S, S > 0.f ? 1.0f / S : 0.f);  // IEEE division
    }
    __syncthreads();
  }
  const bool has_scale = a.scale != nullptr;
  const __amdgpu_buffer_rsrc_t rsc = make_rsrc(a.scale, has_scale ? (uint32_t)(a.K * 4) : 0u);
  const float rg = MODE == MODE_NVFP4 ? 1.0f / a.g : 1.0f;   // RN(1/g), IEEE division
  const bool g_fast = a.g >= kTinyStep && a.g <= kBig;
  float tmax = 0.f;
  for (int64_t row = (int64_t)blockIdx.x * RPB + wave; row < a.R; row += (int64_t)nq * RPB) {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(reinterpret_cast<const char*>(a.x) + (size_t)row * a.ldx * 2, (uint32_t)(a.K * 2));
    SlotRaw<true> raw[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) raw[c] = load_slot<true>(rs, c * 64 + lane);
    const uint4 nopre[1][4] = {};
    quant_row_body<MODE, true, NC, 1>(a, row, raw, lane, wave, 0, nullptr, stab, rsc, rg, g_fast, tmax, nopre);
  }
}

// Row quantizer fused with the low-rank branch projection (Q-WAM abstract:
// the 16-bit branch x L1 L2 next to the 4-bit complement), so x leaves HBM
// once.  A workgroup of eight waves takes four rows at a time and walks
// row groups with a grid-stride loop.  Waves 0..3 quantize, one row each,
// with quant_rows_kernel's body; waves 4..7 compute T = x L1 for the same
// four rows, each over a quarter of K.  The two halves share no data and
// run side by side; both read the rows, the second time from cache.
// * Projection wave p owns the 128-element K chunks p, p + 4, ... and
//   streams each through a private four-slot LDS ring: the chunk of L1
//   (transposed, r x K: r rows of 256 bytes, 16-byte slot s of row j
//   stored at s XOR (j mod 16), so the 16 rows an MFMA fragment reads fall
//   on distinct banks) and the four rows' 256 bytes of the same K range,
//   by buffer-to-LDS copies of whole lines.  Chunks past K are copied as
//   zeros, so every wait is a fixed vmcnt.
// * Per chunk: two 64-element K pairs of bf16 16x16x32 products per
//   16-column block (A = the four rows, read again by the lanes of rows
//   4..15, whose outputs are dropped; within a pair, lane group g holds K
//   elements 16 g .. 16 g + 15 on both operands), then a wait for the
//   slot's LDS reads and the copy of the chunk four ahead into it.
// * A barrier; the four partial 4 x r tiles are added in LDS in wave
//   order and T goes out as the bf16 pair hi = bf16(T), lo = bf16(T - hi)
//   (columns [0, r) and [r, 2r)).
// The barriers wait for LDS operations only (lgkmcnt), never for the
// untracked copies in flight.
constexpr int kLrMaxK = 4096;                  // row length limit (four slots per lane)
constexpr int kLrMaxR = 32;                    // rank limit (two 16-column blocks)
constexpr int kLrChunkK = 128;                 // K elements per chunk
constexpr int kLrRing = 4;                     // chunk slots per projection wave

__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0); vmcnt and expcnt not waited on
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int MODE, int NC, int JB>
__global__ void __launch_bounds__(512) quant_rows_lowrank_kernel(QuantArgs a, LowrankArgs p) {
  asm volatile("" ::"s"(a.x), "s"(a.R), "s"(a.K), "s"(a.ldx), "s"(a.scale), "s"(a.g), "s"(a.rot), "s"(a.order),
               "s"(a.codes), "s"(a.scales), "s"(p.l1t), "s"(p.r), "s"(p.out), "s"(p.ldo));
  constexpr int R16 = 16 * JB;                 // rows of L1 transposed (p.r == R16)
  constexpr int CHB = R16 * kLrChunkK * 2;     // bytes of one chunk of L1
  constexpr int NCP = CHB / 1024;              // its copy instructions
  constexpr int SLOT = CHB + 1024;             // + the four rows' 256 bytes each
  constexpr int PER = NCP + 1;                 // copy instructions per chunk
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool quantizer = wave < 4;             // wave-uniform role
  const int q = wave & 3;                      // row (quantizer) or K share (projection)
  const int lr = lane & 15, lq = lane >> 4;
  const bool has_scale = a.scale != nullptr;
  const int npairs = a.K >> 6;                 // 64-element K pairs
  const int nchunks = (a.K + kLrChunkK - 1) / kLrChunkK;
  const int nsteps = (nchunks + 3) / 4;        // chunks per projection wave (the last ones may lie past K)
  __shared__ __attribute__((aligned(1024))) uint8_t ring[4 * kLrRing * (2 * 16 * kLrChunkK * 2 + 1024)];
  __shared__ float part[4 * JB * 4 * 16];
  __shared__ float2 stab[MODE == MODE_NVFP4 ? 128 : 1];
  if constexpr (MODE == MODE_NVFP4) {
    for (int e = threadIdx.x; e < 128; e += blockDim.x) {
      const float S = e < 0x7F ? e4m3_to_f32((uint32_t)e) * a.g : 0.f;
      stab[e] = make_float2(S, S > 0.f ? 1.0f / S : 0.f);
    }
    __syncthreads();
  }
  const __amdgpu_buffer_rsrc_t rsc = make_rsrc(a.scale, has_scale ? (uint32_t)(a.K * 4) : 0u);
  const float rg = MODE == MODE_NVFP4 ? 1.0f / a.g : 1.0f;
  const bool g_fast = a.g >= kTinyStep && a.g <= kBig;
  float tmax = 0.f;

  // L1 copies: instruction n of a chunk covers chunk bytes [1024 n, 1024 n
  // + 1024), lane l the 16 bytes at 1024 n + 16 l: row 4 n + l / 16,
  // physical slot l % 16.  Row copy: lane l, row l / 16, 16-byte piece
  // l % 16 of the chunk's 256 bytes, unswizzled.
  const v4u rl = rsrc_words(p.l1t, (uint32_t)(R16 * a.K * 2));
  uint32_t coff[NCP], cslot[NCP];
#pragma unroll
  for (int n = 0; n < NCP; ++n) {
    const int row = 4 * n + (lane >> 4);
    cslot[n] = (uint32_t)((lane & 15) ^ (row & 15)) * 16;             // logical slot, bytes
    coff[n] = (uint32_t)(row * a.K * 2) + cslot[n];
  }
  const uint32_t xpiece = (uint32_t)(lane & 15) * 16;
  const uint32_t ring0 = lds_addr(ring) + (uint32_t)(q * kLrRing * SLOT);

  for (int64_t row0 = (int64_t)blockIdx.x * 4; row0 < a.R; row0 += (int64_t)gridDim.x * 4) {
    if (quantizer) {
      const int64_t row = row0 + q;
      if (row < a.R) {
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(reinterpret_cast<const char*>(a.x) + (size_t)row * a.ldx * 2, (uint32_t)(a.K * 2));
        SlotRaw<true> raw[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) raw[c] = load_slot<true>(rs, c * 64 + lane);
        const uint4 nopre[1][4] = {};
        quant_row_body<MODE, true, NC, 1>(a, row, raw, lane, q, 0, nullptr, stab, rsc, rg, g_fast, tmax, nopre);
      }
    } else {
      const int nrows = (int)min((int64_t)4, a.R - row0);
      const v4u rx = rsrc_words(reinterpret_cast<const char*>(a.x) + (size_t)row0 * a.ldx * 2,
                                (uint32_t)(nrows * a.ldx * 2));
      const uint32_t xoff = (uint32_t)((lane >> 4) * a.ldx * 2) + xpiece;
      auto copy_chunk = [&](int step) {        // chunk q + 4 step into slot step % kLrRing
        const int g = q + 4 * step;             // wave-uniform
        const uint32_t dst = ring0 + (uint32_t)((step % kLrRing) * SLOT);
        const uint32_t k0 = g < nchunks ? (uint32_t)(g * 256) : 0u;
#pragma unroll
        for (int n = 0; n < NCP; ++n) {
          // the last chunk may be half a chunk: its other half would be the next row
          const bool ok = g < nchunks && k0 + cslot[n] < (uint32_t)(a.K * 2);
          dma16_at(rl, dst + n * 1024, ok ? coff[n] : kOOB, k0);
        }
        const bool okx = g < nchunks && k0 + xpiece < (uint32_t)(a.K * 2);
        dma16_at(rx, dst + CHB, okx ? xoff : kOOB, k0);
      };
#pragma unroll
      for (int step = 0; step < kLrRing - 1; ++step) copy_chunk(step);
      v4f acc[JB];
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) acc[jb] = v4f{0.f, 0.f, 0.f, 0.f};
      for (int step = 0; step < nsteps; ++step) {
        copy_chunk(step + kLrRing - 1);        // into the slot read two steps ago (its reads waited for)
        wait_vmcnt<(kLrRing - 1) * PER>();     // chunk `step` has landed
        asm volatile("" ::: "memory");
        const int g = q + 4 * step;
        const uint8_t* slot = ring + (q * kLrRing + step % kLrRing) * SLOT;
        const uint8_t* arow = slot + CHB + (lr & 3) * 256 + lq * 32;
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) {
          const int pp = 2 * g + pl;
          if (pp < npairs) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const v8bf af = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(arow + pl * 128 + h * 16));
              const int L = pl * 8 + lq * 2 + h;
#pragma unroll
              for (int jb = 0; jb < JB; ++jb) {
                const uint4 b = *reinterpret_cast<const uint4*>(slot + (jb * 16 + lr) * 256 + ((L ^ lr) * 16));
                acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(v8bf, b), acc[jb], 0, 0, 0);
              }
            }
          }
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0): this slot's reads are done
        asm volatile("" ::: "memory");
      }
      wait_vmcnt<0>();                          // the trailing copies (past K: zeros) have landed
      // lanes 0..15 hold rows 0..3 (one per register) of column lr of each block
      if (lq == 0) {
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
#pragma unroll
          for (int i = 0; i < 4; ++i) part[((q * JB + jb) * 4 + i) * 16 + lr] = acc[jb][i];
      }
    }
    lds_barrier();   // the partial tiles are written
    for (int t = threadIdx.x; t < 4 * R16; t += blockDim.x) {
      const int i = t / R16, j = t - i * R16;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) v += part[((w * JB + (j >> 4)) * 4 + i) * 16 + (j & 15)];
      if (row0 + i < a.R) {
        const uint32_t hi = f32_to_bf16_bits(v);
        const float lo = v - bf16_bits_to_f32(hi);
        uint16_t* o = p.out + (size_t)(row0 + i) * p.ldo;
        o[j] = (uint16_t)hi;
        o[R16 + j] = (uint16_t)f32_to_bf16_bits(lo);
      }
    }
    lds_barrier();   // the partial tiles are written again by the next row group
  }
}

// NVFP4 quantizer for many rows, K a multiple of 64: lane = row.  A wave
// takes 64 consecutive rows and one 64-channel Hadamard block; every
// butterfly stage then runs inside one lane's registers, and the block's 64
// smoothing factors are the same for the whole wave (scalar loads).  NVFP4
// needs no row-wide reduction (its scales are per 16 elements and the tensor
// scale is fixed), so every (rows, block) pair is an independent task.
// The grid is sized to stay resident; each wave walks its tasks and copies
// the next task's tile while it transforms and encodes the current one, so
// the HBM reads overlap the vector work.  NB = 2: two LDS tiles per wave,
// the next copy issued before the current tile is read; NB = 1: one tile,
// the next copy issued as soon as the current tile's reads have returned,
// which halves the LDS per wave and lets twice as many waves share a SIMD
// (the vector work of one wave then hides the stalls of the others).
template <bool BF16IN>
constexpr int nvfp4_lanes_tile() { return 64 * 64 * (BF16IN ? 2 : 4); }

// 16-byte slot swizzle of tile row r (CPR slots per row): 16 consecutive
// rows, read at the same logical slot by 16 lanes of one LDS pass, land on
// 16 distinct 16-byte bank groups of the 256-byte bank window (128-byte
// bf16 rows: two rows per window, so the row pair index picks the slot).
template <int CPR>
__device__ __forceinline__ int tile_swz(int r) {
  return CPR >= 16 ? (r & 15) : ((r >> 1) & (CPR - 1));
}

template <bool BF16IN, bool ROT, int NB>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NB == 1 ? 4 : 1)))
quant_nvfp4_lanes_kernel(QuantArgs a) {
  constexpr int ESZ = BF16IN ? 2 : 4;
  constexpr int RB = 64 * ESZ;              // bytes of one row's 64-element block
  constexpr int TILE = nvfp4_lanes_tile<BF16IN>();   // one wave's 64 x 64 tile
  constexpr int NCOPY = TILE / 1024;        // copy instructions per tile
  __shared__ float2 stab[128];
  __shared__ __attribute__((aligned(16))) uint8_t tiles[4][NB][TILE];
  for (int e = threadIdx.x; e < 128; e += blockDim.x) {
    const float S = e < 0x7F ? e4m3_to_f32((uint32_t)e) * a.g : 0.f;
    stab[e] = make_float2(S, S > 0.f ? 1.0f / S : 0.f);  // IEEE division
  }
  __syncthreads();
  const float rg = 1.0f / a.g;   // RN(1/g)
  const bool g_fast = a.g >= kTinyStep && a.g <= kBig;
  const bool has_scale = a.scale != nullptr;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // task indices fit 32 bits (the launch checks), so (rows, block) comes
  // from a 32-bit division
  const uint32_t nblk = (uint32_t)(a.K >> 6);
  const uint32_t ngrp = (uint32_t)((a.R + 63) >> 6);
  const uint32_t ntask = ngrp * nblk;
  const uint32_t stride = gridDim.x * 4u;
  constexpr int CPR = RB / 16;              // 16-byte chunks per row of the tile

  // Coalesced copy of task t's 64 x 64 tile into buffer `buf` of this
  // wave's LDS slice: copy instruction i covers tile bytes [1024 i,
  // 1024 i + 1024); the chunk at slot q of tile row r holds logical chunk
  // q ^ tile_swz(r) (so that the 64 rows read back by the 64 lanes spread
  // over the banks).  Rows past R read zeros.  The lane's offset inside the
  // tile is fixed; the block's byte offset goes in the scalar operand.
  uint32_t loff[NCOPY];
#pragma unroll
  for (int i = 0; i < NCOPY; ++i) {
    const int p = i * 1024 + lane * 16;
    const int r = p / RB, q = (p % RB) / 16;
    const int L = q ^ tile_swz<CPR>(r);
    loff[i] = (uint32_t)(r * (int)(a.ldx * ESZ) + L * 16);
  }
  const uint32_t tiles_lds = lds_addr(&tiles[wave][0][0]);
  auto copy_tile = [&](uint32_t t, int buf) {
    const uint32_t grp = t / nblk;
    const uint32_t b = t - grp * nblk;
    const v4u rs = rsrc_words(reinterpret_cast<const char*>(a.x) + (size_t)grp * 64 * a.ldx * ESZ,
                              (uint32_t)(min((int64_t)64, a.R - (int64_t)grp * 64) * a.ldx * ESZ));
    const uint32_t tile = tiles_lds + (uint32_t)(buf * TILE);
#pragma unroll
    for (int i = 0; i < NCOPY; ++i) dma16_at(rs, tile + i * 1024, loff[i], b * RB);
  };

  // the kept-channel indices, two per lane (a gather of at most 128)
  int gkeep[2] = {-1, -1};
  if constexpr (BF16IN) {
    if (lane < a.gr) gkeep[0] = a.gidx[lane];
    if (64 + lane < a.gr) gkeep[1] = a.gidx[64 + lane];
  }

  uint32_t task = blockIdx.x * 4u + (uint32_t)wave;
  if (task < ntask) copy_tile(task, 0);
  for (int buf = 0; task < ntask; task += stride, buf ^= (NB - 1)) {
    const uint32_t grp = task / nblk;
    const int b = (int)(task - grp * nblk);
    const int64_t row = (int64_t)grp * 64 + lane;
    const bool live = row < a.R;
    // Start the next task's copy, then wait for this task's tile only:
    // loads complete in order, so at most NCOPY outstanding operations
    // leaves just the copies issued last.
    // (The copies are issued as inline assembly, which the compiler does
    // not track, so these explicit waits are the only ones.)
    if (NB == 2 && task + stride < ntask) {
      copy_tile(task + stride, buf ^ 1);
      wait_vmcnt<NCOPY>();
    } else {
      wait_vmcnt<0>();
    }
    asm volatile("" ::: "memory");
    const uint8_t* tile = tiles[wave][buf];
    float v[64];
#pragma unroll
    for (int c = 0; c < CPR; ++c) {
      const uint4 d = *reinterpret_cast<const uint4*>(tile + lane * RB + ((c ^ tile_swz<CPR>(lane)) * 16));
      if constexpr (BF16IN) {
        const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[8 * c + 2 * k] = __uint_as_float(w[k] << 16);
          v[8 * c + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
      } else {
        v[4 * c] = __uint_as_float(d.x); v[4 * c + 1] = __uint_as_float(d.y);
        v[4 * c + 2] = __uint_as_float(d.z); v[4 * c + 3] = __uint_as_float(d.w);
      }
    }
    // Kept channels inside this 64-channel block, read from the tile: lane
    // j holds gidx[j] and gidx[64 + j]; a ballot names the ones in block b,
    // and for each, every lane (a row) copies its element.  The task of
    // block 0 writes the zeros of indices outside [0, K).
    if constexpr (BF16IN) {
      if (a.gr > 0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int j = 64 * h + lane;
          const int c = gkeep[h];
          const bool in = c >= 0 && c < a.K;
          uint64_t m = __builtin_amdgcn_ballot_w64(j < a.gr && ((in && (c >> 6) == b) || (!in && b == 0)));
          while (m) {
            const int jj = __builtin_ctzll(m);
            m &= m - 1;
            const int cj = __builtin_amdgcn_readlane(c, jj);
            uint16_t val = 0;
            if (cj >= 0 && cj < a.K) {
              const int cc = cj & 63;
              val = *reinterpret_cast<const uint16_t*>(
                  tile + lane * RB + (((cc >> 3) ^ tile_swz<CPR>(lane)) * 16) + (cc & 7) * 2);
            }
            if (live) a.gout[(size_t)row * a.ldg + 64 * h + jj] = val;
          }
        }
      }
    }
    // NB = 2: the copy two tasks ahead overwrites this buffer only after
    // these reads have returned (their values are consumed below).  NB = 1:
    // wait for every LDS read of this tile, then start the next task's copy
    // into it.
    __builtin_amdgcn_wave_barrier();
    if constexpr (NB == 1) {
      if (task + stride < ntask) {
        asm volatile("" ::: "memory");         // every tile read issued above this point
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt and expcnt not waited on
        asm volatile("" ::: "memory");
        copy_tile(task + stride, 0);
      }
    }
    // the block's 64 factors are the same for the whole wave: scalar loads
    const __attribute__((address_space(4))) float* sc =
        (const __attribute__((address_space(4))) float*)(a.scale + (has_scale ? b * 64 : 0));
    if (has_scale && a.order == 0) {
#pragma unroll
      for (int i = 0; i < 64; ++i) v[i] = v[i] * sc[i];
    }
    float fl = 1.0f;
    if constexpr (ROT) {
#pragma unroll
      for (int h = 1; h < 64; h <<= 1) {
#pragma unroll
        for (int j = 0; j < 64; ++j) {
          if ((j & h) == 0) {
            const float x0 = v[j], x1 = v[j + h];
            v[j] = x0 + x1;
            v[j + h] = x0 - x1;
          }
        }
      }
      fl = 0.125f;
      if (a.order == 1) {  // rotate, then smooth: the factor must precede the smoothing product
#pragma unroll
        for (int i = 0; i < 64; ++i) v[i] = v[i] * 0.125f;
        fl = 1.0f;
      }
    }
    if (has_scale && a.order == 1) {
#pragma unroll
      for (int i = 0; i < 64; ++i) v[i] = v[i] * sc[i];
    }
    uint2 c[4];
    uint32_t e4 = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float vb[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) vb[i] = v[16 * q + i];
      e4 |= nvfp4_block16(vb, fl, a.g, rg, g_fast, stab, live, c[q]) << (8 * q);
    }
    if (live) {
      uint4* cp = reinterpret_cast<uint4*>(a.codes + (size_t)row * (a.K >> 1) + b * 32);
      cp[0] = make_uint4(c[0].x, c[0].y, c[1].x, c[1].y);
      cp[1] = make_uint4(c[2].x, c[2].y, c[3].x, c[3].y);
      *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.scales) + (size_t)row * (a.K >> 4) + b * 4) = e4;
    }
  }
}

__global__ void zero_u32_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

template <int MODE, bool BF16IN, int WPR>
static hipError_t launch_nc(int nc, dim3 grid, hipStream_t st, const QuantArgs& a) {
#define W4A4_NC_CASE(N)                                                                         \
  case N:                                                                                      \
    hipLaunchKernelGGL((quant_rows_kernel<MODE, BF16IN, N, WPR>), grid, dim3(WPR > 4 ? 64 * WPR : 256), 0, st, a); \
    break;
  switch (nc) {
    W4A4_NC_CASE(1)
    W4A4_NC_CASE(2)
    W4A4_NC_CASE(3)
    W4A4_NC_CASE(4)
    W4A4_NC_CASE(5)
    W4A4_NC_CASE(6)
    W4A4_NC_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef W4A4_NC_CASE
  return hipGetLastError();
}

static int round_nc(int nc) {
  const int allowed[] = {1, 2, 3, 4, 5, 6, 8};
  for (int v : allowed)
    if (nc <= v) return v;
  return -1;
}

// Largest K a single launch supports: 8 chunks x 64 lanes x 16 elements x 4 waves.
int64_t quant_max_k() { return 8LL * 64 * 16 * 4; }

int64_t quant_lowrank_max_k() { return kLrMaxK; }
int quant_lowrank_max_r() { return kLrMaxR; }
bool quant_lowrank_fits(int64_t K, int64_t r) {
  return K % 64 == 0 && K <= kLrMaxK && (r == 16 || r == 32);
}

template <int MODE, int JB>
static hipError_t launch_lowrank_mode(int nc, dim3 grid, hipStream_t st, const QuantArgs& a, const LowrankArgs& p) {
  switch (nc) {
    case 1: hipLaunchKernelGGL((quant_rows_lowrank_kernel<MODE, 1, JB>), grid, dim3(512), 0, st, a, p); break;
    case 2: hipLaunchKernelGGL((quant_rows_lowrank_kernel<MODE, 2, JB>), grid, dim3(512), 0, st, a, p); break;
    case 3: hipLaunchKernelGGL((quant_rows_lowrank_kernel<MODE, 3, JB>), grid, dim3(512), 0, st, a, p); break;
    case 4: hipLaunchKernelGGL((quant_rows_lowrank_kernel<MODE, 4, JB>), grid, dim3(512), 0, st, a, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_lowrank_r(int nc, int r, dim3 grid, hipStream_t st, const QuantArgs& a, const LowrankArgs& p) {
  return r == 16 ? launch_lowrank_mode<MODE, 1>(nc, grid, st, a, p) : launch_lowrank_mode<MODE, 2>(nc, grid, st, a, p);
}

bool quant_project_fits(int64_t K, int64_t r) { return K % 16 == 0 && K <= 5 * 1024 && r >= 1 && r <= 128; }

template <int MODE>
static hipError_t launch_quant_project_nc(int nc, dim3 grid, hipStream_t st, const QuantArgs& a, const LowrankArgs& p,
                                          int nq, int mt) {
  switch (nc) {
    case 1: hipLaunchKernelGGL((quant_project_kernel<MODE, 1>), grid, dim3(64 * kProjWaves), 0, st, a, p, nq, mt); break;
    case 2: hipLaunchKernelGGL((quant_project_kernel<MODE, 2>), grid, dim3(64 * kProjWaves), 0, st, a, p, nq, mt); break;
    case 3: hipLaunchKernelGGL((quant_project_kernel<MODE, 3>), grid, dim3(64 * kProjWaves), 0, st, a, p, nq, mt); break;
    case 4: hipLaunchKernelGGL((quant_project_kernel<MODE, 4>), grid, dim3(64 * kProjWaves), 0, st, a, p, nq, mt); break;
    case 5: hipLaunchKernelGGL((quant_project_kernel<MODE, 5>), grid, dim3(64 * kProjWaves), 0, st, a, p, nq, mt); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quantize_project(int mode, const void* x, int64_t R, int64_t K, int64_t ldx, const float* scale,
                                   float g, int rot, int order, void* codes, void* scales, const uint16_t* l1t, int r,
                                   uint16_t* out, int64_t ldo, hipStream_t st) {
  if (!quant_project_fits(K, r) || R < 1) return hipErrorInvalidValue;
  QuantArgs a{x, R, (int)K, ldx, scale, g, rot, order, (uint8_t*)codes, scales, nullptr, nullptr, 0, nullptr, 0};
  const LowrankArgs p{l1t, r, out, ldo};
  const int nc = round_nc((int)((K / 16 + 63) / 64));   // slots per lane, one wave per row
  int64_t nq = (R + kProjWaves - 1) / kProjWaves;       // quantizer workgroups (grid-stride beyond 1024)
  if (nq > 1024) nq = 1024;
  const int64_t mt = (R + kProjRows - 1) / kProjRows, ct = (r + 15) / 16;
  const int64_t total = nq + mt * ct;
  if (total > INT32_MAX || mt > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)total);
  switch (mode) {
    case MODE_INT4: return launch_quant_project_nc<MODE_INT4>(nc, grid, st, a, p, (int)nq, (int)mt);
    case MODE_INT8: return launch_quant_project_nc<MODE_INT8>(nc, grid, st, a, p, (int)nq, (int)mt);
    case MODE_INT8W: return launch_quant_project_nc<MODE_INT8W>(nc, grid, st, a, p, (int)nq, (int)mt);
    case MODE_FP8: return launch_quant_project_nc<MODE_FP8>(nc, grid, st, a, p, (int)nq, (int)mt);
    case MODE_NVFP4: return launch_quant_project_nc<MODE_NVFP4>(nc, grid, st, a, p, (int)nq, (int)mt);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quantize_lowrank(int mode, const void* x, int64_t R, int64_t K, int64_t ldx, const float* scale,
                                   float g, int rot, int order, void* codes, void* scales, const uint16_t* l1t, int r,
                                   uint16_t* out, int64_t ldo, hipStream_t st) {
  if (!quant_lowrank_fits(K, r)) return hipErrorInvalidValue;
  QuantArgs a{x, R, (int)K, ldx, scale, g, rot, order, (uint8_t*)codes, scales, nullptr, nullptr, 0, nullptr, 0};
  const LowrankArgs p{l1t, r, out, ldo};
  const int nc = (int)((K / 16 + 63) / 64);       // slots per lane (K <= 4096: at most 4)
  int64_t blocks = (R + 3) / 4;
  if (blocks > 1024) blocks = 1024;               // grid-stride beyond four row groups per CU
  const dim3 grid((unsigned)blocks);
  switch (mode) {
    case MODE_INT4: return launch_lowrank_r<MODE_INT4>(nc, r, grid, st, a, p);
    case MODE_INT8: return launch_lowrank_r<MODE_INT8>(nc, r, grid, st, a, p);
    case MODE_INT8W: return launch_lowrank_r<MODE_INT8W>(nc, r, grid, st, a, p);
    case MODE_FP8: return launch_lowrank_r<MODE_FP8>(nc, r, grid, st, a, p);
    case MODE_NVFP4: return launch_lowrank_r<MODE_NVFP4>(nc, r, grid, st, a, p);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quantize(int mode, bool bf16in, const void* x, int64_t R, int64_t K, int64_t ldx,
                           const float* scale, float g, int rot, int order, void* codes, void* scales,
                           float* amax_out, hipStream_t st, const int32_t* gidx, int gr, void* gout,
                           int64_t ldg) {
  QuantArgs a{x, R, (int)K, ldx, scale, g, rot, order, (uint8_t*)codes, scales, amax_out,
              gidx, gr, (uint16_t*)gout, ldg};
  // The row-per-lane kernel addresses a 64-row tile with 32-bit offsets
  // (64 rows of ldx elements); longer strides take the row kernels, whose
  // resources cover one row each.
  if (mode == MODE_NVFP4 && R >= 256 && K % 64 == 0 && (rot == 0 || rot == 64) &&
      ((R + 63) / 64) * (K / 64) < (1LL << 31) && 64 * ldx * (bf16in ? 2 : 4) < (1LL << 31)) {
    // resident grid: as many four-wave blocks as the tiles' LDS lets every CU hold
    const int64_t tasks = ((R + 63) / 64) * (K / 64);
    constexpr int NB = 1;
    const int per_cu = (160 * 1024) / (NB * 4 * (bf16in ? nvfp4_lanes_tile<true>() : nvfp4_lanes_tile<false>()) + 1024);
    int64_t blocks = (tasks + 3) / 4;
    if (blocks > 256 * per_cu) blocks = 256 * per_cu;
    const dim3 grid((unsigned)blocks);
    if (bf16in) {
      if (rot) hipLaunchKernelGGL((quant_nvfp4_lanes_kernel<true, true, NB>), grid, dim3(256), 0, st, a);
      else hipLaunchKernelGGL((quant_nvfp4_lanes_kernel<true, false, NB>), grid, dim3(256), 0, st, a);
    } else {
      if (rot) hipLaunchKernelGGL((quant_nvfp4_lanes_kernel<false, true, NB>), grid, dim3(256), 0, st, a);
      else hipLaunchKernelGGL((quant_nvfp4_lanes_kernel<false, false, NB>), grid, dim3(256), 0, st, a);
    }
    return hipGetLastError();
  }
  const int64_t nslots = K / 16;
  // One wave per row when there are many rows and the row fits five chunks
  // per lane (the factors then stay in registers); else four waves per row,
  // eight for integer codes of rows longer than 4096.
  const bool intmode = mode == MODE_INT4 || mode == MODE_INT8 || mode == MODE_INT8W || mode == MODE_FP8 ||
                       mode == MODE_Y4 || mode == MODE_Y8;
  int wpr = (R >= 1024 && nslots <= 5 * 64) ? 1 : 4;
  if (wpr == 4 && intmode && nslots > 4 * 64) wpr = 8;
  const int nc = round_nc((int)((nslots + 64 * wpr - 1) / (64 * wpr)));
  if (nc < 0) return hipErrorInvalidValue;
  const int rows_per_block = wpr == 1 ? 4 : 1;
  int64_t blocks = (R + rows_per_block - 1) / rows_per_block;
  const int64_t cap = 256 * 8;  // grid-stride beyond 8 blocks per CU
  if (mode == MODE_AMAX) {
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, st, (uint32_t*)amax_out, (size_t)1);
  }
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  dim3 grid((unsigned)blocks);
  if (wpr == 8) {
    if (mode == MODE_INT4) return bf16in ? launch_nc<MODE_INT4, true, 8>(nc, grid, st, a)
                                         : launch_nc<MODE_INT4, false, 8>(nc, grid, st, a);
    if (mode == MODE_INT8W) return bf16in ? launch_nc<MODE_INT8W, true, 8>(nc, grid, st, a)
                                          : launch_nc<MODE_INT8W, false, 8>(nc, grid, st, a);
    if (mode == MODE_FP8) return bf16in ? launch_nc<MODE_FP8, true, 8>(nc, grid, st, a)
                                        : launch_nc<MODE_FP8, false, 8>(nc, grid, st, a);
    if (mode == MODE_Y4) return bf16in ? launch_nc<MODE_Y4, true, 8>(nc, grid, st, a)
                                       : launch_nc<MODE_Y4, false, 8>(nc, grid, st, a);
    if (mode == MODE_Y8) return bf16in ? launch_nc<MODE_Y8, true, 8>(nc, grid, st, a)
                                       : launch_nc<MODE_Y8, false, 8>(nc, grid, st, a);
    return bf16in ? launch_nc<MODE_INT8, true, 8>(nc, grid, st, a) : launch_nc<MODE_INT8, false, 8>(nc, grid, st, a);
  }
#define W4A4_DISPATCH(MODE)                                                          \
  if (mode == MODE) {                                                                \
    if (bf16in) return wpr == 1 ? launch_nc<MODE, true, 1>(nc, grid, st, a)          \
                                : launch_nc<MODE, true, 4>(nc, grid, st, a);         \
    return wpr == 1 ? launch_nc<MODE, false, 1>(nc, grid, st, a)                     \
                    : launch_nc<MODE, false, 4>(nc, grid, st, a);                    \
  }
  W4A4_DISPATCH(MODE_INT4)
  W4A4_DISPATCH(MODE_INT8)
  W4A4_DISPATCH(MODE_INT8W)
  W4A4_DISPATCH(MODE_FP8)
  W4A4_DISPATCH(MODE_Y4)
  W4A4_DISPATCH(MODE_Y8)
  W4A4_DISPATCH(MODE_NVFP4)
  W4A4_DISPATCH(MODE_AMAX)
#undef W4A4_DISPATCH
  return hipErrorInvalidValue;
}

}  // namespace w4a4
