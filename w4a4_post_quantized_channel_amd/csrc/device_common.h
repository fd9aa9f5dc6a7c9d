// Device-side helpers shared by the gfx950 kernels of the quantized linear.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a4 {

constexpr int kWave = 64;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// Raw buffer resource over [base, base + bytes): loads at offsets outside the
// range return zeros, so edge tiles need no branches around their loads.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOOB = 0x80000000u;  // an offset past every resource used here

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Exact E4M3 (OCP E4M3FN) -> fp32 for codes 0x00..0x7E (no sign used).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 0xF, m = c & 7;
  float normal = __uint_as_float(((e + 120u) << 23) | (m << 20));
  float sub = (float)m * 0.001953125f;  // m * 2^-9
  return e ? normal : sub;
}

// Round a non-negative finite fp32 onto E4M3 (nearest, ties to even
// mantissa, saturating at 448 = code 0x7E).  code = (E + 6) * 8 + r with
// E = max(floor(log2 v), -6) and r = rne(v * 2^(3 - E)).
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float v) {
  if (!(v > 0.f)) return 0u;
  if (v >= 448.f) return 0x7Eu;
  int E = (int)((__float_as_uint(v) >> 23) & 0xFF) - 127;
  E = E < -6 ? -6 : E;
  float q = v * __uint_as_float((uint32_t)(127 + 3 - E) << 23);
  int r = (int)__builtin_rintf(q);
  int code = (E + 6) * 8 + r;
  return (uint32_t)(code > 0x7E ? 0x7E : code);
}

// Round fp32 onto E2M1 (nearest, ties to even mantissa, saturating at 6);
// zero (and anything rounding to zero) encodes as +0.
__device__ __forceinline__ uint32_t f32_to_e2m1_sat(float v) {
  float a = __builtin_fabsf(v);
  uint32_t i = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) +
               (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  uint32_t s = (v < 0.f && i != 0) ? 8u : 0u;
  return s | i;
}

}  // namespace w4a4
