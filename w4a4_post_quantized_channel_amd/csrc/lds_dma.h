// Global -> LDS copies for the gfx950 GEMM kernels.
#pragma once
#include "device_common.h"

namespace w4a4 {

// Global -> LDS copies (buffer loads with the LDS flag: lane l writes its
// bytes at M0 + size * l).  Issued as inline assembly so that the compiler
// does not track them: it would otherwise wait for every copy in flight
// before any LDS read.  The kernel orders them itself (explicit vmcnt wait
// and barrier before a stage's buffer is read).  No register is written.
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4u rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return v4u{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p);
}
// off: per-lane byte offset; soff: wave-uniform byte offset added to it.
__device__ __forceinline__ void dma16(const v4u& rs, uint8_t* lds, uint32_t off, uint32_t soff) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr(lds));   // lds is wave-uniform
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m), "v"(off), "s"(rs), "s"(soff)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const v4u& rs, uint8_t* lds, uint32_t off, uint32_t soff) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr(lds));   // lds is wave-uniform
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(m), "v"(off), "s"(rs), "s"(soff)
               : "memory", "m0");
}

// The same copies with the destination given as a 32-bit LDS byte address
// (wave-uniform): a kernel that forms its LDS addresses from one base
// avoids a generic-to-LDS pointer cast, with its null check, per copy.
__device__ __forceinline__ void dma16_at(const v4u& rs, uint32_t lds, uint32_t off, uint32_t soff) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m), "v"(off), "s"(rs), "s"(soff)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_at(const v4u& rs, uint32_t lds, uint32_t off, uint32_t soff) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(m), "v"(off), "s"(rs), "s"(soff)
               : "memory", "m0");
}

// s_waitcnt with vmcnt <= n and no wait on the other counters.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace w4a4
