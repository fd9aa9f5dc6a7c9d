// The projection t = x L1 of the low-rank branch (Q-WAM abstract: a
// 16-bit low-rank branch beside the 4-bit complement), one 16 x 16 tile of
// t per workgroup of eight waves: the body of project_kernel, and of the
// projection workgroups that quantize_act_project launches beside its
// quantizer workgroups.
#pragma once
#include "device_common.h"
#include "lds_dma.h"

namespace w4a4 {

// t = x L1 for one 16-row x 16-column tile per workgroup of eight waves;
// wave w takes the w-th eighth of K.  A wave copies its operand rows into
// its own LDS area by buffer-to-LDS loads of whole 128-byte row segments
// (8 rows per instruction, 64 K per step), kProjChunk steps at a time, then
// reads the MFMA layout back with ds_read_b128: loading that layout straight
// from global memory touches 16 half-used cache lines per instruction and
// streams about a third as fast.  Chunk c of a row segment sits at position
// c ^ (row & 7).  Copies past K or past the last row or column read as
// zeros.  The eight partial tiles are added in LDS in wave order and
// written as bf16 hi = bf16(t), lo = bf16(t - hi) into columns c and r + c
// of out.  One kernel: no partial products leave the workgroup.
constexpr int kProjRows = 16;                 // rows of x (and of t) per workgroup
constexpr int kProjWaves = 8;
constexpr int kProjChunk = 3;                 // 64-deep steps copied per round
constexpr int kProjStepBytes = 2 * 16 * 128;  // x rows then L1 rows of one step
constexpr int kProjLdsBytes = kProjWaves * kProjChunk * kProjStepBytes;

// Tile (m0, c0) of t; every thread of an eight-wave workgroup calls it.
// area: kProjLdsBytes of LDS, 16-byte aligned.
__device__ __forceinline__ void project_block(const uint16_t* x, int64_t ldx, int M, int K, const uint16_t* l1t,
                                              int r, uint16_t* out, int64_t ldo, int m0, int c0, uint8_t* area) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;
  const int64_t xrow = ldx * 2, lrow = (int64_t)K * 2;   // row bytes
  const v4u rx = rsrc_words(x + (int64_t)m0 * ldx, (uint32_t)(min(kProjRows, M - m0) * xrow));
  const v4u rl = rsrc_words(l1t + (int64_t)c0 * K, (uint32_t)(min(16, r - c0) * lrow));
  const int kw = ((K + 64 * kProjWaves - 1) / (64 * kProjWaves)) * 64;   // K per wave, multiple of 64
  const int k0 = wave * kw, k1 = min(K, k0 + kw);
  uint8_t* const a = area + wave * (kProjChunk * kProjStepBytes);
  // copy instruction d of a step: rows 8 (d & 1) .. + 7 of x (d < 2) or of
  // L1 (d >= 2); lane -> row 8 (d & 1) + lane / 8, chunk position lane % 8
  // (the lane's row and chunk offset are fixed; a step's K byte goes in the
  // scalar operand, and destinations are 32-bit LDS addresses)
  const int crow = lane >> 3, cpos = lane & 7;
  uint32_t loff[4], lcol[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int row = 8 * (d & 1) + crow;
    const int c = cpos ^ (row & 7);                      // logical chunk held at this position
    lcol[d] = 8u * (uint32_t)c;
    loff[d] = (uint32_t)(row * (d < 2 ? xrow : lrow)) + 16u * (uint32_t)c;
  }
  const uint32_t a_lds = lds_addr(a);
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  for (int kc = k0; kc < k1; kc += 64 * kProjChunk) {
#pragma unroll
    for (int u = 0; u < kProjChunk; ++u) {
      const int k = kc + 64 * u;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const bool ok = (uint32_t)k + lcol[d] < (uint32_t)k1;   // chunk of 8 elements inside this wave's range
        dma16_at(d < 2 ? rx : rl, a_lds + (uint32_t)(u * kProjStepBytes + d * 1024), ok ? loff[d] : kOOB,
                 (uint32_t)k * 2u);
      }
    }
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < kProjChunk; ++u) {
      const uint8_t* st = a + u * kProjStepBytes;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int pos = ((4 * h + lq) ^ (lr & 7)) * 16;
        const uint4 xa = *reinterpret_cast<const uint4*>(st + lr * 128 + pos);
        const uint4 lb = *reinterpret_cast<const uint4*>(st + 2048 + lr * 128 + pos);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, xa), __builtin_bit_cast(v8bf, lb),
                                                      acc, 0, 0, 0);
      }
    }
    // the next round's copies overwrite this area only after these reads returned
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  __syncthreads();   // every wave is done with its copy area; reuse it for the partial tiles
  float (*sT)[16][16] = reinterpret_cast<float (*)[16][16]>(area);
#pragma unroll
  for (int q = 0; q < 4; ++q) sT[wave][lq * 4 + q][lr] = acc[q];
  __syncthreads();
  if (tid < 256) {
    const int row = tid >> 4, col = tid & 15, m = m0 + row, c = c0 + col;
    if (m < M && c < r) {
      float t = sT[0][row][col];
#pragma unroll
      for (int w = 1; w < kProjWaves; ++w) t = t + sT[w][row][col];
      const uint32_t hi = f32_to_bf16_bits(t);
      const float lo = t - bf16_bits_to_f32(hi);
      uint16_t* o = out + (int64_t)m * ldo;
      o[c] = (uint16_t)hi;
      o[r + c] = (uint16_t)f32_to_bf16_bits(lo);
    }
  }
}


}  // namespace w4a4
