// Shared epilogue pieces of the GEMM kernels: the 16-bit branch as extra
// bf16 MFMA steps on the fp32 accumulators, and the output store.
#pragma once
#include "device_common.h"
#include "launch.h"

namespace w4a4 {

// 16 consecutive bytes (8 bf16) of row `row`, starting at element k, or
// zeros when the row or the chunk is out of range.
__device__ __forceinline__ v8bf load_bf16x8(const uint16_t* base, int64_t ld, int row, int nrows,
                                            int k, int klen) {
  uint4 d = make_uint4(0, 0, 0, 0);
  if (row < nrows && k < klen) d = *reinterpret_cast<const uint4*>(base + (int64_t)row * ld + k);
  return __builtin_bit_cast(v8bf, d);
}

// acc[i][j] (16x16 fp32 MFMA tiles, lane holds rows 4*(lane/16)+0..3 of
// column lane%16) += A_br[rows, :ra] . B_br[cols, (k mod r)]^T.
// m_base / n_base: first row / column of this wave's tile.
template <int TI, int TJ>
__device__ __forceinline__ void branch_mfma(v4f (&acc)[TI][TJ], const BranchArgs& br, int M, int N,
                                            int m_base, int n_base, int lane) {
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  for (int kk = 0; kk < br.ra; kk += 32) {
    const int ka = kk + lk;
    const int kb = ka % br.r;
    v8bf af[TI], bfr[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) af[i] = load_bf16x8(br.a, br.lda, m_base + i * 16 + lr, M, ka, br.ra);
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      bfr[j] = load_bf16x8(br.b, br.ldb, n_base + j * 16 + lr, N, kb, ka < br.ra ? br.r : 0);
    }
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  }
}

// Epilogue operands a kernel has already staged in LDS for its whole tile:
// the scales of the tile's rows and columns and, for a branch with r and ra
// at most kBrLdsMax, the tile's rows of A_br and B_br.  A branch row holds
// 128 bytes whose 16-byte chunk c sits at position c XOR (row mod 8); chunks
// past ra (A) or r (B) hold zeros.
constexpr int kBrLdsMax = 64;
struct EpiLds {
  const float* sa;       // sa[m - m_tile]
  const float* sw;       // sw[n - n_tile]
  const uint8_t* bra;    // A_br rows of the tile, or null (branch read from global memory)
  const uint8_t* brb;    // B_br rows of the tile
  int m_tile, n_tile;
};

// The A_br operands of a wave's TI row blocks for every K step of an
// LDS-staged branch (ra <= kBrLdsMax = 64: two steps of 32), read once per
// tile; branch_mfma_lds_pre then adds one 16-column block's products.
template <int TI>
struct BrAFrags {
  v8bf a[kBrLdsMax / 32][TI];
};
template <int TI>
__device__ __forceinline__ void load_br_a(BrAFrags<TI>& f, const EpiLds& el, int ra, int m_loc, int lane) {
  const int lr = lane & 15, lk = (lane >> 4) * 8;
#pragma unroll
  for (int s = 0; s < kBrLdsMax / 32; ++s) {
    if (s * 32 >= ra) break;
    const int ka = s * 32 + lk;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int row = m_loc + i * 16 + lr;
      f.a[s][i] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(el.bra + row * 128 + (((ka >> 3) ^ (row & 7)) << 4)));
    }
  }
}
template <int TI>
__device__ __forceinline__ void branch_mfma_lds_pre(v4f (&acc)[TI][1], const BrAFrags<TI>& f, const EpiLds& el, int ra,
                                                    int r, int n_loc, int lane) {
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const int row = n_loc + lr;
#pragma unroll
  for (int s = 0; s < kBrLdsMax / 32; ++s) {
    if (s * 32 >= ra) break;
    const int kb = (s * 32 + lk) % r;
    const v8bf b = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(el.brb + row * 128 + (((kb >> 3) ^ (row & 7)) << 4)));
#pragma unroll
    for (int i = 0; i < TI; ++i) acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[s][i], b, acc[i][0], 0, 0, 0);
  }
}

// Dequantisation scales of a wave's TI x TJ tile grid as the lane uses them:
// sa for its rows 4*(lane/16)+0..3 of each row block, sw for its column
// lane%16 of each 16-column block (0 past M / N).  A kernel that loads
// them before its main loop hides their latency behind it.
template <int TI, int TJ>
struct EpiScales {
  float sa[TI][4];
  float sw[TJ];
};

template <int TI, int TJ>
__device__ __forceinline__ void load_epi_scales(EpiScales<TI, TJ>& s, const GemmArgs& g, int m_base, int n_base,
                                                int lane) {
  const int lr = lane & 15, lq = lane >> 4;
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(g.sa, g.sa ? (uint32_t)g.M * 4u : 0u);
  const __amdgpu_buffer_rsrc_t rsw = make_rsrc(g.sw, g.sw ? (uint32_t)g.N * 4u : 0u);
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m_base + i * 16 + lq * 4 + r;
      s.sa[i][r] = __uint_as_float(buf_load4(rsa, m < g.M ? (uint32_t)m * 4u : kOOB));
    }
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int n = n_base + j * 16 + lr;
    s.sw[j] = __uint_as_float(buf_load4(rsw, n < g.N ? (uint32_t)n * 4u : kOOB));
  }
}

// Epilogue of a wave's TI x TJ grid of 16x16 accumulator tiles, one
// 16-column block at a time (keeps the live register set small):
// dequantise (integer: fp32(fp32(acc) * sa[m]) * sw[n] * alpha, with acc
// shifted right by 8 when both operands are x16-widened int4 and by 4 when
// one is (int8 x int4); float: acc *
// alpha), add the bf16 branch, store.  acc[i][j] covers rows
// m_base + 16 i + [0, 16) and columns n_base + 16 j + [0, 16).
// y_dtype 2 writes the raw integer accumulators.  Stores go through a
// buffer resource over the tile's rows (rows past M fall outside it) with
// 32-bit offsets; columns past N are sent past the resource.
// LDS bytes a wave needs to stage a TI x TJ tile of bf16 output.
template <int TI, int TJ>
constexpr int epilogue_stage_bytes() {
  return TI * 16 * (TJ * 32 + 16);
}

// Accumulator kinds: 0 both int4 (x256), 1 int8, 2 float already scaled
// (NVFP4: times alpha only), 3 int8 x int4 (x16), 4 float with per-row and
// per-column steps (FP8).
template <int KIND, typename T>
__device__ __forceinline__ float epi_acc(T a) {
  if constexpr (KIND == 0) return (float)(a >> 8);
  else if constexpr (KIND == 3) return (float)(a >> 4);
  else return (float)a;
}

// `pre`, when given, holds the scales already loaded (load_epi_scales);
// `el`, when given, the LDS-staged scales and branch rows of the tile.
// GROUPS: the most tiles per group of the grouped branch pass below (0: no
// grouped pass, where its registers cost the kernel's main loop more than
// it saves).
template <int KIND /*0 int4, 1 int8, 2 float, 3 int8 x int4, 4 fp8*/, int GROUPS = 8, typename AccT, int TI,
          int TJ>
__device__ __forceinline__ void epilogue_tiles(AccT (&acc)[TI][TJ], const GemmArgs& g, int m_base, int n_base,
                                               int lane, uint8_t* stage = nullptr,
                                               const EpiScales<TI, TJ>* pre = nullptr, const EpiLds* el = nullptr) {
  const int lr = lane & 15, lq = lane >> 4;
  const int esz = g.y_dtype == 1 ? 2 : 4;
  const int rows = max(0, min(TI * 16, g.M - m_base));
  const uint32_t rstride = (uint32_t)(g.ldy * esz);
  const __amdgpu_buffer_rsrc_t ry =
      make_rsrc(reinterpret_cast<char*>(g.y) + (int64_t)m_base * g.ldy * esz, (uint32_t)rows * rstride);
  uint32_t roff[TI][4];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) roff[i][r] = (uint32_t)(i * 16 + lq * 4 + r) * rstride;

  if constexpr (KIND != 2 && KIND != 4) {
    if (g.y_dtype == 2) {
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int n = n_base + j * 16 + lr;
        const uint32_t coff = n < g.N ? (uint32_t)n * 4u : kOOB;
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int v = KIND == 0 ? (acc[i][j][r] >> 8) : KIND == 3 ? (acc[i][j][r] >> 4) : acc[i][j][r];
            __builtin_amdgcn_raw_buffer_store_b32(v, ry, (int)(roff[i][r] + coff), 0, 0);
          }
      }
      return;
    }
  }
  const float* sa = reinterpret_cast<const float*>(g.sa);
  const float* sw = reinterpret_cast<const float*>(g.sw);
  float sam[TI][4];
  if constexpr (KIND != 2) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m_base + i * 16 + lq * 4 + r;
        sam[i][r] = pre ? pre->sa[i][r] : el ? el->sa[m - el->m_tile] : (m < g.M ? sa[m] : 0.f);
      }
  }
  // LDS-staged branch: its A_br operands once for the whole grid
  const bool br_pre = g.br.r > 0 && el && el->bra;
  BrAFrags<TI> bra_f;
  if (br_pre) load_br_a<TI>(bra_f, *el, g.br.ra, m_base - el->m_tile, lane);
  // The column blocks go in groups of at most eight tiles: a group's tiles
  // are dequantised first and then take the branch products of all of
  // them in one pass, so the products of different tiles overlap instead
  // of waiting on each other; each tile takes the same products in the
  // same order as in the loop below.
  if constexpr (GROUPS) {
    constexpr int GJ = (GROUPS / TI) < 1 ? 1 : (GROUPS / TI);   // column blocks per group
    if (br_pre && stage != nullptr && g.y_dtype == 1) {
      const int lk = lq * 8;
#pragma unroll
      for (int j0 = 0; j0 < TJ; j0 += GJ) {
        v4f yv[TI][GJ];
#pragma unroll
        for (int jj = 0; jj < GJ; ++jj) {
          const int j = j0 + jj;
          if (j >= TJ) break;
          if constexpr (KIND != 2) {
            const int n = n_base + j * 16 + lr;
            const float swn = pre ? pre->sw[j] : el->sw[n - el->n_tile];
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                float v = epi_acc<KIND>(acc[i][j][r]) * sam[i][r];
                v = v * swn;
                yv[i][jj][r] = v * g.alpha;
              }
          } else {
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
              for (int r = 0; r < 4; ++r) yv[i][jj][r] = acc[i][j][r] * g.alpha;
          }
        }
#pragma unroll
        for (int s = 0; s < kBrLdsMax / 32; ++s) {
          if (s * 32 >= g.br.ra) break;
          const int kb = (s * 32 + lk) % g.br.r;
#pragma unroll
          for (int jj = 0; jj < GJ; ++jj) {
            const int j = j0 + jj;
            if (j >= TJ) break;
            const int row = n_base + j * 16 - el->n_tile + lr;
            const v8bf b = __builtin_bit_cast(
                v8bf, *reinterpret_cast<const uint4*>(el->brb + row * 128 + (((kb >> 3) ^ (row & 7)) << 4)));
#pragma unroll
            for (int i = 0; i < TI; ++i)
              yv[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bra_f.a[s][i], b, yv[i][jj], 0, 0, 0);
          }
        }
#pragma unroll
        for (int jj = 0; jj < GJ; ++jj) {
          const int j = j0 + jj;
          if (j >= TJ) break;
#pragma unroll
          for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              *reinterpret_cast<uint16_t*>(stage + (i * 16 + lq * 4 + r) * (TJ * 32 + 16) + (j * 16 + lr) * 2) =
                  (uint16_t)f32_to_bf16_bits(yv[i][jj][r]);
        }
      }
      goto staged_out;
    }
  }
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int n = n_base + j * 16 + lr;
    const uint32_t coff = n < g.N ? (uint32_t)n * (uint32_t)esz : kOOB;
    v4f col[TI][1];
    if constexpr (KIND != 2) {
      const float swn = pre ? pre->sw[j] : el ? el->sw[n - el->n_tile] : (n < g.N ? sw[n] : 0.f);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = epi_acc<KIND>(acc[i][j][r]) * sam[i][r];
          v = v * swn;
          col[i][0][r] = v * g.alpha;
        }
    } else {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) col[i][0][r] = acc[i][j][r] * g.alpha;
    }
    if (g.br.r > 0) {
      if (br_pre)
        branch_mfma_lds_pre<TI>(col, bra_f, *el, g.br.ra, g.br.r, n_base + j * 16 - el->n_tile, lane);
      else
        branch_mfma<TI, 1>(col, g.br, g.M, g.N, m_base, n_base + j * 16, lane);
    }
    if (stage != nullptr && g.y_dtype == 1) {
      // bf16 into the wave's LDS tile (row pitch TJ * 32 + 16 bytes)
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<uint16_t*>(stage + (i * 16 + lq * 4 + r) * (TJ * 32 + 16) + (j * 16 + lr) * 2) =
              (uint16_t)f32_to_bf16_bits(col[i][0][r]);
      continue;
    }
    if (g.y_dtype == 0) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(col[i][0][r]), ry, (int)(roff[i][r] + coff), 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_bits(col[i][0][r]), ry,
                                                (int)(roff[i][r] + coff), 0, 0);
    }
  }
staged_out:
  if (stage != nullptr && g.y_dtype == 1) {
    // Rows back out of LDS, 16 bytes (8 columns) per lane: every row of the
    // tile leaves as whole contiguous segments.
    constexpr int CPR = TJ * 2;                  // 16-byte chunks per row
    constexpr int NCH = TI * 16 * CPR;           // chunks in the tile
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int c0 = 0; c0 < NCH; c0 += 64) {
      const int c = c0 + lane;
      if (NCH % 64 != 0 && c >= NCH) break;
      const int row = c / CPR, ch = c % CPR;
      const uint4 v = *reinterpret_cast<const uint4*>(stage + row * (TJ * 32 + 16) + ch * 16);
      const int n = n_base + ch * 8;
      const uint32_t off = (uint32_t)row * rstride + (uint32_t)n * 2u;
      if (n + 8 <= g.N) {
        // non-temporal (cache policy 2, `nt`): the tile is written once and
        // never read back here, so it need not stay in L2
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, v), ry, (int)off, 0, 2);
      } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (n + e < g.N)
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(w[e >> 1] >> (16 * (e & 1))), ry, (int)(off + 2 * e),
                                                  0, 0);
      }
    }
  }
}

}  // namespace w4a4
