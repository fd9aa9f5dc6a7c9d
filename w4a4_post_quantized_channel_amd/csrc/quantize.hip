// Runtime quantizer for gfx950: smoothing, block-64 Walsh-Hadamard rotation
// and per-row quantization, fused in one pass over the input.
//
// FoldQuantVLA (contribution 2): channel scaling, FWHT with block 64 and
// dynamic per-token quantization.  QuantWAMs sec. 3.1 Eq. 1: the quantizer
// sees A R S^-1.  The same kernel packs weights (one row per output
// channel, multiplying by s instead of 1/s: FoldQuantVLA contribution 1).
//
// Work mapping.  A row of K elements is cut into 16-byte slots of 8
// consecutive elements; slot s of a row lives in lane (s mod 64) of the
// row's wave group, chunk s / (64 * WPR).  A 64-element Hadamard block is
// therefore 8 consecutive lanes: butterfly stages 1, 2, 4 run inside a
// lane's registers and stages 8, 16, 32 across lanes (xor 1, 2, 4).  The
// whole row stays in registers, so the per-row absolute maximum needs no
// second read of HBM.  WPR (waves per row) is 1 for many rows, 4 for few.
#include "device_common.h"
#include "launch.h"

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
};

enum { MODE_INT4 = 0, MODE_INT8 = 1, MODE_NVFP4 = 2, MODE_AMAX = 3 };

template <bool BF16IN>
__device__ __forceinline__ void load_slot(const void* rowp, int s, float (&v)[8]) {
  if constexpr (BF16IN) {
    uint4 d = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(rowp) + s * 8);
    uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(rowp) + s * 8);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Stages h = 1, 2, 4 inside the 8 registers of one slot.
__device__ __forceinline__ void fwht8_local(float (&v)[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if ((j & h) == 0) {
        float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
}

// Stages h = 8, 16, 32: partner slot is lane ^ m (m = 1, 2, 4).  The lane
// holding index j keeps a + b, the lane holding j + h keeps a - b.
__device__ __forceinline__ void fwht8_cross(float (&v)[8], int lane) {
#pragma unroll
  for (int m = 1; m < 8; m <<= 1) {
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float p = __shfl_xor(v[j], m);
      v[j] = upper ? (p - v[j]) : (v[j] + p);
    }
  }
}

template <int MODE, bool BF16IN, int NC, int WPR>
__global__ void __launch_bounds__(256) quant_rows_kernel(QuantArgs a) {
  constexpr int QMAX = MODE == MODE_INT4 ? 7 : 127;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rows_per_block = 4 / WPR;
  const int sub = WPR == 1 ? 0 : wave;            // wave index inside the row group
  const int grp = WPR == 1 ? wave : 0;            // row group inside the block
  const int nslots = a.K >> 3;
  const bool has_scale = a.scale != nullptr;
  const size_t esz = BF16IN ? 2 : 4;
  __shared__ float red[4];

  float sc[NC][8];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int s = (c * WPR + sub) * 64 + lane;
#pragma unroll
    for (int i = 0; i < 8; ++i) sc[c][i] = 1.0f;
    if (has_scale && s < nslots) {
      const float4* p = reinterpret_cast<const float4*>(a.scale + s * 8);
      float4 u = p[0], w = p[1];
      sc[c][0] = u.x; sc[c][1] = u.y; sc[c][2] = u.z; sc[c][3] = u.w;
      sc[c][4] = w.x; sc[c][5] = w.y; sc[c][6] = w.z; sc[c][7] = w.w;
    }
  }

  float tmax = 0.f;  // MODE_AMAX: running max over this wave's rows
  for (int64_t row = (int64_t)blockIdx.x * rows_per_block + grp; row < a.R;
       row += (int64_t)gridDim.x * rows_per_block) {
    const char* rowp = reinterpret_cast<const char*>(a.x) + (size_t)row * a.ldx * esz;
    float v[NC][8];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int s = (c * WPR + sub) * 64 + lane;
      if (s < nslots) {
        load_slot<BF16IN>(rowp, s, v[c]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[c][i] = 0.f;
      }
    }
    // --- transform -------------------------------------------------------
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (a.order == 0 && has_scale) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[c][i] = v[c][i] * sc[c][i];
      }
      if (a.rot) {
        fwht8_local(v[c]);
        fwht8_cross(v[c], lane);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[c][i] = v[c][i] * 0.125f;
      }
      if (a.order == 1 && has_scale) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[c][i] = v[c][i] * sc[c][i];
      }
    }

    if constexpr (MODE == MODE_INT4 || MODE == MODE_INT8 || MODE == MODE_AMAX) {
      float m = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, __builtin_fabsf(v[c][i]));
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      if constexpr (MODE == MODE_AMAX) {
        tmax = fmaxf(tmax, m);
        continue;
      } else {
        if constexpr (WPR > 1) {
          if (lane == 0) red[wave] = m;
          __syncthreads();
          m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
          __syncthreads();
        }
        const float step = m / (float)QMAX;
        if (lane == 0 && sub == 0) reinterpret_cast<float*>(a.scales)[row] = step;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int s = (c * WPR + sub) * 64 + lane;
          if (s >= nslots) continue;
          int q[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            float r = step > 0.f ? __builtin_rintf(v[c][i] / step) : 0.f;
            r = fminf(fmaxf(r, (float)(-QMAX - 1)), (float)QMAX);
            q[i] = (int)r;
          }
          if constexpr (MODE == MODE_INT4) {
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) word |= ((uint32_t)q[i] & 0xFu) << (4 * i);
            *reinterpret_cast<uint32_t*>(a.codes + (size_t)row * (a.K >> 1) + s * 4) = word;
          } else {
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              lo |= ((uint32_t)q[i] & 0xFFu) << (8 * i);
              hi |= ((uint32_t)q[i + 4] & 0xFFu) << (8 * i);
            }
            *reinterpret_cast<uint2*>(a.codes + (size_t)row * a.K + s * 8) = make_uint2(lo, hi);
          }
        }
      }
    } else {  // NVFP4: one E4M3 scale per 16 elements = two neighbouring slots
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int s = (c * WPR + sub) * 64 + lane;
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, __builtin_fabsf(v[c][i]));
        m = fmaxf(m, __shfl_xor(m, 1));
        if (s >= nslots) continue;
        const float sb = m / 6.0f;
        const uint32_t e = f32_to_e4m3_sat(sb / a.g);
        const float S = e4m3_to_f32(e) * a.g;
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint32_t cd = S > 0.f ? f32_to_e2m1_sat(v[c][i] / S) : 0u;
          word |= cd << (4 * i);
        }
        *reinterpret_cast<uint32_t*>(a.codes + (size_t)row * (a.K >> 1) + s * 4) = word;
        if ((s & 1) == 0)
          reinterpret_cast<uint8_t*>(a.scales)[(size_t)row * (a.K >> 4) + (s >> 1)] = (uint8_t)e;
      }
    }
  }
  if constexpr (MODE == MODE_AMAX) {
    if (lane == 0) atomicMax(reinterpret_cast<unsigned int*>(a.amax_out), __float_as_uint(tmax));
  }
}

__global__ void zero_u32_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

template <int MODE, bool BF16IN, int WPR>
static hipError_t launch_nc(int nc, dim3 grid, hipStream_t st, const QuantArgs& a) {
#define W4A4_NC_CASE(N)                                                              \
  case N:                                                                           \
    hipLaunchKernelGGL((quant_rows_kernel<MODE, BF16IN, N, WPR>), grid, dim3(256), 0, st, a); \
    break;
  switch (nc) {
    W4A4_NC_CASE(1)
    W4A4_NC_CASE(2)
    W4A4_NC_CASE(3)
    W4A4_NC_CASE(4)
    W4A4_NC_CASE(6)
    W4A4_NC_CASE(8)
    W4A4_NC_CASE(10)
    W4A4_NC_CASE(12)
    W4A4_NC_CASE(16)
    default:
      return hipErrorInvalidValue;
  }
#undef W4A4_NC_CASE
  return hipGetLastError();
}

static int round_nc(int nc) {
  const int allowed[] = {1, 2, 3, 4, 6, 8, 10, 12, 16};
  for (int v : allowed)
    if (nc <= v) return v;
  return -1;
}

// Largest K a single launch supports: 16 chunks x 64 lanes x 8 elements x 4 waves.
int64_t quant_max_k() { return 16LL * 64 * 8 * 4; }

hipError_t launch_quantize(int mode, bool bf16in, const void* x, int64_t R, int64_t K, int64_t ldx,
                           const float* scale, float g, int rot, int order, void* codes,
                           void* scales, float* amax_out, hipStream_t st) {
  QuantArgs a{x, R, (int)K, ldx, scale, g, rot, order, (uint8_t*)codes, scales, amax_out};
  const int64_t nslots = K / 8;
  // One wave per row when that already gives enough waves and fits in registers.
  int wpr = (R >= 2048 && nslots <= 16 * 64) ? 1 : 4;
  int nc = round_nc((int)((nslots + 64 * wpr - 1) / (64 * wpr)));
  if (nc < 0) return hipErrorInvalidValue;
  const int rows_per_block = 4 / wpr;
  int64_t blocks = (R + rows_per_block - 1) / rows_per_block;
  const int64_t cap = 256 * 8;  // persistent-style cap: 8 blocks per CU
  if (mode == MODE_AMAX) {
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, st, (uint32_t*)amax_out, (size_t)1);
  }
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  dim3 grid((unsigned)blocks);
#define W4A4_DISPATCH(MODE)                                                          \
  if (mode == MODE) {                                                                \
    if (bf16in) return wpr == 1 ? launch_nc<MODE, true, 1>(nc, grid, st, a)          \
                                : launch_nc<MODE, true, 4>(nc, grid, st, a);         \
    return wpr == 1 ? launch_nc<MODE, false, 1>(nc, grid, st, a)                     \
                    : launch_nc<MODE, false, 4>(nc, grid, st, a);                    \
  }
  W4A4_DISPATCH(MODE_INT4)
  W4A4_DISPATCH(MODE_INT8)
  W4A4_DISPATCH(MODE_NVFP4)
  W4A4_DISPATCH(MODE_AMAX)
#undef W4A4_DISPATCH
  return hipErrorInvalidValue;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st) {
  size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (uint32_t*)p, n);
  return hipGetLastError();
}

}  // namespace w4a4
