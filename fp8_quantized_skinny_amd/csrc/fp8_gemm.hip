// FP8 (E4M3FN) weight-only skinny GEMM for gfx950 (MI355X).
//
// y[m][n] = sum_kb S[n/128][kb] * sum_{k in block kb} x[m][k] * e4m3(c[n][k])
//
// The published FP8 regions of a checkpoint are served as FP8 instead of
// being converted to NVFP4 ("NVFP4 on Volta!" author's post, section
// "v1.0 -> v1.1"); the codes are read in their canonical [N][K] order.
//
// A 16-column tile times one 128-K chunk lies inside one 128 x 128 scale
// block, so each chunk is contracted on the matrix cores into a fresh fp32
// partial (E4M3 -> fp16 is exact) and then added to the accumulator times the
// block scale in fp32.  Work split and cross-wavefront reduction follow the
// NVFP4 kernels: CT tiles per workgroup, NW wavefronts splitting K.
//
// Lane (grp, col) of a wavefront loads, per chunk, two 16-byte pieces of
// column col: K = 128kc + 64h + 16grp .. +16 for h = 0, 1, so each load
// instruction covers 64 contiguous bytes of 16 columns.
#include <hip/hip_runtime.h>

#include "common.cuh"
#include "internal.h"

namespace skinny {
namespace {

struct Fp8Args {
  const uint8_t* w;
  const float* scales;
  const _Float16* x;
  _Float16* y;
  int M, K, N;
  int kc, nt, kb;  // K chunks, column tiles, scale blocks along K
};

template <int CT, int NW>
__global__ __launch_bounds__(NW * 64) void fp8_mfma(Fp8Args a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, col = lane & 15;
  const int tile0 = blockIdx.x * CT;
  const int c0 = (a.kc * wave) / NW, c1 = (a.kc * (wave + 1)) / NW;

  f32x4 acc[CT];
#pragma unroll
  for (int t = 0; t < CT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Column of this lane in each tile; columns past N read column N-1 (their
  // results are never stored), so every load stays inside the weights.
  const uint8_t* wp[CT];
  const float* sp[CT];
#pragma unroll
  for (int t = 0; t < CT; ++t) {
    const int n = min((tile0 + t) * kTileCols + col, a.N - 1);
    wp[t] = a.w + static_cast<size_t>(n) * a.K + grp * 16;
    sp[t] = a.scales + static_cast<size_t>(min((tile0 + t) * kTileCols, a.N - 1) / 128) * a.kb;
  }
  const bool xrow = col < a.M;
  const _Float16* xr = a.x + static_cast<size_t>(xrow ? col : 0) * a.K + grp * 16;
  const int kfull = a.K / kChunkK;

  for (int kc = c0; kc < c1; ++kc) {
    const bool full = kc < kfull;
    const int k0 = kc * kChunkK;
    f16x8 xa[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // piece j: h = j >> 1, half s = j & 1 -> K = k0 + 64h + 16grp + 8s
      const int ko = 64 * (j >> 1) + 8 * (j & 1);
      xa[j] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (xrow && (full || k0 + ko + grp * 16 + 8 <= a.K))
        xa[j] = *reinterpret_cast<const f16x8*>(xr + k0 + ko);
    }
    u32x4 w[CT][2];
    float s[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        w[t][h] = u32x4{0u, 0u, 0u, 0u};
        if (full || k0 + 64 * h + grp * 16 + 16 <= a.K) w[t][h] = load16(wp[t] + k0 + 64 * h);
      }
      s[t] = sp[t][kc];
    }
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      f32x4 p = f32x4{0.f, 0.f, 0.f, 0.f};
      p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[0], e4m3x8(w[t][0].x, w[t][0].y), p, 0, 0, 0);
      p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[1], e4m3x8(w[t][0].z, w[t][0].w), p, 0, 0, 0);
      p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[2], e4m3x8(w[t][1].x, w[t][1].y), p, 0, 0, 0);
      p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[3], e4m3x8(w[t][1].z, w[t][1].w), p, 0, 0, 0);
      acc[t] += s[t] * p;
    }
  }

  __shared__ f32x4 red[NW][CT][32];
  if (lane < 32) {
#pragma unroll
    for (int t = 0; t < CT; ++t) red[wave][t][lane] = acc[t];
  }
  __syncthreads();
  if (wave == 0 && lane < 32) {
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      f32x4 v = red[0][t][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) v += red[w][t][lane];
      const int n = (tile0 + t) * kTileCols + col;
      if (tile0 + t < a.nt && n < a.N) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = grp * 4 + r;
          if (m < a.M) a.y[static_cast<size_t>(m) * a.N + n] = static_cast<_Float16>(v[r]);
        }
      }
    }
  }
}

}  // namespace

bool fp8_cfg_supported(const LaunchCfg& c, int M) {
  (void)M;
  return c.engine == 1 && (c.ct == 1 || c.ct == 2 || c.ct == 4) && (c.nw == 4 || c.nw == 8);
}

#define SKINNY_FP8_DISPATCH(CT, NW)                                                   \
  if (cfg.ct == CT && cfg.nw == NW) {                                                 \
    hipLaunchKernelGGL((fp8_mfma<CT, NW>), dim3(grid), dim3(NW * 64), 0, stream, a);  \
    return hipGetLastError();                                                         \
  }

hipError_t launch_fp8(const uint8_t* w, const float* scales, const uint16_t* x, uint16_t* y, int M,
                      int K, int N, const LaunchCfg& cfg, hipStream_t stream) {
  Fp8Args a;
  a.w = w;
  a.scales = scales;
  a.x = reinterpret_cast<const _Float16*>(x);
  a.y = reinterpret_cast<_Float16*>(y);
  a.M = M;
  a.K = K;
  a.N = N;
  a.kc = (K + kChunkK - 1) / kChunkK;
  a.nt = (N + kTileCols - 1) / kTileCols;
  a.kb = (K + 127) / 128;
  const int grid = (a.nt + cfg.ct - 1) / cfg.ct;
  SKINNY_FP8_DISPATCH(1, 4)
  SKINNY_FP8_DISPATCH(1, 8)
  SKINNY_FP8_DISPATCH(2, 4)
  SKINNY_FP8_DISPATCH(2, 8)
  SKINNY_FP8_DISPATCH(4, 4)
  SKINNY_FP8_DISPATCH(4, 8)
  return hipErrorInvalidValue;
}

}  // namespace skinny
