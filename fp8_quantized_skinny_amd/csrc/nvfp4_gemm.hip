// NVFP4 weight-only skinny GEMM kernels for gfx950 (MI355X).
//
// y[m][n] = g * sum_k x[m][k] * e2m1(q[n][k]) * e4m3(s[n][k/16]),  1 <= M <= 8.
//
// The weights are read once, compressed, straight from HBM into VGPRs and
// widened to fp16 in registers just before use; there is no dequantized copy
// anywhere ("NVFP4 on Volta!" author's post, section "What I actually
// built").  Decode at batch 1..8 is bound by that weight stream, so every
// design choice below is about keeping 128-bit loads in flight and keeping
// the ALU work per weight small.
//
// Work split: a workgroup owns CT column tiles (16 columns each) and the
// whole K range; its NW wavefronts split the K chunks (128 K each) evenly and
// their partial sums are added in LDS in wavefront order, so results do not
// depend on timing.  Each lane handles one column and a run of 32 K per tile
// chunk (see internal.h for the packed layout).
//
// Two engines:
//   * VALU (M = 1): v_dot2c_f32_f16 with x shared across each 16-lane row by a
//     DPP row broadcast (lane 16r + i holds the x pair that every lane of row r
//     needs at step i), per-16-block sums scaled by the E4M3 scale in fp32, then
//     the four rows that split a column's K are added with permlane swaps.
//   * MFMA (M = 1..8): v_mfma_f32_16x16x32_f16 with the x rows zero-padded
//     to 16 as operand A and the widened weights (E2M1 * E4M3 in fp16, exact)
//     as operand B.  The 8-row verification tile of the pages (post, on why
//     the M = 8 row matters) fits in half of the 16-row MFMA tile.
// The MFMA engine also carries the lm_head epilogue: per-row argmax over fp32
// logits, ties to the lowest column, merged across workgroups with 64-bit
// atomicMax on (order-preserving key, inverted column) and finished by the
// last workgroup to arrive.
#include <hip/hip_runtime.h>

#include "common.cuh"
#include "internal.h"

namespace skinny {
namespace {

struct Nvfp4Args {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* gptr;
  const _Float16* x;
  _Float16* y;
  int M, K, N;
  int kc, nt, sg;
  int32_t* idx;
  unsigned long long* keys;
  uint32_t* counter;
};

// Chunk range [c0, c1) of wavefront w out of nw for kc chunks (balanced).
__device__ __forceinline__ void wave_range(int kc, int nw, int w, int& c0, int& c1) {
  c0 = (kc * w) / nw;
  c1 = (kc * (w + 1)) / nw;
}

// Scale word (two E4M3 bytes: half 0 in bits 0..7, half 1 in bits 8..15) of
// chunk kc from the 16-byte scale vector of its group.
__device__ __forceinline__ uint32_t scale_word(const u32x4& sv, int kc) {
  const int j = kc & 7;
  const uint32_t d = (j >> 1) == 0 ? sv.x : (j >> 1) == 1 ? sv.y : (j >> 1) == 2 ? sv.z : sv.w;
  return (j & 1) ? (d >> 16) : (d & 0xFFFFu);
}

// ---------------------------------------------------------------------------
// VALU engine, M = 1.
// ---------------------------------------------------------------------------
template <int I>
__device__ __forceinline__ float dot_step(uint32_t xv, uint32_t wd, float acc) {
  const f16x2 xx = __builtin_bit_cast(f16x2, row_bcast<I>(xv));
  return __builtin_amdgcn_fdot2(xx, e2m1x2<(I & 3)>(wd), acc, false);
}

// 16 codes (4 bytes x 2 dwords) of one 16-K block against the broadcast x.
template <int B0>
__device__ __forceinline__ float block_dot(uint32_t xv, uint32_t w0, uint32_t w1) {
  float p = 0.0f;
  p = dot_step<B0 + 0>(xv, w0, p);
  p = dot_step<B0 + 1>(xv, w0, p);
  p = dot_step<B0 + 2>(xv, w0, p);
  p = dot_step<B0 + 3>(xv, w0, p);
  p = dot_step<B0 + 4>(xv, w1, p);
  p = dot_step<B0 + 5>(xv, w1, p);
  p = dot_step<B0 + 6>(xv, w1, p);
  p = dot_step<B0 + 7>(xv, w1, p);
  return p;
}

template <int CT, int NW>
__global__ __launch_bounds__(NW * 64) void nvfp4_valu_m1(Nvfp4Args a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tile0 = blockIdx.x * CT;
  int c0, c1;
  wave_range(a.kc, NW, wave, c0, c1);

  float acc[CT];
#pragma unroll
  for (int t = 0; t < CT; ++t) acc[t] = 0.0f;

  // Tiles past the last one (grid rounding when CT > 1) re-read the last
  // tile; their results are never stored.
  const uint8_t* cptr[CT];
  const uint8_t* sptr[CT];
#pragma unroll
  for (int t = 0; t < CT; ++t) {
    const int tt = min(tile0 + t, a.nt - 1);
    cptr[t] = a.codes + static_cast<size_t>(tt) * a.kc * kTileBytes + lane * 16;
    sptr[t] = a.scales + static_cast<size_t>(tt) * a.sg * kTileBytes + lane * 16;
  }
  const int kfull = a.K / kChunkK;  // chunks whose 128 K are all valid

  u32x4 sv[CT];
  int sg_loaded = -1;
  for (int kc = c0; kc < c1; ++kc) {
    // x pair (k = 128kc + 2 lane, +1) for this chunk; zero past K.
    uint32_t xv = 0;
    if (kc < kfull || kc * kChunkK + 2 * lane < a.K)
      xv = *reinterpret_cast<const uint32_t*>(a.x + kc * kChunkK + 2 * lane);
    if ((kc >> 3) != sg_loaded) {
      sg_loaded = kc >> 3;
#pragma unroll
      for (int t = 0; t < CT; ++t) sv[t] = load16(sptr[t] + (kc >> 3) * kTileBytes);
    }
    u32x4 w[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) w[t] = load16(cptr[t] + kc * kTileBytes);
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      const uint32_t sw = scale_word(sv[t], kc);
      const float s0 = e4m3f<0>(sw), s1 = e4m3f<1>(sw);
      const float p0 = block_dot<0>(xv, w[t].x, w[t].y);
      const float p1 = block_dot<8>(xv, w[t].z, w[t].w);
      acc[t] = __builtin_fmaf(p0, s0, acc[t]);
      acc[t] = __builtin_fmaf(p1, s1, acc[t]);
    }
  }

  __shared__ float red[NW][CT][16];
#pragma unroll
  for (int t = 0; t < CT; ++t) {
    const float v = sum_over_rows(acc[t]);
    if (lane < 16) red[wave][t][lane] = v;
  }
  __syncthreads();
  if (wave == 0 && lane < 16) {
    const float g = *a.gptr;
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      float s = red[0][t][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) s += red[w][t][lane];
      const int n = (tile0 + t) * kTileCols + lane;
      if (tile0 + t < a.nt && n < a.N) a.y[n] = static_cast<_Float16>(g * s);
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA engine, M = 1..8 (and the lm_head argmax epilogue).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ordered_key(float v) {
  if (v == 0.0f) v = 0.0f;  // +0 and -0 compare equal
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int CT, int NW, bool ARGMAX>
__global__ __launch_bounds__(NW * 64) void nvfp4_mfma(Nvfp4Args a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, col = lane & 15;
  const int tile0 = blockIdx.x * CT;
  int c0, c1;
  wave_range(a.kc, NW, wave, c0, c1);

  f32x4 acc[CT];
#pragma unroll
  for (int t = 0; t < CT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Tiles past the last one (grid rounding when CT > 1) re-read the last
  // tile; their results are never stored.
  const uint8_t* cptr[CT];
  const uint8_t* sptr[CT];
#pragma unroll
  for (int t = 0; t < CT; ++t) {
    const int tt = min(tile0 + t, a.nt - 1);
    cptr[t] = a.codes + static_cast<size_t>(tt) * a.kc * kTileBytes + lane * 16;
    sptr[t] = a.scales + static_cast<size_t>(tt) * a.sg * kTileBytes + lane * 16;
  }
  // Operand A: lane (row = col, grp) reads x[row][128kc + 32grp + 8j .. +8].
  const bool xrow = col < a.M;
  const _Float16* xr = a.x + static_cast<size_t>(xrow ? col : 0) * a.K + grp * 32;
  const int kfull = a.K / kChunkK;

  u32x4 sv[CT];
  int sg_loaded = -1;
  for (int kc = c0; kc < c1; ++kc) {
    f16x8 xa[4];
    const int kb = kc * kChunkK + grp * 32;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xa[j] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (xrow && (kc < kfull || kb + 8 * j + 8 <= a.K))
        xa[j] = *reinterpret_cast<const f16x8*>(xr + kc * kChunkK + 8 * j);
    }
    if ((kc >> 3) != sg_loaded) {
      sg_loaded = kc >> 3;
#pragma unroll
      for (int t = 0; t < CT; ++t) sv[t] = load16(sptr[t] + (kc >> 3) * kTileBytes);
    }
    u32x4 w[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) w[t] = load16(cptr[t] + kc * kTileBytes);
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      const f16x2 s = e4m3x2<false>(scale_word(sv[t], kc));
      const f16x8 s0 = f16x8{s.x, s.x, s.x, s.x, s.x, s.x, s.x, s.x};
      const f16x8 s1 = f16x8{s.y, s.y, s.y, s.y, s.y, s.y, s.y, s.y};
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[0], e2m1x8(w[t].x) * s0, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[1], e2m1x8(w[t].y) * s0, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[2], e2m1x8(w[t].z) * s1, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[3], e2m1x8(w[t].w) * s1, acc[t], 0, 0, 0);
    }
  }

  // D layout: lane (grp, col) holds rows 4grp..4grp+3 of column col.  Rows
  // >= 8 are padding, so only lanes 0..31 carry results.
  __shared__ f32x4 red[NW][CT][32];
  if (lane < 32) {
#pragma unroll
    for (int t = 0; t < CT; ++t) red[wave][t][lane] = acc[t];
  }
  __syncthreads();

  if (wave == 0) {
    const float g = *a.gptr;
    float best_v[4];
    int best_n[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) { best_v[r] = -__builtin_inff(); best_n[r] = 0x7fffffff; }
    if (lane < 32) {
#pragma unroll
      for (int t = 0; t < CT; ++t) {
        f32x4 s = red[0][t][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) s += red[w][t][lane];
        const int n = (tile0 + t) * kTileCols + col;
        const bool nok = (tile0 + t) < a.nt && n < a.N;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = grp * 4 + r;
          const float v = g * s[r];
          if (nok && m < a.M) {
            if (a.y) a.y[static_cast<size_t>(m) * a.N + n] = static_cast<_Float16>(v);
            if (ARGMAX && (v > best_v[r] || best_n[r] == 0x7fffffff)) { best_v[r] = v; best_n[r] = n; }
          }
        }
      }
    }
    if (ARGMAX) {
      // Reduce (value, column) over the 16 lanes of each row group; ties keep
      // the lower column.  Columns grow with t for a fixed lane, so the strict
      // '>' above already kept the lowest column within a lane.
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) {
          const float ov = __shfl_xor(best_v[r], off, 16);
          const int on = __shfl_xor(best_n[r], off, 16);
          if (ov > best_v[r] || (ov == best_v[r] && on < best_n[r])) { best_v[r] = ov; best_n[r] = on; }
        }
      }
      if (lane < 32 && col == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = grp * 4 + r;
          if (m < a.M && best_n[r] != 0x7fffffff) {
            const unsigned long long key =
                (static_cast<unsigned long long>(ordered_key(best_v[r])) << 32) |
                static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(best_n[r]));
            atomicMax(a.keys + m, key);
          }
        }
      }
    }
  }
  if (ARGMAX) {
    __shared__ int last;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) last = (atomicAdd(a.counter, 1u) == gridDim.x - 1);
    __syncthreads();
    if (last) {
      __threadfence();
      if (threadIdx.x < a.M) {
        const unsigned long long key = atomicExch(a.keys + threadIdx.x, 0ull);
        a.idx[threadIdx.x] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(key & 0xFFFFFFFFull));
      }
      if (threadIdx.x == 0) atomicExch(a.counter, 0u);
    }
  }
}

template <typename Kern>
hipError_t launch(Kern k, int grid, int block, const Nvfp4Args& a, hipStream_t stream) {
  hipLaunchKernelGGL(k, dim3(grid), dim3(block), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

bool nvfp4_cfg_supported(const LaunchCfg& c, int M, bool argmax) {
  const bool ct_ok = c.ct == 1 || c.ct == 2 || c.ct == 4;
  const bool nw_ok = c.nw == 4 || c.nw == 8;
  if (!ct_ok || !nw_ok) return false;
  if (c.engine == 0) return M == 1 && !argmax;
  return c.engine == 1;
}

#define SKINNY_NVFP4_DISPATCH(CT, NW)                                                         \
  if (cfg.ct == CT && cfg.nw == NW) {                                                         \
    if (cfg.engine == 0) return launch(nvfp4_valu_m1<CT, NW>, grid, NW * 64, a, stream);     \
    if (argmax) return launch(nvfp4_mfma<CT, NW, true>, grid, NW * 64, a, stream);           \
    return launch(nvfp4_mfma<CT, NW, false>, grid, NW * 64, a, stream);                      \
  }

hipError_t launch_nvfp4(const uint8_t* blob, const uint16_t* x, uint16_t* y, int M, int K, int N,
                        const LaunchCfg& cfg, int32_t* idx, void* workspace, hipStream_t stream) {
  const Geometry geo = nvfp4_geometry(K, N);
  Nvfp4Args a;
  a.codes = blob + kHeaderBytes;
  a.scales = blob + kHeaderBytes + geo.codes_bytes;
  a.gptr = reinterpret_cast<const float*>(blob + kGOffset);
  a.x = reinterpret_cast<const _Float16*>(x);
  a.y = reinterpret_cast<_Float16*>(y);
  a.M = M;
  a.K = K;
  a.N = N;
  a.kc = geo.kc;
  a.nt = geo.nt;
  a.sg = geo.sg;
  a.idx = idx;
  a.keys = reinterpret_cast<unsigned long long*>(workspace);
  a.counter = workspace ? reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(workspace) + 8 * kMaxRows)
                        : nullptr;
  const bool argmax = idx != nullptr;
  const int grid = (geo.nt + cfg.ct - 1) / cfg.ct;
  SKINNY_NVFP4_DISPATCH(1, 4)
  SKINNY_NVFP4_DISPATCH(1, 8)
  SKINNY_NVFP4_DISPATCH(2, 4)
  SKINNY_NVFP4_DISPATCH(2, 8)
  SKINNY_NVFP4_DISPATCH(4, 4)
  SKINNY_NVFP4_DISPATCH(4, 8)
  return hipErrorInvalidValue;
}

}  // namespace skinny
