// NVFP4 weight-only skinny GEMM kernels for gfx950 (MI355X).
//
// y[m][n] = g * sum_k x[m][k] * e2m1(q[n][k]) * e4m3(s[n][k/16]),  1 <= M <= 8.
//
// The weights are read once, compressed, straight from HBM into VGPRs (with
// the streaming cache policy: no weight byte is read twice) and widened to
// fp16 in registers just before use; there is no dequantized copy
// anywhere ("NVFP4 on Volta!" author's post, section "What I actually
// built").  Decode at batch 1..8 is bound by that weight stream, so the
// design is about keeping as many 128-bit loads in flight as the chip holds.
//
// Work split.  The packed weights are 9 KiB units (one 16-column tile x 1024
// K: eight 1 KiB code chunks and one 1 KiB scale vector; see internal.h).
// Every wavefront owns exactly one unit: it issues the unit's nine 16-byte
// loads per lane at once, then widens and contracts the eight chunks.  A
// workgroup is CT tiles x S consecutive K spans (nw = CT * S wavefronts);
// the S partial sums of a tile are added in LDS in span order.  When K has
// more spans than a workgroup covers, ksplit workgroups share a tile group:
// each stores its fp32 partial sums with plain stores.  With the plain
// epilogue the splits of a group run on one XCD and the last of them to
// arrive adds all of them in split order (xsplit_add, xsplit.cuh); otherwise a
// second small kernel (reduce.hip) adds them in split order.  Either way the
// result does not depend on timing.  Few registers per wavefront (one unit)
// let the chip keep tens of megabytes of weight loads in flight, which is
// what saturates HBM at these sizes.
//
// Two engines (lane l = 16*grp + c handles column c of the tile and the
// 32-K run 128j + 32grp .. +32 of every chunk j):
//   * VALU (M = 1, 2): v_dot2c_f32_f16 whose x operand is read through DPP
//     row_newbcast (lane 16r + i holds the x pair that every lane of row r
//     needs at step i), each 16-K block's sum scaled by its E4M3 scale in fp32,
//     the four rows that split a column's K added with permlane swaps.  At
//     M = 2 each widened code pair feeds one v_dot2c per x row.  Its balanced
//     layout (engine 3, the Plan's bal_* fields) keeps whole-K tiles for the
//     largest multiple of the CU count and cuts the rest along K, so that
//     every CU reads about the same number of weight bytes: a GEMV with one
//     tile per workgroup lasts as long as its most loaded CUs.
//   * MFMA (M = 1..8): v_mfma_f32_16x16x32_f16 with the widened weights
//     (E2M1 * E4M3 in fp16, exact) as operand B and the x rows, zero-padded to
//     16, as operand A.  The workgroup's x slice is copied into LDS with
//     direct-to-LDS loads (no VGPRs) before the weight loads; A fragments are
//     read from LDS one chunk ahead.  The pages' 8-row verification tile
//     (post, on why the M = 8 row matters) fills half of the 16-row MFMA tile.
// The MFMA engine also carries the lm_head epilogue: each workgroup (or, with
// a K split, each block of the split reduction) writes, per row, the (fp32
// logit, column) of its best column as one ordered 64-bit key; a one-workgroup
// kernel takes the maximum key per row (ties to the lowest column) and writes
// the indices.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.cuh"
#include "internal.h"
#include "xsplit.cuh"

namespace skinny {
namespace {

struct Nvfp4Args {
  const uint8_t* units;
  const float* gptr;
  const _Float16* x;
  _Float16* y;
  int M, K, N;
  int ku, nt, ksplit, S;     // S: K spans per workgroup
  float* part;               // fp32 partial sums of a K split (ksplit > 1): [ksplit][M][N], or with
                             // xsplit one block [M][ct * 16] per (tile group, split)
  unsigned long long* cand;  // [gridDim.x][M] argmax candidates (lm_head, ksplit == 1)
  const float* g2ptr;        // SwiGLU pair: the up projection's scale
  int F;                     // SwiGLU pair: output columns (y is h[M][F])
  int xsplit;                // 1: the K split is added inside the kernel on each tile group's XCD
  int ntg;                   // tile groups (xsplit)
  unsigned* sync;            // xsplit: one arrival counter per tile group, 128 bytes apart (zero at rest)
  // Balanced VALU GEMV (engine 3; bal_small == 0 otherwise): workgroups b <
  // bal_small each take bal_s K spans of one of the last bal_r tiles (bal_ks
  // workgroups per tile, added as an xsplit); the others take one whole tile
  // of the first bal_whole tiles each.
  int bal_small, bal_r, bal_whole, bal_s, bal_ks;
};

// What a kernel does with its finished fp32 tile sums.
enum : int { kEpiPlain = 0, kEpiArgmax = 1, kEpiSwiglu = 2 };

// SwiGLU of a pair-interleaved tile: the lane of gate column c < 8 takes its
// up sum from lane c + 8 (same row group, DPP row_ror:8: a rotation by half a
// row pairs lanes c and c ^ 8 without an LDS round trip) and returns
// silu(g * gate) * (g2 * up); lanes c >= 8 get a value that is never stored.
// Every lane of the 16-lane row must execute this.
__device__ __forceinline__ float swiglu_pair(float sum, float g, float g2) {
  constexpr int kRowRor8 = 0x128;
  const float up = __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, sum), kRowRor8, 0xf, 0xf, false));
  return silu(g * sum) * (g2 * up);
}

// This wavefront's unit and its workgroup's geometry (wave-uniform values).
// Workgroup b of an xsplit grid (1-D, 8 * ceil(ntg / 8) * ksplit workgroups)
// takes tile group and split from xsplit_place (xsplit.cuh): the splits of a
// tile group run on one XCD.
struct Plan {
  int lane, wave, nw, S, tile0, s0, sw;  // sw: spans in this split
  int t, s;                              // local tile and span of this wavefront's unit
  int group, split;                      // tile group and K split of this workgroup
  int ks;                                // workgroups that share the tile group along K
  bool active;
  bool small;                            // a K-split workgroup of the balanced GEMV
  __device__ Plan(const Nvfp4Args& a, int ct) {
    lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    nw = blockDim.x >> 6;
    S = a.S;
    ks = a.ksplit;
    small = false;
    if (a.bal_small > 0) {  // balanced GEMV (ct = 1, nw >= ku, S = nw)
      const int b = blockIdx.x;
      small = b < a.bal_small;
      if (small) {
        ks = a.bal_ks;
        xsplit_place(b, a.bal_ks, group, split);
        tile0 = a.bal_whole + group;
        S = a.bal_s;
        s0 = split * S;
        sw = min(S, a.ku - s0);
      } else {
        ks = 1;
        group = b - a.bal_small;
        split = 0;
        tile0 = group;
        s0 = 0;
        sw = a.ku;
      }
      t = wave / S;
      s = wave % S;
      // Every workgroup of the grid has nw >= ku wavefronts: those past a
      // workgroup's spans (all but S of a small one) idle.
      active = t == 0 && s < sw && (!small || group < a.bal_r);
      return;
    }
    if (a.xsplit) {
      xsplit_place(blockIdx.x, a.ksplit, group, split);
    } else {
      group = blockIdx.x;
      split = blockIdx.y;
    }
    tile0 = group * ct;
    s0 = split * S;
    sw = min(S, a.ku - s0);
    t = wave / S;
    s = wave % S;
    active = s < sw;
  }
  // Units past the last tile (grid rounding) re-read the last tile; their
  // results are never stored.
  __device__ const uint8_t* unit_ptr(const Nvfp4Args& a) const {
    const int tt = min(tile0 + t, a.nt - 1);
    return a.units + (static_cast<size_t>(s0 + s) * a.nt + tt) * kUnitBytes + lane * 16;
  }
};

// Read in place of activation pairs past K by the VALU engine (a global,
// not a constant, so that both choices of address are global loads).
__device__ uint32_t kZeroPair = 0u;

__device__ __forceinline__ uint32_t dword(const u32x4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// ---------------------------------------------------------------------------
// VALU engine, M = 1 and 2.
// ---------------------------------------------------------------------------
// Sixteen codes (two dwords, one 16-K block) against x pairs broadcast from
// lanes 0..7 (lo) or 8..15 (hi) of the lane's own 16-lane row.  One asm block
// widens the codes (v_cvt_scalef32_pk_f16_fp4, byte by byte, low nibble to
// the low half) into eight scratch registers and runs eight v_dot2c_f32_f16
// whose first operand is read through DPP row_newbcast, so the broadcast costs
// no instruction of its own.  Keeping the conversion inside the block stops
// the compiler from converting a whole unit ahead of use.  The compiler cannot
// see hazards inside the asm, so the block carries its own wait states: two
// before the first DPP read (a VALU write of its source may precede the
// block) and two after the last v_dot2c, whose result a following VALU read
// would otherwise miss.
#define SKINNY_BLOCK_DOT(NAME, R0, R1, R2, R3, R4, R5, R6, R7)                                  \
  __device__ __forceinline__ float NAME(uint32_t xv, uint32_t w0, uint32_t w1) {                \
    float p = 0.0f;                                                                             \
    uint32_t t0, t1, t2, t3, t4, t5, t6, t7;                                                    \
    asm("v_cvt_scalef32_pk_f16_fp4 %1, %9, 1.0\n"                                               \
        "v_cvt_scalef32_pk_f16_fp4 %2, %9, 1.0 op_sel:[1,0,0]\n"                                \
        "v_cvt_scalef32_pk_f16_fp4 %3, %9, 1.0 op_sel:[0,1,0]\n"                                \
        "v_cvt_scalef32_pk_f16_fp4 %4, %9, 1.0 op_sel:[1,1,0]\n"                                \
        "v_cvt_scalef32_pk_f16_fp4 %5, %10, 1.0\n"                                              \
        "v_cvt_scalef32_pk_f16_fp4 %6, %10, 1.0 op_sel:[1,0,0]\n"                               \
        "v_cvt_scalef32_pk_f16_fp4 %7, %10, 1.0 op_sel:[0,1,0]\n"                               \
        "v_cvt_scalef32_pk_f16_fp4 %8, %10, 1.0 op_sel:[1,1,0]\n"                               \
        "s_nop 1\n"                                                                             \
        "v_dot2c_f32_f16_dpp %0, %11, %1 row_newbcast:" #R0 " row_mask:0xf bank_mask:0xf\n"     \
        "v_dot2c_f32_f16_dpp %0, %11, %2 row_newbcast:" #R1 " row_mask:0xf bank_mask:0xf\n"     \
        "v_dot2c_f32_f16_dpp %0, %11, %3 row_newbcast:" #R2 " row_mask:0xf bank_mask:0xf\n"     \
        "v_dot2c_f32_f16_dpp %0, %11, %4 row_newbcast:" #R3 " row_mask:0xf bank_mask:0xf\n"     \
        "v_dot2c_f32_f16_dpp %0, %11, %5 row_newbcast:" #R4 " row_mask:0xf bank_mask:0xf\n"     \
        "v_dot2c_f32_f16_dpp %0, %11, %6 row_newbcast:" #R5 " row_mask:0xf bank_mask:0xf\n"     \
        "v_dot2c_f32_f16_dpp %0, %11, %7 row_newbcast:" #R6 " row_mask:0xf bank_mask:0xf\n"     \
        "v_dot2c_f32_f16_dpp %0, %11, %8 row_newbcast:" #R7 " row_mask:0xf bank_mask:0xf\n"     \
        "s_nop 1\n"                                                                             \
        : "+v"(p), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(t5), "=&v"(t6), \
          "=&v"(t7)                                                                             \
        : "v"(w0), "v"(w1), "v"(xv));                                                           \
    return p;                                                                                   \
  }
SKINNY_BLOCK_DOT(block_dot_lo, 0, 1, 2, 3, 4, 5, 6, 7)
SKINNY_BLOCK_DOT(block_dot_hi, 8, 9, 10, 11, 12, 13, 14, 15)
#undef SKINNY_BLOCK_DOT

// The same for two rows of x (M = 2): the codes are widened once and feed
// sixteen v_dot2c, eight per row; the wait states are those of the one-row
// block.
#define SKINNY_BLOCK_DOT2(NAME, R0, R1, R2, R3, R4, R5, R6, R7)                                          \
  __device__ __forceinline__ void NAME(uint32_t x0, uint32_t x1, uint32_t w0, uint32_t w1, float& p0,   \
                                       float& p1) {                                                     \
    p0 = 0.0f;                                                                                          \
    p1 = 0.0f;                                                                                          \
    uint32_t t0, t1, t2, t3, t4, t5, t6, t7;                                                            \
    asm("v_cvt_scalef32_pk_f16_fp4 %2, %10, 1.0\n"                                                     \
        "v_cvt_scalef32_pk_f16_fp4 %3, %10, 1.0 op_sel:[1,0,0]\n"                                      \
        "v_cvt_scalef32_pk_f16_fp4 %4, %10, 1.0 op_sel:[0,1,0]\n"                                      \
        "v_cvt_scalef32_pk_f16_fp4 %5, %10, 1.0 op_sel:[1,1,0]\n"                                      \
        "v_cvt_scalef32_pk_f16_fp4 %6, %11, 1.0\n"                                                     \
        "v_cvt_scalef32_pk_f16_fp4 %7, %11, 1.0 op_sel:[1,0,0]\n"                                      \
        "v_cvt_scalef32_pk_f16_fp4 %8, %11, 1.0 op_sel:[0,1,0]\n"                                      \
        "v_cvt_scalef32_pk_f16_fp4 %9, %11, 1.0 op_sel:[1,1,0]\n"                                      \
        "s_nop 1\n"                                                                                     \
        "v_dot2c_f32_f16_dpp %0, %12, %2 row_newbcast:" #R0 " row_mask:0xf bank_mask:0xf\n"             \
        "v_dot2c_f32_f16_dpp %1, %13, %2 row_newbcast:" #R0 " row_mask:0xf bank_mask:0xf\n"             \
        "v_dot2c_f32_f16_dpp %0, %12, %3 row_newbcast:" #R1 " row_mask:0xf bank_mask:0xf\n"             \
        "v_dot2c_f32_f16_dpp %1, %13, %3 row_newbcast:" #R1 " row_mask:0xf bank_mask:0xf\n"             \
        "v_dot2c_f32_f16_dpp %0, %12, %4 row_newbcast:" #R2 " row_mask:0xf bank_mask:0xf\n"             \
        "v_dot2c_f32_f16_dpp %1, %13, %4 row_newbcast:" #R2 " row_mask:0xf bank_mask:0xf\n"             \
        "v_dot2c_f32_f16_dpp %0, %12, %5 row_newbcast:" #R3 " row_mask:0xf bank_mask:0xf\n"             \
        "v_dot2c_f32_f16_dpp %1, %13, %5 row_newbcast:" #R3 " row_mask:0xf bank_mask:0xf\n"             \
        "v_dot2c_f32_f16_dpp %0, %12, %6 row_newbcast:" #R4 " row_mask:0xf bank_mask:0xf\n"             \
        "v_dot2c_f32_f16_dpp %1, %13, %6 row_newbcast:" #R4 " row_mask:0xf bank_mask:0xf\n"             \
        "v_dot2c_f32_f16_dpp %0, %12, %7 row_newbcast:" #R5 " row_mask:0xf bank_mask:0xf\n"             \
        "v_dot2c_f32_f16_dpp %1, %13, %7 row_newbcast:" #R5 " row_mask:0xf bank_mask:0xf\n"             \
        "v_dot2c_f32_f16_dpp %0, %12, %8 row_newbcast:" #R6 " row_mask:0xf bank_mask:0xf\n"             \
        "v_dot2c_f32_f16_dpp %1, %13, %8 row_newbcast:" #R6 " row_mask:0xf bank_mask:0xf\n"             \
        "v_dot2c_f32_f16_dpp %0, %12, %9 row_newbcast:" #R7 " row_mask:0xf bank_mask:0xf\n"             \
        "v_dot2c_f32_f16_dpp %1, %13, %9 row_newbcast:" #R7 " row_mask:0xf bank_mask:0xf\n"             \
        "s_nop 1\n"                                                                                     \
        : "+v"(p0), "+v"(p1), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(t5),         \
          "=&v"(t6), "=&v"(t7)                                                                          \
        : "v"(w0), "v"(w1), "v"(x0), "v"(x1));                                                          \
  }
SKINNY_BLOCK_DOT2(block_dot2_lo, 0, 1, 2, 3, 4, 5, 6, 7)
SKINNY_BLOCK_DOT2(block_dot2_hi, 8, 9, 10, 11, 12, 13, 14, 15)
#undef SKINNY_BLOCK_DOT2

// MR rows of x (MR = M = 1 or 2), one unit per wavefront.
template <int CT, int EPI, int MR>
__global__ __launch_bounds__(kMaxWaves * 64) void nvfp4_valu(Nvfp4Args a) {
  __shared__ float red[kMaxWaves][MR][16];
  const Plan P(a, CT);
  if (a.xsplit && P.group >= a.ntg) return;  // grid rounding to whole groups of 8 (uniform)
  if (P.small && P.group >= a.bal_r) return;  // the same for the balanced GEMV's split tiles
  float acc[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) acc[r] = 0.0f;
  if (P.active) {
    // The whole unit plus this lane's x pair of each chunk and row (k = 1024g + 128j + 2*lane).
    const uint8_t* p = P.unit_ptr(a);
    const u32x4 sv = load16(p + kChunksPerUnit * kChunkBytes);
    u32x4 c[kChunksPerUnit];
    uint32_t xv[MR][kChunksPerUnit];
    const int kx = (P.s0 + P.s) * kUnitK + 2 * P.lane;
    // A pair past K (k even and K % 16 == 0, so a pair is all in or all out)
    // reads a zero word instead: the packed weights there are zero too, and
    // 0 * 0 adds nothing whatever the row's real activations hold (a clamped
    // real pair would turn an inf or NaN at the end of the row into NaN for
    // every column).  Choosing the address rather than selecting zero after
    // the load keeps the loads independent; a select on loaded data made the
    // first chunk wait for half of the unit's loads.  With two rows a
    // scheduling barrier keeps every load of the unit ahead of the first
    // conversion (the compiler otherwise held back 9 of the 25 loads, which
    // cost 0.3 us on a 17408 x 5120 weight); with one row it issues all 17
    // first by itself, and the barrier measured 0.25 us slower there.
#pragma unroll
    for (int j = 0; j < kChunksPerUnit; ++j) {
      c[j] = load16(p + j * kChunkBytes);
      const int k = kx + j * kChunkK;
#pragma unroll
      for (int r = 0; r < MR; ++r)
        xv[r][j] = *(k < a.K ? reinterpret_cast<const uint32_t*>(a.x + static_cast<size_t>(r) * a.K + k)
                             : &kZeroPair);
    }
    if constexpr (MR == 2) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kChunksPerUnit; ++j) {
      const uint32_t sd = dword(sv, j >> 1);
      const float s0 = (j & 1) ? e4m3f<2>(sd) : e4m3f<0>(sd);
      const float s1 = (j & 1) ? e4m3f<3>(sd) : e4m3f<1>(sd);
      if constexpr (MR == 1) {
        acc[0] = __builtin_fmaf(block_dot_lo(xv[0][j], c[j].x, c[j].y), s0, acc[0]);
        acc[0] = __builtin_fmaf(block_dot_hi(xv[0][j], c[j].z, c[j].w), s1, acc[0]);
      } else {
        float p0, p1;
        block_dot2_lo(xv[0][j], xv[1][j], c[j].x, c[j].y, p0, p1);
        acc[0] = __builtin_fmaf(p0, s0, acc[0]);
        acc[1] = __builtin_fmaf(p1, s0, acc[1]);
        block_dot2_hi(xv[0][j], xv[1][j], c[j].z, c[j].w, p0, p1);
        acc[0] = __builtin_fmaf(p0, s1, acc[0]);
        acc[1] = __builtin_fmaf(p1, s1, acc[1]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    acc[r] = sum_over_rows(acc[r]);
    if (P.lane < 16) red[P.wave][r][P.lane] = acc[r];
  }
  __syncthreads();

  // Wavefront t < CT finishes local tile t: its spans in order, then the
  // outputs or, with a K split, this split's partial sums.
  const bool fin = P.wave < CT && P.lane < 16 && P.tile0 + P.wave < a.nt;
  const int n = (P.tile0 + P.wave) * kTileCols + P.lane;
  float tot[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) tot[r] = 0.0f;
  if (fin) {
    for (int s = 0; s < P.sw; ++s) {
#pragma unroll
      for (int r = 0; r < MR; ++r) tot[r] += red[P.wave * P.S + s][r][P.lane];
    }
  }
  if (P.ks > 1 && (a.xsplit || P.small)) {  // this split's block of the group; the last split adds them
    if (fin) {
      float* blk = a.part + (static_cast<size_t>(P.group) * P.ks + P.split) * MR * (CT * kTileCols);
#pragma unroll
      for (int r = 0; r < MR; ++r) blk[r * (CT * kTileCols) + P.wave * kTileCols + P.lane] = tot[r];
    }
    xsplit_add<CT * kTileCols, true>(a.sync, a.part, a.y, a.gptr, a.M, a.N, P.tile0, P.group, P.ks);
    return;
  }
  if (fin) {
    if (EPI == kEpiSwiglu && a.ksplit == 1) {  // lanes 0..15 of the wavefront are all here
      const int f = (P.tile0 + P.wave) * 8 + P.lane;
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        const float h = swiglu_pair(tot[r], *a.gptr, *a.g2ptr);
        if (P.lane < 8 && f < a.F) a.y[static_cast<size_t>(r) * a.F + f] = static_cast<_Float16>(h);
      }
    } else if (n < a.N) {
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        if (a.ksplit > 1)
          a.part[(static_cast<size_t>(P.split) * MR + r) * a.N + n] = tot[r];
        else if (EPI != kEpiArgmax || a.y)  // the lm_head's logits are optional
          a.y[static_cast<size_t>(r) * a.N + n] = static_cast<_Float16>(*a.gptr * tot[r]);
      }
    }
  }
  if (EPI == kEpiArgmax) {
    // lm_head (no K split): per row, the (fp32 logit, column) key of each of
    // this workgroup's tiles, then of the workgroup, as its candidate.
    // Every lane runs the shuffles; lanes outside a finished tile hold 0.
    __shared__ unsigned long long best[kMaxWaves][MR];
    unsigned long long key[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) key[r] = fin && n < a.N ? argmax_key(*a.gptr * tot[r], n) : 0ull;
    wave_max_keys<MR, 16>(key);
    if (P.lane == 0) {
#pragma unroll
      for (int r = 0; r < MR; ++r) best[P.wave][r] = key[r];
    }
    __syncthreads();
    if (threadIdx.x < MR) {
      unsigned long long k = 0ull;
      for (int t = 0; t < CT; ++t) k = best[t][threadIdx.x] > k ? best[t][threadIdx.x] : k;
      a.cand[static_cast<size_t>(blockIdx.x) * MR + threadIdx.x] = k;
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA engine, M = 1..8 (and the lm_head argmax candidates).
// ---------------------------------------------------------------------------
// LDS copy of x for this workgroup's K spans: rows 0..M-1, row stride
// RS = S*1024 + 8 halves (the pad spreads the rows over LDS banks).
__device__ __forceinline__ int xs_stride(int S) { return S * kUnitK + 8; }

// Copy x[m][1024*s0 .. 1024*(s0+S)) for m < M into LDS with direct-to-LDS
// loads: each wavefront instruction moves one contiguous KiB (64 lanes x 16
// bytes) of one row.  Parts past K are not loaded (those weights are zero);
// that part of the copy is zero-filled with plain stores instead.
__device__ void stage_x(const Nvfp4Args& a, const Plan& P, _Float16* xs) {
  const int RS = xs_stride(P.S);
  const int kbase = P.s0 * kUnitK;
  const int blocks_per_row = P.S * 2;  // 1 KiB blocks = 512 halves
  const int kvalid = a.K - kbase;      // halves of each row that exist
  if (kvalid < P.S * kUnitK) zero_x_tail(xs, a.M, RS, kvalid, P.S * kUnitK);
  const int nblocks = a.M * blocks_per_row;
  for (int b = P.wave; b < nblocks; b += P.nw) {
    const int m = b / blocks_per_row, blk = b % blocks_per_row;
    const int col = blk * 512 + P.lane * 8;
    if (col < kvalid)
      __builtin_amdgcn_global_load_lds(a.x + static_cast<size_t>(m) * a.K + kbase + col, xs + m * RS + blk * 512,
                                       16, 0, 0);
  }
}

// Operand A fragments of chunk j: lane (row c, grp) holds
// x[min(c, M-1)][1024s + 128j + 32grp + 8i .. +8] for MFMA i = 0..3.  Rows
// c >= M of the 16-row tile repeat row M-1 instead of being zeroed: they only
// feed output rows >= M, which are never stored, and reading them costs
// nothing where zeroing costs a branch and sixteen moves per chunk.
__device__ __forceinline__ void read_x_frag(f16x8 (&xa)[4], const _Float16* xrow, int j) {
#pragma unroll
  for (int i = 0; i < 4; ++i) xa[i] = *reinterpret_cast<const f16x8*>(xrow + j * kChunkK + 8 * i);
}

template <int J>
__device__ __forceinline__ f32x4 mfma_chunk(const u32x4& cj, const u32x4& sv, const f16x8 (&xa)[4], f32x4 acc) {
  const f16x2 s = e4m3x2<(J & 1) != 0>(dword(sv, J >> 1));
  const f16x8 s0 = f16x8{s.x, s.x, s.x, s.x, s.x, s.x, s.x, s.x};
  const f16x8 s1 = f16x8{s.y, s.y, s.y, s.y, s.y, s.y, s.y, s.y};
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[0], e2m1x8(cj.x) * s0, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[1], e2m1x8(cj.y) * s0, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[2], e2m1x8(cj.z) * s1, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[3], e2m1x8(cj.w) * s1, acc, 0, 0, 0);
  return acc;
}

template <int J>
__device__ __forceinline__ void mfma_steps(const u32x4 (&c)[kChunksPerUnit], const u32x4& sv, f16x8 (&x0)[4],
                                           f16x8 (&x1)[4], f32x4& acc, const _Float16* xrow) {
  if constexpr (J < kChunksPerUnit) {
    f16x8 (&cur)[4] = (J & 1) ? x1 : x0;
    f16x8 (&nxt)[4] = (J & 1) ? x0 : x1;
    if constexpr (J + 1 < kChunksPerUnit) read_x_frag(nxt, xrow, J + 1);
    acc = mfma_chunk<J>(c[J], sv, cur, acc);
    mfma_steps<J + 1>(c, sv, x0, x1, acc, xrow);
  }
}

template <int CT, int EPI>
__global__ __launch_bounds__(kMaxWaves * 64) void nvfp4_mfma(Nvfp4Args a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const Plan P(a, CT);
  if (a.xsplit && P.group >= a.ntg) return;  // grid rounding to whole groups of 8 (uniform)
  _Float16* xs = reinterpret_cast<_Float16*>(lds);
  f32x4* red = reinterpret_cast<f32x4*>(lds + ((a.M * xs_stride(P.S) * 2 + 15) & ~15));  // [nw][32]

  // x first (the vector-memory counter completes in order), then the unit.
  // Every wavefront loads a unit, an idle one (past the last K span) the
  // blob's unit 0, a cache hit it never uses: with no load under a branch
  // the compiler waits for each chunk alone instead of the whole unit.
  stage_x(a, P, xs);
  u32x4 c[kChunksPerUnit], sv;
  {
    const uint8_t* p = P.active ? P.unit_ptr(a) : a.units + P.lane * 16;
    sv = load16(p + kChunksPerUnit * kChunkBytes);
#pragma unroll
    for (int j = 0; j < kChunksPerUnit; ++j) c[j] = load16(p + j * kChunkBytes);
  }
  // x is in LDS once every wavefront's copies are done; the weights keep arriving.
  lds_copy_barrier<kChunksPerUnit + 1>(true);

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  if (P.active) {
    const int cl = P.lane & 15, grp = P.lane >> 4;
    const _Float16* xrow = xs + min(cl, a.M - 1) * xs_stride(P.S) + P.s * kUnitK + grp * 32;
    f16x8 x0[4], x1[4];
    read_x_frag(x0, xrow, 0);
    mfma_steps<0>(c, sv, x0, x1, acc, xrow);
  }
  if (P.lane < 32) red[P.wave * 32 + P.lane] = acc;
  __syncthreads();

  // Wavefront t < CT finishes local tile t.  D layout: lane (grp, c) holds
  // rows 4grp..4grp+3 of column c; rows >= 8 are padding.
  const bool fin = P.wave < CT && P.tile0 + P.wave < a.nt && P.lane < 32;
  const int cl = P.lane & 15, grp = P.lane >> 4;
  const int n = (P.tile0 + P.wave) * kTileCols + cl;
  f32x4 tot = f32x4{0.f, 0.f, 0.f, 0.f};
  if (fin)
    for (int s = 0; s < P.sw; ++s) tot += red[(P.wave * P.S + s) * 32 + P.lane];
  if (a.ksplit > 1 && a.xsplit) {  // this split's block of the group; the last split adds them
    if (fin) {
      float* blk = a.part + (static_cast<size_t>(P.group) * a.ksplit + P.split) * a.M * (CT * kTileCols);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = grp * 4 + i;
        if (m < a.M) blk[m * (CT * kTileCols) + P.wave * kTileCols + cl] = tot[i];
      }
    }
    xsplit_add<CT * kTileCols, true>(a.sync, a.part, a.y, a.gptr, a.M, a.N, P.tile0, P.group, a.ksplit);
    return;
  }
  if (a.ksplit > 1) {  // this split's partial sums; the split reduction finishes
    if (fin && n < a.N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = grp * 4 + i;
        if (m < a.M) a.part[(static_cast<size_t>(P.split) * a.M + m) * a.N + n] = tot[i];
      }
    }
    return;
  }

  const float g = *a.gptr;
  if (EPI == kEpiSwiglu) {  // lanes 0..31 of the wavefront are all in `fin` or none
    if (fin) {
      const float g2 = *a.g2ptr;
      const int f = (P.tile0 + P.wave) * 8 + cl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = grp * 4 + i;
        const float h = swiglu_pair(tot[i], g, g2);
        if (cl < 8 && m < a.M && f < a.F) a.y[static_cast<size_t>(m) * a.F + f] = static_cast<_Float16>(h);
      }
    }
    return;
  }
  unsigned long long key[4] = {0ull, 0ull, 0ull, 0ull};
  if (fin && n < a.N) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = grp * 4 + i;
      const float v = g * tot[i];
      if (m < a.M) {
        if (a.y) a.y[static_cast<size_t>(m) * a.N + n] = static_cast<_Float16>(v);
        key[i] = argmax_key(v, n);
      }
    }
  }
  if (EPI == kEpiArgmax) {
    // Largest key over the 16 columns of each row group, then over the
    // workgroup's tiles: one candidate per row.
    __shared__ unsigned long long best[kMaxWaves][kMaxRows];
    wave_max_keys<4, 16>(key);
    if (P.wave < CT && P.lane < 32 && cl == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) best[P.wave][grp * 4 + i] = key[i];
    }
    __syncthreads();
    if (threadIdx.x < static_cast<unsigned>(a.M)) {
      unsigned long long k = 0ull;
      for (int t = 0; t < CT; ++t) k = best[t][threadIdx.x] > k ? best[t][threadIdx.x] : k;
      a.cand[static_cast<size_t>(blockIdx.x) * a.M + threadIdx.x] = k;
    }
  }
}

// ---------------------------------------------------------------------------
// Streaming MFMA engine (M = 1..8, K small enough for x to sit in LDS).
// ---------------------------------------------------------------------------
// One workgroup per CU slot copies all of x into LDS once; each wavefront then
// owns whole column tiles (tile t = blockIdx.x + gridDim.x * (wave + nw * i))
// and walks each tile's K spans in order, with the next unit's nine loads
// issued before the current unit is contracted (two units in flight per
// wavefront).  Every tile's sum stays in one wavefront's registers, so there
// is no K split and no second pass; the price is more VGPRs per wavefront
// (two units) and an x copy per workgroup instead of per tile group.
struct Unit {
  u32x4 c[kChunksPerUnit];
  u32x4 sv;
};

__device__ __forceinline__ void load_unit(Unit& u, const uint8_t* p) {
  u.sv = load16(p + kChunksPerUnit * kChunkBytes);
#pragma unroll
  for (int j = 0; j < kChunksPerUnit; ++j) u.c[j] = load16(p + j * kChunkBytes);
}

// Copies x[m][0..K) for m < M into LDS rows of stride RS halves, zero past K.
__device__ void stage_x_all(const Nvfp4Args& a, _Float16* xs, int RS, int wave, int nw, int lane) {
  const int kp = a.ku * kUnitK;
  if (a.K < kp) zero_x_tail(xs, a.M, RS, a.K, kp);
  const int blocks_per_row = kp / 512;  // 1 KiB blocks
  const int nblocks = a.M * blocks_per_row;
  for (int b = wave; b < nblocks; b += nw) {
    const int m = b / blocks_per_row, blk = b % blocks_per_row;
    const int col = blk * 512 + lane * 8;
    if (col < a.K)
      __builtin_amdgcn_global_load_lds(a.x + static_cast<size_t>(m) * a.K + col, xs + m * RS + blk * 512, 16, 0, 0);
  }
}

// The eight chunks of a unit with one set of A fragments, read from LDS just
// before use (the streaming kernel spends its registers on the second unit).
template <int J>
__device__ __forceinline__ void mfma_unit_lean(const Unit& U, f32x4& acc, const _Float16* xrow) {
  if constexpr (J < kChunksPerUnit) {
    f16x8 xa[4];
    read_x_frag(xa, xrow, J);
    acc = mfma_chunk<J>(U.c[J], U.sv, xa, acc);
    mfma_unit_lean<J + 1>(U, acc, xrow);
  }
}

// Per-wavefront state of the streaming kernel.
struct StreamCtx {
  const Nvfp4Args* a;
  const _Float16* xbase;  // this lane's LDS x row (row min(c, M-1)), fragment group offset included
  size_t span_stride;     // bytes from one K span of a tile to its next (span-major units)
  size_t tile_stride;     // bytes from one of this wavefront's tiles to its next
  unsigned long long* best;  // LDS [kMaxRows] running argmax keys of this wavefront
  const uint8_t* spare;      // unit 0 of the blob (this lane's 16 bytes): read in place of a unit past the last tile
  int t0, step, ntiles, lane;
  float g, g2;
};

// Unit J of this wavefront's tile `ti`, whose unit 0 (this lane's 16 bytes)
// is at `base`.  All buffer choices are compile-time: first the loads of the
// wavefront's next unit go out into the other buffer, then unit J is
// contracted.  The next unit is always loaded: after the wavefront's last
// tile it is the blob's unit 0, a cache hit that is never used.  With no
// load under a branch the compiler knows, at every chunk, exactly how many
// loads are still in flight, and waits for the current unit only; a
// conditional prefetch made it wait for the prefetch too, at every tile
// boundary.  After the tile's last span the tile is stored and its logits
// are folded into the wavefront's running argmax keys (kept in LDS, not in
// registers, which the two units in flight already fill).
template <int KU, int J, int PAR, int EPI>
__device__ __forceinline__ void stream_units(const StreamCtx& c, Unit& A, Unit& B, int ti, const uint8_t* base,
                                             f32x4& acc) {
  if constexpr (J < KU) {
    Unit& cur = PAR ? B : A;
    Unit& nxt = PAR ? A : B;
    if constexpr (J + 1 < KU)
      load_unit(nxt, base + (J + 1) * c.span_stride);
    else
      load_unit(nxt, ti + 1 < c.ntiles ? base + c.tile_stride : c.spare);
    // Keep the scheduler from hoisting work across units: it would start later
    // units' LDS reads and conversions early and run out of registers.
    __builtin_amdgcn_sched_barrier(0);
    mfma_unit_lean<0>(cur, acc, c.xbase + J * kUnitK);
    __builtin_amdgcn_sched_barrier(0);
    stream_units<KU, J + 1, 1 - PAR, EPI>(c, A, B, ti, base, acc);
  } else {
    const Nvfp4Args& a = *c.a;
    const int cl = c.lane & 15, grp = c.lane >> 4;
    if (EPI == kEpiSwiglu) {  // every lane is here: pair up gate and up columns
      const int f = (c.t0 + ti * c.step) * 8 + cl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = grp * 4 + i;
        const float h = swiglu_pair(acc[i], c.g, c.g2);
        if (c.lane < 32 && cl < 8 && m < a.M && f < a.F) a.y[static_cast<size_t>(m) * a.F + f] = static_cast<_Float16>(h);
      }
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      return;
    }
    const int n = (c.t0 + ti * c.step) * kTileCols + cl;
    const bool col_ok = c.lane < 32 && n < a.N;
    unsigned long long key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = grp * 4 + i;
      const bool ok = col_ok && m < a.M;
      const float v = c.g * acc[i];
      if (ok && a.y) a.y[static_cast<size_t>(m) * a.N + n] = static_cast<_Float16>(v);
      key[i] = ok ? argmax_key(v, n) : 0ull;
    }
    if (EPI == kEpiArgmax) {
      wave_max_keys<4, 16>(key);
      if (c.lane < 32 && cl == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) c.best[grp * 4 + i] = key[i] > c.best[grp * 4 + i] ? key[i] : c.best[grp * 4 + i];
      }
    }
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

template <int KU, int EPI>
__global__ __launch_bounds__(kMaxWaves * 64) void nvfp4_stream(Nvfp4Args a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int RS = KU * kUnitK + 8;
  _Float16* xs = reinterpret_cast<_Float16*>(lds);
  unsigned long long* best = reinterpret_cast<unsigned long long*>(lds + ((a.M * RS * 2 + 15) & ~15));  // [nw][8]

  StreamCtx c;
  c.a = &a;
  c.lane = lane;
  c.step = gridDim.x * nw;
  c.t0 = blockIdx.x + gridDim.x * wave;
  c.ntiles = c.t0 < a.nt ? (a.nt - 1 - c.t0) / c.step + 1 : 0;
  c.span_stride = static_cast<size_t>(a.nt) * kUnitBytes;
  c.tile_stride = static_cast<size_t>(c.step) * kUnitBytes;
  c.g = *a.gptr;
  c.g2 = EPI == kEpiSwiglu ? *a.g2ptr : 0.0f;
  c.xbase = xs + min(lane & 15, a.M - 1) * RS + (lane >> 4) * 32;
  c.best = best + wave * kMaxRows;
  c.spare = a.units + lane * 16;

  stage_x_all(a, xs, RS, wave, nw, lane);
  if (EPI == kEpiArgmax && lane < kMaxRows) c.best[lane] = 0ull;
  Unit A, B;
  const uint8_t* base = a.units + static_cast<size_t>(c.t0) * kUnitBytes + lane * 16;
  load_unit(A, c.ntiles > 0 ? base : c.spare);
  // x is in LDS once every wavefront's copies are done; the first unit keeps arriving.
  lds_copy_barrier<kChunksPerUnit + 1>(true);

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  // Tiles in pairs, so that every unit's buffer is fixed at compile time
  // (the wavefront's unit u lives in A when u is even): with odd KU the
  // second tile of a pair starts in B.  An odd last tile follows the loop.
  int ti = 0;
  for (; ti + 1 < c.ntiles; ti += 2) {
    stream_units<KU, 0, 0, EPI>(c, A, B, ti, base, acc);
    base += c.tile_stride;
    stream_units<KU, 0, KU % 2, EPI>(c, A, B, ti + 1, base, acc);
    base += c.tile_stride;
  }
  if (ti < c.ntiles) stream_units<KU, 0, 0, EPI>(c, A, B, ti, base, acc);

  if (EPI == kEpiArgmax) {
    // Largest key per row over the workgroup's wavefronts.
    __syncthreads();
    if (threadIdx.x < static_cast<unsigned>(a.M)) {
      unsigned long long k = 0ull;
      for (int w = 0; w < nw; ++w) k = best[w * kMaxRows + threadIdx.x] > k ? best[w * kMaxRows + threadIdx.x] : k;
      a.cand[static_cast<size_t>(blockIdx.x) * a.M + threadIdx.x] = k;
    }
  }
}

template <typename Kern>
hipError_t launch(Kern k, dim3 grid, int nw, size_t lds, const Nvfp4Args& a, hipStream_t stream) {
  hipLaunchKernelGGL(k, grid, dim3(nw * 64), lds, stream, a);
  return hipGetLastError();
}

template <int CT, int EPI>
hipError_t launch_valu(dim3 grid, int nw, const Nvfp4Args& a, hipStream_t stream) {
  return a.M == 2 ? launch(nvfp4_valu<CT, EPI, 2>, grid, nw, 0, a, stream)
                  : launch(nvfp4_valu<CT, EPI, 1>, grid, nw, 0, a, stream);
}

}  // namespace

size_t nvfp4_stream_lds_bytes(int M, int K, int nw) {
  const int ku = (K + kUnitK - 1) / kUnitK;
  return ((static_cast<size_t>(M) * (ku * kUnitK + 8) * 2 + 15) & ~static_cast<size_t>(15)) +
         static_cast<size_t>(nw) * kMaxRows * 8;
}

int nvfp4_stream_groups(const LaunchCfg& c, int N) {
  const int nt = (N + kTileCols - 1) / kTileCols;
  const int per_wg = c.nw;
  const int want = (nt + per_wg - 1) / per_wg;
  return std::max(1, std::min({want, device_cu_count() * c.ct, kMaxStreamGroups}));
}

size_t nvfp4_mfma_lds_bytes(int M, int S, int nw) {
  return ((static_cast<size_t>(M) * (S * kUnitK + 8) * 2 + 15) & ~static_cast<size_t>(15)) +
         static_cast<size_t>(nw) * 32 * sizeof(f32x4);
}

// (engine, ct, nw, ksplit): nw = ct * S wavefronts cover S K spans of ct
// tiles; the ksplit workgroups of a tile group must cover all K spans and
// each must get at least one.
bool nvfp4_cfg_supported(const LaunchCfg& c, int M, int K, bool argmax) {
  if (c.engine == 2)  // streaming: ct = workgroups per CU (1 or 2), no K split, K <= 9 spans
    return (c.ct == 1 || c.ct == 2) && c.nw >= 1 && c.nw <= kMaxWaves && c.ksplit == 1 &&
           (K + kUnitK - 1) / kUnitK <= kMaxStreamSpans && nvfp4_stream_lds_bytes(M, K, c.nw) * c.ct <= kMaxLdsBytes;
  const bool ct_ok = c.ct == 1 || c.ct == 2 || c.ct == 4 || c.ct == 8;
  if (!ct_ok || c.nw < 1 || c.nw > kMaxWaves || c.nw % c.ct != 0 || c.ksplit < 1) return false;
  const int ku = (K + kUnitK - 1) / kUnitK;
  const int S = c.nw / c.ct;
  if (static_cast<long>(c.ksplit) * S < ku || static_cast<long>(c.ksplit - 1) * S >= ku) return false;
  if (c.engine == 0) return M <= 2;
  if (c.engine == 3) return M <= 2 && !argmax && c.ct == 1 && c.ksplit == 1;  // whole K: nw = ku
  if (c.engine != 1) return false;
  return nvfp4_mfma_lds_bytes(M, S, c.nw) <= kMaxLdsBytes;
}

#define SKINNY_NVFP4_DISPATCH(CT)                                                                       \
  if (cfg.ct == CT) {                                                                                   \
    if (cfg.engine == 0)                                                                                \
      return epi == kEpiSwiglu                      ? launch_valu<CT, kEpiSwiglu>(grid, cfg.nw, a, stream) \
             : epi == kEpiArgmax && cfg.ksplit == 1 ? launch_valu<CT, kEpiArgmax>(grid, cfg.nw, a, stream) \
                                                    : launch_valu<CT, kEpiPlain>(grid, cfg.nw, a, stream);  \
    if (epi == kEpiArgmax && cfg.ksplit == 1)                                                           \
      return launch(nvfp4_mfma<CT, kEpiArgmax>, grid, cfg.nw, lds, a, stream);                          \
    if (epi == kEpiSwiglu && cfg.ksplit == 1)                                                           \
      return launch(nvfp4_mfma<CT, kEpiSwiglu>, grid, cfg.nw, lds, a, stream);                          \
    return launch(nvfp4_mfma<CT, kEpiPlain>, grid, cfg.nw, lds, a, stream);                             \
  }

namespace {

hipError_t launch_gemm(const Nvfp4Args& a, const LaunchCfg& cfg, int epi, hipStream_t stream) {
  if (cfg.engine == 2) {
    const dim3 grid(nvfp4_stream_groups(cfg, a.N));
    const size_t lds = nvfp4_stream_lds_bytes(a.M, a.K, cfg.nw);
    switch (a.ku) {
#define SKINNY_STREAM_KU(KU) \
  case KU:                   \
    return epi == kEpiArgmax   ? launch(nvfp4_stream<KU, kEpiArgmax>, grid, cfg.nw, lds, a, stream) \
           : epi == kEpiSwiglu ? launch(nvfp4_stream<KU, kEpiSwiglu>, grid, cfg.nw, lds, a, stream) \
                               : launch(nvfp4_stream<KU, kEpiPlain>, grid, cfg.nw, lds, a, stream);
      SKINNY_STREAM_KU(1)
      SKINNY_STREAM_KU(2)
      SKINNY_STREAM_KU(3)
      SKINNY_STREAM_KU(4)
      SKINNY_STREAM_KU(5)
      SKINNY_STREAM_KU(6)
      SKINNY_STREAM_KU(7)
      SKINNY_STREAM_KU(8)
      SKINNY_STREAM_KU(9)
#undef SKINNY_STREAM_KU
      default:
        return hipErrorInvalidValue;
    }
  }
  const dim3 grid = a.xsplit ? dim3(8 * ((a.ntg + 7) / 8) * cfg.ksplit) : dim3((a.nt + cfg.ct - 1) / cfg.ct, cfg.ksplit);
  const size_t lds = nvfp4_mfma_lds_bytes(a.M, a.S, cfg.nw);
  SKINNY_NVFP4_DISPATCH(1)
  SKINNY_NVFP4_DISPATCH(2)
  SKINNY_NVFP4_DISPATCH(4)
  SKINNY_NVFP4_DISPATCH(8)
  return hipErrorInvalidValue;
}

}  // namespace

#undef SKINNY_NVFP4_DISPATCH

hipError_t launch_nvfp4(const uint8_t* blob, const uint16_t* x, uint16_t* y, int M, int K, int N,
                        const LaunchCfg& cfg, int32_t* idx, void* workspace, hipStream_t stream, int swiglu_F,
                        const int32_t* drafts, int32_t* verify) {
  const Geometry geo = nvfp4_geometry(K, N);
  const bool argmax = idx != nullptr;
  const WorkspaceLayout wl = nvfp4_workspace_layout(cfg, M, K, N, argmax);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  Nvfp4Args a;
  a.units = blob + kHeaderBytes;
  a.gptr = reinterpret_cast<const float*>(blob + kGOffset);
  a.x = reinterpret_cast<const _Float16*>(x);
  a.y = reinterpret_cast<_Float16*>(y);
  a.M = M;
  a.K = K;
  a.N = N;
  a.ku = geo.ku;
  a.nt = geo.nt;
  a.ksplit = cfg.ksplit;
  a.S = cfg.nw / cfg.ct;
  a.part = wl.part_bytes ? reinterpret_cast<float*>(ws + wl.part_off) : nullptr;
  a.cand = argmax ? reinterpret_cast<unsigned long long*>(ws + wl.keys_off) : nullptr;
  a.g2ptr = reinterpret_cast<const float*>(blob + kG2Offset);
  a.F = swiglu_F;
  const bool swiglu = swiglu_F > 0;
  a.xsplit = nvfp4_uses_xsplit(cfg, N, !argmax && !swiglu) ? 1 : 0;
  a.ntg = (geo.nt + cfg.ct - 1) / cfg.ct;
  a.sync = reinterpret_cast<unsigned*>(ws + wl.sync_off);
  a.bal_small = a.bal_r = a.bal_whole = a.bal_s = a.bal_ks = 0;
  if (cfg.engine == 3) {  // plain epilogue only (checked by the callers)
    BalancedLayout b;
    LaunchCfg c0 = cfg;
    c0.engine = 0;
    if (!nvfp4_balanced_layout(geo.nt, geo.ku, device_cu_count(), &b))
      return launch_gemm(a, c0, kEpiPlain, stream);  // whole tiles spread evenly already
    a.bal_whole = b.whole;
    a.bal_r = geo.nt - b.whole;
    a.bal_s = b.spans;
    a.bal_ks = b.splits;
    a.bal_small = 8 * ((a.bal_r + 7) / 8) * b.splits;
    a.part = reinterpret_cast<float*>(ws + wl.part_off);
    return launch_valu<1, kEpiPlain>(dim3(a.bal_small + b.whole), cfg.nw, a, stream);
  }
  hipError_t e = launch_gemm(a, cfg, argmax ? kEpiArgmax : swiglu ? kEpiSwiglu : kEpiPlain, stream);
  if (e != hipSuccess || a.xsplit) return e;
  int groups = cfg.engine == 2 ? nvfp4_stream_groups(cfg, N) : (geo.nt + cfg.ct - 1) / cfg.ct;
  if (cfg.ksplit > 1 && swiglu)
    return launch_finalize_swiglu(a.part, cfg.ksplit, M, N, swiglu_F, a.gptr, a.g2ptr, y, stream);
  if (cfg.ksplit > 1) {
    e = launch_finalize(a.part, cfg.ksplit, M, N, a.gptr, y, a.cand, stream);
    if (e != hipSuccess) return e;
    groups = finalize_groups(N);
  }
  return argmax ? launch_argmax_reduce(a.cand, groups, M, idx, stream, drafts, verify) : hipSuccess;
}

}  // namespace skinny
