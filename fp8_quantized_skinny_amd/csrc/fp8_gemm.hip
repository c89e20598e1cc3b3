// FP8 (E4M3FN) weight-only skinny GEMM for gfx950 (MI355X).
//
// y[m][n] = sum_kb S[n/128][kb] * sum_{k in block kb} x[m][k] * e4m3(c[n][k])
//
// The published FP8 regions of a checkpoint are served as FP8 instead of
// being converted to NVFP4 ("NVFP4 on Volta!" author's post, section
// "v1.0 -> v1.1"); the codes are read in their canonical [N][K] order.
//
// A 16-column tile times one 128-K chunk lies inside one 128 x 128 scale
// block, so each chunk is contracted into a fresh fp32 partial (E4M3 -> fp16
// is exact) that is then added to the accumulator times the block scale in
// fp32.  Two engines contract a chunk:
//   * MFMA (M = 1..8): v_mfma_f32_16x16x32_f16 with x rows, padded to 16,
//     from an LDS copy as operand A (the default from M = 3);
//   * VALU (M <= 4): v_dot2c_f32_f16 with each row's x pairs read from
//     global memory and broadcast across 16 lanes by DPP row_newbcast, as in
//     the NVFP4 GEMV; no LDS copy of x (the default at M <= 2).
//
// Work split follows the NVFP4 kernels: a unit is one 16-column tile x 512 K
// (four chunks, 8 KiB of codes); every wavefront loads one unit at once and
// contracts it; a workgroup is CT tiles x S units along K (nw = CT * S), with
// a K split over workgroups when K has more units (partial sums stored with
// plain stores and added in split order by the reduction kernel).  The MFMA
// engine copies x into LDS once per workgroup with direct-to-LDS loads.
// Both engines contract, per chunk j, lane (grp, c)'s two 16-byte pieces
// K = 128j + 32grp + 16h .. +16 (h = 0, 1) of column 8(c % 2) + c / 2 of the
// tile.  Canonical codes are not loaded in that layout (it would read every
// 128-byte line as two halves from two instructions): each load reads eight
// whole lines, and selects with one-lane DPP shifts merge a chunk's two loads
// into the pieces.  Pieces past K or columns past N read a clamped valid address and
// are zeroed.
//
// The packed variant reads the same pieces from a blob of fp8_pack: 8 KiB
// units (one tile x 512 K) in span-major order, in which piece 2j + h of a
// unit holds each lane's 16 bytes next to each other, so every load
// instruction is one contiguous KiB, as for NVFP4 (padding is zero codes).
// Canonical and packed codes give the same registers, hence the same bits.
#include <hip/hip_runtime.h>

#include "common.cuh"
#include "internal.h"
#include "xsplit.cuh"

namespace skinny {
namespace {

constexpr int kFp8UnitChunks = 4;
constexpr int kFp8UnitK = kFp8UnitChunks * kChunkK;  // 512
static_assert(kFp8UnitK == kFp8PackK && 2 * kFp8UnitChunks * 1024 == kFp8UnitBytes, "FP8 packed unit");

struct Fp8Args {
  const uint8_t* w;  // canonical codes [N][K], or the packed units (fp8_pack) of the blob
  const float* scales;
  const _Float16* x;
  _Float16* y;
  int M, K, N;
  int nt, kb, ku;  // column tiles, scale blocks along K, units along K
  int ksplit, S;
  float* part;  // fp32 partial sums (ksplit > 1): [ksplit][M][N], or xsplit one block [M][ct * 16] per (tile group, split)
  int xsplit;      // 1: the K split is added inside the kernel on each tile group's XCD (MFMA engine)
  int ntg;         // tile groups (xsplit)
  unsigned* sync;  // xsplit: one arrival counter per tile group, 128 bytes apart (zero at rest)
};

// This wavefront's unit and its workgroup's geometry (wave-uniform values).
// An xsplit grid is one-dimensional: tile group and split from xsplit_place
// (xsplit.cuh), so that the splits of a group run on one XCD; otherwise
// blockIdx.x is the tile group and blockIdx.y the split.
struct Fp8Plan {
  int lane, wave, nw, S, tile0, s0, sw, t, s;
  int group, split;
  bool active;
  __device__ Fp8Plan(const Fp8Args& a, int ct) {
    lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    nw = blockDim.x >> 6;
    S = a.S;
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
};

__device__ __forceinline__ int fp8_xs_stride(int S) { return S * kFp8UnitK + 8; }

__device__ void fp8_stage_x(const Fp8Args& a, const Fp8Plan& P, _Float16* xs) {
  const int RS = fp8_xs_stride(P.S);
  const int kbase = P.s0 * kFp8UnitK;
  const int kvalid = a.K - kbase;
  if (kvalid < P.S * kFp8UnitK) zero_x_tail(xs, a.M, RS, kvalid, P.S * kFp8UnitK);
  const int nblocks = a.M * P.S;  // 1 KiB blocks = 512 halves = one unit of K
  for (int b = P.wave; b < nblocks; b += P.nw) {
    const int m = b / P.S, blk = b % P.S;
    const int col = blk * 512 + P.lane * 8;
    if (col < kvalid)
      __builtin_amdgcn_global_load_lds(a.x + static_cast<size_t>(m) * a.K + kbase + col, xs + m * RS + blk * 512,
                                       16, 0, 0);
  }
}

// Column of the tile held by lane c of a 16-lane row in the compute layout:
// even lanes hold columns 0..7, odd lanes 8..15, so that both canonical
// loads of a chunk merge into it with one-lane shifts (below).
__device__ __forceinline__ int fp8_lane_col(int c) { return 8 * (c & 1) + (c >> 1); }

// Canonical codes, whole lines per load: load i of a unit (tile t, K range
// 512u ..) gives lane 16q + i' the 16 bytes K = 512u + 128(i % 4) + 16p .. +16
// with p = 2q + i' % 2 of column 16t + 8(i / 4) + i' / 2: each lane pair reads
// 32 consecutive bytes and each instruction eight whole 128-byte lines.
// (Reading the tile in the compute layout instead, sixteen half lines per
// instruction and two instructions per line, ran at about three quarters of
// the whole-line read rate.)  Loads go out in the order 0, 4, 1, 5, ... so
// that chunk j (loads j and 4 + j) is complete after its first 2(j + 1)
// loads.  Pieces past K read the row start instead (K % 16 == 0: a piece is
// all in or all out); their x is zero.
__device__ __forceinline__ void fp8_load_lines(u32x4 (&v)[2 * kFp8UnitChunks], const Fp8Args& a, int tt, int u,
                                               int lane) {
  const int c8 = (lane & 15) >> 1, p = 2 * (lane >> 4) + (lane & 1);
#pragma unroll
  for (int j = 0; j < kFp8UnitChunks; ++j) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int n = min(tt * kTileCols + 8 * g + c8, a.N - 1);
      const int k = u * kFp8UnitK + kChunkK * j + 16 * p;
      v[4 * g + j] = load16(a.w + static_cast<size_t>(n) * a.K + (k < a.K ? k : 0));
    }
  }
}

// Both pieces of a chunk in the compute (and packed) layout from its two
// whole-line loads lo (columns 0..7) and hi (columns 8..15).  In row grp,
// lanes 2c and 2c + 1 of lo hold pieces 2grp and 2grp + 1 of column c, and
// the same lanes of hi those of column 8 + c.  w0 (piece 2grp) keeps lo's
// even lanes and takes hi's even lanes one lane up; w1 (piece 2grp + 1) keeps
// hi's odd lanes and takes lo's odd lanes one lane down.  The shifts (DPP
// row_shr:1 / row_shl:1) run in every lane, since a DPP read of a lane that
// a branch switched off gives 0; only the selects depend on the lane.  (The
// same merge as v_cndmask_b32 with a DPP operand in inline asm, half the
// instructions, measured no faster at M = 4 and 0.1 us slower at M = 1.)
constexpr int kRowShl1 = 0x101, kRowShr1 = 0x111;
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_shift(uint32_t from) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(from), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ void fp8_line_merge(const u32x4& lo, const u32x4& hi, u32x4& w0, u32x4& w1) {
  const bool odd = (threadIdx.x & 1) != 0;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t up = dpp_shift<kRowShr1>(hi[d]), down = dpp_shift<kRowShl1>(lo[d]);
    w0[d] = odd ? up : lo[d];
    w1[d] = odd ? hi[d] : down;
  }
}

// Per-wavefront LDS slot of the MFMA engine: the wavefront's partial tile
// sums (32 lanes x 16 bytes).
constexpr int kWaveSlotBytes = 32 * 16;

// A fragments of chunk j: lane (row c, grp) holds, for MFMA i = 2h + s,
// x[min(c, M-1)][512u + 128j + 32grp + 16h + 8s .. +8], i.e. the 32 halves
// from 128j + 32grp in order.  Rows c >= M only feed output rows that are
// never stored, so they repeat row M-1.
__device__ __forceinline__ void fp8_read_x(f16x8 (&xa)[4], const _Float16* xrow, int j) {
  const _Float16* p = xrow + j * kChunkK;
#pragma unroll
  for (int i = 0; i < 4; ++i) xa[i] = *reinterpret_cast<const f16x8*>(p + 8 * i);
}

// Chunk J and on; canonical codes are merged into the compute layout just
// before their chunk, so a chunk waits for its own two loads only.
template <int J, bool PACKED>
__device__ __forceinline__ void fp8_steps(u32x4 (&w)[kFp8UnitChunks][2], const u32x4 (&v)[2 * kFp8UnitChunks],
                                          const float (&sc)[kFp8UnitChunks], f16x8 (&x0)[4], f16x8 (&x1)[4],
                                          f32x4& acc, const _Float16* xrow) {
  if constexpr (J < kFp8UnitChunks) {
    f16x8 (&cur)[4] = (J & 1) ? x1 : x0;
    f16x8 (&nxt)[4] = (J & 1) ? x0 : x1;
    if constexpr (J + 1 < kFp8UnitChunks) fp8_read_x(nxt, xrow, J + 1);
    if constexpr (!PACKED) fp8_line_merge(v[J], v[4 + J], w[J][0], w[J][1]);
    f32x4 p = f32x4{0.f, 0.f, 0.f, 0.f};
    p = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur[0], e4m3x8(w[J][0].x, w[J][0].y), p, 0, 0, 0);
    p = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur[1], e4m3x8(w[J][0].z, w[J][0].w), p, 0, 0, 0);
    p = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur[2], e4m3x8(w[J][1].x, w[J][1].y), p, 0, 0, 0);
    p = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur[3], e4m3x8(w[J][1].z, w[J][1].w), p, 0, 0, 0);
    acc += sc[J] * p;
    fp8_steps<J + 1, PACKED>(w, v, sc, x0, x1, acc, xrow);
  }
}

template <int CT, bool PACKED>
__global__ __launch_bounds__(kMaxWaves * 64) __attribute__((amdgpu_waves_per_eu(8))) void fp8_mfma(Fp8Args a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const Fp8Plan P(a, CT);
  if (a.xsplit && P.group >= a.ntg) return;  // grid rounding to whole groups of 8 (uniform)
  _Float16* xs = reinterpret_cast<_Float16*>(lds);
  unsigned char* slots = lds + ((a.M * fp8_xs_stride(P.S) * 2 + 15) & ~15);  // [nw][kWaveSlotBytes]
  unsigned char* slot = slots + P.wave * kWaveSlotBytes;

  fp8_stage_x(a, P, xs);
  const int cl = P.lane & 15, grp = P.lane >> 4;
  const int tt = min(P.tile0 + P.t, a.nt - 1);
  u32x4 w[kFp8UnitChunks][2];
  u32x4 v[2 * kFp8UnitChunks];  // canonical codes as loaded (whole lines)
  float sc[kFp8UnitChunks];
  // Every wavefront loads, an idle one (past the last K span) clamped
  // addresses it never uses: with no load under a branch the compiler waits
  // for each chunk alone instead of the whole unit.
  {
    const int u = P.s0 + P.s;
    // Scales of the tile's 128-column block for this unit's four K blocks,
    // loaded before the weights so that reading them waits for nothing else.
    // A K block past the end contributes nothing (its x is zero in LDS), so
    // the last block's scale stands in for it.
    const float* srow = a.scales + static_cast<size_t>(min(tt * kTileCols, a.N - 1) / 128) * a.kb;
#pragma unroll
    for (int j = 0; j < kFp8UnitChunks; ++j) sc[j] = srow[min(u * kFp8UnitChunks + j, a.kb - 1)];
    __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the codes'
    // Codes: pieces past K load from the row start instead (x is zero there,
    // so they add exact zeros); no select on loaded data, which would make
    // every load wait for the previous one.
    if (PACKED) {
      // Unit (tt, u) of the span-major blob; an idle wavefront's u (past the
      // last unit) is clamped to a real unit it never uses.
      const uint8_t* up =
          a.w + (static_cast<size_t>(min(u, a.ku - 1)) * a.nt + tt) * kFp8UnitBytes + P.lane * 16;
#pragma unroll
      for (int j = 0; j < kFp8UnitChunks; ++j) {
#pragma unroll
        for (int h = 0; h < 2; ++h) w[j][h] = load16(up + (2 * j + h) * 1024);
      }
    } else {
      fp8_load_lines(v, a, tt, min(u, a.ku - 1), P.lane);
    }
  }
  // x is in LDS once every wavefront's copies are done; the weights keep arriving.
  lds_copy_barrier<2 * kFp8UnitChunks>(true);

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  if (P.active) {
    const _Float16* xrow = xs + min(cl, a.M - 1) * fp8_xs_stride(P.S) + P.s * kFp8UnitK + grp * 32;
    f16x8 x0[4], x1[4];
    fp8_read_x(x0, xrow, 0);
    fp8_steps<0, PACKED>(w, v, sc, x0, x1, acc, xrow);
  }
  if (P.lane < 32) reinterpret_cast<f32x4*>(slot)[P.lane] = acc;
  __syncthreads();

  const bool fin = P.wave < CT && P.tile0 + P.wave < a.nt && P.lane < 32;
  const int col = P.wave * kTileCols + fp8_lane_col(cl);  // column within the tile group
  const int n = P.tile0 * kTileCols + col;
  if (fin && n < a.N) {
    f32x4 tot = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < P.sw; ++s)
      tot += reinterpret_cast<const f32x4*>(slots + (P.wave * P.S + s) * kWaveSlotBytes)[P.lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = grp * 4 + i;
      if (m >= a.M) continue;
      if (a.xsplit)  // this split's block of the group; the last split adds them
        a.part[((static_cast<size_t>(P.group) * a.ksplit + P.split) * a.M + m) * (CT * kTileCols) + col] = tot[i];
      else if (a.ksplit > 1)
        a.part[(static_cast<size_t>(P.split) * a.M + m) * a.N + n] = tot[i];
      else
        a.y[static_cast<size_t>(m) * a.N + n] = static_cast<_Float16>(tot[i]);
    }
  }
  if (a.xsplit) xsplit_add<CT * kTileCols, false>(a.sync, a.part, a.y, nullptr, a.M, a.N, P.tile0, P.group, a.ksplit);
}

// ---------------------------------------------------------------------------
// VALU engine, M = 1.
// ---------------------------------------------------------------------------
// Half a chunk of one lane (16 E4M3 codes in four dwords, 16 consecutive K)
// against the x pairs of MR rows, each broadcast from lanes 0..7 (lo) or
// 8..15 (hi) of the lane's 16-lane row, accumulated into p[m].  As in the
// NVFP4 GEMV, one asm block widens the codes once (v_cvt_scalef32_pk_f16_fp8,
// exact, two per instruction, low half of each dword first) and runs MR x 8
// v_dot2c_f32_f16 whose x operand is read through DPP row_newbcast, with its
// own wait states: two before the first DPP read and two after the last
// v_dot2c.  Keeping the widening inside the block stops the compiler from
// widening a whole unit ahead of use.
__device__ __forceinline__ void fp8_half_dot1_lo(float (&p)[1], const uint32_t (&xv)[1], const u32x4& w) {
  uint32_t t0, t1, t2, t3, t4, t5, t6, t7;
  asm("v_cvt_scalef32_pk_f16_fp8 %1, %9, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %2, %9, 1.0 op_sel:[1,0,0]\n"
      "v_cvt_scalef32_pk_f16_fp8 %3, %10, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %4, %10, 1.0 op_sel:[1,0,0]\n"
      "v_cvt_scalef32_pk_f16_fp8 %5, %11, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %6, %11, 1.0 op_sel:[1,0,0]\n"
      "v_cvt_scalef32_pk_f16_fp8 %7, %12, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %8, %12, 1.0 op_sel:[1,0,0]\n"
      "s_nop 1\n"
      "v_dot2c_f32_f16_dpp %0, %13, %1 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %13, %2 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %13, %3 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %13, %4 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %13, %5 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %13, %6 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %13, %7 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %13, %8 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      : "+v"(p[0]), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(t5), "=&v"(t6), "=&v"(t7)
      : "v"(w.x), "v"(w.y), "v"(w.z), "v"(w.w), "v"(xv[0]));
}
__device__ __forceinline__ void fp8_half_dot1_hi(float (&p)[1], const uint32_t (&xv)[1], const u32x4& w) {
  uint32_t t0, t1, t2, t3, t4, t5, t6, t7;
  asm("v_cvt_scalef32_pk_f16_fp8 %1, %9, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %2, %9, 1.0 op_sel:[1,0,0]\n"
      "v_cvt_scalef32_pk_f16_fp8 %3, %10, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %4, %10, 1.0 op_sel:[1,0,0]\n"
      "v_cvt_scalef32_pk_f16_fp8 %5, %11, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %6, %11, 1.0 op_sel:[1,0,0]\n"
      "v_cvt_scalef32_pk_f16_fp8 %7, %12, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %8, %12, 1.0 op_sel:[1,0,0]\n"
      "s_nop 1\n"
      "v_dot2c_f32_f16_dpp %0, %13, %1 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %13, %2 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %13, %3 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %13, %4 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %13, %5 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %13, %6 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %13, %7 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %13, %8 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      : "+v"(p[0]), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(t5), "=&v"(t6), "=&v"(t7)
      : "v"(w.x), "v"(w.y), "v"(w.z), "v"(w.w), "v"(xv[0]));
}
__device__ __forceinline__ void fp8_half_dot2_lo(float (&p)[2], const uint32_t (&xv)[2], const u32x4& w) {
  uint32_t t0, t1, t2, t3, t4, t5, t6, t7;
  asm("v_cvt_scalef32_pk_f16_fp8 %2, %10, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %3, %10, 1.0 op_sel:[1,0,0]\n"
      "v_cvt_scalef32_pk_f16_fp8 %4, %11, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %5, %11, 1.0 op_sel:[1,0,0]\n"
      "v_cvt_scalef32_pk_f16_fp8 %6, %12, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %7, %12, 1.0 op_sel:[1,0,0]\n"
      "v_cvt_scalef32_pk_f16_fp8 %8, %13, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %9, %13, 1.0 op_sel:[1,0,0]\n"
      "s_nop 1\n"
      "v_dot2c_f32_f16_dpp %0, %14, %2 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %14, %3 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %14, %4 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %14, %5 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %14, %6 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %14, %7 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %14, %8 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %14, %9 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %15, %2 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %15, %3 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %15, %4 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %15, %5 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %15, %6 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %15, %7 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %15, %8 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %15, %9 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      : "+v"(p[0]), "+v"(p[1]), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(t5), "=&v"(t6), "=&v"(t7)
      : "v"(w.x), "v"(w.y), "v"(w.z), "v"(w.w), "v"(xv[0]), "v"(xv[1]));
}
__device__ __forceinline__ void fp8_half_dot2_hi(float (&p)[2], const uint32_t (&xv)[2], const u32x4& w) {
  uint32_t t0, t1, t2, t3, t4, t5, t6, t7;
  asm("v_cvt_scalef32_pk_f16_fp8 %2, %10, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %3, %10, 1.0 op_sel:[1,0,0]\n"
      "v_cvt_scalef32_pk_f16_fp8 %4, %11, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %5, %11, 1.0 op_sel:[1,0,0]\n"
      "v_cvt_scalef32_pk_f16_fp8 %6, %12, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %7, %12, 1.0 op_sel:[1,0,0]\n"
      "v_cvt_scalef32_pk_f16_fp8 %8, %13, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %9, %13, 1.0 op_sel:[1,0,0]\n"
      "s_nop 1\n"
      "v_dot2c_f32_f16_dpp %0, %14, %2 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %14, %3 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %14, %4 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %14, %5 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %14, %6 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %14, %7 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %14, %8 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %14, %9 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %15, %2 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %15, %3 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %15, %4 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %15, %5 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %15, %6 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %15, %7 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %15, %8 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %15, %9 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      : "+v"(p[0]), "+v"(p[1]), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(t5), "=&v"(t6), "=&v"(t7)
      : "v"(w.x), "v"(w.y), "v"(w.z), "v"(w.w), "v"(xv[0]), "v"(xv[1]));
}
__device__ __forceinline__ void fp8_half_dot4_lo(float (&p)[4], const uint32_t (&xv)[4], const u32x4& w) {
  uint32_t t0, t1, t2, t3, t4, t5, t6, t7;
  asm("v_cvt_scalef32_pk_f16_fp8 %4, %12, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %5, %12, 1.0 op_sel:[1,0,0]\n"
      "v_cvt_scalef32_pk_f16_fp8 %6, %13, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %7, %13, 1.0 op_sel:[1,0,0]\n"
      "v_cvt_scalef32_pk_f16_fp8 %8, %14, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %9, %14, 1.0 op_sel:[1,0,0]\n"
      "v_cvt_scalef32_pk_f16_fp8 %10, %15, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %11, %15, 1.0 op_sel:[1,0,0]\n"
      "s_nop 1\n"
      "v_dot2c_f32_f16_dpp %0, %16, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %16, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %16, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %16, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %16, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %16, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %16, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %16, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %17, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %17, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %17, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %17, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %17, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %17, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %17, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %17, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %2, %18, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %2, %18, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %2, %18, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %2, %18, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %2, %18, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %2, %18, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %2, %18, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %2, %18, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %3, %19, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %3, %19, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %3, %19, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %3, %19, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %3, %19, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %3, %19, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %3, %19, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %3, %19, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(t5), "=&v"(t6), "=&v"(t7)
      : "v"(w.x), "v"(w.y), "v"(w.z), "v"(w.w), "v"(xv[0]), "v"(xv[1]), "v"(xv[2]), "v"(xv[3]));
}
__device__ __forceinline__ void fp8_half_dot4_hi(float (&p)[4], const uint32_t (&xv)[4], const u32x4& w) {
  uint32_t t0, t1, t2, t3, t4, t5, t6, t7;
  asm("v_cvt_scalef32_pk_f16_fp8 %4, %12, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %5, %12, 1.0 op_sel:[1,0,0]\n"
      "v_cvt_scalef32_pk_f16_fp8 %6, %13, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %7, %13, 1.0 op_sel:[1,0,0]\n"
      "v_cvt_scalef32_pk_f16_fp8 %8, %14, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %9, %14, 1.0 op_sel:[1,0,0]\n"
      "v_cvt_scalef32_pk_f16_fp8 %10, %15, 1.0\n"
      "v_cvt_scalef32_pk_f16_fp8 %11, %15, 1.0 op_sel:[1,0,0]\n"
      "s_nop 1\n"
      "v_dot2c_f32_f16_dpp %0, %16, %4 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %16, %5 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %16, %6 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %16, %7 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %16, %8 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %16, %9 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %16, %10 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %0, %16, %11 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %17, %4 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %17, %5 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %17, %6 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %17, %7 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %17, %8 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %17, %9 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %17, %10 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %1, %17, %11 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %2, %18, %4 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %2, %18, %5 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %2, %18, %6 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %2, %18, %7 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %2, %18, %8 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %2, %18, %9 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %2, %18, %10 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %2, %18, %11 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %3, %19, %4 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %3, %19, %5 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %3, %19, %6 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %3, %19, %7 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %3, %19, %8 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %3, %19, %9 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %3, %19, %10 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_dot2c_f32_f16_dpp %3, %19, %11 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(t5), "=&v"(t6), "=&v"(t7)
      : "v"(w.x), "v"(w.y), "v"(w.z), "v"(w.w), "v"(xv[0]), "v"(xv[1]), "v"(xv[2]), "v"(xv[3]));
}

template <int MR>
__device__ __forceinline__ void fp8_half_dot(float (&p)[MR], const uint32_t (&xv)[MR], const u32x4& w, bool hi) {
  if constexpr (MR == 1) {
    if (hi) fp8_half_dot1_hi(p, xv, w); else fp8_half_dot1_lo(p, xv, w);
  } else if constexpr (MR == 2) {
    if (hi) fp8_half_dot2_hi(p, xv, w); else fp8_half_dot2_lo(p, xv, w);
  } else {
    if (hi) fp8_half_dot4_hi(p, xv, w); else fp8_half_dot4_lo(p, xv, w);
  }
}

// One unit per wavefront, as in the MFMA engine; lane 16r + q holds, for each
// chunk j and row m, the x pair the lanes of its row r need at step q % 8 of
// half q / 8: x[m][512u + 128j + 32r + 16(q/8) + 2(q%8) ..+2], which is
// x[m][512u + 128j + 32r + 2q ..+2].  Each chunk's
// sum over its 128 K is multiplied by its block scale in fp32.  x needs no
// LDS copy.  MR rows per instance (M = 3 runs as MR = 4: its fourth row
// reads row 2 again and is never stored).
template <int CT, bool PACKED, int MR>
__global__ __launch_bounds__(kMaxWaves * 64) void fp8_valu(Fp8Args a) {
  __shared__ float red[kMaxWaves][MR][16];
  const Fp8Plan P(a, CT);
  const int q = P.lane & 15, r = P.lane >> 4;
  const int tt = min(P.tile0 + P.t, a.nt - 1);
  const int u = min(P.s0 + P.s, a.ku - 1);  // an idle wavefront loads a real unit it never uses
  // Block scales first (wave-uniform); a K block past K gets scale 0 (its
  // x pairs are zero or its codes are, below).
  float sc[kFp8UnitChunks];
  {
    const float* srow = a.scales + static_cast<size_t>(min(tt * kTileCols, a.N - 1) / 128) * a.kb;
#pragma unroll
    for (int j = 0; j < kFp8UnitChunks; ++j) {
      const int kb = u * kFp8UnitChunks + j;
      sc[j] = kb < a.kb ? srow[kb] : 0.0f;
    }
  }
  u32x4 w[kFp8UnitChunks][2];
  u32x4 v[2 * kFp8UnitChunks];  // canonical codes as loaded (whole lines)
  uint32_t xv[kFp8UnitChunks][MR];
  const int kx = u * kFp8UnitK + 32 * r + 2 * q;
  const _Float16* xr[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) xr[m] = a.x + static_cast<size_t>(min(m, a.M - 1)) * a.K;
  // A pair past K reads the last pair of its row (index in [0, K-2], even,
  // so the 4-byte load stays in the row); below, it is replaced by zero
  // where that matters.
  if (PACKED) {
    const uint8_t* up = a.w + (static_cast<size_t>(u) * a.nt + tt) * kFp8UnitBytes + P.lane * 16;
#pragma unroll
    for (int j = 0; j < kFp8UnitChunks; ++j) {
      w[j][0] = load16(up + (2 * j) * 1024);
      w[j][1] = load16(up + (2 * j + 1) * 1024);
#pragma unroll
      for (int m = 0; m < MR; ++m)
        xv[j][m] = *reinterpret_cast<const uint32_t*>(xr[m] + min(kx + j * kChunkK, a.K - 2));
    }
  } else {
    fp8_load_lines(v, a, tt, u, P.lane);
#pragma unroll
    for (int j = 0; j < kFp8UnitChunks; ++j) {
#pragma unroll
      for (int m = 0; m < MR; ++m)
        xv[j][m] = *reinterpret_cast<const uint32_t*>(xr[m] + min(kx + j * kChunkK, a.K - 2));
    }
  }
  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.0f;
  const bool straddles = (u + 1) * kFp8UnitK > a.K;
  if (P.active) {
#pragma unroll
    for (int j = 0; j < kFp8UnitChunks; ++j) {
      // Canonical codes past K are real codes of the row start: their x pairs
      // must be zero; selected here, where these x words are needed anyway.
      // Packed codes past K are zero, but a clamped pair holding inf or NaN
      // would still give 0 * x = NaN: a unit that straddles K (wave-uniform)
      // selects too, which no full unit does.
      const bool in = (!PACKED || straddles) ? kx + j * kChunkK < a.K : true;
      if (!PACKED) fp8_line_merge(v[j], v[4 + j], w[j][0], w[j][1]);
      uint32_t x[MR];
      float p[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        x[m] = in ? xv[j][m] : 0u;
        p[m] = 0.0f;
      }
      fp8_half_dot<MR>(p, x, w[j][0], false);
      fp8_half_dot<MR>(p, x, w[j][1], true);
#pragma unroll
      for (int m = 0; m < MR; ++m) acc[m] = __builtin_fmaf(p[m], sc[j], acc[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const float v = sum_over_rows(acc[m]);
    if (P.lane < 16) red[P.wave][m][fp8_lane_col(P.lane)] = v;
  }
  __syncthreads();

  // Wavefront t < CT finishes local tile t: its K units in order, then the
  // output rows or, with a K split, this split's partial sums.
  if (P.wave < CT && P.lane < 16 && P.tile0 + P.wave < a.nt) {
    const int n = (P.tile0 + P.wave) * kTileCols + P.lane;
    if (n < a.N) {
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        if (m >= a.M) break;
        float tot = 0.0f;
        for (int s = 0; s < P.sw; ++s) tot += red[P.wave * P.S + s][m][P.lane];
        if (a.ksplit > 1)
          a.part[(static_cast<size_t>(P.split) * a.M + m) * a.N + n] = tot;
        else
          a.y[static_cast<size_t>(m) * a.N + n] = static_cast<_Float16>(tot);
      }
    }
  }
}

size_t fp8_lds_bytes(int M, int S, int nw) {
  return ((static_cast<size_t>(M) * (S * kFp8UnitK + 8) * 2 + 15) & ~static_cast<size_t>(15)) +
         static_cast<size_t>(nw) * kWaveSlotBytes;
}

}  // namespace

// (engine, ct, nw, ksplit): engine 1 = MFMA (M <= 8), engine 0 = VALU (M <= 4).
bool fp8_cfg_supported(const LaunchCfg& c, int M, int K) {
  if (!(c.engine == 1 || (c.engine == 0 && M <= 4))) return false;
  if (!(c.ct == 1 || c.ct == 2 || c.ct == 4 || c.ct == 8)) return false;
  if (c.nw < 1 || c.nw > kMaxWaves || c.nw % c.ct != 0 || c.ksplit < 1) return false;
  const int ku = (K + kFp8UnitK - 1) / kFp8UnitK;
  const int S = c.nw / c.ct;
  if (static_cast<long>(c.ksplit) * S < ku || static_cast<long>(c.ksplit - 1) * S >= ku) return false;
  return c.engine == 0 || fp8_lds_bytes(M, S, c.nw) <= kMaxLdsBytes;
}

// The VALU engine's instance for M rows (M = 3 runs as four rows).
template <int CT, bool PACKED>
void launch_fp8_valu_rows(const Fp8Args& a, dim3 grid, dim3 blk, hipStream_t stream) {
  if (a.M == 1)
    hipLaunchKernelGGL((fp8_valu<CT, PACKED, 1>), grid, blk, 0, stream, a);
  else if (a.M == 2)
    hipLaunchKernelGGL((fp8_valu<CT, PACKED, 2>), grid, blk, 0, stream, a);
  else
    hipLaunchKernelGGL((fp8_valu<CT, PACKED, 4>), grid, blk, 0, stream, a);
}

template <int CT>
hipError_t launch_fp8_valu(const Fp8Args& a, dim3 grid, int nw, bool packed, hipStream_t stream) {
  if (packed)
    launch_fp8_valu_rows<CT, true>(a, grid, dim3(nw * 64), stream);
  else
    launch_fp8_valu_rows<CT, false>(a, grid, dim3(nw * 64), stream);
  return hipGetLastError();
}

#define SKINNY_FP8_DISPATCH(CT)                                                           \
  if (cfg.ct == CT && cfg.engine == 0) {                                                  \
    e = launch_fp8_valu<CT>(a, grid, cfg.nw, packed, stream);                             \
  } else if (cfg.ct == CT) {                                                              \
    if (packed)                                                                           \
      hipLaunchKernelGGL((fp8_mfma<CT, true>), grid, dim3(cfg.nw * 64), lds, stream, a);  \
    else                                                                                  \
      hipLaunchKernelGGL((fp8_mfma<CT, false>), grid, dim3(cfg.nw * 64), lds, stream, a); \
    e = hipGetLastError();                                                                \
  }

hipError_t launch_fp8(const uint8_t* w, const float* scales, const uint16_t* x, uint16_t* y, int M,
                      int K, int N, const LaunchCfg& cfg, void* workspace, hipStream_t stream, bool packed) {
  const WorkspaceLayout wl = fp8_workspace_layout(cfg, M, K, N);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  Fp8Args a;
  a.w = packed ? w + kHeaderBytes : w;
  a.scales = scales;
  a.x = reinterpret_cast<const _Float16*>(x);
  a.y = reinterpret_cast<_Float16*>(y);
  a.M = M;
  a.K = K;
  a.N = N;
  a.nt = (N + kTileCols - 1) / kTileCols;
  a.kb = (K + 127) / 128;
  a.ku = (K + kFp8UnitK - 1) / kFp8UnitK;
  a.ksplit = cfg.ksplit;
  a.S = cfg.nw / cfg.ct;
  a.part = wl.part_bytes ? reinterpret_cast<float*>(ws + wl.part_off) : nullptr;
  a.ntg = (a.nt + cfg.ct - 1) / cfg.ct;
  a.xsplit = fp8_uses_xsplit(cfg, N) ? 1 : 0;
  a.sync = wl.sync_bytes ? reinterpret_cast<unsigned*>(ws) : nullptr;
  const dim3 grid = a.xsplit ? dim3(8 * ((a.ntg + 7) / 8) * cfg.ksplit) : dim3(a.ntg, cfg.ksplit);
  const size_t lds = fp8_lds_bytes(M, a.S, cfg.nw);
  hipError_t e = hipErrorInvalidValue;
  SKINNY_FP8_DISPATCH(1)
  SKINNY_FP8_DISPATCH(2)
  SKINNY_FP8_DISPATCH(4)
  SKINNY_FP8_DISPATCH(8)
  if (e != hipSuccess || cfg.ksplit == 1 || a.xsplit) return e;
  return launch_finalize(a.part, cfg.ksplit, M, N, nullptr, y, nullptr, stream);
}

}  // namespace skinny
