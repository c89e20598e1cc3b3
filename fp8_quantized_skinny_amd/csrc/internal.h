// Internal declarations shared by the host code and the kernel translation units.
#ifndef SKINNY_INTERNAL_H
#define SKINNY_INTERNAL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace skinny {

// ---------------------------------------------------------------------------
// Packed NVFP4 blob.
//
//   [0, 256)     header (Nvfp4Header, zero padded)
//   [256, ...)   units: G x NT units of 9216 bytes, span-major: unit (t, g)
//                at 256 + (g * NT + t) * 9216
//
// A unit covers one column tile t (columns 16t .. 16t+15) and one K span g
// (K 1024g .. 1024g+1023): eight 1 KiB code chunks followed by one 1 KiB
// scale vector, so a wavefront streams a unit with nine contiguous 1 KiB
// accesses of one 16-byte load per lane.
//
// Code chunk j (K 1024g + 128j ..): lane l = 16*grp + c (grp 0..3, c 0..15)
// owns bytes [16l, 16l+16): the 32 E2M1 codes of column 16t+c at
// K = 1024g + 128j + 32grp + i (i = 0..31), two per byte, low nibble first.
// Scale vector: lane l owns bytes [16l, 16l+16); byte 2j + h is the E4M3
// scale of that lane's codes in chunk j, half h (16 K each).
//
// Span-major order puts the units of one K span of consecutive tiles next to
// each other, so wavefronts that walk their tiles span by span in step (the
// streaming engine) read one contiguous region at a time; the one-unit-per-
// wavefront kernels read consecutive tiles of every span, which is as dense.
//
// K is padded to a multiple of 1024 and N to a multiple of 16 with zero codes
// and zero scales, so padded weights are exactly 0.
//
// A SwiGLU pair blob (kind 1) holds two weights of F columns each, gate and
// up, interleaved by eight: tile t has gate columns 8t .. 8t+7 as its columns
// 0..7 and up columns 8t .. 8t+7 as its columns 8..15 (zero past F), so
// N = 16 * ceil(F / 8) and every gate column meets its up column in the same
// wavefront, eight lanes apart.  g is the gate's per-tensor scale, g2 the
// up's.  A plain blob (kind 0) has g2 = g.
// ---------------------------------------------------------------------------
constexpr uint32_t kBlobMagic = 0x344E4B53u;  // "SKN4" little-endian
constexpr uint32_t kBlobVersion = 4;
constexpr size_t kHeaderBytes = 256;
constexpr int kTileCols = 16;
constexpr int kChunkK = 128;
constexpr int kChunksPerUnit = 8;
constexpr int kUnitK = kChunkK * kChunksPerUnit;  // 1024
constexpr size_t kChunkBytes = 1024;
constexpr size_t kUnitBytes = kChunkBytes * (kChunksPerUnit + 1);  // 9216

struct Nvfp4Header {
  uint32_t magic;
  uint32_t version;
  uint32_t K, N;
  uint32_t ku;  // K spans of 1024 (ceil)
  uint32_t nt;  // column tiles of 16 (ceil)
  uint32_t unit_bytes;
  float g;      // per-tensor scale; byte offset 28
  uint64_t units_off, units_bytes;
  float g2;       // up scale of a SwiGLU pair (= g otherwise); byte offset 48
  uint32_t kind;  // 0 plain, 1 SwiGLU pair
  uint32_t F;     // SwiGLU pair: columns of each of gate and up (0 otherwise)
};
static_assert(sizeof(Nvfp4Header) <= kHeaderBytes, "header too large");
constexpr size_t kGOffset = 28;
constexpr size_t kG2Offset = 48;
constexpr uint32_t kKindPlain = 0, kKindSwiglu = 1;
// Columns of the packed blob of a SwiGLU pair of F columns each.
constexpr int swiglu_packed_cols(int F) { return 16 * ((F + 7) / 8); }

struct Geometry {
  int ku, nt;
  size_t units_bytes, total_bytes;
};
Geometry nvfp4_geometry(int K, int N);

// ---------------------------------------------------------------------------
// Packed FP8 blob (fp8_pack), optional: the canonical [N][K] codes work too.
//
//   [0, 256)     header (Fp8Header, zero padded)
//   [256, ...)   units: KU x NT units of 8192 bytes, span-major: unit (t, u)
//                at 256 + (u * NT + t) * 8192
//
// Unit (t, u) covers columns 16t .. 16t+15 and K 512u .. 512u+511: eight
// 1 KiB pieces q = 2j + h; in piece q, lane l = 16*grp + c owns bytes
// [16l, 16l+16): the E4M3 codes of column 16t + 8(c%2) + c/2 at K = 512u +
// 128j + 32grp + 16h + i (i = 0..15).  K is padded to a multiple of 512 and N to a
// multiple of 16 with zero codes.
// ---------------------------------------------------------------------------
constexpr uint32_t kFp8BlobMagic = 0x38464B53u;  // "SKF8" little-endian
constexpr uint32_t kFp8BlobVersion = 2;
constexpr int kFp8PackK = 512;
constexpr size_t kFp8UnitBytes = 8192;
struct Fp8Header {
  uint32_t magic, version, K, N, ku, nt, unit_bytes, reserved;
  uint64_t units_off, units_bytes;
};
static_assert(sizeof(Fp8Header) <= kHeaderBytes, "header too large");

// Launch parameters picked by the host for one call.
struct LaunchCfg {
  int engine;  // 0 = VALU dot2 (NVFP4 M <= 2, FP8 M <= 4), 1 = MFMA 16x16x32 f16, 2 = streaming MFMA,
               // 3 = the NVFP4 VALU GEMV with whole K per tile, balanced over the CUs (see BalancedLayout)
  int ct;      // engines 0, 1: column tiles (of 16) per workgroup; engine 2: workgroups per CU
  int nw;      // wavefronts per workgroup (1..16); engines 0, 1: ct * K spans per workgroup
  int ksplit;  // workgroups that split K (1 = no split; engine 2 never splits)
};
constexpr int kMaxWaves = 16;
constexpr size_t kMaxLdsBytes = 160 * 1024;

// Workspace of one call (offsets in bytes, 256-aligned).  Every workspace
// that is not empty starts with the same kSyncBytes: arrival counters of the
// in-kernel K-split reduction, one per tile group and 128 bytes apart (a
// cache line each).  They must be zero before a workspace's first use, and
// every call leaves them zero; no other data is ever placed there, so one
// workspace can serve calls of every kind.  After them: argmax candidate
// keys (lm_head) and the fp32 partial sums of a K split.  Those are written
// by the call before they are read, so they need no initialisation.
constexpr int kMaxSyncGroups = 1024;
constexpr size_t kSyncLineBytes = 128;
constexpr size_t kSyncBytes = kMaxSyncGroups * kSyncLineBytes;
struct WorkspaceLayout {
  size_t sync_off, sync_bytes, keys_off, keys_bytes, part_off, part_bytes, total;
};
WorkspaceLayout nvfp4_workspace_layout(const LaunchCfg& cfg, int M, int K, int N, bool argmax);
// The balanced VALU GEMV (engine 3).  The one-tile-whole-K GEMV puts nt
// workgroups of ku wavefronts on the CUs; when nt is not a multiple of the
// CU count, some CUs get one whole tile more than the others (ku units of
// 9 KiB), and the call lasts as long as those CUs take.  The balanced layout
// keeps `whole` = the largest multiple of the CU count of tiles as whole-K
// workgroups and cuts each of the other nt - whole tiles into `splits`
// workgroups of `spans` K spans, at most one per CU, added inside the kernel
// (as an in-kernel K split).  False when nothing is to gain or the layout does
// not fit: nt a multiple of the CU count, more than four whole tiles per CU
// (the grid would no longer be resident at once), or more split workgroups
// than CUs (or than kMaxSyncGroups).
struct BalancedLayout {
  int whole, spans, splits;
};
bool nvfp4_balanced_layout(int nt, int ku, int cus, BalancedLayout* out);

// True when an NVFP4 call with this choice adds its K split inside the GEMM
// kernel (the VALU or MFMA engine, plain epilogue, at most kMaxSyncGroups tile
// groups).
bool nvfp4_uses_xsplit(const LaunchCfg& cfg, int N, bool plain_epilogue);
// The same for the FP8 GEMM (MFMA engine only).
bool fp8_uses_xsplit(const LaunchCfg& cfg, int N);
WorkspaceLayout fp8_workspace_layout(const LaunchCfg& cfg, int M, int K, int N);

// Kernel launchers (defined in the .hip files).  Arguments are validated.
// swiglu_F > 0: the blob is a SwiGLU pair of swiglu_F columns each (N is its
// packed column count) and y is h[M][swiglu_F] = silu(gate) * up.
hipError_t launch_nvfp4(const uint8_t* blob, const uint16_t* x, uint16_t* y,
                        int M, int K, int N, const LaunchCfg& cfg,
                        int32_t* idx, void* workspace, hipStream_t stream, int swiglu_F = 0,
                        const int32_t* drafts = nullptr, int32_t* verify = nullptr);
// packed: w is an fp8_pack blob (header included) instead of canonical codes.
hipError_t launch_fp8(const uint8_t* w, const float* scales, const uint16_t* x,
                      uint16_t* y, int M, int K, int N, const LaunchCfg& cfg,
                      void* workspace, hipStream_t stream, bool packed = false);
bool nvfp4_cfg_supported(const LaunchCfg& cfg, int M, int K, bool argmax);
bool fp8_cfg_supported(const LaunchCfg& cfg, int M, int K);
size_t nvfp4_mfma_lds_bytes(int M, int S, int nw);

// Streaming engine: LDS bytes per workgroup (all of x plus the argmax
// scratch) and the grid size, at most kMaxStreamGroups workgroups.
constexpr int kMaxStreamGroups = 1024;
constexpr int kMaxStreamSpans = 9;
size_t nvfp4_stream_lds_bytes(int M, int K, int nw);
int nvfp4_stream_groups(const LaunchCfg& cfg, int N);

// Read-bandwidth probes (probe.hip).  launch_read_probe reads bytes / 9216
// blocks of 9216 bytes, one per single-wavefront workgroup; the patterns of
// launch_read_probe_pattern are those of skinny_read_probe_pattern (skinny.h),
// with arguments already checked.
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_read_probe_pattern(const void* buf, size_t bytes, int pattern, int a, int b, uint32_t* sink,
                                     hipStream_t stream);

// Compute units of the current device (256 if it cannot be queried).
int device_cu_count();

// Second pass of a K split (reduce.hip): adds part[split][m][n] over the
// splits in order, scales by *gptr (1 if null) and writes fp16 y (if non-null)
// and, if cand is non-null, one argmax key per row for each of the
// finalize_groups(N) column blocks.  launch_argmax_reduce turns `groups`
// candidate keys per row into idx.
int finalize_groups(int N);
hipError_t launch_finalize(const float* part, int ksplit, int M, int N, const float* gptr, uint16_t* y,
                           unsigned long long* cand, hipStream_t stream);
// With result non-null it also verifies the speculative round whose drafts
// rows 1 .. M-1 carry (drafts[M-1], greedy acceptance): result[0] = accepted
// drafts L, result[1 .. L+1] = committed tokens, result[L+2 .. M] = -1.
hipError_t launch_argmax_reduce(const unsigned long long* cand, int groups, int M, int32_t* idx,
                                hipStream_t stream, const int32_t* drafts = nullptr, int32_t* result = nullptr);
// Second pass of a K split of a SwiGLU pair: h[m][f] = silu(g * gate) * (g2 *
// up), both sums taken over the splits in order from part[split][m][n] of
// the packed columns (n = 16 * (f / 8) + f % 8 and n + 8).
hipError_t launch_finalize_swiglu(const float* part, int ksplit, int M, int N, int F, const float* gptr,
                                  const float* g2ptr, uint16_t* h, hipStream_t stream);

// Largest row count (the target token plus seven drafts).
constexpr int kMaxRows = 8;

// Every host-side check of nvfp4_gemm except the workspace's, and the
// workspace bytes its default kernel choice needs (host.cpp).
int nvfp4_gemm_host_checks(const void* w_packed, const uint16_t* x, const uint16_t* y, int M, int K, int N,
                           size_t* workspace_need);

}  // namespace skinny

#endif
