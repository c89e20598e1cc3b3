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
//   [0, 256)               header (Nvfp4Header, zero padded)
//   [256, 256 + CB)        code tiles: NT x KC tiles of 1024 bytes, tile-major
//                          (tile t = columns 16t..16t+15, chunk kc = K 128kc..)
//   [256 + CB, +SB)        scale groups: NT x SG groups of 1024 bytes
//
// Inside a code tile, lane l = 16*grp + c (grp 0..3, c 0..15) of a wavefront
// owns bytes [16l, 16l+16): the 32 E2M1 codes of column 16t+c at
// K = 128kc + 32grp + i (i = 0..31), two per byte, low nibble first.  One
// 16-byte load per lane therefore reads the whole tile with one contiguous
// 1 KiB wavefront access.
//
// Inside a scale group (8 chunks, 1024 K), lane l owns bytes [16l, 16l+16):
// byte 2j + h is the E4M3 scale of the same lane's codes in chunk 8sg + j,
// half h (K = 128(8sg+j) + 32grp + 16h .. +16).  One 16-byte load per lane
// gives the scales of eight chunks.
//
// K is padded to a multiple of 128 and N to a multiple of 16 with zero codes
// and zero scales; padded weights are exactly 0.
// ---------------------------------------------------------------------------
constexpr uint32_t kBlobMagic = 0x344E4B53u;  // "SKN4" little-endian
constexpr uint32_t kBlobVersion = 1;
constexpr size_t kHeaderBytes = 256;
constexpr int kTileCols = 16;
constexpr int kChunkK = 128;
constexpr int kChunksPerScaleGroup = 8;
constexpr size_t kTileBytes = 1024;

struct Nvfp4Header {
  uint32_t magic;
  uint32_t version;
  uint32_t K, N;
  uint32_t kc;  // K chunks of 128 (ceil)
  uint32_t nt;  // column tiles of 16 (ceil)
  uint32_t sg;  // scale groups per tile (ceil(kc / 8))
  float g;      // per-tensor scale; byte offset 28
  uint64_t codes_off, codes_bytes, scales_off, scales_bytes;
};
static_assert(sizeof(Nvfp4Header) <= kHeaderBytes, "header too large");
constexpr size_t kGOffset = 28;

struct Geometry {
  int kc, nt, sg;
  size_t codes_bytes, scales_bytes, total_bytes;
};
Geometry nvfp4_geometry(int K, int N);

// Launch parameters picked by the host for one call.
struct LaunchCfg {
  int engine;  // 0 = VALU dot2 (M = 1 only), 1 = MFMA 16x16x32 f16
  int ct;      // column tiles (of 16) per workgroup
  int nw;      // wavefronts per workgroup (they split K)
};

// Kernel launchers (defined in the .hip files).  Arguments are validated.
hipError_t launch_nvfp4(const uint8_t* blob, const uint16_t* x, uint16_t* y,
                        int M, int K, int N, const LaunchCfg& cfg,
                        int32_t* idx, void* workspace, hipStream_t stream);
hipError_t launch_fp8(const uint8_t* w, const float* scales, const uint16_t* x,
                      uint16_t* y, int M, int K, int N, const LaunchCfg& cfg,
                      hipStream_t stream);
bool nvfp4_cfg_supported(const LaunchCfg& cfg, int M, bool argmax);
bool fp8_cfg_supported(const LaunchCfg& cfg, int M);

// lm_head workspace: kMaxRows x u64 per-row argmax keys, then one u32 arrival counter.
constexpr int kMaxRows = 8;
constexpr size_t kArgmaxWorkspaceBytes = 256;

}  // namespace skinny

#endif
