// Read-bandwidth probes: the measured HBM read ceiling that the GEMM kernels
// are compared with (the author's post rates its kernels against a measured
// read-only ceiling of its cards, section "What I actually built").
//
// Every probe reads whole blocks of 1 KiB per wavefront instruction (one
// 16-byte non-temporal load per lane, the weight loads of the GEMM kernels)
// and folds the data into one value so that no load can be dropped.  Nothing
// is written unless the folded value hits a 2^-64 chance, so a probe moves the
// bytes it reads and nothing else.  Patterns:
//   * blocks: every wavefront reads one block of B KiB with B loads issued
//     together, W wavefronts per workgroup, block order = wavefront order.
//     B = 9, W = 1 is the default probe: the fastest pattern measured at the
//     decode sizes (50 MB on MI355X: 8.26 us against 8.43 us for W = 4 and
//     8.67 us for the GEMV's own shape below).
//   * tiles: the NVFP4 GEMV's shape: 9 KiB units in span-major order, one
//     workgroup per 16-column tile with one wavefront per K span.
//   * persistent: G workgroups of W wavefronts walk the blocks (wavefront w
//     reads blocks w, w + all wavefronts, ...) with two, three or four 9 KiB
//     blocks in flight each.
#include <hip/hip_runtime.h>

#include "common.cuh"
#include "internal.h"

namespace skinny {
namespace {

__device__ __forceinline__ void fold_and_sink(u32x4 h, uint32_t* sink) {
  const uint64_t lo = static_cast<uint64_t>(h.x) | (static_cast<uint64_t>(h.y) << 32);
  const uint64_t hi = static_cast<uint64_t>(h.z) | (static_cast<uint64_t>(h.w) << 32);
  if ((lo ^ hi) == 0x9E3779B97F4A7C15ull) sink[0] = h.x;
}

template <int B>
__global__ __launch_bounds__(1024) void read_blocks(const uint8_t* buf, size_t blocks, uint32_t* sink) {
  const size_t wave = (static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  if (wave >= blocks) return;
  const uint8_t* p = buf + wave * (B * 1024) + (threadIdx.x & 63) * 16;
  u32x4 v[B];
#pragma unroll
  for (int j = 0; j < B; ++j) v[j] = load16(p + j * 1024);
  u32x4 h = v[0];
#pragma unroll
  for (int j = 1; j < B; ++j) h ^= v[j];
  fold_and_sink(h, sink);
}

// Tile t of nt, span s = wavefront index: unit (s, t) at (s * nt + t) * 9216.
__global__ __launch_bounds__(1024) void read_tiles(const uint8_t* buf, int nt, uint32_t* sink) {
  const uint8_t* p = buf + (static_cast<size_t>(threadIdx.x >> 6) * nt + blockIdx.x) * kUnitBytes +
                     (threadIdx.x & 63) * 16;
  u32x4 v[9];
#pragma unroll
  for (int j = 0; j < 9; ++j) v[j] = load16(p + j * 1024);
  u32x4 h = v[0];
#pragma unroll
  for (int j = 1; j < 9; ++j) h ^= v[j];
  fold_and_sink(h, sink);
}

// IN blocks in flight per wavefront: wavefront w of W reads blocks w, w + W,
// ...; each block's loads go out IN blocks ahead of its use.  Past the end a
// wavefront re-reads its first block (never used), so every address stays
// inside the blocks.
template <int IN>
__global__ __launch_bounds__(1024) void read_persistent(const uint8_t* buf, size_t blocks, uint32_t* sink) {
  const size_t W = (static_cast<size_t>(gridDim.x) * blockDim.x) >> 6;
  const size_t w = (static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  if (w >= blocks) return;
  const uint8_t* base = buf + (threadIdx.x & 63) * 16;
  u32x4 v[IN][9], h = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < IN; ++i) {
    const size_t b = w + i * W < blocks ? w + i * W : w;
#pragma unroll
    for (int j = 0; j < 9; ++j) v[i][j] = load16(base + b * kUnitBytes + j * 1024);
  }
  for (size_t b0 = w; b0 < blocks; b0 += IN * W) {
#pragma unroll
    for (int i = 0; i < IN; ++i) {
#pragma unroll
      for (int j = 0; j < 9; ++j) h ^= v[i][j];
      const size_t nb = b0 + (i + IN) * W < blocks ? b0 + (i + IN) * W : w;
#pragma unroll
      for (int j = 0; j < 9; ++j) v[i][j] = load16(base + nb * kUnitBytes + j * 1024);
    }
  }
  fold_and_sink(h, sink);
}

template <int B>
void launch_blocks(const uint8_t* buf, size_t bytes, int waves, uint32_t* sink, hipStream_t stream) {
  const size_t blocks = bytes / (B * 1024);
  const size_t groups = (blocks + waves - 1) / waves;
  hipLaunchKernelGGL(read_blocks<B>, dim3(static_cast<unsigned>(groups)), dim3(64 * waves), 0, stream, buf, blocks,
                     sink);
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  launch_blocks<9>(static_cast<const uint8_t*>(buf), bytes, 1, sink, stream);
  return hipGetLastError();
}

hipError_t launch_read_probe_pattern(const void* buf, size_t bytes, int pattern, int a, int b, uint32_t* sink,
                                     hipStream_t stream) {
  const uint8_t* p = static_cast<const uint8_t*>(buf);
  switch (pattern) {
    case 0: launch_blocks<9>(p, bytes, a, sink, stream); break;
    case 1: launch_blocks<4>(p, bytes, a, sink, stream); break;
    case 2: launch_blocks<18>(p, bytes, a, sink, stream); break;
    case 3: {
      const int nt = static_cast<int>(bytes / (static_cast<size_t>(a) * kUnitBytes));
      hipLaunchKernelGGL(read_tiles, dim3(nt), dim3(64 * a), 0, stream, p, nt, sink);
      break;
    }
    case 4:
      hipLaunchKernelGGL(read_persistent<2>, dim3(a), dim3(64 * b), 0, stream, p, bytes / kUnitBytes, sink);
      break;
    case 5:
      hipLaunchKernelGGL(read_persistent<3>, dim3(a), dim3(64 * b), 0, stream, p, bytes / kUnitBytes, sink);
      break;
    case 6:
      hipLaunchKernelGGL(read_persistent<4>, dim3(a), dim3(64 * b), 0, stream, p, bytes / kUnitBytes, sink);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace skinny
