// Read-bandwidth probe: the measured HBM read ceiling that the GEMM kernels
// are compared with (the author's post rates its kernels against a measured
// read-only ceiling of its cards, section "What I actually built").
//
// Every wavefront reads one 9 KiB block with nine 16-byte loads per lane,
// issued together, exactly like one NVFP4 unit of the GEMM kernels, and
// folds the data into one value so that no load can be dropped.  Nothing is
// written unless the folded value hits a 2^-64 chance, so the probe moves
// the block bytes and nothing else.
#include <hip/hip_runtime.h>

#include "common.cuh"
#include "internal.h"

namespace skinny {
namespace {

constexpr int kProbeBlock = 9216;

__global__ __launch_bounds__(256) void read_probe(const uint8_t* buf, size_t blocks, uint32_t* sink) {
  const size_t wave = (static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  if (wave >= blocks) return;
  const uint8_t* p = buf + wave * kProbeBlock + (threadIdx.x & 63) * 16;
  u32x4 v[9];
#pragma unroll
  for (int j = 0; j < 9; ++j) v[j] = load16(p + j * 1024);
  u32x4 h = v[0];
#pragma unroll
  for (int j = 1; j < 9; ++j) h ^= v[j];
  const uint64_t lo = static_cast<uint64_t>(h.x) | (static_cast<uint64_t>(h.y) << 32);
  const uint64_t hi = static_cast<uint64_t>(h.z) | (static_cast<uint64_t>(h.w) << 32);
  if ((lo ^ hi) == 0x9E3779B97F4A7C15ull) sink[0] = h.x;
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const size_t blocks = bytes / kProbeBlock;
  const size_t groups = (blocks + 3) / 4;
  hipLaunchKernelGGL(read_probe, dim3(static_cast<unsigned>(groups)), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(buf), blocks, sink);
  return hipGetLastError();
}

}  // namespace skinny
