// In-kernel K-split reduction shared by the GEMM kernels.
//
// When the K spans of a tile group do not fit one workgroup, ksplit
// workgroups share the group and each stores its fp32 partial sums.  The
// grid is one-dimensional and workgroup b takes tile group
// 8 * (b / (8 * ksplit)) + b % 8 and split (b % (8 * ksplit)) / 8, so all
// splits of a group are congruent mod 8: the hardware deals the workgroups
// of a kernel to the 8 XCDs in turn, so they run on one XCD and share its L2.
// Plain stores, a workgroup-scope atomic (executed in that L2) and loads that
// skip the CU's L1 then see each other without any cache write-back.
#ifndef SKINNY_XSPLIT_CUH_
#define SKINNY_XSPLIT_CUH_

#include <hip/hip_runtime.h>

#include "internal.h"

namespace skinny {

__device__ __forceinline__ void xsplit_place(int b, int ksplit, int& group, int& split) {
  const int per = 8 * ksplit;
  group = (b / per) * 8 + (b & 7);
  split = (b % per) >> 3;
}

// The end of a split workgroup: its block of tile group `group` (M rows of
// COLS fp32 sums from column 16 * tile0 on, at part + (group * ks + split)
// * M * COLS, already stored) is published with an arrival count on the
// group's counter (sync, 128 bytes per group, zero at rest).  The workgroup
// that arrives last adds the ks blocks in split order, scales by *g (SCALED:
// the NVFP4 global scale; FP8 sums are already scaled) and writes the columns
// below N of y [M][N] as fp16; it then sets the counter back to zero for the
// next call.  Nothing waits on another workgroup, and the order of the sums
// does not depend on which split arrives last.  Every thread of the
// workgroup must call this.
template <int COLS, bool SCALED>
__device__ void xsplit_add(unsigned* sync, const float* part, _Float16* y, const float* g, int M, int N, int tile0,
                           int group, int ks) {
  __shared__ int last;
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have reached L2
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* cnt = sync + static_cast<size_t>(group) * (kSyncLineBytes / 4);
    const unsigned old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    last = old == static_cast<unsigned>(ks - 1);
    if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __syncthreads();
  if (!last) return;
  const size_t block = static_cast<size_t>(M) * COLS;
  const float* base = part + static_cast<size_t>(group) * ks * block;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(base), 0, static_cast<int>(ks * block * sizeof(float)), 0x00020000);
  const float scale = SCALED ? *g : 1.0f;
  for (int o = threadIdx.x; o < static_cast<int>(block); o += blockDim.x) {
    const int m = o / COLS, n = tile0 * kTileCols + o % COLS;
    // Sixteen splits per batch, all loads issued before the first add; a
    // split past the last reads 0 (outside the buffer's range) and adds 0.
    constexpr int kBatch = 16;
    float sum = 0.0f;
    for (int k0 = 0; k0 < ks; k0 += kBatch) {
      float v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i)  // sc0: past this CU's L1, from the XCD's L2
        v[i] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rsrc, static_cast<int>(((k0 + i) * block + o) * 4), 0, 1));
#pragma unroll
      for (int i = 0; i < kBatch; ++i) sum += v[i];
    }
    if (n < N) y[static_cast<size_t>(m) * N + n] = static_cast<_Float16>(scale * sum);
  }
}

}  // namespace skinny

#endif
