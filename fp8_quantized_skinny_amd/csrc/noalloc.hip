// nvfp4_gemm for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc): the
// same kernels, with the scratch a K split needs taken from a file-scope
// device array instead of a caller's workspace.
//
// The array is part of the library's code object, so each GPU the library
// runs on holds its own copy from the first call on that GPU until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host that name is only a stand-in): the first call on each device looks up
// the device address with hipGetSymbolAddress, with that device current, and
// every call on the device passes that address.  Calls that overlap in time
// on one GPU share the array and race.  The array's first
// SKINNY_WORKSPACE_SYNC_BYTES hold the K split's arrival counters, which must
// be zero when a call starts and are zero again when it ends; the first call
// on each device clears them with a small kernel on its stream (static
// storage starts zeroed as well).  The kernels write every other scratch byte
// they read within a call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"
#include "skinny.h"

namespace {

constexpr size_t kScratchBytes = SKINNY_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch`, per device (null until looked up)

static_assert(SKINNY_WORKSPACE_SYNC_BYTES % 4 == 0 && SKINNY_WORKSPACE_SYNC_BYTES <= kScratchBytes, "sync region");

__global__ void clear_words(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// This device's address of `scratch`, looked up (and its counters cleared on
// `stream`) on the first call on the device.
int scratch_address(void** out, hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SKINNY_EHIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SKINNY_EHIP;
    constexpr int kWords = SKINNY_WORKSPACE_SYNC_BYTES / 4;
    hipLaunchKernelGGL(clear_words, dim3((kWords + 255) / 256), dim3(256), 0, stream, static_cast<uint32_t*>(p),
                       kWords);
    if (hipGetLastError() != hipSuccess) return SKINNY_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SKINNY_OK;
}

}  // namespace

extern "C" int nvfp4_gemm_noalloc(const void* w_packed, const uint16_t* x, uint16_t* y, int M, int K, int N,
                                  hipStream_t stream) {
  // Every host-side check before any HIP call, as for nvfp4_gemm.
  size_t need = 0;
  int s = skinny::nvfp4_gemm_host_checks(w_packed, x, y, M, K, N, &need);
  if (s) return s;
  if (need > kScratchBytes) return SKINNY_ESIZE;
  void* ws = nullptr;
  s = scratch_address(&ws, stream);
  if (s) return s;
  return nvfp4_gemm(w_packed, x, y, M, K, N, ws, kScratchBytes, stream);
}
