// Second-pass kernels of the skinny GEMM: the K-split reduction (plain, or
// the SwiGLU of a gate/up pair) and the lm_head argmax over workgroup
// candidates.
//
// When K is split over several workgroups, each one stores its fp32 partial
// sums with plain stores, part[split][m][n], and exits.  finalize_splits then
// adds the splits in split order (so results never depend on timing),
// applies the per-tensor scale and rounds to fp16.  (Plain NVFP4 calls on the
// VALU and MFMA engines add their splits inside the GEMM kernel instead; these
// kernels serve FP8, SwiGLU pairs and the lm_head.)  For the lm_head it also
// takes, per row and per block of 256 columns, the largest logit as one
// ordered 64-bit key (logit bits above the inverted column, so a larger key is
// a larger logit or the same logit at a lower column); argmax_reduce then
// takes the largest key per row over all blocks.  The argmax is taken on the
// fp32 logits before fp16 rounding (author's post, section "This is a server,
// not a GEMM screenshot": the drafter proposes greedy, local-argmax tokens).
#include <hip/hip_runtime.h>

#include "common.cuh"
#include "internal.h"

namespace skinny {
namespace {

constexpr int kFinalizeThreads = 256;

// Block (x, m): columns 256x .. 256x+255 of row m, one column per thread.
// Each thread adds its column's partials in split order.  One column per
// thread gives four times the wavefronts of four columns per thread (16-byte
// loads); on MI355X that took a nine-way split of the down projection at
// M = 8 from 15.2 to 14.9 us per call (before such splits moved into the
// GEMM kernel).
template <bool ARGMAX>
__global__ __launch_bounds__(kFinalizeThreads) void finalize_splits(const float* part, int ksplit, int M, int N,
                                                                    const float* gptr, _Float16* y,
                                                                    unsigned long long* cand) {
  __shared__ unsigned long long best[kFinalizeThreads / 64];
  const int n = blockIdx.x * kFinalizeThreads + threadIdx.x;
  const int m = blockIdx.y;
  unsigned long long key = 0ull;
  if (n < N) {
    const float* p = part + static_cast<size_t>(m) * N + n;
    const size_t stride = static_cast<size_t>(M) * N;
    // Batches of kBatch splits: the loads of a batch are all issued before
    // the first add, so a call with ksplit <= kBatch (the library's own
    // choices split at most nine ways) waits for memory only once.
    constexpr int kBatch = 16;
    float s = 0.0f;
    for (int k0 = 0; k0 < ksplit; k0 += kBatch) {
      float v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) v[i] = k0 + i < ksplit ? p[(k0 + i) * stride] : 0.0f;
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        if (k0 + i < ksplit) s += v[i];
    }
    const float v = (gptr ? *gptr : 1.0f) * s;
    if (y) y[static_cast<size_t>(m) * N + n] = static_cast<_Float16>(v);
    key = argmax_key(v, n);
  }
  if (ARGMAX) {
    key = wave_max_key(key);
    if ((threadIdx.x & 63) == 0) best[threadIdx.x >> 6] = key;
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long k = 0ull;
      for (int w = 0; w < kFinalizeThreads / 64; ++w) k = best[w] > k ? best[w] : k;
      cand[static_cast<size_t>(blockIdx.x) * M + m] = k;
    }
  }
}

// idx[m] = column of the largest candidate key of row m.  Every thread
// issues the loads of all its rows before reducing any of them, so the kernel
// waits for memory about once instead of once per row.
//
// With `result` (greedy verification of a speculative round), row m of x is
// the target model's state after the last accepted token (m = 0) or after
// draft m (m >= 1), so idx[m] is the target's greedy choice for the token
// that follows.  Draft m + 1 is accepted while it equals idx[m] for every
// earlier row; the round commits the L accepted drafts and then idx[L]
// (greedy speculative decoding: Leviathan, Kalman and Matias, "Fast Inference
// from Transformers via Speculative Decoding", 2023; the author's post runs
// rounds of k = 7 drafts, M = 8 rows, with greedy local-argmax proposals).
// result[0] = L, result[1 .. L+1] = the committed tokens, the rest -1.
__global__ __launch_bounds__(256) void argmax_reduce(const unsigned long long* cand, int groups, int M,
                                                     int32_t* idx, const int32_t* drafts, int32_t* result) {
  __shared__ unsigned long long red[4][kMaxRows];
  __shared__ int32_t top[kMaxRows];
  unsigned long long k[kMaxRows];
#pragma unroll
  for (int m = 0; m < kMaxRows; ++m) k[m] = 0ull;
  for (int g = threadIdx.x; g < groups; g += blockDim.x) {
    unsigned long long v[kMaxRows];
#pragma unroll
    for (int m = 0; m < kMaxRows; ++m) v[m] = m < M ? cand[static_cast<size_t>(g) * M + m] : 0ull;
#pragma unroll
    for (int m = 0; m < kMaxRows; ++m) k[m] = v[m] > k[m] ? v[m] : k[m];
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  wave_max_keys<kMaxRows>(k);
  if (lane == 0) {
#pragma unroll
    for (int m = 0; m < kMaxRows; ++m) red[wave][m] = k[m];
  }
  __syncthreads();
  if (threadIdx.x < static_cast<unsigned>(M)) {
    unsigned long long best = 0ull;
    for (int w = 0; w < 4; ++w) best = red[w][threadIdx.x] > best ? red[w][threadIdx.x] : best;
    // No candidate at all (every logit NaN) leaves the all-ones index -1.
    const int32_t i = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(best & 0xFFFFFFFFull));
    idx[threadIdx.x] = i;
    top[threadIdx.x] = i;
  }
  if (result) {
    __syncthreads();
    if (threadIdx.x == 0) {
      int L = 0;
      while (L < M - 1 && drafts[L] == top[L]) ++L;
      result[0] = L;
      for (int j = 0; j < M; ++j) result[1 + j] = j < L ? drafts[j] : j == L ? top[L] : -1;
    }
  }
}

// One row (M = 1), up to tens of thousands of candidates (one per workgroup
// of the lm_head GEMV): every thread reads 16 keys per round before
// comparing any, so 16384 candidates cost one memory round trip.  Reads
// past the last candidate repeat it (a maximum does not change).  With
// `result`, a round of M = 1 has no drafts: it commits idx[0].
constexpr int kRowReduceThreads = 1024;
constexpr int kRowReduceDepth = 16;
__global__ __launch_bounds__(kRowReduceThreads) void argmax_reduce_row(const unsigned long long* cand, int groups,
                                                                    int32_t* idx, int32_t* result) {
  __shared__ unsigned long long red[kRowReduceThreads / 64];
  unsigned long long k = 0ull;
  for (int g0 = threadIdx.x; g0 < groups; g0 += kRowReduceThreads * kRowReduceDepth) {
    unsigned long long v[kRowReduceDepth];
#pragma unroll
    for (int b = 0; b < kRowReduceDepth; ++b) v[b] = cand[min(g0 + b * kRowReduceThreads, groups - 1)];
#pragma unroll
    for (int b = 0; b < kRowReduceDepth; ++b) k = v[b] > k ? v[b] : k;
  }
  k = wave_max_key(k);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = k;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long best = 0ull;
    for (int w = 0; w < kRowReduceThreads / 64; ++w) best = red[w] > best ? red[w] : best;
    // No candidate at all (every logit NaN) leaves the all-ones index -1.
    const int32_t i = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(best & 0xFFFFFFFFull));
    idx[0] = i;
    if (result) {
      result[0] = 0;
      result[1] = i;
    }
  }
}

// SwiGLU pair of a K split: thread f of block (x, m) adds the split partials
// of gate column 16 * (f / 8) + f % 8 and of its up column eight further on,
// each in split order, and writes h[m][f] = silu(g * gate) * (g2 * up).
__global__ __launch_bounds__(kFinalizeThreads) void finalize_swiglu(const float* part, int ksplit, int M, int N,
                                                                    int F, const float* gptr, const float* g2ptr,
                                                                    _Float16* h) {
  const int f = blockIdx.x * kFinalizeThreads + threadIdx.x;
  const int m = blockIdx.y;
  if (f >= F) return;
  const int n = (f / 8) * kTileCols + f % 8;
  const float* p = part + static_cast<size_t>(m) * N + n;
  const size_t stride = static_cast<size_t>(M) * N;
  float gate = 0.0f, up = 0.0f;
  for (int s = 0; s < ksplit; ++s) {
    gate += p[s * stride];
    up += p[s * stride + 8];
  }
  h[static_cast<size_t>(m) * F + f] = static_cast<_Float16>(silu(*gptr * gate) * (*g2ptr * up));
}

}  // namespace

int finalize_groups(int N) { return (N + kFinalizeThreads - 1) / kFinalizeThreads; }

hipError_t launch_finalize(const float* part, int ksplit, int M, int N, const float* gptr, uint16_t* y,
                           unsigned long long* cand, hipStream_t stream) {
  _Float16* yh = reinterpret_cast<_Float16*>(y);
  const dim3 grid(finalize_groups(N), M), block(kFinalizeThreads);
  if (cand)
    hipLaunchKernelGGL(finalize_splits<true>, grid, block, 0, stream, part, ksplit, M, N, gptr, yh, cand);
  else
    hipLaunchKernelGGL(finalize_splits<false>, grid, block, 0, stream, part, ksplit, M, N, gptr, yh, cand);
  return hipGetLastError();
}

hipError_t launch_finalize_swiglu(const float* part, int ksplit, int M, int N, int F, const float* gptr,
                                  const float* g2ptr, uint16_t* h, hipStream_t stream) {
  const dim3 grid((F + kFinalizeThreads - 1) / kFinalizeThreads, M), block(kFinalizeThreads);
  hipLaunchKernelGGL(finalize_swiglu, grid, block, 0, stream, part, ksplit, M, N, F, gptr, g2ptr,
                     reinterpret_cast<_Float16*>(h));
  return hipGetLastError();
}

hipError_t launch_argmax_reduce(const unsigned long long* cand, int groups, int M, int32_t* idx,
                                hipStream_t stream, const int32_t* drafts, int32_t* result) {
  if (M == 1)
    hipLaunchKernelGGL(argmax_reduce_row, dim3(1), dim3(kRowReduceThreads), 0, stream, cand, groups, idx, result);
  else
    hipLaunchKernelGGL(argmax_reduce, dim3(1), dim3(256), 0, stream, cand, groups, M, idx, drafts, result);
  return hipGetLastError();
}

}  // namespace skinny
