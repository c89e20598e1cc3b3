// Device helpers shared by the gfx950 kernels.
#ifndef SKINNY_COMMON_CUH
#define SKINNY_COMMON_CUH

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skinny {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Two E2M1 codes (byte B of w: low nibble -> .x, high nibble -> .y) to fp16.
// The hardware scale operand of this conversion only uses its power-of-two
// part, so it is fed 1.0 and block scales are applied separately.
template <int B>
__device__ __forceinline__ f16x2 e2m1x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, B);
}

// Eight E2M1 codes (one dword) to eight fp16 values, k order preserved.
__device__ __forceinline__ f16x8 e2m1x8(uint32_t w) {
  const f16x2 a = e2m1x2<0>(w), b = e2m1x2<1>(w), c = e2m1x2<2>(w), d = e2m1x2<3>(w);
  return f16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Two E4M3FN bytes (the low or high 16 bits of w) to fp16 (exact).
template <bool HI>
__device__ __forceinline__ f16x2 e4m3x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// Eight E4M3FN codes (two dwords) to eight fp16 values.
__device__ __forceinline__ f16x8 e4m3x8(uint32_t lo, uint32_t hi) {
  const f16x2 a = e4m3x2<false>(lo), b = e4m3x2<true>(lo), c = e4m3x2<false>(hi), d = e4m3x2<true>(hi);
  return f16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// One E4M3FN byte (byte B of w) to fp32 (exact).
template <int B>
__device__ __forceinline__ float e4m3f(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8(w, B);
}

// Lane (16r + i) receives lane (16r + I)'s value: DPP row_newbcast.
template <int I>
__device__ __forceinline__ uint32_t row_bcast(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x150 + I, 0xf, 0xf, true));
}

// Sum of v over lanes {l, l^16, l^32, l^48}: the four 16-lane rows of a
// wavefront, exchanged with ds_bpermute lane shuffles.  Every lane ends with
// the same value, (v0 + v2) + (v1 + v3) for rows 0..3.
__device__ __forceinline__ float sum_over_rows(float v) {
  v += __shfl_xor(v, 32);
  v += __shfl_xor(v, 16);
  return v;
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Cross-workgroup hand-off without cache write-backs.  Data that another
// workgroup (possibly on another XCD, with its own L2) reads back is written
// and read with system-scope atomic accesses, which go to the coherence point
// instead of a private L2 copy; wait_stores() makes them complete before the
// arrival counter is bumped.  Counters and keys are system-scope atomic
// read-modify-writes whose results are waited for, so each one is performed
// before the next is issued.
__device__ __forceinline__ void store_shared(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ float load_shared(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ uint32_t counter_add(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ uint32_t counter_exch(uint32_t* p, uint32_t v) {
  return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ unsigned long long key_max(unsigned long long* p, unsigned long long v) {
  return __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ unsigned long long key_exch(unsigned long long* p, unsigned long long v) {
  return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace skinny

#endif
