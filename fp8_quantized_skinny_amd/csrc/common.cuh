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

// Sum of v over lanes {l, l^16, l^32, l^48}: the four 16-lane rows of a
// wavefront.  Every lane ends with the same value, (v0 + v2) + (v1 + v3) for
// rows 0..3.  The rows move with gfx950's permlane swaps, which run in the
// VALU: v_permlane32_swap of two copies of v leaves rows (0, 1, 0, 1) in one
// and (2, 3, 2, 3) in the other, v_permlane16_swap then rows (0, 0, 2, 2) and
// (1, 1, 3, 3).  Lane shuffles (ds_bpermute) gave the same sums but waited for
// an LDS round trip each.  Every lane of the wavefront must be active.
__device__ __forceinline__ float sum_over_rows(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto h = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  v = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  const uint32_t w = __float_as_uint(v);
  const auto q = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// s_waitcnt immediate (gfx9 encoding) that waits until at most `vm` vector
// memory and `lgkm` LDS/scalar operations are outstanding.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 0xF) | (((vm >> 4) & 3) << 14) | (7 << 4) | ((lgkm & 0xF) << 8);
}

// Workgroup barrier after direct-to-LDS copies (global_load_lds) that each
// wavefront issued before `pending` newer loads of its own.  The vector-memory
// counter completes in order, so waiting until at most PENDING loads are
// outstanding finishes this wavefront's copies without waiting for its newer
// loads; __syncthreads() would wait for all of them (a full fence), which
// holds the whole workgroup until its slowest weight load has arrived.  The
// wait is the compiler's own s_waitcnt, not inline asm: the compiler then
// knows the copies have landed, whereas after an opaque wait it treats them
// as outstanding and, at its next wait on a newer load, waits for every load
// in flight.  The empty asm keeps LDS reads from moving above the barrier.
template <int PENDING>
__device__ __forceinline__ void lds_copy_barrier(bool pending) {
  if (pending)
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(PENDING, 0));
  else
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// SiLU in fp32, v * sigmoid(v), the activation of a SwiGLU MLP (Shazeer,
// "GLU Variants Improve Transformer").  exp(-v) overflows to inf for
// v < -88, which gives the right limit -0.
__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }

// 16 bytes of weights whose cache lines no other load of the call touches
// (each wavefront instruction reads whole lines): every such byte is read once
// per call, so the load is non-temporal (streaming cache policy).  On MI355X a
// pure read of 50 MB in this pattern ran at 5.99 TB/s with it against 5.45
// TB/s without (100 MB: 6.65 against 6.08 TB/s).  x and partial sums, which
// are re-read, use plain loads.
__device__ __forceinline__ u32x4 load16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Zeroes halves [from, to) of rows 0..M-1 of an LDS copy of x (row stride RS
// halves) with 16-byte stores: the part of the copy past K, which the
// direct-to-LDS loads leave untouched.  from, to and RS are multiples of 8.
__device__ __forceinline__ void zero_x_tail(_Float16* xs, int M, int RS, int from, int to) {
  from = from < 0 ? 0 : from;
  const int per_row = (to - from) >> 3;
  if (per_row <= 0) return;
  for (int c = threadIdx.x; c < M * per_row; c += blockDim.x) {
    const int m = c / per_row, j = c - m * per_row;
    *reinterpret_cast<u32x4*>(xs + m * RS + from + 8 * j) = u32x4{0u, 0u, 0u, 0u};
  }
}

// Ordered argmax key of logit v at column n: the top 32 bits order like the
// fp32 value (+0 and -0 made equal), the low 32 bits are the inverted column,
// so the larger key is the larger logit or, on a tie, the lower column.  A
// NaN logit is no score: it gets key 0, the "no candidate" key, which every
// number (even -inf, whose key is 0x007FFFFF...) beats, so a NaN never wins
// and a row of NaN alone leaves the index at 0xFFFFFFFF - 0 = -1.
__device__ __forceinline__ unsigned long long argmax_key(float v, int n) {
  if (v != v) return 0ull;
  if (v == 0.0f) v = 0.0f;
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (static_cast<unsigned long long>(ord) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(n));
}

// The larger of lane l's key and its partner's in one step of a max
// reduction over lane groups: the partner is lane l ^ 32 (OFF = 32) or
// l ^ 16 (OFF = 16), exchanged with gfx950's permlane swaps, or lane
// (l - OFF) mod 16 of the same 16-lane row (OFF = 8, 4, 2, 1), read through
// DPP row_ror.  Rotating by 8, 4, 2 and 1 covers a row as xor partners do, so
// steps OFF = WIDTH/2 .. 1 leave every lane with the largest key of its WIDTH
// lanes.  Both halves of the 64-bit key move the same way.  All VALU, no LDS
// round trip; every lane of the wavefront must be active.
template <int OFF>
__device__ __forceinline__ unsigned long long max_with_partner(unsigned long long k) {
  static_assert(OFF == 32 || OFF == 16 || OFF == 8 || OFF == 4 || OFF == 2 || OFF == 1, "partner offset");
  const uint32_t lo = static_cast<uint32_t>(k), hi = static_cast<uint32_t>(k >> 32);
  unsigned long long a, b;
  if constexpr (OFF >= 16) {
    // Each swap of two copies leaves the lane's own value in one result and
    // its partner's in the other.
    const auto l = OFF == 32 ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                             : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto h = OFF == 32 ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                             : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    a = (static_cast<unsigned long long>(h[0]) << 32) | l[0];
    b = (static_cast<unsigned long long>(h[1]) << 32) | l[1];
  } else {
    constexpr int kRowRor = 0x120 + OFF;  // DPP row_ror:OFF
    const uint32_t plo = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(lo), kRowRor, 0xf, 0xf, false));
    const uint32_t phi = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(hi), kRowRor, 0xf, 0xf, false));
    a = (static_cast<unsigned long long>(phi) << 32) | plo;
    b = k;
  }
  return a > b ? a : b;
}

// Largest key of each of R independent values over the WIDTH lanes (16 or 64)
// of each lane group; every lane gets them.  Every lane must be active.
template <int R, int WIDTH = 64>
__device__ __forceinline__ void wave_max_keys(unsigned long long (&k)[R]) {
  static_assert(WIDTH == 16 || WIDTH == 64, "lane group");
  if constexpr (WIDTH == 64) {
#pragma unroll
    for (int r = 0; r < R; ++r) k[r] = max_with_partner<1>(max_with_partner<2>(max_with_partner<4>(
                                        max_with_partner<8>(max_with_partner<16>(max_with_partner<32>(k[r]))))));
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r)
      k[r] = max_with_partner<1>(max_with_partner<2>(max_with_partner<4>(max_with_partner<8>(k[r]))));
  }
}

// The same for one value.
template <int WIDTH = 64>
__device__ __forceinline__ unsigned long long wave_max_key(unsigned long long k) {
  unsigned long long one[1] = {k};
  wave_max_keys<1, WIDTH>(one);
  return one[0];
}

}  // namespace skinny

#endif
