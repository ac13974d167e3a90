// Internal helpers shared by the gfx950 kernels of the library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// bfloat16 bits -> float (exact).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bfloat16 pair (round to nearest even), lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Order-preserving map of a float to uint32 (larger float -> larger key); -0.0 maps
// like +0.0 so that the two tie.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = (s == 0.0f) ? 0u : __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Number of set bits of a 64-bit lane mask below the calling lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Work-group id remap so that consecutive logical tiles share an XCD.
// The dispatcher hands work-group w to XCD (w mod 8); the logical tile of w is chosen so
// that XCD x runs the contiguous range [x*per, (x+1)*per) of logical tiles. Tiles that read
// the same K/V (same batch and KV head) are contiguous, so they share that XCD's L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t w, uint32_t total) {
  constexpr uint32_t kXcd = 8;
  const uint32_t per = total / kXcd;          // full rounds
  const uint32_t full = per * kXcd;
  if (w >= full) return w;                    // ragged tail keeps its own order
  return (w % kXcd) * per + (w / kXcd);
}

}  // namespace bsattn
