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

// Reductions within aligned groups of lanes through DPP moves (VALU, no LDS): xor 1 and xor 2
// inside a quad, then the mirrored quad of the 8-lane half row, then the mirrored half of the
// 16-lane row. Every lane of a group ends with the group's value; all lanes of a group must be
// active.
template <int CTRL, typename T>
__device__ __forceinline__ T dpp_mov(T v) {
  static_assert(sizeof(T) == 4, "32-bit lanes");
  return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                           0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;                // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;                // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;         // lane i <-> 7 - i within each 8 lanes
constexpr int kDppMirror = 0x140;             // lane i <-> 15 - i within each 16 lanes

template <int LG, typename T>                 // LG = 8 or 16
__device__ __forceinline__ T group_sum(T a) {
  static_assert(LG == 8 || LG == 16, "DPP groups of 8 or 16 lanes");
  a += dpp_mov<kDppXor1>(a);
  a += dpp_mov<kDppXor2>(a);
  a += dpp_mov<kDppHalfMirror>(a);
  if constexpr (LG == 16) a += dpp_mov<kDppMirror>(a);
  return a;
}

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

// Storage kinds: 0 fp32, 1 bf16, 2 OCP fp8 e4m3. Vec<KIND>: elements per 16-byte vector and
// their fp32 values folded into an accumulator array (add: sums; vmax: elementwise maxima).
template <int KIND> struct Vec;
template <> struct Vec<0> {            // fp32
  static constexpr int E = 4;
  __device__ static void add(const u32x4& w, float* a) {
    a[0] += __uint_as_float(w.x); a[1] += __uint_as_float(w.y);
    a[2] += __uint_as_float(w.z); a[3] += __uint_as_float(w.w);
  }
  __device__ static void vmax(const u32x4& w, float* a) {
    a[0] = fmaxf(a[0], __uint_as_float(w.x)); a[1] = fmaxf(a[1], __uint_as_float(w.y));
    a[2] = fmaxf(a[2], __uint_as_float(w.z)); a[3] = fmaxf(a[3], __uint_as_float(w.w));
  }
};
template <> struct Vec<1> {            // bf16
  static constexpr int E = 8;
  __device__ static void add(const u32x4& w, float* a) {
    a[0] += bf16lo(w.x); a[1] += bf16hi(w.x); a[2] += bf16lo(w.y); a[3] += bf16hi(w.y);
    a[4] += bf16lo(w.z); a[5] += bf16hi(w.z); a[6] += bf16lo(w.w); a[7] += bf16hi(w.w);
  }
  __device__ static void vmax(const u32x4& w, float* a) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[2 * i] = fmaxf(a[2 * i], bf16lo(ws[i]));
      a[2 * i + 1] = fmaxf(a[2 * i + 1], bf16hi(ws[i]));
    }
  }
};
template <> struct Vec<2> {            // OCP fp8 e4m3 (gfx950 converts the OCP format)
  static constexpr int E = 16;
  __device__ static void add(const u32x4& w, float* a) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[i], false);
      auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[i], true);
      a[4 * i + 0] += lo[0]; a[4 * i + 1] += lo[1];
      a[4 * i + 2] += hi[0]; a[4 * i + 3] += hi[1];
    }
  }
  __device__ static void vmax(const u32x4& w, float* a) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[i], false);
      auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[i], true);
      a[4 * i + 0] = fmaxf(a[4 * i + 0], lo[0]); a[4 * i + 1] = fmaxf(a[4 * i + 1], lo[1]);
      a[4 * i + 2] = fmaxf(a[4 * i + 2], hi[0]); a[4 * i + 3] = fmaxf(a[4 * i + 3], hi[1]);
    }
  }
};

// Element n (0-based) of the SplitMix64 sequence seeded with `seed` (Steele, Lea, Flood,
// "Fast splittable pseudorandom number generators", OOPSLA 2014): the state after n + 1 Weyl
// steps of the golden-ratio increment, through the published 64-bit finaliser.
__device__ __forceinline__ uint64_t splitmix64(uint64_t seed, uint64_t n) {
  uint64_t z = seed + (n + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Overlapping key blocks (the MSA page's §5.3 overlap remedy): key block j holds the tokens
// [j*stride, min(j*stride + SB, N)) with SB/2 <= stride <= SB, so only neighbouring blocks share
// tokens. Attention reads the SB-token tile that starts at key_tile_start (the last block's
// tile moves back to end at token N, so every tile lies inside the sequence) and leaves out
// its first key_tile_skip keys: tokens before the block's start, and tokens that the selected
// block j-1 already holds (the union of a row's blocks counts each token once). Each block
// has at least one token of its own, so the skip is below SB.
__device__ __forceinline__ int64_t key_tile_start(int j, int stride, int SB, int64_t N) {
  const int64_t s = (int64_t)j * stride;
  return s < N - SB ? s : N - SB;
}
__device__ __forceinline__ int key_tile_skip(int j, int stride, int SB, int64_t N,
                                             bool prev_selected) {
  const int64_t first = prev_selected ? (int64_t)(j - 1) * stride + SB : (int64_t)j * stride;
  return (int)(first - key_tile_start(j, stride, SB, N));
}

// Bitmap (LDS, (nkb + 31) / 32 words) of the key blocks named by the first `count` entries
// of a row; entries outside [0, nkb) are left out. All threads of the work-group take part.
__device__ __forceinline__ void mark_selected(uint32_t* bits, const int32_t* row, int count,
                                              int nkb, int tid, int nthreads) {
  for (int w = tid; w < (nkb + 31) / 32; w += nthreads) bits[w] = 0u;
  __syncthreads();
  for (int p = tid; p < count; p += nthreads) {
    const int j = row[p];
    if ((unsigned)j < (unsigned)nkb) atomicOr(&bits[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
}
__device__ __forceinline__ bool is_selected(const uint32_t* bits, int j) {
  return j >= 0 && ((bits[j >> 5] >> (j & 31)) & 1u);
}

// Selection options (flags of the extended entry points)
constexpr unsigned kCausal = 1u;     // key blocks j <= i only, own block forced
constexpr unsigned kPoolMax = 2u;    // in-block elementwise maximum instead of the mean
constexpr unsigned kGroup = 4u;      // one selection per KV head from the group's summed scores

}  // namespace bsattn
