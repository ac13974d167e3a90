// Achievable-peak probes (measurement support, declared in include/bsattn_probe.h): what this
// chip sustains for the two resources the path is bound by, to set next to the vendor peaks.
// Built into its own library, libbsattn_probe.so, which only the benchmark loads; the
// method's library (libbsattn.so) does not contain it.
//
// mfma_bf16_kernel: every wave issues chains of independent v_mfma_f32_32x32x16_bf16 (eight
// accumulators, so that each MFMA waits on nothing) for `iters` rounds; the operands stay in
// registers, so nothing but the matrix cores is exercised. Each chain has its own operands,
// pseudo-random values of unit scale (as attention's bf16 operands are), so consecutive MFMAs
// switch data as real work does: constant or tiny operands draw less power and let the chip
// hold a clock that real data does not. The accumulators are summed into one float per lane
// at the end so that the work is not optimised away. mfma_fp8_kernel: the same on the fp8 MFMA.
// read_kernel: a sum of a large buffer with 16-byte nontemporal loads (HBM read rate);
// copy_kernel: 16-byte loads and stores (read + write rate).
#include <stdarg.h>
#include <stdio.h>

#include "../../include/bsattn_probe.h"
#include "common.h"

namespace bsattn {
namespace {

constexpr int kChains = 8;

// pseudo-random value in [-2, 2) from an integer (a 32-bit integer hash)
__device__ __forceinline__ float unit_value(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352dU; x ^= x >> 15; x *= 0x846ca68bU; x ^= x >> 16;
  return (float)(x >> 8) * (4.0f / 16777216.0f) - 2.0f;
}

__global__ __launch_bounds__(256) void mfma_bf16_kernel(int64_t iters, float* __restrict__ sink) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8 a[kChains], b[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[c][e] = (__bf16)unit_value(t * 131u + c * 17u + e);
      b[c][e] = (__bf16)unit_value(t * 131u + c * 17u + e + 0x9e3779b9u);
    }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[c], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// the same stream on the fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, e4m3 operands, unit
// scales); operand bytes are pseudo-random e4m3 codes of unit scale (exponent field 5..8)
__global__ __launch_bounds__(256) void mfma_fp8_kernel(int64_t iters, float* __restrict__ sink) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  i32x8 a[kChains], b[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t ra = __float_as_uint(unit_value(t * 131u + c * 17u + e));
      const uint32_t rb = __float_as_uint(unit_value(t * 131u + c * 17u + e + 0x9e3779b9u));
      // four codes per word: sign and mantissa from the hash, exponent field 5 + (bits & 3)
      a[c][e] = (int)((ra & 0x87878787u) | (((ra >> 3) & 0x03030303u) + 0x05050505u) << 3);
      b[c][e] = (int)((rb & 0x87878787u) | (((rb >> 3) & 0x03030303u) + 0x05050505u) << 3);
    }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[c], b[c], acc[c], 0, 0, 0, 127,
                                                               0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Each work-group streams one contiguous range (as the path's pooling and attention read
// whole blocks); 16 loads of 16 bytes in flight per thread.
constexpr int kStreamUnroll = 16;

__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                   float* __restrict__ sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t begin = (int64_t)blockIdx.x * per;
  const int64_t end = begin + per < n16 ? begin + per : n16;
  int64_t i = begin + threadIdx.x;
  uint32_t x = 0;
  for (; i + (kStreamUnroll - 1) * 256 < end; i += kStreamUnroll * 256) {
    u32x4 w[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) w[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) x ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
  for (; i < end; i += 256) {
    const u32x4 w = __builtin_nontemporal_load(src + i);
    x ^= w.x ^ w.y ^ w.z ^ w.w;
  }
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = (float)(x & 0xffff);
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, int64_t n16) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t begin = (int64_t)blockIdx.x * per;
  const int64_t end = begin + per < n16 ? begin + per : n16;
  int64_t i = begin + threadIdx.x;
  constexpr int kU = kStreamUnroll / 2;
  for (; i + (kU - 1) * 256 < end; i += kU * 256) {
    u32x4 w[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) w[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
    for (int u = 0; u < kU; ++u) __builtin_nontemporal_store(w[u], dst + i + u * 256);
  }
  for (; i < end; i += 256) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

static hipError_t launch_probe_mfma_bf16(int64_t iters, int groups, float* sink, hipStream_t stream) {
  mfma_bf16_kernel<<<groups, 256, 0, stream>>>(iters, sink);
  return hipGetLastError();
}

static hipError_t launch_probe_mfma_fp8(int64_t iters, int groups, float* sink, hipStream_t stream) {
  mfma_fp8_kernel<<<groups, 256, 0, stream>>>(iters, sink);
  return hipGetLastError();
}

static hipError_t launch_probe_read(const void* src, int64_t n16, int groups, float* sink,
                             hipStream_t stream) {
  read_kernel<<<groups, 256, 0, stream>>>((const u32x4*)src, n16, sink);
  return hipGetLastError();
}

static hipError_t launch_probe_copy(const void* src, void* dst, int64_t n16, int groups,
                             hipStream_t stream) {
  copy_kernel<<<groups, 256, 0, stream>>>((const u32x4*)src, (u32x4*)dst, n16);
  return hipGetLastError();
}

}  // namespace bsattn

namespace {

thread_local char g_err[256] = "";

int fail(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return 1;   // BSATTN_E_INVALID
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return 0;
  snprintf(g_err, sizeof(g_err), "%s: %s", what, hipGetErrorString(e));
  return 4;   // BSATTN_E_HIP
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

const char* bsattn_probe_last_error(void) { return g_err; }

size_t bsattn_probe_sink_floats(int groups) { return groups > 0 ? (size_t)groups * 256 : 0; }

int bsattn_probe_mfma_bf16(int64_t iters, int groups, float* sink, double* flops, void* stream) {
  if (iters < 1 || iters > ((int64_t)1 << 30) || groups < 1 || groups > 65535)
    return fail("iters in [1, 2^30] and groups in [1, 65535] required");
  if (!sink || ((uintptr_t)sink & 3u)) return fail("sink null or unaligned");
  if (flops) *flops = 2.0 * 32 * 32 * 16 * 8 * 4 * (double)groups * (double)iters;
  return hip_status(bsattn::launch_probe_mfma_bf16(iters, groups, sink, (hipStream_t)stream),
                    "mfma probe launch");
}

int bsattn_probe_mfma_fp8(int64_t iters, int groups, float* sink, double* flops, void* stream) {
  if (iters < 1 || iters > ((int64_t)1 << 30) || groups < 1 || groups > 65535)
    return fail("iters in [1, 2^30] and groups in [1, 65535] required");
  if (!sink || ((uintptr_t)sink & 3u)) return fail("sink null or unaligned");
  if (flops) *flops = 2.0 * 32 * 32 * 64 * 8 * 4 * (double)groups * (double)iters;
  return hip_status(bsattn::launch_probe_mfma_fp8(iters, groups, sink, (hipStream_t)stream),
                    "mfma fp8 probe launch");
}

int bsattn_probe_read(const void* src, size_t bytes, int groups, float* sink, void* stream) {
  if (!src || !sink || !aligned16(src) || ((uintptr_t)sink & 3u) || bytes == 0 || bytes % 16 ||
      groups < 1 || groups > 65535)
    return fail("read probe: bad pointer, size or group count");
  return hip_status(bsattn::launch_probe_read(src, (int64_t)(bytes / 16), groups, sink,
                                              (hipStream_t)stream),
                    "read probe launch");
}

int bsattn_probe_copy(const void* src, void* dst, size_t bytes, int groups, void* stream) {
  if (!src || !dst || !aligned16(src) || !aligned16(dst) || bytes == 0 || bytes % 16 ||
      groups < 1 || groups > 65535)
    return fail("copy probe: bad pointer, size or group count");
  const char *s0 = (const char*)src, *d0 = (const char*)dst;
  if (s0 < d0 + bytes && d0 < s0 + bytes) return fail("copy probe: overlap");
  return hip_status(bsattn::launch_probe_copy(src, dst, (int64_t)(bytes / 16), groups,
                                              (hipStream_t)stream),
                    "copy probe launch");
}

}  // extern "C"
