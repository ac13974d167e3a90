// Decode step: one new query token per sequence against a KV cache, with the pooled key
// blocks of the cache kept up to date as blocks complete.
//
// SparseFormer page ("2026 新一代卷积与Transformer网络架构技术演进与性能对比"), "SparseFormer
// 注意力实现": mean-pooled key blocks, top-k blocks by the product with the (here single-token)
// query, attention over the chosen blocks with scale 1/sqrt(D). MSA page
// ("从M2.7到M3：多模态模型稀疏注意力架构设计与实现全解析") §5.2: first-token latency comes from
// an unoptimised block-scoring step. Step rule for a sequence of L cached tokens (the query is
// token L-1): its own block (L-1)/b is always used; the other min(k, own+1) - 1 places go to
// the complete blocks j < own with the largest q . kbar_j (ties to the lower j).
//
// Kernels (bf16 caches [B, Lmax, Hkv, D], fp32 pooled cache [B, Hkv, Lmax/b, D]):
//   pool_new_kernel    one work-group per (sequence, block): pools the blocks completed
//                      between the old and the new length (all complete blocks without old
//                      lengths).
//   dselect_kernel     one work-group per (sequence, query head): fp32 scores of the complete
//                      earlier blocks (one thread per block, fixed summation order), the same
//                      bitwise threshold search as the prefill selection, ascending output.
//   dattn_kernel       split-K over the chosen blocks (flash-decoding): one wave per
//                      (sequence, query head, split); per block, lanes own keys for the scores
//                      (16-byte row loads), the weights go through LDS, then lanes own pairs of
//                      d for the weighted value sum (coalesced 4-byte loads per key row).
//                      Writes the split's (max, sum, unnormalised output).
//   dcombine_kernel    per (sequence, query head): merges the splits, writes bf16.
// The work is HBM-bound (each key and value of a chosen block is read once per query head);
// the single query row leaves nothing for the matrix cores.
#include "common.h"
#include "launch.h"

namespace bsattn {
namespace {

// ---------------------------------------------------------------- pooling of new blocks
__global__ __launch_bounds__(256) void pool_new_kernel(const uint16_t* __restrict__ kc,
                                                       const int32_t* __restrict__ lens_old,
                                                       const int32_t* __restrict__ lens_new,
                                                       float* __restrict__ kbar, int64_t Lmax,
                                                       int Hkv, int D, int block, int nbmax) {
  const int b = blockIdx.y, j = blockIdx.x;
  const int64_t Ln = lens_new[b];
  const int64_t Lo = lens_old ? lens_old[b] : 0;
  if (Ln < 1 || Ln > Lmax || Lo < 0 || Lo > Ln) return;
  if (j < Lo / block || j >= Ln / block) return;
  const int V = Hkv * D / 8;                            // 16-byte chunks per token row
  const int64_t rs = (int64_t)Hkv * D;
  const float inv = 1.0f / (float)block;
  for (int c = threadIdx.x; c < V; c += blockDim.x) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const uint16_t* p = kc + ((int64_t)b * Lmax + (int64_t)j * block) * rs + 8 * c;
    for (int t = 0; t < block; ++t) Vec<1>::add(*(const u32x4*)(p + t * rs), acc);
    const int g = (8 * c) / D, d0 = (8 * c) % D;
    float* o = kbar + (((int64_t)b * Hkv + g) * nbmax + j) * D + d0;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = acc[e] * inv;
  }
}

// ---------------------------------------------------------------- selection
constexpr int kSelThreads = 256;
constexpr int kSelPer = 32;                   // columns per thread: nb <= 8192

__device__ __forceinline__ int block_sum(int v, int* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  const int total = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return total;
}

__device__ __forceinline__ int block_exclusive_scan(int v, int* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) red[w] = incl;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += red[i];
  __syncthreads();
  return before + incl - v;
}

template <int D>
__global__ __launch_bounds__(kSelThreads) void dselect_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ kbar,
    const int32_t* __restrict__ lens, int32_t* __restrict__ idx, int64_t Lmax, int Hq, int Hkv,
    int block, int nbmax, int topk) {
  __shared__ float qs[D];
  __shared__ int red[4];
  const int bh = blockIdx.x;
  const int b = bh / Hq, h = bh % Hq, g = h / (Hq / Hkv);
  const int tid = threadIdx.x;
  int32_t* out = idx + (int64_t)bh * topk;
  const int64_t L = lens[b];
  if (L < 1 || L > Lmax) {                    // invalid length: no block
    for (int p = tid; p < topk; p += kSelThreads) out[p] = -1;
    return;
  }
  const int own = (int)((L - 1) / block);
  const int kb = own + 1 < topk ? own + 1 : topk;
  const int need_k = kb - 1;                  // places for complete earlier blocks
  for (int d = tid; d < D; d += kSelThreads) {
    const uint16_t w = q[(int64_t)bh * D + d];
    qs[d] = __uint_as_float((uint32_t)w << 16);
  }
  __syncthreads();
  const float* K = kbar + ((int64_t)b * Hkv + g) * nbmax * D;
  uint32_t key[kSelPer];
#pragma unroll
  for (int e = 0; e < kSelPer; ++e) {
    const int j = e * kSelThreads + tid;     // columns strided: a warp's loads share lines
    key[e] = 0u;
    if (j < own) {
      const float* row = K + (int64_t)j * D;
      float s = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; d += 4) {
        const f32x4 kv = *(const f32x4*)(row + d);
        s = __builtin_fmaf(qs[d], kv[0], s);
        s = __builtin_fmaf(qs[d + 1], kv[1], s);
        s = __builtin_fmaf(qs[d + 2], kv[2], s);
        s = __builtin_fmaf(qs[d + 3], kv[3], s);
      }
      key[e] = order_key(s);
    }
  }
  // threshold T: the need_k-th largest key (keys 0 = no column never count)
  uint32_t T = 0;
  if (need_k > 0) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      int c = 0;
#pragma unroll
      for (int e = 0; e < kSelPer; ++e) c += key[e] >= cand;
      const int cnt = block_sum(c, red);
      if (cnt >= need_k) T = cand;
      if (cnt == need_k) break;
    }
  }
  // selected: key > T, then keys == T by ascending column; columns are strided over threads,
  // so ranks go column by column: e outer, threads inner
  int gt = 0;
#pragma unroll
  for (int e = 0; e < kSelPer; ++e) gt += need_k > 0 && key[e] > T;
  const int tot_gt = block_sum(gt, red);
  int eq_seen = 0, pos_seen = 0;
  for (int e = 0; e < kSelPer; ++e) {
    if (e * kSelThreads >= own) break;       // uniform
    const int j = e * kSelThreads + tid;
    const bool valid = need_k > 0 && j < own;
    const bool is_eq = valid && T != 0 && key[e] == T;
    const int eq_before = eq_seen + block_exclusive_scan(is_eq ? 1 : 0, red);
    const bool sel = valid && (key[e] > T || (is_eq && eq_before < need_k - tot_gt));
    const int p_before = pos_seen + block_exclusive_scan(sel ? 1 : 0, red);
    if (sel) out[p_before] = j;
    eq_seen += block_sum(is_eq ? 1 : 0, red);
    pos_seen += block_sum(sel ? 1 : 0, red);
  }
  if (tid == 0) out[kb - 1] = own;
  for (int p = kb + tid; p < topk; p += kSelThreads) out[p] = -1;
}

// ---------------------------------------------------------------- split-K attention
template <int D>
__global__ __launch_bounds__(64) void dattn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ lens, float* __restrict__ part, int64_t Lmax, int Hq, int Hkv,
    int block, int topk, int splits, float c) {
  constexpr int DP = D / 2;                   // bf16 pairs per row
  __shared__ float qs[D];
  __shared__ float ps[128];                   // weights of one block (block <= 128)
  const int bh = blockIdx.x / splits, sp = blockIdx.x % splits;
  const int b = bh / Hq, h = bh % Hq, g = h / (Hq / Hkv);
  const int lane = threadIdx.x;
  const int64_t L = lens[b];
  const int64_t rs = (int64_t)Hkv * D;
  float* my = part + ((int64_t)bh * splits + sp) * (D + 2);
  for (int d = lane; d < D; d += 64) {
    const uint16_t w = q[(int64_t)bh * D + d];
    qs[d] = __uint_as_float((uint32_t)w << 16);
  }
  __syncthreads();
  const int32_t* row = idx + (int64_t)bh * topk;
  const int per = (topk + splits - 1) / splits;
  const int e0 = sp * per, e1 = e0 + per < topk ? e0 + per : topk;
  float m = -__builtin_inff(), l = 0.f;
  // value accumulators: D = 128: lane owns pair (lane); D = 64: lanes 0..31 own pairs of even
  // keys, lanes 32..63 the same pairs of odd keys (summed at the end)
  const int pair = D == 128 ? lane : (lane & 31);
  const int kpar = D == 128 ? 0 : (lane >> 5);
  float o0 = 0.f, o1 = 0.f;
  const uint16_t* kb0 = kc + (int64_t)b * Lmax * rs + (int64_t)g * D;
  const uint16_t* vb0 = vc + (int64_t)b * Lmax * rs + (int64_t)g * D;
  const bool len_ok = L >= 1 && L <= Lmax;
  for (int e = e0; e < e1 && len_ok; ++e) {
    const int j = row[e];
    if (j < 0 || (int64_t)j * block >= L) continue;   // unused place or beyond the cache
    const int64_t t0 = (int64_t)j * block;
    const int nk = (int)(L - t0 < block ? L - t0 : block);   // own block: tokens < L
    // scores: lane owns keys lane and lane + 64
    float s[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = lane + 64 * u;
      s[u] = -__builtin_inff();
      if (t < nk) {
        const uint16_t* kr = kb0 + (t0 + t) * rs;
        float a = 0.f;
#pragma unroll
        for (int d = 0; d < D; d += 8) {
          const u32x4 w = *(const u32x4*)(kr + d);
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            a = __builtin_fmaf(qs[d + 2 * x], bf16lo(w[x]), a);
            a = __builtin_fmaf(qs[d + 2 * x + 1], bf16hi(w[x]), a);
          }
        }
        s[u] = a * c;                         // exp2 domain
      }
    }
    float mb = fmaxf(s[0], s[1]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mb = fmaxf(mb, __shfl_xor(mb, o));
    const float mn = fmaxf(m, mb);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);    // 0 on the first block
    m = mn;
    float lp = 0.f;
    __syncthreads();                          // previous block done with ps
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = lane + 64 * u;
      const float p = t < nk ? __builtin_amdgcn_exp2f(s[u] - m) : 0.f;
      if (t < block) ps[t] = p;
      lp += p;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lp += __shfl_xor(lp, o);
    l = l * alpha + lp;
    o0 *= alpha;
    o1 *= alpha;
    __syncthreads();
    const int step = D == 128 ? 1 : 2;
    for (int t = kpar; t < nk; t += step) {
      const uint32_t w = *(const uint32_t*)(vb0 + (t0 + t) * rs + 2 * pair);
      const float p = ps[t];
      o0 = __builtin_fmaf(p, bf16lo(w), o0);
      o1 = __builtin_fmaf(p, bf16hi(w), o1);
    }
  }
  if (D == 64) {                              // fold the odd-key half into lanes 0..31
    o0 += __shfl_down(o0, 32);
    o1 += __shfl_down(o1, 32);
  }
  if (lane < DP) {
    my[2 + 2 * pair] = o0;
    my[2 + 2 * pair + 1] = o1;
  }
  if (lane == 0) {
    my[0] = m;
    my[1] = l;
  }
}

template <int D>
__global__ __launch_bounds__(64) void dcombine_kernel(const float* __restrict__ part,
                                                      const int32_t* __restrict__ lens,
                                                      uint16_t* __restrict__ out, int64_t Lmax,
                                                      int Hq, int splits) {
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const float* pp = part + (int64_t)bh * splits * (D + 2);
  float M = -__builtin_inff();
  for (int s = 0; s < splits; ++s) M = fmaxf(M, pp[s * (D + 2)]);
  float lsum = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float ms = pp[s * (D + 2)];
    if (ms != -__builtin_inff()) lsum += __builtin_amdgcn_exp2f(ms - M) * pp[s * (D + 2) + 1];
  }
  const int64_t L = lens[b];
  const bool ok = L >= 1 && L <= Lmax && lsum > 0.f;
  for (int d = threadIdx.x; d < D; d += 64) {
    float acc = 0.f;
    for (int s = 0; s < splits; ++s) {
      const float ms = pp[s * (D + 2)];
      if (ms != -__builtin_inff()) acc += __builtin_amdgcn_exp2f(ms - M) * pp[s * (D + 2) + 2 + d];
    }
    const float v = ok ? acc / lsum : __builtin_nanf("");
    out[(int64_t)bh * D + d] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xFFFFu);
  }
}

}  // namespace

int decode_splits(int64_t B, int Hq, int topk) {
  const int64_t heads = B * Hq;
  int64_t s = (2048 + heads - 1) / heads;     // aim at >= 2048 waves on 256 CUs
  if (s > topk) s = topk;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return (int)s;
}

size_t decode_workspace_bytes(int64_t B, int Hq, int D, int topk) {
  return (size_t)B * Hq * decode_splits(B, Hq, topk) * (D + 2) * sizeof(float);
}

bool decode_supported(int D, int block) {
  return (D == 64 || D == 128) && (block == 64 || block == 128);
}

hipError_t launch_decode_pool(int64_t B, int64_t Lmax, int Hkv, int D, int block,
                              const void* k_cache, const int32_t* lens_old,
                              const int32_t* lens_new, float* kbar, hipStream_t stream) {
  const int nbmax = (int)(Lmax / block);
  pool_new_kernel<<<dim3((unsigned)nbmax, (unsigned)B), 256, 0, stream>>>(
      (const uint16_t*)k_cache, lens_old, lens_new, kbar, Lmax, Hkv, D, block, nbmax);
  return hipGetLastError();
}

hipError_t launch_decode(int64_t B, int64_t Lmax, int Hq, int Hkv, int D, int block, int topk,
                         const void* q, const void* k_cache, const void* v_cache,
                         const float* kbar, const int32_t* lens, float scale, void* out,
                         int32_t* idx, void* workspace, hipStream_t stream) {
  const int nbmax = (int)(Lmax / block);
  const int splits = decode_splits(B, Hq, topk);
  const float c = (float)((double)scale * 1.4426950408889634);
  float* part = (float*)workspace;
  const unsigned heads = (unsigned)(B * Hq);
  if (D == 64)
    dselect_kernel<64><<<heads, kSelThreads, 0, stream>>>((const uint16_t*)q, kbar, lens, idx,
                                                           Lmax, Hq, Hkv, block, nbmax, topk);
  else
    dselect_kernel<128><<<heads, kSelThreads, 0, stream>>>((const uint16_t*)q, kbar, lens, idx,
                                                            Lmax, Hq, Hkv, block, nbmax, topk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (D == 64)
    dattn_kernel<64><<<heads * splits, 64, 0, stream>>>(
        (const uint16_t*)q, (const uint16_t*)k_cache, (const uint16_t*)v_cache, idx, lens, part,
        Lmax, Hq, Hkv, block, topk, splits, c);
  else
    dattn_kernel<128><<<heads * splits, 64, 0, stream>>>(
        (const uint16_t*)q, (const uint16_t*)k_cache, (const uint16_t*)v_cache, idx, lens, part,
        Lmax, Hq, Hkv, block, topk, splits, c);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (D == 64)
    dcombine_kernel<64><<<heads, 64, 0, stream>>>(part, lens, (uint16_t*)out, Lmax, Hq, splits);
  else
    dcombine_kernel<128><<<heads, 64, 0, stream>>>(part, lens, (uint16_t*)out, Lmax, Hq, splits);
  return hipGetLastError();
}

}  // namespace bsattn
