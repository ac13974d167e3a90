// Steps 2-3 of block selection for many key blocks (nb > 1024): the score matrix is built in
// the workspace by a matrix product with fp32 accuracy (three-part bf16 split on the bf16
// MFMA), then each row's top-k is found by one work-group.
//
// SparseFormer page ("2026 新一代卷积与Transformer网络架构技术演进与性能对比"), section
// "SparseFormer 注意力实现": block_scores = einsum over d of the pooled query and key blocks
// (no scale), then torch.topk with k = int(topk_ratio * num_blocks) per row. MSA page
// ("从M2.7到M3：多模态模型稀疏注意力架构设计与实现全解析") §3.2: 1M-token context at block 128, i.e.
// 8192 key blocks per row; §3.3: block scores as a matrix product.
//
// score_gemm_kernel: S[b,h] = qbar[b,h] (nb x D) * kbar[b,g]^T, fp32, unscaled (details at the
// kernel).
//
// topk_rows_kernel: one work-group (256 threads) per row; thread t holds the 32-column chunk
// j = 32t .. 32t+31 (nb = 8192) as order-preserving keys. The k-th largest key T is found from
// key-bucket counts and the keys of one bucket (details at the kernel); keys > T are kept
// and keys == T fill the remaining places in ascending j (the lower index wins).
// Output positions come from block-wide exclusive scans, so the row is written in ascending j.
// Causal option: as in the fused kernel, columns j > i get key 0, column i the largest key,
// the row keeps min(topk, i+1) blocks and its remaining places are set to -1; a row with
// i + 1 <= topk keeps all of 0..i and is written without reading its scores.
//
// Group-shared selection (GQA, MSA §3.1): group_sum_kernel adds the pooled queries of each
// group's G heads into the rows of its first head (the scores of the sum are the sum of the
// heads' scores), the product runs once per (batch, KV head) on those rows, and each row's
// top-k is written to the idx rows of all G heads.
#include "common.h"
#include "launch.h"

namespace bsattn {
namespace {

// ---------------------------------------------------------------- score GEMM
// fp32 products on the bf16 MFMA: every pooled value x is split into three bf16 parts
// x = x0 + x1 + x2 (x0 = bf16(x), x1 = bf16(x - x0), x2 = x - x0 - x1; exact for normal
// values, each part carrying the next 8 of x's 24 significant bits), and
//   q.k = q0.k0 + (q0.k1 + q1.k0 + q0.k2 + q1.k1 + q2.k0) + (q1.k2 + q2.k1 + q2.k2).
// The six products go to one fp32 accumulator, the smallest first; the last three are left
// out: they are below 2^-23 of sum_d |q_d k_d|, fp32 rounding level. A product of two bf16
// parts is exact in fp32, and the accumulator's rounding is that of an fp32 product (a CPU
// simulation of this order: at most 5e-7 of sum_d |q_d k_d|, an fp32 matrix product 2e-7).
// (A second accumulator for the five smaller products halves that error but takes 64 more
// registers: 2 instead of 3 waves per SIMD, 5 % slower at 8192 key blocks.) The bf16 MFMA
// does 16 times the fp32 one's work per cycle, so the six products take 3/8 of an fp32
// product's matrix time.
//
// One work-group (4 waves) computes a 128 x 128 tile of S, each wave a 64 x 64 quarter as
// 2 x 2 tiles of v_mfma_f32_32x32x16_bf16 (A = query rows, B = key rows; lane l takes row
// l % 32 and d = 16c + 8(l / 32) .. +7 of k-step c on both operands). The pooled rows go
// through LDS 16 values of d at a time: every thread loads two 16-byte pieces of query rows and
// two of key rows, splits them and stores the parts (two buffers, one barrier per step; the
// next step's loads fly during the current step's products). Part p of an operand is
// [128 rows][16 bf16]; the 16-byte half h of row r sits at half h ^ ((r >> 3) & 1), so the 16
// lanes of a row read touch every bank once. Every score goes through the same instruction
// sequence, so equal pooled key blocks give bit-equal scores.
constexpr int kGemmTile = 128;

__device__ __forceinline__ void split3(const f32x4& v, u32x2 part[3]) {
  float r[4];
  const uint32_t a0 = pack_bf16x2(v[0], v[1]), a1 = pack_bf16x2(v[2], v[3]);
  r[0] = v[0] - bf16lo(a0); r[1] = v[1] - bf16hi(a0);
  r[2] = v[2] - bf16lo(a1); r[3] = v[3] - bf16hi(a1);
  const uint32_t b0 = pack_bf16x2(r[0], r[1]), b1 = pack_bf16x2(r[2], r[3]);
  r[0] -= bf16lo(b0); r[1] -= bf16hi(b0);
  r[2] -= bf16lo(b1); r[3] -= bf16hi(b1);
  part[0] = u32x2{a0, a1};
  part[1] = u32x2{b0, b1};
  part[2] = u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
}

template <int D>
__global__ __launch_bounds__(256) void score_gemm_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, float* __restrict__ S,
    int Hq, int Hkv, int nb, int tiles, bool group, bool causal) {
  constexpr int NC = D / 16;                  // k-steps
  constexpr int PART = kGemmTile * 32;        // bytes of one part of one operand
  constexpr int BUF = 6 * PART;               // q parts 0..2, k parts 0..2
  __shared__ __attribute__((aligned(16))) char lds[2 * BUF];

  // tile index: (b*HS + s) * per + u, s a selection head (a query head, or a KV head whose
  // group's summed queries sit in the rows of its first head), u the tile (ti, tj) of that
  // head's matrix in row-major order: u = ti * tiles + tj, or, causal, over the lower triangle
  // only, u = ti (ti + 1) / 2 + tj with tj <= ti. A causal row i reads columns up to the end of
  // i's 32-column chunk, inside i's own 128-column tile, so the tiles above the diagonal are
  // never read and not formed. Tiles of one (batch, selection head) share their pooled rows:
  // keep them on one XCD's L2.
  const int G = Hq / Hkv, HS = group ? Hkv : Hq;
  const int64_t per = causal ? (int64_t)tiles * (tiles + 1) / 2 : (int64_t)tiles * tiles;
  const int64_t t = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bh = t / per;                         // b * HS + s
  const int u = (int)(t - bh * per);
  int ti, tj;
  if (causal) {   // float root, then one step either way puts ti (ti+1)/2 <= u < (ti+1)(ti+2)/2
    ti = (int)((sqrtf(8.f * (float)u + 1.f) - 1.f) * 0.5f);
    if (ti * (ti + 1) / 2 > u) --ti;
    if ((ti + 1) * (ti + 2) / 2 <= u) ++ti;
    tj = u - ti * (ti + 1) / 2;
  } else {
    ti = u / tiles;
    tj = u - ti * tiles;
  }
  const int sh = (int)(bh % HS), b = (int)(bh / HS);
  const int hq = group ? sh * G : sh;                 // query head of the pooled rows
  const int g = group ? sh : sh / G;
  const float* Q = qbar + ((int64_t)b * Hq + hq) * nb * D;
  const float* K = kbar + ((int64_t)b * Hkv + g) * nb * D;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, half = lane >> 5;

  // loads: rows lr and lr + 64 of the tile (clamped to the last pooled row; the scores of
  // rows and columns past nb are not stored), d = 16c + 4 * quad .. +3
  const int lr = tid >> 2, quad = tid & 3;
  const float* src[2][2];                     // [q or k][row]
  int soff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = lr + 64 * u;
    const int qr = ti * kGemmTile + r, kr = tj * kGemmTile + r;
    src[0][u] = Q + (int64_t)(qr < nb ? qr : nb - 1) * D + 4 * quad;
    src[1][u] = K + (int64_t)(kr < nb ? kr : nb - 1) * D + 4 * quad;
    soff[u] = r * 32 + 16 * ((quad >> 1) ^ ((r >> 3) & 1)) + 8 * (quad & 1);
  }
  int aoff[2], boff[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int ra = 64 * (wave >> 1) + 32 * a + l32, rb = 64 * (wave & 1) + 32 * a + l32;
    aoff[a] = ra * 32 + 16 * (half ^ ((ra >> 3) & 1));
    boff[a] = 3 * PART + rb * 32 + 16 * (half ^ ((rb >> 3) & 1));
  }
  f32x4 st[2][2];
  auto load = [&](int c) {
#pragma unroll
    for (int o = 0; o < 2; ++o)
#pragma unroll
      for (int u = 0; u < 2; ++u) st[o][u] = *(const f32x4*)(src[o][u] + 16 * c);
  };
  auto store = [&](char* buf) {
#pragma unroll
    for (int o = 0; o < 2; ++o)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u32x2 part[3];
        split3(st[o][u], part);
#pragma unroll
        for (int p = 0; p < 3; ++p) *(u32x2*)(buf + (3 * o + p) * PART + soff[u]) = part[p];
      }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][c][r] = 0.f;

  load(0);
  store(lds);
  __syncthreads();
  for (int c = 0; c < NC; ++c) {
    const char* cur = lds + (c & 1) * BUF;
    if (c + 1 < NC) load(c + 1);
    bf16x8 qa[3][2], kb[3][2];
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        qa[p][a] = *(const bf16x8*)(cur + p * PART + aoff[a]);
        kb[p][a] = *(const bf16x8*)(cur + p * PART + boff[a]);
      }
    // smallest products first
    constexpr int PQ[6] = {2, 1, 0, 1, 0, 0}, PK[6] = {0, 1, 2, 0, 1, 0};
#pragma unroll
    for (int x = 0; x < 6; ++x)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
          acc[a][cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[PQ[x]][a], kb[PK[x]][cc], acc[a][cc], 0, 0, 0);
    if (c + 1 < NC) store(lds + ((c + 1) & 1) * BUF);
    __syncthreads();
  }

  // acc[a][c][r]: row 64(wave/2) + 32a + 8(r/4) + 4*half + r%4, column 64(wave%2) + 32c + l32.
  // The scores go out past the caches (nontemporal stores: 2.9 % faster selection at 8192 key
  // blocks); the top-k kernel reads them back with ordinary loads (nontemporal loads there
  // were 15 % slower).
  float* Sbh = S + bh * nb * nb;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int row0 = ti * kGemmTile + 64 * (wave >> 1) + 32 * a;
      const int col = tj * kGemmTile + 64 * (wave & 1) + 32 * cc + l32;
      if (row0 >= nb || col - l32 >= nb) continue;   // the half tile past nb (nb % 128 = 64)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + 8 * (r >> 2) + 4 * half + (r & 3);
        __builtin_nontemporal_store(acc[a][cc][r], Sbh + (int64_t)row * nb + col);
      }
    }
}

// ---------------------------------------------------------------- per-row top-k
constexpr int kTopkThreads = 256;
constexpr int kPerThread = 32;             // columns per thread: nb <= 8192
static_assert(kGemmTile % kPerThread == 0, "a causal row's chunk must lie in its own tile");

__device__ __forceinline__ int block_sum(int v, int* red) {
  // wave sum (DPP within 16 lanes, then across 16 and 32 lanes), then the 4 wave sums
  // through LDS (caller syncs around reuse)
  v = group_sum<16>(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const int total = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return total;
}

// exclusive prefix of v over threads in thread order, and the block total
__device__ __forceinline__ int block_exclusive_scan(int v, int* red, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) red[w] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < w) before += red[i];
    tot += red[i];
  }
  __syncthreads();
  *total = tot;
  return before + incl - v;
}

constexpr int kBinBits = 11;
constexpr int kBins = 1 << kBinBits;       // key buckets per level
constexpr int kMaxCand = 4 * kWave;        // bucket size one wave resolves (4 keys per lane)

// m * 2 + (a < b), unsigned: one compare into VCC and one add with that carry (shifts a
// comparison bit into a mask from the bottom; the compiler forms this with three instructions)
__device__ __forceinline__ uint32_t shift_in_lt(uint32_t m, uint32_t a, uint32_t b) {
  asm("v_cmp_lt_u32 vcc, %1, %2\n\tv_addc_co_u32 %0, vcc, %0, %0, vcc"
      : "+v"(m) : "v"(a), "v"(b) : "vcc");
  return m;
}
__device__ __forceinline__ uint32_t shift_in_eq(uint32_t m, uint32_t a, uint32_t b) {
  asm("v_cmp_eq_u32 vcc, %1, %2\n\tv_addc_co_u32 %0, vcc, %0, %0, vcc"
      : "+v"(m) : "v"(a), "v"(b) : "vcc");
  return m;
}

// Order-preserving key of a float (as order_key): -0.0 becomes +0.0 by adding +0.0, then the
// sign bit decides between flipping every bit (negative) and setting the top bit.
__device__ __forceinline__ uint32_t order_key_fast(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// rows of S: (b * HS + s) * nb + i; the top-k of a row goes to the idx rows of the G query
// heads s*G .. s*G+G-1 of a group (group), or of query head s
//
// The k-th largest key T is found by counting keys into buckets of equal key width (LDS
// counts): bucket = (key - base) >> shift, so a bucket is a key range, equal keys share one
// and every key of a higher bucket is larger than every key of a lower one. A scan from the
// top finds the bucket holding the k-th largest key. If it holds more than kMaxCand keys, its
// range is cut into buckets again (11 bits narrower, at most three levels over the 32-bit
// keys); otherwise its keys go to LDS and one wave finds T among them bit by bit with ballots.
// A bucket one key wide holds equal keys only, and that key is T. CAUSAL: the row's own forced
// block (all-ones key) falls into the top bucket of every level and columns past the row's
// admissible range (key 0) are not counted. nb is a multiple of 64, so a thread's 32 columns
// are all inside the row or all past it.
template <bool CAUSAL>
__global__ __launch_bounds__(kTopkThreads) void topk_rows_kernel(const float* __restrict__ S,
                                                                 int32_t* __restrict__ idx,
                                                                 int nb, int topk, int G) {
  __shared__ int red[4];
  __shared__ uint32_t redu[8];
  __shared__ int hist[kBins];
  __shared__ uint32_t cand[kMaxCand];
  __shared__ int found[3];                 // bucket of the k-th key, keys above it, candidates
  __shared__ uint32_t t_found[2];          // T, candidates above T
  const int64_t row = blockIdx.x;
  const int i = (int)(row % nb);           // query block of this row
  const int kr = CAUSAL && i + 1 < topk ? i + 1 : topk;
  const float* srow = S + row * nb;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  if (CAUSAL && kr == i + 1) {   // (block-uniform) the row keeps all its blocks 0..i, in order
    const int64_t bs = row / nb;
    for (int hh = 0; hh < G; ++hh) {
      int32_t* out = idx + ((bs * G + hh) * nb + i) * topk;
      for (int p = t; p < topk; p += kTopkThreads) out[p] = p <= i ? p : -1;
    }
    return;
  }
  const int j0 = t * kPerThread;
  const bool has = j0 < (CAUSAL ? i + 1 : nb);   // some admissible column (all, unless causal)
  uint32_t key[kPerThread];
  if (has) {
    f32x4 v[kPerThread / 4];
#pragma unroll
    for (int e = 0; e < kPerThread / 4; ++e) v[e] = *(const f32x4*)(srow + j0 + 4 * e);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) key[e] = order_key_fast(v[e / 4][e % 4]);
    if constexpr (CAUSAL) {                  // columns past the row: 0; the own block: all ones
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) {
        const int j = j0 + e;
        key[e] = j > i ? 0u : j == i ? 0xFFFFFFFFu : key[e];
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) key[e] = 0u;
  }

  // ---- key range of the scored columns (causal: key - 1 takes the uncounted 0 to all ones and
  // key + 1 takes the forced all-ones key to 0, so neither bounds the range)
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  if (has) {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      kmin = min(kmin, CAUSAL ? key[e] - 1u : key[e]);
      kmax = max(kmax, CAUSAL ? key[e] + 1u : key[e]);
    }
  }
  for (int b = t; b < kBins; b += kTopkThreads) hist[b] = 0;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
  }
  if (lane == 0) { redu[w] = kmin; redu[4 + w] = kmax; }
  if (t == 0) { found[0] = 0; found[1] = 0; found[2] = 0; }
  __syncthreads();
  kmin = min(min(redu[0], redu[1]), min(redu[2], redu[3]));
  kmax = max(max(redu[4], redu[5]), max(redu[6], redu[7]));
  if (CAUSAL) { kmin += 1u; kmax -= 1u; }

  // ---- bucket levels
  uint32_t base = kmin;                    // first key of the current range
  const uint32_t span = kmax > kmin ? kmax - kmin : 0u;
  int shift = span ? 32 - __builtin_clz(span) - kBinBits : 0;
  if (shift < 0) shift = 0;
  bool open = true;                        // the range has no upper end (top bucket so far)
  int above = 0;                           // keys above the current range
  int bT = 0, cb = 0;
  for (int level = 0;; ++level) {
    if (has) {
      if (level == 0) {                      // every counted key lies in the first range
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) {
          const uint32_t b = min((key[e] - base) >> shift, (uint32_t)(kBins - 1));
          if (!CAUSAL || key[e] != 0u) atomicAdd(&hist[b], 1);
        }
      } else {
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) {
          const uint32_t kk = key[e];
          const uint32_t b = (kk - base) >> shift;
          if (kk != 0u && kk >= base && (b < (uint32_t)kBins || open))
            atomicAdd(&hist[min(b, (uint32_t)(kBins - 1))], 1);
        }
      }
    }
    __syncthreads();
    // thread t scans the 8 buckets [kBins - 8(t+1), kBins - 8t) from the top
    const int b_top = kBins - 8 * t - 1;
    int cnt8[8], local = 0;
#pragma unroll
    for (int m = 0; m < 8; ++m) { cnt8[m] = hist[b_top - m]; local += cnt8[m]; }
    int total;
    int run = above + block_exclusive_scan(local, red, &total);   // keys above my buckets
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (run < kr && run + cnt8[m] >= kr) { found[0] = b_top - m; found[1] = run; }
      run += cnt8[m];
    }
    __syncthreads();
    bT = found[0];
    above = found[1];
    cb = hist[bT];
    if (cb <= kMaxCand || shift == 0) break;   // (block-uniform)
    // cut bucket bT into kBins narrower buckets (every thread has read found and hist first)
    base += (uint32_t)bT << shift;
    open = open && bT == kBins - 1;
    shift = shift > kBinBits ? shift - kBinBits : 0;
    __syncthreads();
    for (int b = t; b < kBins; b += kTopkThreads) hist[b] = 0;
    __syncthreads();
  }

  // ---- T from the keys of bucket bT: the keys in [lo, lo + 2^shift), or every key >= lo for
  // the open top bucket
  uint32_t T;
  int tot_gt;                              // keys > T
  const uint32_t lo = base + ((uint32_t)bT << shift);
  const bool top_open = open && bT == kBins - 1;
  if (cb <= kMaxCand) {
    uint32_t cm = 0;                       // bit e: key e is in the bucket
    if (has) {
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) {
        const uint32_t kk = key[e];
        const bool in = kk != 0u && (top_open ? kk >= lo : ((kk - lo) >> shift) == 0u);
        cm |= (uint32_t)in << e;
      }
    }
    if (cm) {
      int p = atomicAdd(&found[2], __builtin_popcount(cm));
      for (uint32_t m = cm; m; m &= m - 1u) cand[p++] = key[__builtin_ctz(m)];
    }
    __syncthreads();
    if (w == 0) {
      const int need = kr - above;          // places left for the bucket's keys (>= 1)
      uint32_t c4[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) c4[m] = lane + kWave * m < cb ? cand[lane + kWave * m] : 0u;
      // the need-th largest candidate key itself (no early exit: T must be a key of the bucket,
      // so that no key of a lower bucket exceeds it)
      uint32_t Tc = 0;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t probe = Tc | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int m = 0; m < 4; ++m) cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(c4[m] >= probe));
        if (cnt >= need) Tc = probe;
      }
      int gtc = 0;
#pragma unroll
      for (int m = 0; m < 4; ++m) gtc += __builtin_popcountll(__builtin_amdgcn_ballot_w64(c4[m] > Tc));
      if (lane == 0) { t_found[0] = Tc; t_found[1] = (uint32_t)gtc; }
    }
    __syncthreads();
    T = t_found[0];
    tot_gt = above + (int)t_found[1];
  } else {                                  // a one-key-wide bucket: all its keys equal T
    T = lo;
    tot_gt = above;
  }

  // ---- the row: keys > T, then keys == T in ascending j until kr places are filled
  uint32_t gtm = 0, eqm = 0;               // bit e: key e > T, key e == T
  if (has) {
#pragma unroll
    for (int e = kPerThread - 1; e >= 0; --e) {   // shifted in from the top: bit e = key e
      gtm = shift_in_lt(gtm, T, key[e]);
      eqm = shift_in_eq(eqm, T, key[e]);
    }
  }
  int tot_eq;
  const int eq_before = block_exclusive_scan(__builtin_popcount(eqm), red, &tot_eq);
  uint32_t selm = gtm;                     // plus this thread's first (need - eq_before) ties
  int nn = kr - tot_gt - eq_before;
  for (uint32_t m = eqm; m && nn > 0; m &= m - 1u, --nn) selm |= m & (0u - m);
  int tot_sel;
  const int pos0 = block_exclusive_scan(__builtin_popcount(selm), red, &tot_sel);
  const int64_t bs = row / nb;             // b * HS + s
  for (int hh = 0; hh < G; ++hh) {
    int32_t* out = idx + ((bs * G + hh) * nb + i) * topk;
    int pos = pos0;
    // (pos < kr holds for consistent counts; it also bounds rows of NaN scores)
    for (uint32_t m = selm; m && pos < kr; m &= m - 1u) out[pos++] = j0 + __builtin_ctz(m);
    for (int p = kr + t; p < topk; p += kTopkThreads) out[p] = -1;   // unused causal places
  }
}

// in place: rows of head g*G of each group += rows of heads g*G+1 .. g*G+G-1, in head order
__global__ __launch_bounds__(256) void group_sum_kernel(float* __restrict__ qbar, int64_t B,
                                                        int Hq, int Hkv, int64_t per_head) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (b, g, element)
  if (e >= B * Hkv * per_head) return;
  const int G = Hq / Hkv;
  const int64_t bg = e / per_head, x = e % per_head;
  float* first = qbar + bg * G * per_head + x;       // head g*G of batch b
  float s = first[0];
  for (int hh = 1; hh < G; ++hh) s += first[hh * per_head];
  first[0] = s;
}

}  // namespace

hipError_t launch_scores_large(int64_t B, int Hq, int Hkv, int nb, int D, float* qbar,
                               const float* kbar, float* S, bool group, bool causal,
                               hipStream_t stream) {
  if (group && Hq > Hkv) {
    const int64_t n = B * Hkv * (int64_t)nb * D;
    group_sum_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, stream>>>(
        qbar, B, Hq, Hkv, (int64_t)nb * D);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int tiles = (nb + kGemmTile - 1) / kGemmTile;
  const int64_t per = causal ? (int64_t)tiles * (tiles + 1) / 2 : (int64_t)tiles * tiles;
  const int64_t n = B * (group ? Hkv : Hq) * per;
  if (D == 64)
    score_gemm_kernel<64><<<dim3((unsigned)n), 256, 0, stream>>>(qbar, kbar, S, Hq, Hkv, nb,
                                                                  tiles, group, causal);
  else
    score_gemm_kernel<128><<<dim3((unsigned)n), 256, 0, stream>>>(qbar, kbar, S, Hq, Hkv, nb,
                                                                   tiles, group, causal);
  return hipGetLastError();
}

hipError_t launch_topk_rows(int64_t rows, int nb, int topk, const float* S, int32_t* idx,
                            bool causal, int G, hipStream_t stream) {
  if (causal)
    topk_rows_kernel<true><<<dim3((unsigned)rows), kTopkThreads, 0, stream>>>(S, idx, nb, topk, G);
  else
    topk_rows_kernel<false><<<dim3((unsigned)rows), kTopkThreads, 0, stream>>>(S, idx, nb, topk, G);
  return hipGetLastError();
}

}  // namespace bsattn
