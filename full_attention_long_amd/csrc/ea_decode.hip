// Decode with a mode-aware KV cache: one new token per sequence attends to
// its cached keys, FA heads to all of them, SA heads to the sink blocks and
// the local window only, so an SA head's cache slot holds just those blocks.
//
// Pages: the FA and SA equations of the preliminaries and the hybrid-head
// output equation of "Elastic Attention: Test-time Adaptive Sparsity Ratios
// for Efficient Transformers" (the same visibility rule as the prefill, for a
// query at the last position of a sequence one token longer), and the KV-cache
// memory limits its long-context experiments report for baselines at 256K.
//
// Cache slot of (sequence b, KV head g): cap blocks of 64 tokens, K and V
// each.  FA: ceil(max_len / 64) blocks, logical block kb at physical kb.  SA:
// n_sink + R blocks, R = w at max_len (the window only grows with the length,
// by at most one block per block, so its start never moves back): a sink block
// kb < n_sink stays at kb, a later block at n_sink + (kb - n_sink) mod R, where
// it overwrites a block no later query can see.  (When n_sink + R covers the
// whole length the slot is not a ring.)  The query at position p sees, as in
// the prefill of a sequence of length p + 1: every key j <= p (FA), or the
// sinks and the w(ceil((p + 1) / 64)) blocks ending at its own (SA).
#include "ea_internal.h"

#include <math.h>

namespace ea {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kDecodeWaves = 4;
constexpr int kDecodeThreads = kDecodeWaves * 64;

__host__ __device__ inline int sa_window(int N, int n_sink, int window_blocks, float keep) {
  if (window_blocks > 0) return window_blocks;
  const double k = floor(static_cast<double>(keep) * static_cast<double>(N) + 0.5);
  const int kk = static_cast<int>(k);
  return (n_sink + 1 > kk ? n_sink + 1 : kk) - n_sink;
}

// 64-token block pb of the cache: K rows, then V rows 64 * d elements later.
__device__ __forceinline__ int64_t block_offset(const CacheView& c, int64_t pb) {
  return pb * 2 * kBlock * c.d;
}

__device__ __forceinline__ int64_t phys_block(const CacheView& c, int64_t slot, int kb) {
  const int ring = c.ring[slot];
  const int pb = (ring == 0 || kb < c.n_sink) ? kb : c.n_sink + (kb - c.n_sink) % ring;
  return c.base[slot] + pb;
}

// Slot table: capacity, ring size and first block of every (b, g), by an
// exclusive scan of the capacities in one workgroup; lengths start at 0.
__global__ __launch_bounds__(1024) void cache_init_kernel(CacheView c, const int8_t* __restrict__ modes) {
  __shared__ int64_t part[1024];
  const int nslot = c.B * c.Hkv;
  const int NB = (c.max_len + kBlock - 1) / kBlock;
  const int R = sa_window(NB, c.n_sink, c.window_blocks, c.keep_fraction);
  const int per = (nslot + 1023) / 1024;
  const int s0 = threadIdx.x * per, s1 = min(nslot, s0 + per);
  int64_t sum = 0;
  for (int s = s0; s < s1; ++s) {
    const bool sa = modes[s] != 0 && c.n_sink + R < NB;
    c.cap[s] = sa ? c.n_sink + R : NB;
    c.ring[s] = sa ? R : 0;
    c.mode[s] = modes[s] != 0 ? 1 : 0;
    sum += c.cap[s];
  }
  part[threadIdx.x] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t acc = 0;
    for (int i = 0; i < 1024; ++i) {
      const int64_t t = part[i];
      part[i] = acc;
      acc += t;
    }
  }
  __syncthreads();
  int64_t acc = part[threadIdx.x];
  for (int s = s0; s < s1; ++s) {
    c.base[s] = acc;
    acc += c.cap[s];
  }
  for (int b = threadIdx.x; b < c.B; b += blockDim.x) c.lengths[b] = 0;
  if (threadIdx.x == 1023) c.valid[0] = acc <= c.area_blocks ? 1 : 0;  // acc = total blocks
}

// Zero-fill of the K/V blocks (rows not yet written are masked out by the
// attention, and must be finite there).
__global__ __launch_bounds__(256) void zero_kernel(u32x4* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = u32x4{0, 0, 0, 0};
}

__device__ __forceinline__ int find_seq(const int32_t* cu, int B, int64_t t) {
  int lo = 0, hi = B;  // invariant: cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Prompt rows into the cache: row (t, g) of K and V, if its block is one a
// later query can see (FA: all; SA ring: the sinks and the last R blocks).
// One thread per 16-byte chunk.
__global__ __launch_bounds__(256) void cache_fill_kernel(CacheView c, const int32_t* __restrict__ cu,
                                                         int64_t T, const uint16_t* __restrict__ K,
                                                         const uint16_t* __restrict__ V) {
  const int cpr = c.d / 8;
  const int64_t total = T * c.Hkv * cpr;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = i / cpr;
    const int ch = static_cast<int>(i - row * cpr);
    const int64_t t = row / c.Hkv;
    const int g = static_cast<int>(row - t * c.Hkv);
    const int b = find_seq(cu, c.B, t);
    const int L = cu[b + 1] - cu[b];
    const int p = static_cast<int>(t - cu[b]);
    // precondition violated (a sequence past max_len, or cu_seqlens not
    // non-decreasing): leave the slot alone
    if (L > c.max_len || p < 0 || p >= L || !c.valid[0]) continue;
    const int64_t slot = static_cast<int64_t>(b) * c.Hkv + g;
    const int kb = p / kBlock;
    const int ring = c.ring[slot];
    if (ring != 0 && kb >= c.n_sink && kb <= (L - 1) / kBlock - ring) continue;
    const int64_t dst = block_offset(c, phys_block(c, slot, kb)) + (p % kBlock) * c.d + ch * 8;
    const int64_t src = row * c.d + ch * 8;
    *reinterpret_cast<u32x4*>(c.K + dst) = *reinterpret_cast<const u32x4*>(K + src);
    *reinterpret_cast<u32x4*>(c.V + dst) = *reinterpret_cast<const u32x4*>(V + src);
  }
  if (blockIdx.x == 0)
    for (int b = threadIdx.x; b < c.B; b += blockDim.x) {
      // a length outside [0, max_len] (contents that break the precondition)
      // marks the sequence full, so that no decode step writes its slot
      const int L = cu[b + 1] - cu[b];
      c.lengths[b] = (L >= 0 && L <= c.max_len) ? L : c.max_len;
    }
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ i16x4 ds_read_tr(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// One workgroup per (chunk of visible key blocks, KV head, sequence); each of
// its 4 waves takes every 4th block of the chunk.  A wave holds the G <= 16
// query heads of the group as the B operand of S^T = K Q^T (16x16x32 bf16
// MFMA, K rows loaded straight from the cache as the A operand), keeps an
// online softmax per head, and accumulates O^T += V^T P^T with V^T read from a
// per-wave LDS copy of the block by transposing reads.  The chunk's partial
// (normalised O and LSE per head) goes to the workspace for the combine.
template <int D>
__global__ __launch_bounds__(kDecodeThreads) void decode_attn_kernel(CacheView c, DecodeArgs a) {
  constexpr int NU = D / 32;     // 32-wide d steps of S^T
  constexpr int NM = D / 16;     // 16-row d tiles of O^T
  constexpr int VROW = D + 16;   // padded LDS row of V (elements)
  // per-wave V copies; after the block loop the same memory holds the
  // cross-wave reduction
  __shared__ __attribute__((aligned(16))) uint16_t Vs[kDecodeWaves][kBlock * VROW];
  static_assert(sizeof(Vs) >= sizeof(float) * kDecodeWaves * 16 * (D + 3), "reduction must fit");

  const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int64_t slot = static_cast<int64_t>(b) * c.Hkv + g;
  const int pos = c.lengths[b];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, lg = lane / 16, li = lane % 16;
  const int64_t part0 = (static_cast<int64_t>(b) * a.Hq + static_cast<int64_t>(g) * a.G) * a.n_chunks;
  const bool full = pos < 0 || pos >= c.max_len || !c.valid[0];
  const int qb = pos / kBlock;
  const int mode = c.mode[slot];
  const int w = sa_window(qb + 1, c.n_sink, c.window_blocks, c.keep_fraction);
  const KeyRange kr = key_range(mode, qb, qb, c.n_sink, w);
  const int n_vis = full ? 0 : kr.count();
  const int v0 = chunk * a.chunk_blocks, v1 = min(n_vis, v0 + a.chunk_blocks);

  // The new token's K and V rows go to position pos of the slot, written by
  // the workgroup whose chunk holds that block (the last visible one), before
  // its waves read the block.
  if (!full && chunk == (n_vis - 1) / a.chunk_blocks) {
    const int64_t dst = block_offset(c, phys_block(c, slot, qb)) + (pos % kBlock) * D;
    for (int ch = threadIdx.x; ch < D / 8; ch += kDecodeThreads) {
      *reinterpret_cast<u32x4*>(c.K + dst + ch * 8) = *reinterpret_cast<const u32x4*>(a.k_new + slot * D + ch * 8);
      *reinterpret_cast<u32x4*>(c.V + dst + ch * 8) = *reinterpret_cast<const u32x4*>(a.v_new + slot * D + ch * 8);
    }
    __syncthreads();
  }

  if (v0 >= v1) {  // nothing visible in this chunk
    if (threadIdx.x < a.G) a.lse_part[(part0 + static_cast<int64_t>(threadIdx.x) * a.n_chunks) + chunk] = -INFINITY;
    return;
  }

  // Q^T as the B operand: lane (lg, li) holds head li, dims 32u + 8 lg .. + 7.
  bf16x8 qf[NU];
  {
    const bool hv = li < a.G;
    const uint16_t* qrow = a.q + (static_cast<int64_t>(b) * a.Hq + g * a.G + (hv ? li : 0)) * D;
#pragma unroll
    for (int u = 0; u < NU; ++u)
      qf[u] = hv ? *reinterpret_cast<const bf16x8*>(qrow + 32 * u + 8 * lg) : bf16x8{};
  }

  f32x4 o[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) o[m] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;
  const float cs = a.scale * kLog2e;
  uint16_t* vs = Vs[wave];

  for (int vi = v0 + wave; vi < v1; vi += kDecodeWaves) {
    const int kb = vi < kr.r1_end ? vi : kr.r2_beg + (vi - kr.r1_end);
    const int64_t blk = block_offset(c, phys_block(c, slot, kb));
    const uint16_t* Kb = c.K + blk;
    const uint16_t* Vb = c.V + blk;
    // V block -> registers now, LDS after the scores
    constexpr int NV = kBlock * D / 8 / 64;  // 16-byte chunks per lane
    u32x4 vreg[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) vreg[k] = *reinterpret_cast<const u32x4*>(Vb + (k * 64 + lane) * 8);
    // S^T tiles: 16 keys each; lane holds keys 16t + 4 lg + i for head li
    f32x4 s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      s[t] = f32x4{};
#pragma unroll
      for (int u = 0; u < NU; ++u)
        s[t] = mfma16(*reinterpret_cast<const bf16x8*>(Kb + (16 * t + li) * D + 32 * u + 8 * lg), qf[u], s[t]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = kb * kBlock + 16 * t + 4 * lg + i;
        const float sc = j <= pos ? s[t][i] * cs : -INFINITY;
        s[t][i] = sc;
        mx = fmaxf(mx, sc);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - mn);  // 0 on the first block
    m_run = mn;
    float ls = 0.f;
    bf16x8 pb[2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[t][i] - mn);
        ls += p;
        pb[t / 2][4 * (t & 1) + i] = static_cast<__bf16>(p);
      }
    l_run = l_run * alpha + ls;
#pragma unroll
    for (int m = 0; m < NM; ++m) o[m] *= alpha;
    // V rows into this wave's LDS copy (the wave's previous reads of it are
    // done: LDS serves one wave's instructions in order)
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int ci = k * 64 + lane, row = ci / (D / 8), col = (ci % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(vs + row * VROW + col) = vreg[k];
    }
    // O^T += V^T P^T over two 32-key steps: keys 32 c2 + 4 lg + 0..3 and
    // 32 c2 + 16 + 4 lg + 0..3, the order P^T holds them in
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint16_t* base = vs + (32 * c2 + 4 * lg + li / 4) * VROW + 16 * m + 4 * (li & 3);
        const i16x4 lo = ds_read_tr(base);
        const i16x4 hi = ds_read_tr(base + 16 * VROW);
        const i16x8 v8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[m] = mfma16(__builtin_bit_cast(bf16x8, v8), pb[c2], o[m]);
      }
    }
  }

  // Combine the 4 waves: per head li, (m, l) and O^T rows 16 m + 4 lg + i.
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  __syncthreads();  // every wave is done with its V copy
  float (*red_m)[16] = reinterpret_cast<float (*)[16]>(&Vs[0][0]);
  float (*red_l)[16] = red_m + kDecodeWaves;
  float (*red_o)[16][D + 1] = reinterpret_cast<float (*)[16][D + 1]>(red_l + kDecodeWaves);
  if (lg == 0) {
    red_m[wave][li] = m_run;
    red_l[wave][li] = l_run;
  }
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) red_o[wave][li][16 * m + 4 * lg + i] = o[m][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < a.G * D; idx += kDecodeThreads) {
    const int h = idx / D, dim = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kDecodeWaves; ++k) M = fmaxf(M, red_m[k][h]);
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int k = 0; k < kDecodeWaves; ++k) {
      const float e = red_m[k][h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(red_m[k][h] - M);
      L += e * red_l[k][h];
      acc += e * red_o[k][h][dim];
    }
    const int64_t pi = part0 + static_cast<int64_t>(h) * a.n_chunks + chunk;
    a.o_part[pi * D + dim] = acc / L;
    if (dim == 0) a.lse_part[pi] = (M + __log2f(L)) * kLn2;
  }
}

// Final O and LSE of one (sequence, query head) from its chunks' partials,
// one workgroup per 32 of the D dims: thread group q of 8 (32 threads, one
// per dim) owns chunks q, q + 8, ..., and loads their LSEs and partial rows
// at once (one memory latency), then the chunk-LSE max and the weight sum are
// reduced over the workgroup and each group's weighted sums are added.  The
// (b, 0, 0) workgroup then advances lengths[b] past the new token.
constexpr int kCombineDims = 32;
constexpr int kCombineGroups = 256 / kCombineDims;
constexpr int kCombinePer = 16;  // chunks per thread held in registers

template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(CacheView c, DecodeArgs a) {
  __shared__ float red[2][kCombineGroups];
  __shared__ float acc_s[kCombineGroups][kCombineDims];
  const int hq = blockIdx.x, b = blockIdx.y, slice = blockIdx.z, tid = threadIdx.x;
  const int64_t p0 = (static_cast<int64_t>(b) * a.Hq + hq) * a.n_chunks;
  const int nc = a.n_chunks;  // <= 2048, checked on the host
  const int dl = tid % kCombineDims, grp = tid / kCombineDims;
  const int dim = slice * kCombineDims + dl;
  // this thread's chunks: grp + 8 m; the first kCombinePer in registers,
  // any further ones (nc > 128) read in a second pass
  float lk[kCombinePer], ok[kCombinePer];
  float mx = -INFINITY;
#pragma unroll
  for (int m = 0; m < kCombinePer; ++m) {
    const int k = grp + kCombineGroups * m;
    lk[m] = k < nc ? a.lse_part[p0 + k] : -INFINITY;
    ok[m] = k < nc ? a.o_part[(p0 + k) * D + dim] : 0.f;
    mx = fmaxf(mx, lk[m]);
  }
  for (int k = grp + kCombineGroups * kCombinePer; k < nc; k += kCombineGroups)
    mx = fmaxf(mx, a.lse_part[p0 + k]);
  // lanes of one group hold the same chunks: the group's max is any lane's
  if (dl == 0) red[0][grp] = mx;
  __syncthreads();
  float M = red[0][0];
#pragma unroll
  for (int q = 1; q < kCombineGroups; ++q) M = fmaxf(M, red[0][q]);
  float ls = 0.f, acc = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int m = 0; m < kCombinePer; ++m) {
      if (lk[m] != -INFINITY) {
        const float e = expf(lk[m] - M);
        ls += e;
        acc += e * ok[m];
      }
    }
    for (int k = grp + kCombineGroups * kCombinePer; k < nc; k += kCombineGroups) {
      const float l = a.lse_part[p0 + k];
      if (l != -INFINITY) {
        const float e = expf(l - M);
        ls += e;
        acc += e * a.o_part[(p0 + k) * D + dim];
      }
    }
  }
  if (dl == 0) red[1][grp] = ls;
  acc_s[grp][dl] = acc;
  __syncthreads();
  if (grp == 0) {
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int q = 0; q < kCombineGroups; ++q) {
      L += red[1][q];
      o += acc_s[q][dl];
    }
    const int64_t orow = (static_cast<int64_t>(b) * a.Hq + hq) * D;
    a.O[orow + dim] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(L > 0.f ? o / L : 0.f));
    if (dim == 0 && a.lse) a.lse[static_cast<int64_t>(b) * a.Hq + hq] = L > 0.f ? M + logf(L) : -INFINITY;
    if (hq == 0 && dim == 0 && c.valid[0] && c.lengths[b] < c.max_len) c.lengths[b] += 1;
  }
}

}  // namespace

CacheLayout cache_layout(int32_t B, int32_t Hkv) {
  auto align = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const size_t ns = static_cast<size_t>(B) * Hkv;
  CacheLayout l{};
  size_t off = 0;
  l.lengths = off; off = align(off + sizeof(int32_t) * B);
  l.cap = off;     off = align(off + sizeof(int32_t) * ns);
  l.ring = off;    off = align(off + sizeof(int32_t) * ns);
  l.base = off;    off = align(off + sizeof(int64_t) * ns);
  l.mode = off;    off = align(off + ns);
  l.valid = off;   off = align(off + sizeof(int32_t));
  l.blocks = off;
  return l;
}

int32_t cache_slot_blocks(int mode, int32_t max_len, int32_t n_sink, int32_t window_blocks,
                          float keep_fraction) {
  const int NB = (max_len + kBlock - 1) / kBlock;
  const int R = sa_window(NB, n_sink, window_blocks, keep_fraction);
  return mode != 0 && n_sink + R < NB ? n_sink + R : NB;
}

hipError_t launch_cache_init(const CacheView& c, const int8_t* modes, hipStream_t st) {
  hipLaunchKernelGGL(cache_init_kernel, dim3(1), dim3(1024), 0, st, c, modes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = c.area_blocks * 2 * kBlock * c.d / 8;  // 16-byte chunks of the block area
  if (n == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>(n / 256 + 1 < 65536 ? n / 256 + 1 : 65536);
  hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, st, reinterpret_cast<u32x4*>(c.K), n);
  return hipGetLastError();
}

hipError_t launch_cache_fill(const CacheView& c, const int32_t* cu, int64_t T, const void* K,
                             const void* V, hipStream_t st) {
  const int64_t n = T * c.Hkv * (c.d / 8);
  const unsigned grid = static_cast<unsigned>(n / 256 + 1 < 65536 ? n / 256 + 1 : 65536);
  hipLaunchKernelGGL(cache_fill_kernel, dim3(grid), dim3(256), 0, st, c, cu, T,
                     static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V));
  return hipGetLastError();
}

hipError_t launch_decode(const CacheView& c, const DecodeArgs& a, hipStream_t st) {
  // append + chunked attention, then the merge of the chunks (a kernel
  // boundary makes the partials of every XCD visible to the merge)
  const dim3 grid(static_cast<unsigned>(a.n_chunks), static_cast<unsigned>(c.Hkv),
                  static_cast<unsigned>(c.B));
  if (c.d == 128) {
    hipLaunchKernelGGL((decode_attn_kernel<128>), grid, dim3(kDecodeThreads), 0, st, c, a);
    hipLaunchKernelGGL((decode_combine_kernel<128>), dim3(a.Hq, c.B, 128 / kCombineDims), dim3(256),
                       0, st, c, a);
  } else {
    hipLaunchKernelGGL((decode_attn_kernel<64>), grid, dim3(kDecodeThreads), 0, st, c, a);
    hipLaunchKernelGGL((decode_combine_kernel<64>), dim3(a.Hq, c.B, 64 / kCombineDims), dim3(256),
                       0, st, c, a);
  }
  return hipGetLastError();
}

}  // namespace ea
