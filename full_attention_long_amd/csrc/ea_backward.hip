// Backward of the hybrid attention layer: dQ, dK and dV for an upstream
// gradient dO, every head in its routed mode (FA or SA key set), bf16 in and
// out with float32 accumulation.
//
// Pages: the FA and SA equations of the preliminaries and the hybrid-head
// output equation of "Elastic Attention: Test-time Adaptive Sparsity Ratios
// for Efficient Transformers"; the router is trained behind a frozen backbone
// in every layer (training paragraphs), so gradients flow through the
// attention of each routed head to the layers below.
//
// With P = exp(S - LSE) rebuilt from the forward's LSE, and
// D = rowsum(dO * O) = rowsum(P * dP):
//   dV = P^T dO, dP = dO V^T, dS = P * (dP - D), dQ = scale dS K,
//   dK = scale dS^T Q   (dK, dV summed over the G query heads of a KV head).
// Three kernels: bwd_pre_kernel (D and LSE in log2 units per row),
// bwd_dq_kernel (query-tile stationary, the forward's work list and K/V
// tiles: S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T with 32x32x16 MFMAs)
// and bwd_dkv_kernel (key stationary: each pair of waves owns 32 keys of its
// KV head and walks the query blocks that can see them, head by head, one
// wave computing S, P and dV += P^T dO, the other dP and dK += dS^T Q, with
// 16x16x32 MFMAs).
#include "ea_internal.h"

#include <math.h>

#include <type_traits>

namespace ea {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ i16x4 ds_read_tr(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}
__device__ __forceinline__ bf16x8 tr_pair(const uint16_t* lo, const uint16_t* hi) {
  const i16x4 a = ds_read_tr(lo), b = ds_read_tr(hi);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// D[hq, t] = sum_d dO * O and LSE in log2 units, per (token, query head) row;
// the d / 8 threads of a row sit in one wave.
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ O,
                                                      const uint16_t* __restrict__ dO,
                                                      const float* __restrict__ lse, int64_t T,
                                                      int32_t Hq, int32_t d, float* __restrict__ Dv,
                                                      float* __restrict__ lse2) {
  const int cpr = d / 8;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t row = i / cpr;
  const bool ok = row < T * Hq;
  float acc = 0.f;
  if (ok) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(O + i * 8);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(dO + i * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += static_cast<float>(a[e]) * static_cast<float>(b[e]);
  }
  for (int off = cpr / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (ok && i % cpr == 0) {
    const int64_t t = row / Hq;
    const int hq = static_cast<int>(row - t * Hq);
    Dv[static_cast<int64_t>(hq) * T + t] = acc;
    lse2[static_cast<int64_t>(hq) * T + t] = lse[static_cast<int64_t>(hq) * T + t] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dQ: one work item (the forward's query tile of 256 rows, 32 per wave) over
// its visible key blocks.  Per block: K in the row layout (S^T = K Q^T) and in
// the transposing layout (dQ^T += K^T dS^T), V in the row layout
// (dP^T = V dO^T), all three by direct buffer-to-LDS loads one block ahead.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kAttnWaves * 64, 2) void bwd_dq_kernel(BwdArgs a) {
  constexpr int CPR = D / 8;
  constexpr int TILE = kBlock * D;
  constexpr int RPI = 1024 / (2 * D);
  constexpr int NDMA = kBlock / RPI / kAttnWaves;
  constexpr int DT = D / 32;
  constexpr int NQ = D / 16;
  constexpr int KGS = RPI * D + 32;
  constexpr int KTILE = (kBlock / RPI) * KGS;
  constexpr int VSW = (CPR / 4) - 1;
  auto kfold = [](int j) { return D == 128 ? j : (j >> 1); };
  __shared__ __attribute__((aligned(1024))) uint16_t Kr0[KTILE], Kr1[KTILE], Vr0[KTILE], Vr1[KTILE],
      Kt0[TILE], Kt1[TILE];

  const int64_t pos_in_list = list_position(blockIdx.x);
  if (a.meta[kMetaStamp] != a.stamp) return;
  if (pos_in_list >= static_cast<int64_t>(a.meta[kMetaTiles]) * a.Hkv) return;
  const Item it = a.items[a.order[pos_in_list]];
  const int b = it.b, kvh = it.kvh, mode = it.mode;
  const int tok0 = a.cu[b];
  const int L = a.cu[b + 1] - tok0;
  const int ns = a.n_sink, w = a.seq_w[b];
  const int p0 = it.qt * a.BMq;
  const int p1 = min(p0 + a.BMq, L) - 1;
  const int qb0 = p0 / kBlock, qb1 = p1 / kBlock;
  const KeyRange kr = key_range(mode, qb0, qb1, ns, w);
  const int nblk = kr.count();
  auto kb_of = [&](int n) { return n < kr.r1_end ? n : kr.r2_beg + (n - kr.r1_end); };

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, h = lane / 32, lq = lane % 32;
  const int row = wave * 32 + lq;
  const int hh = row / a.BMq;
  const int pos = p0 + row % a.BMq;
  const bool rvalid = hh < a.G && pos < L;
  const int hq = kvh * a.G + hh;
  const int qblk = pos / kBlock;

  bf16x8 qf[NQ], of[NQ];
  {
    const int64_t r = (static_cast<int64_t>(tok0 + pos) * a.Hq + hq) * D;
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      qf[u] = rvalid ? *reinterpret_cast<const bf16x8*>(a.Q + r + 16 * u + 8 * h) : bf16x8{};
      of[u] = rvalid ? *reinterpret_cast<const bf16x8*>(a.dO + r + 16 * u + 8 * h) : bf16x8{};
    }
  }
  const int64_t li = static_cast<int64_t>(hq) * a.T + tok0 + pos;
  const float lrow = rvalid ? a.lse2[li] : INFINITY;  // an invalid row's P is 0
  const float drow = rvalid ? a.Dv[li] : 0.f;
  const float c = a.scale * kLog2e;

  const int rs = a.Hkv * D;
  const uint16_t* Kseq = a.K + (static_cast<int64_t>(tok0) * a.Hkv + kvh) * D;
  const uint16_t* Vseq = a.V + (static_cast<int64_t>(tok0) * a.Hkv + kvh) * D;
  int dma_roff[NDMA], dma_toff[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int r = (wave * NDMA + i) * RPI + lane / CPR;
    dma_roff[i] = (r * rs + ((lane % CPR) ^ kfold(lane / CPR)) * 8) * 2;
    dma_toff[i] = (r * rs + ((lane % CPR) ^ (4 * ((r & 3) & VSW))) * 8) * 2;
  }
  auto dma = [&](const uint16_t* seq, const int* off, uint16_t* tile, int gstride, int kb) {
    const int key0 = kb * kBlock;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(seq + static_cast<int64_t>(key0) * rs), 0,
        static_cast<unsigned>(L - key0) * static_cast<unsigned>(rs) * 2u, kBufferWord3);
#pragma unroll
    for (int i = 0; i < NDMA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)(tile + (wave * NDMA + i) * gstride), 16,
          off[i], 0, 0, 0);
  };
  int koff_e, koff_o;
  {
    const int j = lq % RPI, f = kfold(j), bb = f >> 1, e = f & 1;
    const int base = (lq / RPI) * KGS + j * D + (h ^ e) * 8;
    koff_e = base + 16 * bb;
    koff_o = base - 16 * bb;
  }
  int toff[DT];
  {
    const int vr = 4 * h + (lane & 15) / 4;
    const int clow = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int j = ((lane >> 2) & 3) & VSW;
#pragma unroll
    for (int t = 0; t < DT; ++t) toff[t] = vr * D + (4 * (t ^ j) + clow) * 8 + 4 * (lane & 1);
  }
  // A-operand rows of a row-layout tile times the B fragments, added to init
  auto rowmm = [&](const uint16_t* tile, const bf16x8* bf, f32x16& x0, f32x16& x1, float init) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      x0[e] = init;
      x1[e] = init;
    }
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int o0 = ((u & 1) ? koff_o : koff_e) + 16 * u;
      x0 = mfma32(*reinterpret_cast<const bf16x8*>(tile + o0), bf[u], x0);
      x1 = mfma32(*reinterpret_cast<const bf16x8*>(tile + o0 + (32 / RPI) * KGS), bf[u], x1);
    }
  };

  f32x16 dq[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) dq[t] = f32x16{};

  auto block = [&](int kb, const uint16_t* kr_, const uint16_t* vr_, const uint16_t* kt_) {
    f32x16 s0, s1, p0v, p1v;
    rowmm(kr_, qf, s0, s1, 0.f);
    // dP^T needs only LDS operands: issued here, its products run in the
    // matrix pipe while the exponentials below wait on and consume S
    // dP^T - D straight from the products (the accumulators start at -D; the
    // start value passes through an empty asm so that its 32 broadcast
    // registers are set here rather than hoisted out of the block loop):
    // 32 subtractions per block become 16 register moves
    float nd = -drow;
    asm volatile("" : "+v"(nd));
    rowmm(vr_, of, p0v, p1v, nd);
    // a block every row of the tile sees (the common case) skips the
    // per-element visibility test
    if (block_full(mode, kb, p0, qb0, qb1, ns, w)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], c, -lrow));
        s1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c, -lrow));
      }
    } else {
      const bool blk_ok = block_visible(mode, kb, qblk, ns, w);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = kb * kBlock + 8 * (i / 4) + 4 * h + (i % 4);
        const bool v0 = blk_ok && j <= pos, v1 = blk_ok && j + 32 <= pos;
        s0[i] = v0 ? __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], c, -lrow)) : 0.f;
        s1[i] = v1 ? __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c, -lrow)) : 0.f;
      }
    }
    bf16x8 dsb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x8 t;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = 8 * (q & 1) + e;
        t[e] = q < 2 ? s0[k] * p0v[k] : s1[k] * p1v[k];
      }
      dsb[q] = __builtin_convertvector(t, bf16x8);
    }
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        dq[t] = mfma32(tr_pair(kt_ + toff[t] + 16 * u * D, kt_ + toff[t] + (16 * u + 8) * D),
                       dsb[u], dq[t]);
  };

  if (nblk > 0) {
    dma(Kseq, dma_roff, Kr0, KGS, kb_of(0));
    dma(Vseq, dma_roff, Vr0, KGS, kb_of(0));
    dma(Kseq, dma_toff, Kt0, RPI * D, kb_of(0));
    __syncthreads();
    for (int n = 0; n < nblk; n += 2) {
      const int nx = kb_of(min(n + 1, nblk - 1));
      dma(Kseq, dma_roff, Kr1, KGS, nx);
      dma(Vseq, dma_roff, Vr1, KGS, nx);
      dma(Kseq, dma_toff, Kt1, RPI * D, nx);
      block(kb_of(n), Kr0, Vr0, Kt0);
      __syncthreads();
      if (n + 1 < nblk) {
        const int nx2 = kb_of(min(n + 2, nblk - 1));
        dma(Kseq, dma_roff, Kr0, KGS, nx2);
        dma(Vseq, dma_roff, Vr0, KGS, nx2);
        dma(Kseq, dma_toff, Kt0, RPI * D, nx2);
        block(kb_of(n + 1), Kr1, Vr1, Kt1);
        __syncthreads();
      }
    }
  }

  if (rvalid) {
    uint16_t* dst = a.dQ + (static_cast<int64_t>(tok0 + pos) * a.Hq + hq) * D;
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = dq[t][4 * q + e] * a.scale;
        *reinterpret_cast<bf16x4*>(dst + 32 * t + 8 * q + 4 * h) = __builtin_convertvector(v, bf16x4);
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV: a workgroup owns kDkvKeys keys of one KV head of one sequence and
// walks the query blocks that can see them, each block once per query head of
// the group: tile t = (block qb_hi - t / G, head t % G) is that head's 64 Q
// and dO rows with their LSE and D.  The walk runs downwards from the last
// block, where every key chunk of a head starts, so the workgroups of one head
// that run together read the same Q and dO tiles at about the same time and
// share them in the cache.  The 8 waves form 4 pairs, waves p and
// p + 4 (one SIMD), each pair owning 32 keys as two 16-key tiles, and split
// the work of a tile in two balanced halves:
//   wave p     (A): S = Q K^T, P = exp(S - LSE) (bf16) into LDS, dV += P^T dO;
//   wave p + 4 (B): dP = dO V^T, dS = P (dP - D) with P from LDS, dK += dS^T Q.
// S and dP are formed once per key and query (four products instead of the
// five of separate dK and dV kernels), and each Q / dO operand read from LDS
// feeds the MFMAs of both key tiles.  B works one tile behind A, so a single
// barrier per step orders everything: in step k, A takes tile k, B tile k - 1
// (whose P A wrote in step k - 1), and all threads write tile k + 1 from
// registers into the third buffer of a three-tile LDS ring, then load tile
// k + 2 into those registers.
// ---------------------------------------------------------------------------
constexpr int kDkvThreads = 64 * kDkvWaves;
constexpr int kDkvPairs = kDkvWaves / 2;
static_assert(kDkvKeys == 32 * kDkvPairs, "two 16-key tiles per wave pair");

template <int D>
__global__ __launch_bounds__(kDkvThreads) void bwd_dkv_kernel(BwdArgs a) {
  constexpr int NU = D / 32;    // 32-wide d steps
  constexpr int NM = D / 16;    // 16-wide d tiles of dK, dV
  constexpr int QROW = D + 16;  // padded LDS rows of the Q and dO tiles
  constexpr int TILE = kBlock * QROW;
  constexpr int NCH = kBlock * D / 8 / kDkvThreads;  // 16-byte chunks per thread per tile
  static_assert(NCH * kDkvThreads * 8 == kBlock * D, "tile must split evenly");
  // ring of 3 tiles: [buffer][Q, dO] rows, [buffer][LSE, -D]
  __shared__ __attribute__((aligned(16))) uint16_t Ts[3][2][TILE];
  __shared__ __attribute__((aligned(16))) float Ls[3][2][kBlock];
  // P of each pair as bf16 A operands: [tile parity][pair][2 half + key tile][lane]
  __shared__ __attribute__((aligned(16))) bf16x8 Px[2][kDkvPairs][4][64];

  // raw item ((b Hkv + g) npair + grp), taken in the list's cost order, in
  // chunks of consecutive entries per XCD: within a cost band the list holds
  // the key chunks of one head in a row, so those share the XCD's cache
  // The item's values are the same for the whole workgroup; they are read
  // with vector loads (the kernel writes global memory, so the compiler cannot
  // read them as constants) and made scalar by readfirstlane, so that every
  // tile address and buffer resource derived from them stays in SGPRs.
  auto uni = [](int v) __attribute__((always_inline)) { return __builtin_amdgcn_readfirstlane(v); };
  const int64_t pos = list_position(blockIdx.x);
  if (pos >= a.dkv_n) return;
  const int64_t item = uni(a.dkv_order[pos]);
  const int grp = static_cast<int>(item % a.npair);
  const int64_t rest = item / a.npair;
  const int g = static_cast<int>(rest % a.Hkv);
  const int b = static_cast<int>(rest / a.Hkv);
  if (uni(a.meta[kMetaStamp]) != a.stamp) return;  // the planner rejected the device contents
  const int tok0 = uni(a.cu[b]);
  const int L = uni(a.cu[b + 1]) - tok0;
  if (grp * kDkvKeys >= L) return;
  const int mode = uni(a.modes[static_cast<int64_t>(b) * a.Hkv + g]) != 0 ? kModeSA : kModeFA;
  const int ns = a.n_sink, w = uni(a.seq_w[b]);
  const int N = (L + kBlock - 1) / kBlock;
  const int kb0 = grp * (kDkvKeys / kBlock);
  const int kb1 = min(N - 1, kb0 + kDkvKeys / kBlock - 1);
  const int qb_lo = kb0;
  const int qb_hi = (mode == kModeSA && kb0 >= ns) ? min(N - 1, kb1 + w - 1) : N - 1;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, lg = lane / 16, li = lane % 16;
  const bool role_a = wave < kDkvPairs;  // wave-uniform
  const int pw = wave % kDkvPairs;       // the pair, and its 32 keys
  // this lane's key of key tile c as a B column; the pair's 32 keys lie in
  // one 64-key block, kbj (computed from wave-uniform values, so that the
  // loop bounds derived from it stay scalar)
  int key_b[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) key_b[c] = grp * kDkvKeys + pw * 32 + 16 * c + li;
  const int kbj = (grp * kDkvKeys + pw * 32) / kBlock;
  // K (wave A) or V (wave B) rows as the B operands of S = Q K^T or dP = dO V^T
  bf16x8 bfr[2][NU];
  {
    const uint16_t* src = role_a ? a.K : a.V;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bool kv = key_b[c] < L;
      const int64_t r = (static_cast<int64_t>(tok0 + (kv ? key_b[c] : 0)) * a.Hkv + g) * D;
#pragma unroll
      for (int u = 0; u < NU; ++u)
        bfr[c][u] = kv ? *reinterpret_cast<const bf16x8*>(src + r + 32 * u + 8 * lg) : bf16x8{};
    }
  }
  f32x4 acc[2][NM];  // dV (wave A) or dK (wave B)
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[c][m] = f32x4{};
  const float cl = a.scale * kLog2e;

  // tile t -> registers -> ring buffer.  Buffer loads: a resource per tile
  // (uniform) whose range ends at the sequence end, so rows past it read as
  // zeros without a branch, and per-thread offsets that stay the same from
  // tile to tile.
  u32x4 qreg[NCH], oreg[NCH];
  float lreg = 0.f, dreg = 0.f;
  int toff[NCH];  // byte offset of this thread's chunks inside a tile's rows
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int ci = k * kDkvThreads + tid, r = ci / (D / 8), col = (ci % (D / 8)) * 8;
    toff[k] = (r * a.Hq * D + col) * 2;
  }
  auto fetch = [&](int t) __attribute__((always_inline)) {
    const int qb = qb_hi - t / a.G;
    const int hq = g * a.G + t % a.G;
    const int rows = L - qb * kBlock;  // > 0: qb is a block of the sequence
    const int64_t row0 = (static_cast<int64_t>(tok0) + qb * kBlock) * a.Hq + hq;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.Q + row0 * D), 0, static_cast<unsigned>(rows) * a.Hq * D * 2u, kBufferWord3);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.dO + row0 * D), 0, static_cast<unsigned>(rows) * a.Hq * D * 2u, kBufferWord3);
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      qreg[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, toff[k], 0, 0));
      oreg[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, toff[k], 0, 0));
    }
    if (tid < kBlock) {
      const int64_t ix = static_cast<int64_t>(hq) * a.T + tok0 + qb * kBlock;
      const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(a.lse2 + ix), 0, static_cast<unsigned>(rows) * 4u, kBufferWord3);
      const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(a.Dv + ix), 0, static_cast<unsigned>(rows) * 4u, kBufferWord3);
      lreg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, tid * 4, 0, 0));
      dreg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, tid * 4, 0, 0));
      // a row past the end: LSE +inf, so that its P is 0 (its Q and dO are 0)
      if (tid >= rows) lreg = INFINITY;
    }
  };
  auto stage = [&](int t) __attribute__((always_inline)) {
    const int buf = t % 3;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int ci = k * kDkvThreads + tid, r = ci / (D / 8), col = (ci % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(&Ts[buf][0][r * QROW + col]) = qreg[k];
      *reinterpret_cast<u32x4*>(&Ts[buf][1][r * QROW + col]) = oreg[k];
    }
    if (tid < kBlock) {
      Ls[buf][0][tid] = lreg;
      Ls[buf][1][tid] = -dreg;
    }
  };

  // The products of a half hf (the tile's query rows 32 hf .. 32 hf + 31):
  //  rows: S = Q K^T (wave A) or dP = dO V^T (wave B), 2 query tiles of 16
  //        rows x 2 key tiles; lane holds key li of tile c, rows 16 qt + 4 lg + i;
  //  cols: acc += X^T T with X (P for wave A, dS for wave B) as bf16 A
  //        operands (keys x the half's 32 queries) and T (dO, Q) by
  //        transposing reads, query rows 32 hf + 4 lg + 0..3 and + 16, the
  //        order the operands hold them in.
  // Each operand read from LDS feeds both key tiles.  Reads are issued as a
  // group ahead of their MFMAs (load_* / mma_*), so the waves' LDS latency
  // hides behind other work.
  typedef bf16x8 RowOps[2][NU];
  typedef bf16x8 ColOps[NM];
  // this lane's part of each read's LDS address, formed once: every read of
  // a step is then one tile base plus this plus a constant
  const int row_lane = li * QROW + 8 * lg;
  const int col_lane = (4 * lg + li / 4) * QROW + 4 * (li & 3);
  auto load_rows = [&](const uint16_t* src, int hf, RowOps& qa) __attribute__((always_inline)) {
    const uint16_t* base = src + row_lane;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int u = 0; u < NU; ++u)
        qa[t2][u] = *reinterpret_cast<const bf16x8*>(base + 16 * (2 * hf + t2) * QROW + 32 * u);
  };
  auto mma_rows = [&](const RowOps& qa, f32x4 (*x)[2], const f32x4* init) __attribute__((always_inline)) {
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
      for (int c = 0; c < 2; ++c) x[t2][c] = init ? init[t2] : f32x4{};
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int c = 0; c < 2; ++c) x[t2][c] = mfma16(qa[t2][u], bfr[c][u], x[t2][c]);
    }
  };
  // (tile = ring slot 2 buf + tensor; the lane's offset into it goes through
  // an empty asm so that it stays one register and each read's constant part
  // folds into the instruction's offset field, where the compiler would
  // otherwise keep 16 per-read lane offsets and add the slot to each)
  auto load_cols = [&](int tile, int hf, ColOps& bt) __attribute__((always_inline)) {
    int off = tile * TILE + col_lane;
    asm("" : "+v"(off));
    const uint16_t* base = &Ts[0][0][0] + off;
#pragma unroll
    for (int m = 0; m < NM; ++m)
      bt[m] = tr_pair(base + 32 * hf * QROW + 16 * m, base + (32 * hf + 16) * QROW + 16 * m);
  };
  // m in [m0, m1)
  auto mma_cols = [&](const bf16x8* xa, const ColOps& bt, int m0, int m1) __attribute__((always_inline)) {
#pragma unroll
    for (int m = m0; m < m1; ++m)
#pragma unroll
      for (int c = 0; c < 2; ++c) acc[c][m] = mfma16(xa[c], bt[m], acc[c][m]);
  };
  auto fence = []() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };

  // wave A, tile t: P = exp(S - LSE) as bf16, to LDS for wave B, and
  // dV += P^T dO.  MASKED: some key of the pair is invisible to some row of
  // the block (the diagonal block, the window's edge, the sequence's end); the
  // mask then sends the exponent to -inf.  `between` runs after the second
  // half's MFMAs are issued.
  auto tile_a = [&](int t, auto masked, auto between) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    const int qb = qb_hi - t / a.G;
    const uint16_t* Qt = Ts[t % 3][0];
    const uint16_t* Ot = Ts[t % 3][1];
    const float* Lt = Ls[t % 3][0];
    RowOps qa;
    ColOps bt;
    load_rows(Qt, 0, qa);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x4 s[2][2];
      fence();
      mma_rows(qa, s, nullptr);
      fence();
      load_cols(2 * (t % 3) + 1, hf, bt);
      fence();
      bf16x8 pa[2];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int qt = 2 * hf + t2;
        const f32x4 lv = *reinterpret_cast<const f32x4*>(Lt + 16 * qt + 4 * lg);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float e = __builtin_fmaf(s[t2][c][i], cl, -lv[i]);
            if constexpr (MASKED) {
              const int p = qb * kBlock + 16 * qt + 4 * lg + i;
              const bool vis = key_b[c] <= p && p < L &&
                               (mode == kModeFA || kbj < ns || p / kBlock - kbj < w);
              e = vis ? e : -INFINITY;
            }
            pa[c][4 * t2 + i] = static_cast<__bf16>(__builtin_amdgcn_exp2f(e));
          }
        }
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) Px[t & 1][pw][2 * hf + c][lane] = pa[c];
      fence();
      mma_cols(pa, bt, 0, NM / 2);
      fence();
      if (hf == 0) load_rows(Qt, 1, qa);  // into the registers the first MFMAs freed
      fence();
      mma_cols(pa, bt, NM / 2, NM);
      fence();
      if (hf == 1) between();
    }
  };
  // wave B, tile t: dS = P (dP - D), then dK += dS^T Q
  auto tile_b = [&](int t, auto between) __attribute__((always_inline)) {
    const uint16_t* Qt = Ts[t % 3][0];
    const uint16_t* Ot = Ts[t % 3][1];
    const float* Dt = Ls[t % 3][1];
    RowOps qa;
    ColOps bt;
    load_rows(Ot, 0, qa);
    // -D of the tile's rows (the ring holds D negated): the dP accumulators
    // start there, so the products give dP - D (16 subtractions per half
    // fewer)
    f32x4 nd[2][2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) nd[hf][t2] = *reinterpret_cast<const f32x4*>(Dt + 16 * (2 * hf + t2) + 4 * lg);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x4 dp[2][2];
      fence();
      mma_rows(qa, dp, nd[hf]);
      fence();
      load_cols(2 * (t % 3), hf, bt);
      bf16x8 pa[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) pa[c] = Px[t & 1][pw][2 * hf + c][lane];
      fence();
      bf16x8 ds[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            ds[c][4 * t2 + i] = static_cast<__bf16>(static_cast<float>(pa[c][4 * t2 + i]) * dp[t2][c][i]);
      fence();
      mma_cols(ds, bt, 0, NM / 2);
      fence();
      if (hf == 0) load_rows(Ot, 1, qa);
      fence();
      mma_cols(ds, bt, NM / 2, NM);
      fence();
      if (hf == 1) between();
    }
  };

  const int nsteps = (qb_hi - qb_lo + 1) * a.G;
  fetch(0);
  stage(0);
  if (nsteps > 1) fetch(1);
  __syncthreads();
  // Step k: wave A takes tile k and wave B tile k - 1; after their second
  // halves all threads write tile k + 1 (loaded a step earlier) into the ring
  // and start the loads of tile k + 2 (at the end of the step rather than
  // between the halves: 0.4% faster; at its start: 2% slower).  Both roles
  // pass nsteps + 1 barriers.
  auto ring = [&](int k) __attribute__((always_inline)) {
    if (k + 1 < nsteps) {
      stage(k + 1);
      if (k + 2 < nsteps) fetch(k + 2);
    }
  };
  if (role_a) {
    // Every row of block qb sees every key of the pair exactly when
    // kbj < qb <= qf: past the diagonal block, inside the sequence's whole
    // blocks and, for a window, inside the window.  Those tiles (qb walks
    // down, so a middle range of k) take the unmasked variant; each variant
    // runs in a loop of its own, so each is register-allocated alone.
    int qf = L / kBlock - 1;
    if (mode == kModeSA && kbj >= ns) qf = min(qf, kbj + w - 1);
    const int m1 = min(nsteps, max(0, (qb_hi - kbj) * a.G));
    const int m0 = min(m1, max(0, (qb_hi - qf) * a.G));
    int k = 0;
    for (; k < m0; ++k) {
      tile_a(k, std::true_type{}, [&]() __attribute__((always_inline)) { ring(k); });
      __syncthreads();
    }
    for (; k < m1; ++k) {
      tile_a(k, std::false_type{}, [&]() __attribute__((always_inline)) { ring(k); });
      __syncthreads();
    }
    for (; k < nsteps; ++k) {
      tile_a(k, std::true_type{}, [&]() __attribute__((always_inline)) { ring(k); });
      __syncthreads();
    }
    __syncthreads();  // step nsteps: wave B's last tile
  } else {
    ring(0);
    __syncthreads();
    for (int k = 1; k <= nsteps; ++k) {
      tile_b(k - 1, [&]() __attribute__((always_inline)) { ring(k); });
      __syncthreads();
    }
  }

  // lane holds keys 16 c + 4 lg + i of the pair's 32, dims 16 m + li
  uint16_t* const out = role_a ? a.dV : a.dK;
  const float osc = role_a ? 1.f : a.scale;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = grp * kDkvKeys + pw * 32 + 16 * c + 4 * lg + i;
      if (key >= L) continue;
      const int64_t r = (static_cast<int64_t>(tok0 + key) * a.Hkv + g) * D;
#pragma unroll
      for (int m = 0; m < NM; ++m)
        out[r + 16 * m + li] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[c][m][i] * osc));
    }
  }
}

// Cost (query blocks walked) of every dK/dV item, as a sort key: most
// expensive first, empty items last.  The key counts the cost in units of
// kDkvCostUnit blocks, so a band spans 2^kCostBandShift such units: 64 key
// chunks of one FA head in a row (their costs step by 2 blocks), and an XCD's
// 32 consecutive list entries are key chunks of a single head that walk the
// same Q and dO tiles (1% faster on the 128K 2/8 layer than bands of 32
// blocks, whose chunks mixed two heads).
constexpr int kDkvCostUnit = 4;
__global__ __launch_bounds__(256) void dkv_items_kernel(BwdArgs a, int32_t maxcost,
                                                        uint32_t* __restrict__ keys) {
  const int64_t x = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (x >= a.dkv_n) return;
  const int pair = static_cast<int>(x % a.npair);
  const int64_t rest = x / a.npair;
  const int g = static_cast<int>(rest % a.Hkv);
  const int b = static_cast<int>(rest / a.Hkv);
  const int L = a.cu[b + 1] - a.cu[b];
  if (a.meta[kMetaStamp] != a.stamp || pair * kDkvKeys >= L) {
    keys[x] = empty_key((maxcost + kDkvCostUnit - 1) / kDkvCostUnit);
    return;
  }
  const int N = (L + kBlock - 1) / kBlock;
  const int kb0 = pair * (kDkvKeys / kBlock);
  const int kb1 = min(N - 1, kb0 + kDkvKeys / kBlock - 1);
  const bool sa = a.modes[static_cast<int64_t>(b) * a.Hkv + g] != 0;
  const int qb_hi = (sa && kb0 >= a.n_sink) ? min(N - 1, kb1 + a.seq_w[b] - 1) : N - 1;
  const int cost = qb_hi - kb0 + 1;
  keys[x] = cost_key((cost + kDkvCostUnit - 1) / kDkvCostUnit, (maxcost + kDkvCostUnit - 1) / kDkvCostUnit);
}

}  // namespace

DkvList dkv_list_layout(const Shape& s) {
  auto align = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  DkvList l{};
  l.npair = static_cast<int32_t>((static_cast<int64_t>(s.max_seqlen) + kDkvKeys - 1) / kDkvKeys);
  l.n = static_cast<int64_t>(s.B) * s.Hkv * l.npair;
  l.maxcost = (s.max_seqlen + kBlock - 1) / kBlock;
  size_t off = 0;
  l.keys = off;  off = align(off + sizeof(uint32_t) * l.n);
  l.order = off; off = align(off + sizeof(int32_t) * l.n);
  l.total = off;
  return l;
}

hipError_t launch_backward(const Shape& s, const Geometry& g, BwdArgs args, const DkvList& l,
                           char* list_base, hipStream_t st) {
  uint32_t* keys = reinterpret_cast<uint32_t*>(list_base + l.keys);
  int32_t* order = reinterpret_cast<int32_t*>(list_base + l.order);
  args.dkv_order = order;
  args.dkv_n = l.n;
  args.npair = l.npair;
  hipLaunchKernelGGL(dkv_items_kernel, dim3(static_cast<unsigned>((l.n + 255) / 256)), dim3(256), 0,
                     st, args, l.maxcost, keys);
  hipError_t e0 = launch_key_sort(keys, l.n, order, st);
  if (e0 != hipSuccess) return e0;
  const int64_t dkv_items = l.n;
  const int64_t rows = s.T * s.Hq * (s.d / 8);
  hipLaunchKernelGGL(bwd_pre_kernel, dim3(static_cast<unsigned>((rows + 255) / 256)), dim3(256), 0, st,
                     args.O, args.dO, args.lse, s.T, s.Hq, s.d, args.Dv, args.lse2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int64_t span = static_cast<int64_t>(kNumXcd) * kXcdChunk;
  const unsigned grid = static_cast<unsigned>((args.max_items + span - 1) / span * span);
  const dim3 dkv_grid(static_cast<unsigned>((dkv_items + span - 1) / span * span));
  if (s.d == 128) {
    hipLaunchKernelGGL((bwd_dq_kernel<128>), dim3(grid), dim3(kAttnWaves * 64), 0, st, args);
    hipLaunchKernelGGL((bwd_dkv_kernel<128>), dkv_grid, dim3(kDkvThreads), 0, st, args);
  } else {
    hipLaunchKernelGGL((bwd_dq_kernel<64>), dim3(grid), dim3(kAttnWaves * 64), 0, st, args);
    hipLaunchKernelGGL((bwd_dkv_kernel<64>), dkv_grid, dim3(kDkvThreads), 0, st, args);
  }
  return hipGetLastError();
}

}  // namespace ea
