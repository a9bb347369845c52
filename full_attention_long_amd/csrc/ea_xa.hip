// XAttention (XA) block selection for the XA heads of the hybrid prefill.
//
// Pages: "Elastic Attention: Test-time Adaptive Sparsity Ratios for Efficient
// Transformers" runs retrieval or sparse heads in XAttention mode (experimental
// setup, baselines paragraph: threshold tau = 0.9, XAttention's other settings
// at their defaults; head configurations FA-XA and XA-SSA).  The selection
// restates "XAttention: Block Sparse Attention with Antidiagonal Scoring"
// (method section) at its default block 128 and stride 8:
//
//   group score   sum_t <q[aS + S-1-t], k[cS + t]> over the antidiagonal of
//                 the S x S tile of position groups a (queries) and c (keys),
//                 positions past the sequence end reading as zero;
//   softmax       of score * scale / S over the groups c <= a of row a;
//   block mass    A[i][j] = sum of those probabilities over the 16 x 16 group
//                 tile of XA query block i and key block j;
//   selection     block 0 and block i, then blocks in decreasing mass (ties
//                 to the lower index) until the kept mass reaches tau times
//                 the row total.
//
// One workgroup of 8 waves per (sequence, KV head, pair of XA query blocks
// 2p + 1 and 2p): waves 0-3 score block 2p + 1, waves 4-7 block 2p, for the
// KV group's query heads 4 at a time (one per wave).  A wave keeps its head's
// 16 group rows of its block in registers as the A operand of 16x16x32 bf16
// MFMAs: the contraction runs over the S * d values of a group (S query rows
// in reversed order, d dims each), so one 16 x 16 tile of group scores is
// S d / 32 MFMAs.  Key blocks j = 0..2p + 1 stream through LDS once for both
// blocks (128 key rows, the 8 rows of each group contiguous and groups padded
// by 32 bytes, so that the B-operand reads are free of bank conflicts and
// every read is one base register plus an immediate offset), by direct
// buffer-to-LDS loads into a ring of four tiles three blocks ahead.  Per key
// block, each group row's log2-sum-exp2 over the block's 16 groups (DPP
// reductions over the 16 lanes of the row) goes to the workspace and updates
// the row's running total; once the totals are known, A[i][j] = sum over the
// rows of 2^(block lse - row total).
// The selection then runs in the same workgroup, a wave per (head, block)
// row: the row's masses, a bitonic sort of its candidates (mass bits above
// the inverted block index, so equal masses keep ascending index; the rows'
// sorts share one pass of barriers), a prefix sum in sorted order and the
// threshold test in float32.  The per-head keep flags of the KV group are
// OR-ed into one mask per key block, and the kept blocks are written as one
// ascending list of (j | head mask << 16) for the attention kernel, which
// walks the union once and masks each head to its own blocks.
#include "ea_internal.h"

#include <math.h>

namespace ea {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kXaThreads = 512;
// elements of padding after each 8-row key group in the LDS key tiles
constexpr int kXaGroupPad = 16;
constexpr int kXaWaves = kXaThreads / 64;
// s_waitcnt immediate that waits until at most N vector-memory operations of
// the wave are outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14;
// expcnt and lgkmcnt at their maxima, i.e. not waited for)
constexpr int kReadsAhead = 6;  // B-operand reads in flight ahead of the MFMAs
template <int N>
constexpr int kVmcntAhead = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kMinusBig = -1.0e30f;
// word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data, no swizzle)
constexpr int kBufferWord3 = 0x00020000;

struct XaArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const int8_t* modes;
  const int32_t* cu;
  const int32_t* meta;   // meta[kMetaXaRows]: number of XA rows
  const int32_t* rows;   // the XA (sequence, KV head) rows, b * Hkv + kvh
  int32_t* cnt;     // [B * Hkv * nqb]
  float* lse;       // [B, Hq, xa_row_offset(nqb), 16] log2-sum-exp2 of each group row per key block
  int32_t* list;    // [B * Hkv * xa_row_offset(nqb)]
  float* mass;      // [B, Hq, nqb, nqb] or null
  uint8_t* keep;    // [B, Hq, nqb, nqb] or null
  int32_t B, Hq, Hkv, G, nqb, nqb_pad, head_config;
  float cs;         // softmax scale * log2(e) / S
  float tau;
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Max / sum over the 16 lanes of a DPP row, the result in every lane of it:
// swap neighbours, swap pairs, mirror within 8, mirror within 16.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppSwap1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int kDppSwap2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;   // row_half_mirror
constexpr int kDppMirror = 0x140;       // row_mirror
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<kDppSwap1>(v));
  v = fmaxf(v, dpp<kDppSwap2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  return fmaxf(v, dpp<kDppMirror>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kDppSwap1>(v);
  v += dpp<kDppSwap2>(v);
  v += dpp<kDppHalfMirror>(v);
  return v + dpp<kDppMirror>(v);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Exclusive prefix over the workgroup of one value per thread, in thread
// order (red: kXaWaves + 1 floats); returns the prefix, *total the sum.
template <typename T>
__device__ T block_exclusive(T v, T* red, T* total) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  T x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const T y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  __syncthreads();
  if (lane == 63) red[wave] = x;
  __syncthreads();
  T before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kXaWaves; ++w) {
    if (w < wave) before += red[w];
    all += red[w];
  }
  *total = all;
  return before + x - v;
}

// The (sequence, KV head) rows whose heads run in XA mode, in order, and
// their count (one workgroup).
__global__ __launch_bounds__(kXaThreads) void xa_rows_kernel(const int8_t* __restrict__ modes,
                                                              const int32_t* __restrict__ cu,
                                                              int32_t B, int32_t Hkv,
                                                              int32_t head_config,
                                                              int32_t* __restrict__ rows,
                                                              int32_t* __restrict__ meta) {
  __shared__ int32_t red[kXaWaves + 1];
  int32_t base = 0;
  // invalid device contents (the planner's checks ran first): no XA row at all
  const int n = meta[kMetaError] != 0 ? 0 : B * Hkv;
  for (int r0 = 0; r0 < n; r0 += kXaThreads) {
    const int r = r0 + static_cast<int>(threadIdx.x);
    const bool x = r < n && cu[r / Hkv + 1] > cu[r / Hkv] &&
                   computation_mode(head_config, modes[r] != 0) == kModeXA;
    int32_t all;
    const int32_t pos = block_exclusive(static_cast<int32_t>(x), red, &all);
    if (x) rows[base + pos] = r;
    base += all;
    __syncthreads();
  }
  if (threadIdx.x == 0) meta[kMetaXaRows] = base;
}

template <int D>
__global__ __launch_bounds__(kXaThreads) void xa_plan_kernel(XaArgs a) {
  constexpr int S = kXaStride;
  constexpr int KS = S * D / 32;                     // 32-wide k-steps of one group
  constexpr int KGS = S * D + kXaGroupPad;           // elements per padded key group
  constexpr int KT = kXaGroupsPerBlock * KGS;        // elements of one key tile
  constexpr int RPI = 1024 / (2 * D);                // key rows per 1 KiB load instruction
  constexpr int IPG = S / RPI;                       // load instructions per key group
  constexpr int NDMA = kXaBlock / RPI / kXaWaves;    // load instructions per wave per tile
  constexpr int AHEAD = 3;                           // key tiles in flight beyond the one read
  static_assert(IPG >= 1 && IPG * RPI == S, "a key group is whole load instructions");
  static_assert(NDMA * RPI * kXaWaves == kXaBlock, "key tile must split evenly");
  static_assert(kXaGroupsPerBlock == 16, "one 16-row MFMA tile of groups per XA block");
  static_assert(kXaWaves == 8, "two quads of waves, one per query block of the pair");

  // a ring of four key tiles, each addressed only through its own name, so
  // that the direct loads into three of them can be in flight while the
  // fourth is read; after the scoring they hold the selection's sort keys
  __shared__ __attribute__((aligned(1024))) uint16_t Kt0[KT], Kt1[KT], Kt2[KT], Kt3[KT];
  __shared__ float rlt[kXaWaves][kXaGroupsPerBlock];  // group-row totals of the waves' (head, block)
  __shared__ int32_t redi[kXaWaves + 1];
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // [2][nqb] 16-bit masks of the heads keeping key block j, for the pair's
  // upper and lower block (a group has at most 16 query heads), two to a
  // 32-bit word so that the waves of different heads set bits by LDS atomics
  uint32_t* hmw = reinterpret_cast<uint32_t*>(smem);
  // keep mask of the pair's block qd (0 upper, 1 lower) at key block j
  auto hm_at = [&](int qd, int j) __attribute__((always_inline)) {
    const int x = qd * a.nqb + j;
    return (hmw[x >> 1] >> (16 * (x & 1))) & 0xFFFFu;
  };

  // Work item t = the workgroup's position in the XCD-chunked order
  // (list_position): a pair of query blocks (2 p + 1, 2 p) of one XA row;
  // items run in bands of kXcdChunk pairs, the costliest (largest p) band
  // first; inside a band, one XA row after the other, kXcdChunk consecutive
  // pairs each, so that the workgroups an XCD runs together stream the same
  // key blocks through its L2.
  const int64_t t = list_position(blockIdx.x);
  const int n_rows = a.meta[kMetaXaRows];
  const int nqp = (a.nqb + 1) / 2;
  if (t >= static_cast<int64_t>(n_rows) * a.nqb_pad) return;
  const int64_t band = t / (static_cast<int64_t>(kXcdChunk) * n_rows);
  const int rem = static_cast<int>(t - band * kXcdChunk * n_rows);
  const int bk = a.rows[rem / kXcdChunk];
  const int pp = a.nqb_pad - 1 - static_cast<int>(band * kXcdChunk + rem % kXcdChunk);
  const int b = bk / a.Hkv, kvh = bk % a.Hkv;
  const int tok0 = a.cu[b];
  const int L = a.cu[b + 1] - tok0;
  if (pp < 0 || pp >= nqp) return;
  // the pair's blocks: quad 0 takes 2 p + 1, quad 1 takes 2 p; a block past
  // the sequence end (or past nqb) has no work
  int ib[2];
  bool bv[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    ib[q] = 2 * pp + 1 - q;
    bv[q] = ib[q] < a.nqb && static_cast<int64_t>(ib[q]) * kXaBlock < L;
  }
  if (!bv[1]) return;  // then block 2 p + 1 lies past the end too
  const int jmax = bv[0] ? ib[0] : ib[1];  // key blocks 0 .. jmax are walked
  const int ng = (L + S - 1) / S;  // position groups of the sequence

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int quad = wave / 4, wq = wave % 4;
  const int i = ib[quad];         // this wave's query block
  const bool iv = bv[quad];
  const int r = lane % 16, kq = lane / 16;
  for (int j = tid; j < a.nqb; j += kXaThreads) hmw[j] = 0u;  // 2 nqb 16-bit masks

  // Direct loads of key block j: instruction q = wave NDMA + n of the tile
  // fills rows (q % IPG) RPI .. + RPI - 1 of group q / IPG, lane l writing
  // 16-byte chunk l % (D / 8) of row l / (D / 8).  The buffer resource ends at
  // the sequence end (rows past it read as zeros; the whole offset is in the
  // range-checked vector offset).  LDS: the 8 rows of a group contiguous,
  // groups padded by 32 bytes (an odd multiple of 32 bytes apart): a B-operand
  // read's lanes r and kq (groups r, 16-byte column kq) then land on distinct
  // 16-byte bank groups within each set of lanes the LDS serves together (with
  // 16-byte padding, lanes of adjacent kq collided: the bank-conflict counter
  // read 28% of the kernel's time, and the selection took 10.0 ms instead of
  // 8.1 at 128K).
  const int rs2 = a.Hkv * D * 2;  // bytes between key rows
  const uint16_t* kseq = a.K + (static_cast<int64_t>(tok0) * a.Hkv + kvh) * D;
  int dma_off[NDMA];
#pragma unroll
  for (int n = 0; n < NDMA; ++n) {
    const int q = wave * NDMA + n;
    dma_off[n] = ((q / IPG) * S + (q % IPG) * RPI + lane / (D / 8)) * rs2 + (lane % (D / 8)) * 16;
  }
  // (the offsets come in as a parameter: a lambda capturing a local array
  // by reference makes the host pass drop this kernel's launch stub).  Key
  // blocks past jmax load nothing, but every wave still counts NDMA loads per
  // step: a block past the end reads the range-checked zero page.
  auto dma = [&](uint16_t* tile, int j, const int* off) __attribute__((always_inline)) {
    const int jj = min(j, jmax);
    const int key0 = jj * kXaBlock;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(kseq + static_cast<int64_t>(key0) * a.Hkv * D), 0,
        j <= jmax ? static_cast<unsigned>(L - key0) * static_cast<unsigned>(rs2) : 0u, kBufferWord3);
#pragma unroll
    for (int n = 0; n < NDMA; ++n) {
      const int q = wave * NDMA + n;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)(tile + (q / IPG) * KGS + (q % IPG) * RPI * D),
          16, off[n], 0, 0, 0);
    }
  };

  for (int g0 = 0; g0 < a.G; g0 += 4) {
    const int gg = g0 + wq;
    const bool hv = gg < a.G && iv;
    const int hq = kvh * a.G + min(gg, a.G - 1);
    // A operand: group row 16 i + r, contraction index 32 kk + 8 kq + e =
    // t D + dim, i.e. query position (16 i + r) S + S-1-t
    bf16x8 qa[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int tt = (32 * kk) / D, dim = (32 * kk) % D + 8 * kq;
      const int p = (16 * i + r) * S + S - 1 - tt;
      qa[kk] = (hv && p < L) ? *reinterpret_cast<const bf16x8*>(
                                   a.Q + (static_cast<int64_t>(tok0 + p) * a.Hq + hq) * D + dim)
                             : bf16x8{};
    }
    // Lane holds group rows 16 i + 4 kq + e (e = 0..3), key group 16 j + r,
    // of each score tile.  Per key block: each row's log2-sum-exp2 over the
    // block's 16 groups goes to the workspace and the row's running sum
    // absorbs it.  The sums are taken against a running reference R of the
    // row (uniform over its 16 lanes), not the block's own max: only when a
    // sum passes 2^64 (or R is unset) does a rare branch take the block max,
    // raise R and rescale the running sum.
    float R_e[4], L_e[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      R_e[e] = kMinusBig;
      L_e[e] = 0.f;
    }
    float* const lrow = a.lse + ((static_cast<int64_t>(b) * a.Hq + hq) * xa_row_offset(a.nqb) +
                                 xa_row_offset(i)) * kXaGroupsPerBlock;
    // step j: load block j + AHEAD into the tile block j - 1 used, score
    // block j from kt, then wait for this wave's loads of block j + 1 (the
    // AHEAD - 1 newer tiles may stay in flight) and meet the other waves
    auto step = [&](int j, const uint16_t* kt, uint16_t* kload) __attribute__((always_inline)) {
      dma(kload, j + AHEAD, dma_off);
      if (hv && j <= i) {
        // B operand: key group column r (positions (16 j + r) S + t), same
        // k-slice: group r, row t, dims 32 kk % D + 8 kq, i.e. element
        // r KGS + 32 kk + 8 kq; two independent accumulation chains (a
        // product's result is ready before its chain's next MFMA issues)
        // The B-operand reads run kReadsAhead MFMAs ahead of their use,
        // pinned there by scheduling fences (left alone, the compiler reads
        // each one into the same registers right before its MFMA, which then
        // waits out the whole LDS latency).
        f32x4 sc[2] = {f32x4{}, f32x4{}};
        bf16x8 kb[KS];
        auto kread = [&](int kk) __attribute__((always_inline)) {
          kb[kk] = *reinterpret_cast<const bf16x8*>(kt + r * KGS + 32 * kk + 8 * kq);
        };
#pragma unroll
        for (int kk = 0; kk < kReadsAhead; ++kk) kread(kk);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          if (kk + kReadsAhead < KS) kread(kk + kReadsAhead);
          __builtin_amdgcn_sched_barrier(0);
          sc[kk & 1] = mfma16(qa[kk], kb[kk], sc[kk & 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
        const f32x4 s = sc[0] + sc[1];
        const int c = 16 * j + r;  // this lane's key group
        f32x4 x, ps;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ag = 16 * i + 4 * kq + e;
          x[e] = (c <= ag && ag < ng) ? s[e] * a.cs : -INFINITY;
          ps[e] = row16_sum(__builtin_amdgcn_exp2f(x[e] - R_e[e]));
        }
        const bool big = !(ps[0] <= 0x1p64f) || !(ps[1] <= 0x1p64f) || !(ps[2] <= 0x1p64f) ||
                         !(ps[3] <= 0x1p64f);
        if (__builtin_expect(__ballot(big) != 0, 0)) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float rn = fmaxf(R_e[e], row16_max(x[e]));
            L_e[e] *= __builtin_amdgcn_exp2f(R_e[e] - rn);
            R_e[e] = rn;
            ps[e] = row16_sum(__builtin_amdgcn_exp2f(x[e] - rn));
          }
        }
        f32x4 blse;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // an all-masked row of the block: ps = 0, lse -inf, no change
          blse[e] = R_e[e] + __log2f(ps[e]);
          L_e[e] += ps[e];
        }
        if (r == 0) *reinterpret_cast<f32x4*>(lrow + j * kXaGroupsPerBlock + 4 * kq) = blse;
      }
      // this wave's loads of block j + 1 are done once at most the loads of
      // the AHEAD - 1 tiles after it are outstanding.  Then the barrier, which
      // the compiler may move no memory access across (a fence would also wait
      // for the loads still meant to be in flight).
      __builtin_amdgcn_s_waitcnt(kVmcntAhead<NDMA * (AHEAD - 1)>);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    dma(Kt0, 0, dma_off);
    dma(Kt1, 1, dma_off);
    dma(Kt2, 2, dma_off);
    __builtin_amdgcn_s_waitcnt(kVmcntAhead<NDMA * (AHEAD - 1)>);
    __syncthreads();
    for (int j = 0; j <= jmax; j += 4) {
      step(j, Kt0, Kt3);
      if (j + 1 <= jmax) step(j + 1, Kt1, Kt0);
      if (j + 2 <= jmax) step(j + 2, Kt2, Kt1);
      if (j + 3 <= jmax) step(j + 3, Kt3, Kt2);
    }
    // no load may still be writing a tile when the first one becomes the
    // sort buffer
    __builtin_amdgcn_s_waitcnt(kVmcntAhead<0>);
    // the group-row totals (uniform over the 16 lanes of a row)
    if (hv && r == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) rlt[wave][4 * kq + e] = R_e[e] + __log2f(L_e[e]);
    }
    __syncthreads();  // totals and workspace rows written; the key tiles are free

    // Threshold selection of the (head, block) rows of the two quads, row w =
    // (block of quad w / 4, head g0 + w % 4), wave w taking row w.  Block
    // masses A[i][j] = sum over the group rows (those before the sequence's
    // last group) of 2^(block lse - row total).  Each wave forms its row's
    // masses and sort keys; one bitonic sort over the whole workgroup then
    // orders the keys of up to 8 rows at once (a barrier per stage for all of
    // them rather than per row), and each wave takes its row's prefix sums in
    // sorted order and sets its head's keep bits.
    {
      int P2 = 1;
      while (P2 < jmax - 1) P2 <<= 1;
      const int rpt = (KT / 4) / P2 >= 2 ? 2 : 1;  // rows whose keys fit one key tile
      const int nr = 4 * rpt;                      // rows per sort batch
      auto row_keys = [&](int rr) __attribute__((always_inline)) {
        const int t = rr / rpt;
        uint16_t* tile = t == 0 ? Kt0 : t == 1 ? Kt1 : t == 2 ? Kt2 : Kt3;
        return reinterpret_cast<uint64_t*>(tile) + (rr % rpt) * P2;
      };
      for (int r0 = 0; r0 < kXaWaves; r0 += nr) {
        const bool mine = wave >= r0 && wave < r0 + nr;  // wave-uniform
        const int qd = wave / 4, gw = g0 + wave % 4;
        const bool rv = mine && gw < a.G && bv[qd];
        const int iw = ib[qd];
        const int m = iw - 1;  // candidates: blocks 1 .. iw-1
        const int hqw = kvh * a.G + min(gw, a.G - 1);
        const uint32_t bit = 1u << gw;
        float target = 0.f, forced = 0.f;
        if (mine) {
          uint64_t* keys = row_keys(wave - r0);
          float part = 0.f, f0 = 0.f, fi = 0.f;
          if (rv) {
            const float* srow = a.lse + ((static_cast<int64_t>(b) * a.Hq + hqw) * xa_row_offset(a.nqb) +
                                         xa_row_offset(iw)) * kXaGroupsPerBlock;
            for (int j = lane; j <= iw; j += 64) {
              float mj = 0.f;
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(srow + j * kXaGroupsPerBlock + 4 * q);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (16 * iw + 4 * q + e < ng) mj += __builtin_amdgcn_exp2f(v[e] - rlt[wave][4 * q + e]);
              }
              part += mj;
              if (a.mass) a.mass[((static_cast<int64_t>(b) * a.Hq + hqw) * a.nqb + iw) * a.nqb + j] = mj;
              if (j == 0) f0 = mj;
              if (j == iw) fi = mj;
              if (j >= 1 && j < iw)
                keys[j - 1] = (static_cast<uint64_t>(__float_as_uint(mj)) << 32) |
                              static_cast<uint64_t>(0xFFFFFFFFu - static_cast<uint32_t>(j));
            }
          }
          // the rest of the row's P2 slots (all of them for an empty row) sort last
          for (int p = (rv ? max(m, 0) : 0) + lane; p < P2; p += 64) keys[p] = 0ull;
          target = a.tau * wave_sum(part);
          f0 = wave_sum(f0);  // one lane holds each, the others 0
          fi = wave_sum(fi);
          forced = iw > 0 ? f0 + fi : f0;
        }
        __syncthreads();  // every row's keys written
        // bitonic sort of each row's P2 keys, descending; stage (k, jj) pairs
        // slot p (bit jj clear) with p + jj
        for (int k = 2; k <= P2; k <<= 1) {
          for (int jj = k >> 1; jj > 0; jj >>= 1) {
            for (int x = tid; x < nr * (P2 / 2); x += kXaThreads) {
              const int rr = x / (P2 / 2), y = x % (P2 / 2);
              const int p = ((y & ~(jj - 1)) << 1) | (y & (jj - 1)), q = p | jj;
              uint64_t* keys = row_keys(rr);
              const uint64_t x0 = keys[p], x1 = keys[q];
              const bool desc = (p & k) == 0;
              if (desc ? (x0 < x1) : (x0 > x1)) {
                keys[p] = x1;
                keys[q] = x0;
              }
            }
            __syncthreads();
          }
        }
        if (rv && m > 0) {
          // exclusive prefix of the sorted masses (each lane a run of slots);
          // keep entry p while the mass kept before it is short of the target
          const uint64_t* keys = row_keys(wave - r0);
          const int per = (P2 + 63) / 64;
          const int p0 = lane * per;
          float mine_sum = 0.f;
          for (int p = p0; p < min(p0 + per, m); ++p)
            mine_sum += __uint_as_float(static_cast<uint32_t>(keys[p] >> 32));
          float incl = mine_sum;
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(incl, off, 64);
            if (lane >= off) incl += y;
          }
          float before = incl - mine_sum;
          for (int p = p0; p < min(p0 + per, m); ++p) {
            const float v = __uint_as_float(static_cast<uint32_t>(keys[p] >> 32));
            if (forced + before < target) {
              const int j = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(keys[p]));
              atomicOr(&hmw[(qd * a.nqb + j) >> 1], bit << (16 * ((qd * a.nqb + j) & 1)));
            }
            before += v;
          }
        }
        if (rv && lane == 0) {
          atomicOr(&hmw[(qd * a.nqb) >> 1], bit << (16 * ((qd * a.nqb) & 1)));
          atomicOr(&hmw[(qd * a.nqb + iw) >> 1], bit << (16 * ((qd * a.nqb + iw) & 1)));
        }
        __syncthreads();  // keep bits set; the key tiles are free for the next batch
        if (rv && a.keep) {
          uint8_t* krow = a.keep + ((static_cast<int64_t>(b) * a.Hq + hqw) * a.nqb + iw) * a.nqb;
          for (int j = lane; j <= iw; j += 64) krow[j] = (hm_at(qd, j) & bit) ? 1 : 0;
        }
      }
    }
    __syncthreads();  // the key tiles are free again
  }

  // Ascending list of the key blocks some head of the group keeps, for each
  // block of the pair.
  for (int qd = 0; qd < 2; ++qd) {
    if (!bv[qd]) continue;  // workgroup-uniform
    const int iw = ib[qd];
    const int per = (iw + 1 + kXaThreads - 1) / kXaThreads;
    const int j0 = tid * per;
    int32_t mine = 0;
    for (int j = j0; j < min(j0 + per, iw + 1); ++j) mine += hm_at(qd, j) != 0u;
    int32_t count;
    int32_t pos = block_exclusive(mine, redi, &count);
    int32_t* lrow = a.list + static_cast<int64_t>(bk) * xa_row_offset(a.nqb) + xa_row_offset(iw);
    for (int j = j0; j < min(j0 + per, iw + 1); ++j) {
      const uint32_t h = hm_at(qd, j);
      if (h != 0u) lrow[pos++] = j | static_cast<int32_t>(h << 16);
    }
    if (tid == 0) a.cnt[static_cast<int64_t>(bk) * a.nqb + iw] = count;
    __syncthreads();  // redi is reused by the next block's prefix
  }
}

}  // namespace

size_t xa_plan_lds_bytes(const Shape& s) {
  const int nqb = (s.max_seqlen + kXaBlock - 1) / kXaBlock;
  int P2 = 1;
  while (P2 < nqb) P2 <<= 1;
  // the sort keys of one query block reuse the first key tile
  const size_t ktile = static_cast<size_t>(kXaGroupsPerBlock) * (kXaStride * s.d + kXaGroupPad) * 2;
  if (nqb > 4096 || 8u * static_cast<size_t>(P2) > ktile) return 0;
  return 2 * sizeof(uint16_t) * static_cast<size_t>(nqb);
}

hipError_t launch_xa_plan(const Shape& s, const Geometry& g, float tau, const void* Q,
                          const void* K, const int8_t* modes, const int32_t* cu,
                          const Workspace& ws, char* base, float* mass, uint8_t* keep,
                          hipStream_t st) {
  XaArgs a;
  a.Q = static_cast<const uint16_t*>(Q);
  a.K = static_cast<const uint16_t*>(K);
  a.modes = modes;
  a.cu = cu;
  int32_t* meta = reinterpret_cast<int32_t*>(base + ws.meta);
  int32_t* rows = reinterpret_cast<int32_t*>(base + ws.xa_rows);
  a.meta = meta;
  a.rows = rows;
  a.cnt = reinterpret_cast<int32_t*>(base + ws.xa_cnt);
  a.list = reinterpret_cast<int32_t*>(base + ws.xa_list);
  a.lse = reinterpret_cast<float*>(base + ws.xa_lse);
  a.mass = mass;
  a.keep = keep;
  a.B = s.B;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.G = s.G;
  a.nqb = ws.xa_nqb;
  // pairs of query blocks, in whole bands of kXcdChunk
  a.nqb_pad = ((ws.xa_nqb + 1) / 2 + kXcdChunk - 1) / kXcdChunk * kXcdChunk;
  a.head_config = s.head_config;
  a.cs = g.scale * kLog2e / kXaStride;
  a.tau = tau;
  const size_t lds = xa_plan_lds_bytes(s);
  if (lds == 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(xa_rows_kernel, dim3(1), dim3(kXaThreads), 0, st, modes, cu, s.B, s.Hkv,
                     s.head_config, rows, meta);
  // one workgroup per (XA row, pair of query blocks) at most, rounded up to
  // whole rounds of the XCD-chunked order
  constexpr int64_t span = static_cast<int64_t>(kNumXcd) * kXcdChunk;
  const int64_t items = static_cast<int64_t>(a.nqb_pad) * s.B * s.Hkv;
  const unsigned grid = static_cast<unsigned>((items + span - 1) / span * span);
  const void* fn = s.d == 128 ? reinterpret_cast<const void*>(&xa_plan_kernel<128>)
                               : reinterpret_cast<const void*>(&xa_plan_kernel<64>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  if (s.d == 128) hipLaunchKernelGGL(xa_plan_kernel<128>, dim3(grid), dim3(kXaThreads), lds, st, a);
  else hipLaunchKernelGGL(xa_plan_kernel<64>, dim3(grid), dim3(kXaThreads), lds, st, a);
  return hipGetLastError();
}

}  // namespace ea
