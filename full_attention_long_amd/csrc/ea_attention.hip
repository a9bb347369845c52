// Fused hybrid GQA attention forward for gfx950: every work item, FA or SA, in
// one launch.
//
// Pages: FA and SA equations of the preliminaries and the hybrid-head output
// equation (with its GQA footnote) in "Elastic Attention: Test-time Adaptive
// Sparsity Ratios for Efficient Transformers"; the single fused pass over
// mixed-mode heads is "Technical Summary: Elastic Attention", Sec. 2.3.  The
// sparse pattern (sink blocks + causal local window, 64-token blocks) and the
// softmax scale 1/sqrt(d) are the readings stated in ea.h.
//
// Work item = query tile of one KV-head group: 256 rows = G heads x BMq
// positions, one wave per 32 rows, 8 waves per workgroup, so every K/V block
// brought into LDS serves 256 query rows.  Each wave computes the transposed
// score tile S^T = K Q^T (keys x queries) with 32x32 MFMAs so that every lane
// owns one query row: the row max needs one cross-half exchange per key block
// and the row sum none until the epilogue.  Probabilities P^T stay in
// registers in the MFMA result layout and feed O^T += V^T P^T directly; the
// V^T operand is read from the row-major V tile with gfx950's transposing LDS
// read (ds_read_b64_tr_b16), whose 4-key groups also match the key order the
// MFMA result leaves in each lane.  K and V blocks of 64 keys are
// double-buffered through LDS, the next blocks' loads in flight during the
// current block's MFMAs, one barrier per block.
//
// Work-list entries are mapped onto the XCDs in chunks of C = kXcdChunk
// consecutive entries (one per CU of an XCD), dealt to the 8 XCDs in snake
// order (list_position).  The workgroups resident on one XCD then hold runs of
// consecutive entries, which the banded cost sort keeps in query-tile order
// within a KV head, so they stream the same K/V blocks through that XCD's L2 at
// about the same time.
//
// Online softmax in base 2 (scale * log2 e folded into one FMA per score) with
// a lazy running max: the float32 kernel moves it, and rescales O and l, only
// when a row's block max exceeds it by more than 8; the bf16 kernel only when
// a row's probabilities sum past 2^20.  Either way the ratio O / l is exact.
#include "ea_internal.h"

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

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
// bf16 kernel: a row's probabilities may sum to 2^20 before O and l are
// rescaled (fp32 accumulators and bf16 operands keep their relative precision
// at any scale; the sum over a whole sequence stays far below float range)
constexpr float kSumLimit = 1048576.0f;
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kValuPerMfma = 5;
constexpr int kDsAhead = 4;
constexpr int kPvAhead = 4;
// word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data, no swizzle)
constexpr int kBufferWord3 = 0x00020000;
constexpr float kMinusBig = -1.0e30f;      // finite "minus infinity" for the running max

struct AttnArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;          // outputs of FA and SA items
  float* lse;
  void* O_mid;      // outputs of middle-set items (dual-mode forward)
  float* lse_mid;
  const int32_t* cu;
  const int32_t* seq_w;
  const Item* items;
  const int32_t* order;
  const int32_t* meta;
  const int32_t* xa_list;  // XA mode: kept key blocks per (sequence, KV head, XA query block)
  const int32_t* xa_cnt;
  int64_t T;
  int32_t Hq, Hkv, G, BMq, n_sink, stamp, parts, xa_nqb;
  float scale_log2;
};

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Four bf16 of one V column, rows r..r+3 of a 4-row group, per lane of each
// 16-lane group (gfx950 transposing LDS read).
__device__ __forceinline__ i16x4 ds_read_tr(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// ---------------------------------------------------------------------------
// float32 kernel (the correctness path): 32x32x2 fp32 MFMAs, K and V tiles
// staged through registers into padded LDS rows, double-buffered.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kAttnWaves * 64, 2) void attention_kernel_f32(AttnArgs a) {
  using E = float;
  constexpr int NT = kAttnWaves * 64;      // threads per workgroup
  constexpr int CH = 16 / sizeof(E);       // elements per 16-byte chunk
  constexpr int KROW = D + CH;             // padded LDS row of K (elements)
  constexpr int VROW = D + CH;             // padded LDS row of V (elements)
  constexpr int NLD = kBlock * D / CH / NT;  // 16-byte chunks per thread per block (K and V each)
  constexpr int DT = D / 32;               // 32-wide dim tiles of O^T
  static_assert(NLD * NT * CH == kBlock * D, "tile must split evenly over the workgroup");

  __shared__ __attribute__((aligned(16))) E Ks[2][kBlock * KROW];
  __shared__ __attribute__((aligned(16))) E Vs[2][kBlock * VROW];

  // XCD-chunked position in the cost-sorted work list
  const int64_t pos_in_list = list_position(blockIdx.x);
  if (a.meta[kMetaStamp] != a.stamp) return;  // workspace not planned for these sizes
  if (pos_in_list >= static_cast<int64_t>(a.meta[kMetaTiles]) * a.Hkv * a.parts) return;
  const Item it = a.items[a.order[pos_in_list]];
  const int b = it.b, kvh = it.kvh;
  const int tok0 = a.cu[b];
  const int L = a.cu[b + 1] - tok0;
  const int mode = it.mode;
  const int ns = a.n_sink;
  const int w = a.seq_w[b];
  const int p0 = it.qt * a.BMq;
  const int p1 = min(p0 + a.BMq, L) - 1;
  const int qb0 = p0 / kBlock, qb1 = p1 / kBlock;

  // Visible key blocks: [0, r1_end) then [r2_beg, r2_beg + nblk - r1_end).
  const KeyRange kr = key_range(mode, qb0, qb1, ns, w);
  const int r1_end = kr.r1_end, r2_beg = kr.r2_beg;
  const int nblk = kr.count();
  E* const Oout = static_cast<E*>(mode == kModeMiddle ? a.O_mid : a.O);
  float* const lse_out = mode == kModeMiddle ? a.lse_mid : a.lse;

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, h = lane / 32, lq = lane % 32;
  const int row = wave * 32 + lq;
  const int hh = row / a.BMq;
  const int pos = p0 + row % a.BMq;
  const bool rvalid = hh < a.G && pos < L;
  const int hq = kvh * a.G + hh;
  const int qblk = pos / kBlock;

  const E* Qp = static_cast<const E*>(a.Q);
  const E* Kp = static_cast<const E*>(a.K);
  const E* Vp = static_cast<const E*>(a.V);

  // ---- Q fragments (B operand of S^T = K Q^T), kept in registers ----
  using QFrag = f32x4;
  constexpr int NQ = D / 8;
  QFrag qf[NQ];
  {
    const E* qrow = Qp + (static_cast<int64_t>(tok0 + pos) * a.Hq + hq) * D;
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      if (rvalid) {
        qf[u] = *reinterpret_cast<const QFrag*>(qrow + 8 * u + 4 * h);
      } else {
        qf[u] = QFrag{};
      }
    }
  }

  // ---- global -> register -> LDS staging of one key block ----
  u32x4 kreg[NLD], vreg[NLD];
  auto gload = [&](int kb) {
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      const int c = n * NT + tid;
      const int row = c / (D / CH), col = (c % (D / CH)) * CH;
      const int key = kb * kBlock + row;
      if (key < L) {
        const int64_t off = (static_cast<int64_t>(tok0 + key) * a.Hkv + kvh) * D + col;
        kreg[n] = *reinterpret_cast<const u32x4*>(Kp + off);
        vreg[n] = *reinterpret_cast<const u32x4*>(Vp + off);
      } else {
        kreg[n] = u32x4{0, 0, 0, 0};
        vreg[n] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      const int c = n * NT + tid;
      const int row = c / (D / CH), col = (c % (D / CH)) * CH;
      *reinterpret_cast<u32x4*>(&Ks[buf][row * KROW + col]) = kreg[n];
      *reinterpret_cast<u32x4*>(&Vs[buf][row * VROW + col]) = vreg[n];
    }
  };
  auto kb_of = [&](int n) { return n < r1_end ? n : r2_beg + (n - r1_end); };

  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = f32x16{};
  float m_run = kMinusBig, l_run = 0.f;
  const float c = a.scale_log2;

  gload(kb_of(0));
  lstore(0);
  __syncthreads();

  for (int n = 0; n < nblk; ++n) {
    const int kb = kb_of(n);
    const int buf = n & 1;
    if (n + 1 < nblk) gload(kb_of(n + 1));

    // ---- S^T tiles: keys [0,32) and [32,64) of the block x this wave's 32 queries ----
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    const E* k0 = &Ks[buf][lq * KROW];
    const E* k1 = &Ks[buf][(32 + lq) * KROW];
#pragma unroll
    for (int g = 0; g < D / 8; ++g) {
      const f32x4 ka = *reinterpret_cast<const f32x4*>(k0 + 8 * g + 4 * h);
      const f32x4 kb2 = *reinterpret_cast<const f32x4*>(k1 + 8 * g + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s0 = mfma_f32(ka[e], qf[g][e], s0);
        s1 = mfma_f32(kb2[e], qf[g][e], s1);
      }
    }

    // ---- mask the diagonal and window-edge blocks (element (i) is key 8(i/4)+4h+(i%4)) ----
    const bool full = block_full(mode, kb, p0, qb0, qb1, ns, w);
    if (!full) {
      const bool blk_ok = block_visible(mode, kb, qblk, ns, w);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = kb * kBlock + 8 * (i / 4) + 4 * h + (i % 4);
        if (!(blk_ok && j <= pos)) s0[i] = -INFINITY;
        if (!(blk_ok && j + 32 <= pos)) s1[i] = -INFINITY;
      }
    }

    // ---- online softmax (base 2, lazy rescale) ----
    float mx = s0[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s0[i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s1[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mc = mx * c;
    if (__ballot(mc > m_run + kRescaleThreshold)) {
      const float mn = fmaxf(m_run, mc);
      const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < DT; ++t) o[t] *= alpha;
    }
    const float nm = -m_run;
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], c, nm));
      s1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c, nm));
      ls += s0[i] + s1[i];
    }
    l_run += ls;

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const E* vcol = &Vs[buf][32 * t + lq];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i / 4) + 4 * h + (i % 4);
        o[t] = mfma_f32(vcol[key * VROW], s0[i], o[t]);
        o[t] = mfma_f32(vcol[(key + 32) * VROW], s1[i], o[t]);
      }
    }

    if (n + 1 < nblk) lstore((n + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, written in place in [T, Hq, D]; LSE ----
  // (a row that sees no key of a middle-set item gets O = 0 and LSE = -inf)
  const float lt = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (rvalid) {
    E* orow = Oout + (static_cast<int64_t>(tok0 + pos) * a.Hq + hq) * D;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int dim = 32 * t + 8 * q + 4 * h;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = o[t][4 * q + e] * inv;
        *reinterpret_cast<f32x4*>(orow + dim) = v;
      }
    }
    if (h == 0 && lse_out)
      lse_out[static_cast<int64_t>(hq) * a.T + tok0 + pos] = lt > 0.f ? (m_run + __log2f(lt)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// bf16 kernel.
//
// Software pipeline over the item's visible key blocks 0..nblk-1.  Iteration n
// computes, in one basic block, the score MFMAs of block n + 1 (S = K Q^T)
// with the softmax VALU work of block n interleaved between them
// (exponentials, bf16 conversion, row sums), then O^T += V_n^T P_n^T.  The
// exponentials use the row's running offset m of earlier blocks; only when a
// row's probabilities sum past kSumLimit (or m is unset) does a rare branch
// take the row max, rescale O and l, and recompute P.
//
// K and V tiles of 64 keys reach LDS by direct buffer-to-LDS loads (no
// register staging) one iteration ahead: iteration n loads K_{n+2} into the
// buffer K_n left free and V_{n+1} into the buffer V_{n-1} left free, while it
// reads K_{n+1} and V_n.  Each 1 KiB load instruction of a wave fills 4
// (d = 128) or 8 (d = 64) consecutive rows.  K rows sit in groups of one
// instruction's rows, each group padded by 64 bytes, with the 16-byte chunks
// of a row XOR-swizzled inside its group; V rows are unpadded with chunks
// swizzled by 4 (row % 4).  Both spread the 16-byte K reads and the
// transposing V reads over the 64 LDS banks.  The buffer range ends at the
// sequence end, so rows past it read as zeros.  LDS operand reads run a few
// MFMAs ahead of their use.
// ---------------------------------------------------------------------------
template <int D, bool XA>
__global__ __launch_bounds__(kAttnWaves * 64, 2) void attention_kernel_bf16(AttnArgs a) {
  constexpr int CPR = D / 8;                     // 16-byte chunks per row
  constexpr int TILE = kBlock * D;               // elements of one K or V tile
  constexpr int RPI = 1024 / (2 * D);            // rows per 1 KiB load instruction
  constexpr int NDMA = kBlock / RPI / kAttnWaves;  // load instructions per wave per tile
  constexpr int DT = D / 32;
  constexpr int NQ = D / 16;
  // K tile: groups of RPI rows (one load instruction each) padded by 64 bytes;
  // within a group, row j's chunks are XOR-swizzled by kfold(j) in 0..3.
  constexpr int KGS = RPI * D + 32;              // K group stride (elements)
  constexpr int KTILE = (kBlock / RPI) * KGS;    // elements of one K tile
  constexpr int VSW = (CPR / 4) - 1;             // V: chunk ^ 4 ((row & 3) & VSW)
  static_assert(NDMA >= 1 && NDMA * RPI * kAttnWaves == kBlock, "tile must split evenly");
  auto kfold = [](int j) { return D == 128 ? j : (j >> 1); };

  // four separate LDS arrays, each addressed only through its own name, so that
  // the compiler can tell a direct load into one from reads of another
  __shared__ __attribute__((aligned(1024))) uint16_t Ks0[KTILE], Ks1[KTILE], Vs0[TILE], Vs1[TILE];

  const int64_t pos_in_list = list_position(blockIdx.x);
  if (a.meta[kMetaStamp] != a.stamp) return;  // workspace not planned for these sizes
  if (pos_in_list >= static_cast<int64_t>(a.meta[kMetaTiles]) * a.Hkv * a.parts) return;
  const Item it = a.items[a.order[pos_in_list]];
  const int b = it.b, kvh = it.kvh;
  const int tok0 = a.cu[b];
  const int L = a.cu[b + 1] - tok0;
  const int mode = it.mode;
  const int ns = a.n_sink;
  const int w = a.seq_w[b];
  const int p0 = it.qt * a.BMq;
  const int p1 = min(p0 + a.BMq, L) - 1;
  const int qb0 = p0 / kBlock, qb1 = p1 / kBlock;
  const KeyRange kr = key_range(mode, qb0, qb1, ns, w);
  const int r1_end = kr.r1_end, r2_beg = kr.r2_beg;
  int nblk = kr.count();
  // XA item: the ascending list of the tile's XA query block (entries
  // j | head mask << 16 for kept 128-blocks j, each two 64-blocks), less the
  // diagonal block's second half when the tile ends before it
  // (read through the constant address space: the list does not change
  // during the launch, so its entries come by scalar loads, which the DMA
  // loads' vmcnt does not count; as ordinary global loads, every entry read
  // waited for all the tile loads in flight)
  typedef const __attribute__((address_space(4))) int32_t cint32;
  cint32* xl = nullptr;
  if constexpr (XA) {
    if (mode == kModeXA) {
      const int xi = p0 / kXaBlock;
      const int64_t bk = static_cast<int64_t>(b) * a.Hkv + kvh;
      xl = (cint32*)(a.xa_list + bk * xa_row_offset(a.xa_nqb) + xa_row_offset(xi));
      nblk = 2 * a.xa_cnt[bk * a.xa_nqb + xi] - (2 * xi + 1 > qb1 ? 1 : 0);
    }
  }
  // The entries m = n / 2 and m + 1 that the pair of blocks n, n + 1 and
  // their loads ahead need stay in registers, and the next one is loaded a
  // pair ahead (read where it is needed, each entry's scalar load was waited
  // for at once, after the barrier, before any matrix work of the block).
  int xm = 0, xe0 = 0, xe1 = 0, xlast = 0;
  if constexpr (XA) {
    if (mode == kModeXA && nblk > 0) {
      xlast = (nblk + 1) / 2 - 1;
      xe0 = xl[0];
      xe1 = xl[min(1, xlast)];
    }
  }
  // (for n in [2 xm, 2 xm + 3], the range every caller stays in)
  auto kb_of = [&](int n) {
    if constexpr (XA) {
      if (mode == kModeXA) return 2 * (((n >> 1) == xm ? xe0 : xe1) & 0xFFFF) + (n & 1);
    }
    return n < r1_end ? n : r2_beg + (n - r1_end);
  };
  uint16_t* const Oout = static_cast<uint16_t*>(mode == kModeMiddle ? a.O_mid : a.O);
  float* const lse_out = mode == kModeMiddle ? a.lse_mid : a.lse;
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, h = lane / 32, lq = lane % 32;
  const int row = wave * 32 + lq;
  const int hh = row / a.BMq;
  const int pos = p0 + row % a.BMq;
  const bool rvalid = hh < a.G && pos < L;
  const int hq = kvh * a.G + hh;
  const int qblk = pos / kBlock;

  bf16x8 qf[NQ];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.Q) + (static_cast<int64_t>(tok0 + pos) * a.Hq + hq) * D;
#pragma unroll
    for (int u = 0; u < NQ; ++u)
      qf[u] = rvalid ? *reinterpret_cast<const bf16x8*>(qrow + 16 * u + 8 * h) : bf16x8{};
  }

  // Direct loads of one tile: instruction i of this wave fills rows
  // r0 .. r0 + RPI - 1 (r0 = (wave NDMA + i) RPI); lane l writes physical chunk
  // l % CPR of row r0 + l / CPR, i.e. logical chunk (l % CPR) ^ swizzle(row).
  const int rs = a.Hkv * D;  // row stride; L * rs < 2^31 is checked on the host
  const uint16_t* Kseq = static_cast<const uint16_t*>(a.K) + (static_cast<int64_t>(tok0) * a.Hkv + kvh) * D;
  const uint16_t* Vseq = static_cast<const uint16_t*>(a.V) + (static_cast<int64_t>(tok0) * a.Hkv + kvh) * D;
  int dma_koff[NDMA], dma_voff[NDMA];  // byte offsets within a tile's rows
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int r = (wave * NDMA + i) * RPI + lane / CPR;
    dma_koff[i] = (r * rs + ((lane % CPR) ^ kfold(lane / CPR)) * 8) * 2;
    dma_voff[i] = (r * rs + ((lane % CPR) ^ (4 * ((r & 3) & VSW))) * 8) * 2;
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

  // Per-lane LDS offsets (elements) of the swizzled reads.
  // K: row lq (+32), in group g = lq / RPI at j = lq % RPI, chunk
  // (2u + h) ^ f = 2 (u ^ b) + (h ^ e) with f = kfold(j) = 2b + e: an even-u
  // and an odd-u lane offset plus a uniform 16u.  Over any 16 consecutive rows
  // the 16-byte reads of one chunk land on 16 distinct bank groups.
  int koff_e, koff_o;
  {
    const int j = lq % RPI, f = kfold(j), bb = f >> 1, e = f & 1;
    const int base = (lq / RPI) * KGS + j * D + (h ^ e) * 8;
    koff_e = base + 16 * bb;
    koff_o = base - 16 * bb;
  }
  // V: rows 16u + 4h + (lane & 15) / 4 (+8), column 32t + 16 ((lane >> 4) & 1) + 4 (lane & 3);
  // chunk 4t + c_low becomes 4 (t ^ j) + c_low with j = ((lane >> 2) & 3) & VSW.
  int voff[DT];
  {
    const int vr = 4 * h + (lane & 15) / 4;
    const int clow = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int j = ((lane >> 2) & 3) & VSW;
#pragma unroll
    for (int t = 0; t < DT; ++t) voff[t] = vr * D + (4 * (t ^ j) + clow) * 8 + 4 * (lane & 1);
  }

  auto scores = [&](const uint16_t* kt, f32x16& s0, f32x16& s1) {
    s0 = f32x16{};
    s1 = f32x16{};
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int o0 = ((u & 1) ? koff_o : koff_e) + 16 * u;
      s0 = mfma_bf16(*reinterpret_cast<const bf16x8*>(kt + o0), qf[u], s0);
      s1 = mfma_bf16(*reinterpret_cast<const bf16x8*>(kt + o0 + (32 / RPI) * KGS), qf[u], s1);
    }
  };

  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = f32x16{};
  float m_run = kMinusBig, l_run = 0.f;
  const float c = a.scale_log2;

  auto pv = [&](const uint16_t* vt, const bf16x8* pb) {
#pragma unroll
    for (int t = 0; t < DT; ++t) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const i16x4 lo = ds_read_tr(vt + voff[t] + 16 * u * D);
        const i16x4 hi = ds_read_tr(vt + voff[t] + (16 * u + 8) * D);
        const i16x8 v8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[t] = mfma_bf16(__builtin_bit_cast(bf16x8, v8), pb[u], o[t]);
      }
    }
    // keep the transposing reads kPvAhead MFMAs ahead of their use
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kPvAhead, 0);
#pragma unroll
    for (int i = 0; i < 4 * DT; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (i + kPvAhead < 4 * DT) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
  };

  // hmask: XA heads of the group that kept block kb (XA items only)
  auto mask = [&](int kb, uint32_t hmask, f32x16& s0, f32x16& s1) {
    bool blk_ok;
    if constexpr (XA) {
      blk_ok = mode == kModeXA ? ((hmask >> hh) & 1u) != 0u : block_visible(mode, kb, qblk, ns, w);
    } else {
      blk_ok = block_visible(mode, kb, qblk, ns, w);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = kb * kBlock + 8 * (i / 4) + 4 * h + (i % 4);
      if (!(blk_ok && j <= pos)) s0[i] = -INFINITY;
      if (!(blk_ok && j + 32 <= pos)) s1[i] = -INFINITY;
    }
  };

  // P = exp2(s c - m) as bf16 MFMA operands; returns the row sum of the
  // unrounded values (LSE keeps float32 accuracy).
  auto expcvt = [&](const f32x16& s0, const f32x16& s1, float nm, bf16x8* pb) {
    float ls = 0.f;
    f32x8 t;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x16& sv = q < 2 ? s0 : s1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        t[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[8 * (q & 1) + e], c, nm));
        ls += t[e];
      }
      pb[q] = __builtin_convertvector(t, bf16x8);
    }
    return ls;
  };

  // Softmax of one block (scores s0, s1) into pb; rescales O and l when needed.
  auto softmax = [&](f32x16& s0, f32x16& s1, bf16x8* pb) {
    float ls = expcvt(s0, s1, -m_run, pb);
    float row_sum;
    {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(ls), __float_as_uint(ls), false, false);
      row_sum = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    // Interleave the next block's score MFMAs (each fed by an LDS read issued
    // a few MFMAs ahead) with this block's exponentials.
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kDsAhead, 0);
#pragma unroll
    for (int i = 0; i < 2 * NQ; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (i + kDsAhead < 2 * NQ) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, kValuPerMfma, 0);
    }
    const bool upd = row_sum > kSumLimit;
    if (__ballot(upd)) {
      float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
      const float mn = upd ? fmaxf(m_run, mx * c) : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < DT; ++t) o[t] *= alpha;
      bf16x8 pn[4];
      const float ln = expcvt(s0, s1, -m_run, pn);
#pragma unroll
      for (int u = 0; u < 4; ++u) pb[u] = upd ? pn[u] : pb[u];
      ls = upd ? ln : ls;
    }
    l_run += ls;
  };

  // A middle-set tile can have no block at all (its rows see no key beyond the
  // SA set): it skips straight to the epilogue and writes O = 0, LSE = -inf.
  if (nblk > 0) {
  // Prologue: K_0, K_1 and V_0 into LDS, scores of block 0.
  dma(Kseq, dma_koff, Ks0, KGS, kb_of(0));
  dma(Kseq, dma_koff, Ks1, KGS, kb_of(min(1, nblk - 1)));
  dma(Vseq, dma_voff, Vs0, RPI * D, kb_of(0));
  __syncthreads();
  f32x16 sa0, sa1, sb0, sb1;
  scores(Ks0, sa0, sa1);
  __syncthreads();  // K_0 fully read before K_2 replaces it

  // Iteration n: loads of K_{n+2} (into the K buffer of parity n) and V_{n+1}
  // (into the V buffer of parity n + 1) in flight; scores of block n + 1 from
  // the other K buffer interleaved with the softmax of block n; then
  // O += V_n P_n.  Even and odd iterations are written out separately so that
  // every LDS array is named statically.
  auto iter = [&](int n, f32x16& c0, f32x16& c1, f32x16& x0, f32x16& x1, uint16_t* kload,
                  const uint16_t* kread, uint16_t* vload, const uint16_t* vread) {
    const int kb = kb_of(n);
    uint32_t hmask = 0u;
    bool full;
    if constexpr (XA) {
      if (mode == kModeXA) {
        hmask = static_cast<uint32_t>(xe0) >> 16;  // entry n / 2 = xm
        full = hmask == (1u << a.G) - 1u && kb * kBlock + kBlock - 1 <= p0;
      } else {
        full = block_full(mode, kb, p0, qb0, qb1, ns, w);
      }
    } else {
      full = block_full(mode, kb, p0, qb0, qb1, ns, w);
    }
    if (!full) mask(kb, hmask, c0, c1);
    dma(Kseq, dma_koff, kload, KGS, kb_of(min(n + 2, nblk - 1)));
    dma(Vseq, dma_voff, vload, RPI * D, kb_of(min(n + 1, nblk - 1)));
    // a wave in the score / softmax phase issues ahead of one in the O += V P
    // phase on the same SIMD (its VALU work is what the other's MFMAs hide)
    __builtin_amdgcn_s_setprio(1);
    scores(kread, x0, x1);
    bf16x8 pb[4];
    softmax(c0, c1, pb);
    __builtin_amdgcn_s_setprio(0);
    pv(vread, pb);
    __syncthreads();
  };
  for (int n = 0; n < nblk; n += 2) {
    int xe2 = 0;
    if constexpr (XA) {
      if (mode == kModeXA) xe2 = xl[min(xm + 2, xlast)];
    }
    iter(n, sa0, sa1, sb0, sb1, Ks0, Ks1, Vs1, Vs0);
    if (n + 1 < nblk) iter(n + 1, sb0, sb1, sa0, sa1, Ks1, Ks0, Vs0, Vs1);
    if constexpr (XA) {
      ++xm;
      xe0 = xe1;
      xe1 = xe2;
    }
  }
  }

  // Epilogue: O = O^T / l in place in [T, Hq, D]; LSE.
  float lt;
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    lt = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;  // no visible key (middle set): O = 0
  if (rvalid) {
    uint16_t* orow = Oout + (static_cast<int64_t>(tok0 + pos) * a.Hq + hq) * D;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = o[t][4 * q + e] * inv;
        *reinterpret_cast<bf16x4*>(orow + 32 * t + 8 * q + 4 * h) = __builtin_convertvector(v, bf16x4);
      }
    }
    if (h == 0 && lse_out)
      lse_out[static_cast<int64_t>(hq) * a.T + tok0 + pos] = lt > 0.f ? (m_run + __log2f(lt)) * kLn2 : -INFINITY;
  }
}

template <bool BF16, int D>
void launch(const AttnArgs& args, unsigned grid, bool xa, hipStream_t st) {
  if constexpr (BF16) {
    if (xa)
      hipLaunchKernelGGL((attention_kernel_bf16<D, true>), dim3(grid), dim3(kAttnWaves * 64), 0, st, args);
    else
      hipLaunchKernelGGL((attention_kernel_bf16<D, false>), dim3(grid), dim3(kAttnWaves * 64), 0, st, args);
  } else {
    hipLaunchKernelGGL((attention_kernel_f32<D>), dim3(grid), dim3(kAttnWaves * 64), 0, st, args);
  }
}

}  // namespace

hipError_t launch_attention(const Shape& s, const Geometry& g, const void* Q, const void* K,
                            const void* V, const int32_t* cu, const AttnOut& out,
                            const Workspace& ws, char* base, hipStream_t st) {
  AttnArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = out.O;
  a.lse = out.lse;
  a.O_mid = out.O_mid;
  a.lse_mid = out.lse_mid;
  a.cu = cu;
  a.seq_w = reinterpret_cast<const int32_t*>(base + ws.seq_w);
  a.items = reinterpret_cast<const Item*>(base + ws.items_raw);
  a.order = reinterpret_cast<const int32_t*>(base + ws.order);
  a.meta = reinterpret_cast<const int32_t*>(base + ws.meta);
  a.T = s.T;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.G = s.G;
  a.BMq = s.BMq;
  a.n_sink = g.n_sink;
  a.stamp = plan_stamp(s);
  a.parts = s.parts;
  a.scale_log2 = g.scale_log2;
  a.xa_list = s.xa ? reinterpret_cast<const int32_t*>(base + ws.xa_list) : nullptr;
  a.xa_cnt = s.xa ? reinterpret_cast<const int32_t*>(base + ws.xa_cnt) : nullptr;
  a.xa_nqb = ws.xa_nqb;
  constexpr int64_t span = static_cast<int64_t>(kNumXcd) * kXcdChunk;
  const unsigned grid = static_cast<unsigned>((ws.max_items + span - 1) / span * span);
  const bool bf16 = s.elem_bytes == 2;
  // XA items exist only in bf16 (the caller rejects float32 with XA heads)
  const bool xa = s.xa != 0;
  if (xa && !bf16) return hipErrorInvalidValue;
  if (bf16 && s.d == 128) launch<true, 128>(a, grid, xa, st);
  else if (bf16 && s.d == 64) launch<true, 64>(a, grid, xa, st);
  else if (!bf16 && s.d == 128) launch<false, 128>(a, grid, xa, st);
  else launch<false, 64>(a, grid, xa, st);
  return hipGetLastError();
}

}  // namespace ea
