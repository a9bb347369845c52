// Per-launch work list of the fused hybrid attention forward, and the
// transposed copy of V its inner product with the probabilities reads.
//
// One work item is a query tile of one KV-head group of one sequence: all G
// query heads of the group for BMq = 128 / G consecutive positions, so the
// heads that share a K/V block also share its trip through LDS (GQA; footnote
// of the hybrid-head output equation in "Elastic Attention: Test-time Adaptive
// Sparsity Ratios for Efficient Transformers").  The item's cost is the number
// of 64-token key blocks its rows can see: all causal blocks for an FA head,
// sink blocks plus the local window for an SA head.  Items are counting-sorted
// by descending cost so the largest start first (longest-processing-time
// order) and FA and SA tiles balance over the compute units in one launch,
// without splitting any tile or recombining partial results (the fused kernel
// of "Technical Summary: Elastic Attention", Sec. 2.3).
//
// Everything runs on the device, stream-ordered after the router, with no
// host round trip: the host only knows upper bounds of the item count.
#include "ea_internal.h"

#include <math.h>

namespace ea {
namespace {

constexpr int kScanThreads = 1024;

// Exclusive scan of n int32 values in place by one workgroup; returns the total.
__device__ int32_t block_exclusive_scan(int32_t* a, int64_t n, int32_t* tmp /* [kScanThreads/64 + 1] */) {
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  int32_t carry = 0;
  for (int64_t base = 0; base < n; base += kScanThreads) {
    const int64_t i = base + tid;
    const int32_t v = i < n ? a[i] : 0;
    int32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) tmp[wave] = x;
    __syncthreads();
    if (tid == 0) {
      int32_t s = 0;
      for (int w = 0; w < kScanThreads / 64; ++w) {
        const int32_t t = tmp[w];
        tmp[w] = s;
        s += t;
      }
      tmp[kScanThreads / 64] = s;
    }
    __syncthreads();
    if (i < n) a[i] = carry + tmp[wave] + x - v;
    carry += tmp[kScanThreads / 64];
    __syncthreads();
  }
  return carry;
}

// Per-sequence sizes: tiles, key blocks, window; zero the cost histogram.
__global__ __launch_bounds__(kScanThreads) void setup_kernel(
    const int32_t* __restrict__ cu, int32_t B, int32_t BMq, int32_t n_sink, int32_t window_blocks,
    float keep_fraction, int32_t* __restrict__ meta, int32_t* __restrict__ tile_prefix,
    int32_t* __restrict__ vblk_prefix, int32_t* __restrict__ seq_w, int32_t* __restrict__ hist,
    int32_t nbins) {
  __shared__ int32_t tmp[kScanThreads / 64 + 1];
  for (int i = threadIdx.x; i < nbins; i += kScanThreads) hist[i] = 0;
  for (int b = threadIdx.x; b < B; b += kScanThreads) {
    const int L = max(0, cu[b + 1] - cu[b]);
    const int N = (L + kBlock - 1) / kBlock;
    tile_prefix[b] = (L + BMq - 1) / BMq;
    vblk_prefix[b] = N;
    int w = window_blocks;
    if (w <= 0) {
      // keep = max(n_sink + 1, floor(rho * N + 1/2)), in double on the float value
      const double keep = floor(static_cast<double>(keep_fraction) * static_cast<double>(N) + 0.5);
      const int k = max(n_sink + 1, static_cast<int>(keep));
      w = k - n_sink;
    }
    seq_w[b] = w;
  }
  __syncthreads();
  const int32_t tiles = block_exclusive_scan(tile_prefix, B, tmp);
  const int32_t vblocks = block_exclusive_scan(vblk_prefix, B, tmp);
  if (threadIdx.x == 0) {
    tile_prefix[B] = tiles;
    vblk_prefix[B] = vblocks;
    meta[kMetaTiles] = tiles;
    meta[kMetaVBlocks] = vblocks;
  }
}

// Index of the last prefix entry <= x (prefix is non-decreasing, prefix[0] = 0).
__device__ __forceinline__ int find_seq(const int32_t* prefix, int B, int32_t x) {
  int lo = 0, hi = B;  // invariant: prefix[lo] <= x < prefix[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ int item_cost(int mode, int p0, int p1, int n_sink, int w) {
  const int qb0 = p0 / kBlock, qb1 = p1 / kBlock;
  if (mode == 0) return qb1 + 1;
  const int ws = max(0, qb0 - w + 1);
  return min(n_sink, ws) + (qb1 + 1 - ws);
}

__global__ __launch_bounds__(256) void items_kernel(
    const int32_t* __restrict__ cu, const int8_t* __restrict__ modes, int32_t B, int32_t Hkv,
    int32_t BMq, int32_t n_sink, const int32_t* __restrict__ meta,
    const int32_t* __restrict__ tile_prefix, const int32_t* __restrict__ seq_w,
    int32_t* __restrict__ hist, int32_t nbins, Item* __restrict__ raw) {
  const int64_t x = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int32_t tiles = meta[kMetaTiles];
  if (x >= static_cast<int64_t>(tiles) * Hkv) return;
  const int kvh = static_cast<int>(x / tiles);
  const int32_t rem = static_cast<int32_t>(x - static_cast<int64_t>(kvh) * tiles);
  const int b = find_seq(tile_prefix, B, rem);
  const int qt = rem - tile_prefix[b];
  const int L = cu[b + 1] - cu[b];
  const int p0 = qt * BMq, p1 = min(p0 + BMq, L) - 1;
  const int mode = modes[static_cast<int64_t>(b) * Hkv + kvh] != 0 ? 1 : 0;
  const int cost = item_cost(mode, p0, p1, n_sink, seq_w[b]);
  Item it;
  it.b = b;
  it.kvh = kvh;
  it.qt = qt;
  it.cost = cost;
  raw[x] = it;
  const int bin = nbins - 1 - min(cost, nbins - 1);  // bin 0 = most expensive
  atomicAdd(&hist[bin], 1);
}

__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    int32_t* __restrict__ meta, const int32_t* __restrict__ hist, int32_t* __restrict__ cursor,
    int32_t nbins) {
  __shared__ int32_t tmp[kScanThreads / 64 + 1];
  for (int i = threadIdx.x; i < nbins; i += kScanThreads) cursor[i] = hist[i];
  __syncthreads();
  const int32_t n = block_exclusive_scan(cursor, nbins, tmp);
  if (threadIdx.x == 0) meta[kMetaItems] = n;
}

__global__ __launch_bounds__(256) void scatter_kernel(
    const int32_t* __restrict__ meta, int32_t Hkv, int32_t* __restrict__ cursor, int32_t nbins,
    const Item* __restrict__ raw, Item* __restrict__ items) {
  const int64_t x = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (x >= static_cast<int64_t>(meta[kMetaTiles]) * Hkv) return;
  const Item it = raw[x];
  const int bin = nbins - 1 - min(it.cost, nbins - 1);
  const int32_t pos = atomicAdd(&cursor[bin], 1);
  items[pos] = it;
}

// V [T, Hkv, d] -> Vt [Hkv][d][tpad]: each sequence starts at a 64-aligned
// column (its key-block prefix * 64), padding columns are zero, and within
// every aligned group of 16 keys the columns hold keys in the order
// 0-3, 8-11, 4-7, 12-15.  That order is the one in which a 32x32 MFMA result
// tile leaves probabilities in the lanes (lane half h holds keys 4h..4h+3 and
// 8+4h..8+4h+3 of each 16), so the probability-times-V product reads each
// lane's 8 keys as one contiguous 16-byte row segment.
template <typename E, int D>
__global__ __launch_bounds__(256) void transpose_v_kernel(
    const E* __restrict__ V, const int32_t* __restrict__ cu, int32_t B, int32_t Hkv,
    const int32_t* __restrict__ meta, const int32_t* __restrict__ vblk_prefix, int64_t tpad,
    E* __restrict__ Vt) {
  constexpr int CH = 16 / sizeof(E);       // elements per 16-byte chunk
  constexpr int ROW = D + CH;              // padded LDS row
  __shared__ __attribute__((aligned(16))) E tile[kBlock * ROW];
  const int kvh = blockIdx.y;
  const int32_t x = blockIdx.x;
  if (x >= meta[kMetaVBlocks]) return;
  const int b = find_seq(vblk_prefix, B, x);
  const int kb = x - vblk_prefix[b];
  const int s0 = cu[b];
  const int L = cu[b + 1] - s0;
  const int n = min(kBlock, L - kb * kBlock);
  // load 64 rows x D (zero past the sequence end)
  constexpr int CHUNKS = kBlock * D / CH;
  for (int c = threadIdx.x; c < CHUNKS; c += 256) {
    const int row = c / (D / CH), col = (c % (D / CH)) * CH;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < n) {
      const int64_t off = (static_cast<int64_t>(s0 + kb * kBlock + row) * Hkv + kvh) * D + col;
      v = *reinterpret_cast<const uint4*>(V + off);
    }
    *reinterpret_cast<uint4*>(&tile[row * ROW + col]) = v;
  }
  __syncthreads();
  // write D rows x 64 columns in the permuted key order
  constexpr int OCHUNKS = D * kBlock / CH;
  const int64_t col0 = static_cast<int64_t>(x) * kBlock;
  for (int c = threadIdx.x; c < OCHUNKS; c += 256) {
    const int dim = c / (kBlock / CH), p0 = (c % (kBlock / CH)) * CH;
    E vals[CH];
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      const int p = p0 + e;                       // storage position in the block
      const int g16 = p & ~15, q = p & 15;        // 16-group base, position in group
      const int half = q >> 3, j = q & 7;
      const int key = g16 + ((j >> 2) << 3) + (half << 2) + (j & 3);
      vals[e] = tile[key * ROW + dim];
    }
    *reinterpret_cast<uint4*>(Vt + (static_cast<int64_t>(kvh) * D + dim) * tpad + col0 + p0) =
        *reinterpret_cast<const uint4*>(vals);
  }
}

}  // namespace

Workspace plan_workspace(const Shape& s) {
  auto align = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  Workspace w{};
  w.nbins = (s.max_seqlen + kBlock - 1) / kBlock + 1;
  w.max_items = static_cast<int64_t>(s.Hkv) * ((s.T + s.BMq - 1) / s.BMq + s.B);
  w.tpad = ((s.T + kBlock - 1) / kBlock + s.B) * kBlock;
  size_t off = 0;
  w.meta = off;        off = align(off + sizeof(int32_t) * kMetaSlots);
  w.tile_prefix = off; off = align(off + sizeof(int32_t) * (s.B + 1));
  w.vblk_prefix = off; off = align(off + sizeof(int32_t) * (s.B + 1));
  w.seq_w = off;       off = align(off + sizeof(int32_t) * s.B);
  w.hist = off;        off = align(off + sizeof(int32_t) * w.nbins);
  w.cursor = off;      off = align(off + sizeof(int32_t) * w.nbins);
  w.items_raw = off;   off = align(off + sizeof(Item) * w.max_items);
  w.items = off;       off = align(off + sizeof(Item) * w.max_items);
  w.vt = off;          off = align(off + static_cast<size_t>(s.elem_bytes) * s.Hkv * s.d * w.tpad);
  w.total = off;
  return w;
}

hipError_t launch_worklist(const Shape& s, const Geometry& g, const int8_t* modes,
                           const int32_t* cu, const Workspace& ws, char* base, hipStream_t st) {
  int32_t* meta = reinterpret_cast<int32_t*>(base + ws.meta);
  int32_t* tile_prefix = reinterpret_cast<int32_t*>(base + ws.tile_prefix);
  int32_t* vblk_prefix = reinterpret_cast<int32_t*>(base + ws.vblk_prefix);
  int32_t* seq_w = reinterpret_cast<int32_t*>(base + ws.seq_w);
  int32_t* hist = reinterpret_cast<int32_t*>(base + ws.hist);
  int32_t* cursor = reinterpret_cast<int32_t*>(base + ws.cursor);
  Item* raw = reinterpret_cast<Item*>(base + ws.items_raw);
  Item* items = reinterpret_cast<Item*>(base + ws.items);
  hipLaunchKernelGGL(setup_kernel, dim3(1), dim3(kScanThreads), 0, st, cu, s.B, s.BMq, g.n_sink,
                     g.window_blocks, g.keep_fraction, meta, tile_prefix, vblk_prefix, seq_w, hist,
                     ws.nbins);
  const unsigned grid = static_cast<unsigned>((ws.max_items + 255) / 256);
  hipLaunchKernelGGL(items_kernel, dim3(grid), dim3(256), 0, st, cu, modes, s.B, s.Hkv, s.BMq,
                     g.n_sink, meta, tile_prefix, seq_w, hist, ws.nbins, raw);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, st, meta, hist, cursor,
                     ws.nbins);
  hipLaunchKernelGGL(scatter_kernel, dim3(grid), dim3(256), 0, st, meta, s.Hkv, cursor, ws.nbins,
                     raw, items);
  return hipGetLastError();
}

hipError_t launch_transpose_v(const Shape& s, const void* V, const int32_t* cu,
                              const Workspace& ws, char* base, hipStream_t st) {
  const int32_t* meta = reinterpret_cast<const int32_t*>(base + ws.meta);
  const int32_t* vblk_prefix = reinterpret_cast<const int32_t*>(base + ws.vblk_prefix);
  const dim3 grid(static_cast<unsigned>(ws.tpad / kBlock), static_cast<unsigned>(s.Hkv));
  if (s.elem_bytes == 2) {
    using E = uint16_t;
    E* vt = reinterpret_cast<E*>(base + ws.vt);
    if (s.d == 64)
      hipLaunchKernelGGL((transpose_v_kernel<E, 64>), grid, dim3(256), 0, st,
                         static_cast<const E*>(V), cu, s.B, s.Hkv, meta, vblk_prefix, ws.tpad, vt);
    else
      hipLaunchKernelGGL((transpose_v_kernel<E, 128>), grid, dim3(256), 0, st,
                         static_cast<const E*>(V), cu, s.B, s.Hkv, meta, vblk_prefix, ws.tpad, vt);
  } else {
    using E = float;
    E* vt = reinterpret_cast<E*>(base + ws.vt);
    if (s.d == 64)
      hipLaunchKernelGGL((transpose_v_kernel<E, 64>), grid, dim3(256), 0, st,
                         static_cast<const E*>(V), cu, s.B, s.Hkv, meta, vblk_prefix, ws.tpad, vt);
    else
      hipLaunchKernelGGL((transpose_v_kernel<E, 128>), grid, dim3(256), 0, st,
                         static_cast<const E*>(V), cu, s.B, s.Hkv, meta, vblk_prefix, ws.tpad, vt);
  }
  return hipGetLastError();
}

}  // namespace ea
