// Per-launch work list of the fused hybrid attention forward.
//
// One work item is a query tile of one KV-head group of one sequence: all G
// query heads of the group for BMq = kTileRows / G consecutive positions, so
// the heads that share a K/V block also share its trip through LDS (GQA;
// footnote of the hybrid-head output equation in "Elastic Attention:
// Test-time Adaptive Sparsity Ratios for Efficient Transformers").  The
// item's cost is the number of 64-token key blocks its rows can see: all
// causal blocks for an FA head, sink blocks plus the local window for an SA
// head.  The dual-mode (training) forward lists every tile twice, once over
// its head's SA set and once over the causal blocks outside it, whose partial
// results the merge kernel combines into the FA output (ea_dual.hip).
//
// Items are sorted by descending cost with a stable counting sort over the raw
// order (KV head, sequence, query tile), so the list is longest-processing-
// time first, items of equal cost stay in query order within a head, and the
// whole layer, FA and SA tiles together, runs as one launch without splitting
// any tile or recombining partial results (the fused kernel of "Technical
// Summary: Elastic Attention", Sec. 2.3).  The attention kernel maps the list
// onto the XCDs in chunks of consecutive entries (see ea_attention.hip).
//
// Everything runs on the device, stream-ordered after the router, with no
// host round trip: the host only sizes buffers from upper bounds.
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

// Per-sequence query tiles and sparse window, after the device-content checks:
// cu_seqlens starts at 0, never decreases and ends at T, no sequence is longer
// than max_seqlen (buffers are sized from it), and every mode is 0 or 1.  On
// a failed check the header gets the MetaError bits, zero tiles and stamp 0,
// which every later kernel of the call takes as "do nothing".
__global__ __launch_bounds__(kScanThreads) void setup_kernel(
    const int32_t* __restrict__ cu, const int8_t* __restrict__ modes, int32_t B, int32_t Hkv,
    int64_t T, int32_t max_seqlen, int32_t BMq, int32_t n_sink, int32_t window_blocks,
    float keep_fraction, int32_t stamp, int32_t* __restrict__ meta,
    int32_t* __restrict__ tile_prefix, int32_t* __restrict__ seq_w) {
  __shared__ int32_t tmp[kScanThreads / 64 + 1];
  __shared__ int32_t err;
  if (threadIdx.x == 0) err = 0;
  __syncthreads();
  int32_t bad = 0;
  if (threadIdx.x == 0) {
    if (cu[0] != 0) bad |= kErrCuStart;
    if (static_cast<int64_t>(cu[B]) != T) bad |= kErrCuEnd;
  }
  for (int b = threadIdx.x; b < B; b += kScanThreads) {
    const int64_t len = static_cast<int64_t>(cu[b + 1]) - cu[b];
    if (len < 0) bad |= kErrCuOrder;
    if (len > max_seqlen) bad |= kErrSeqLen;
    const int L = len > 0 ? static_cast<int>(len) : 0;
    const int N = (L + kBlock - 1) / kBlock;
    tile_prefix[b] = (L + BMq - 1) / BMq;
    int w = window_blocks;
    if (w <= 0) {
      // keep = max(n_sink + 1, floor(rho * N + 1/2)), in double on the float value
      const double keep = floor(static_cast<double>(keep_fraction) * static_cast<double>(N) + 0.5);
      const int k = max(n_sink + 1, static_cast<int>(keep));
      w = k - n_sink;
    }
    // a window of N blocks already covers every causal key of the sequence;
    // the clamp keeps sums such as (last key block + w) inside int32
    seq_w[b] = min(w, max(N, 1));
  }
  if (modes) {
    const int64_t n = static_cast<int64_t>(B) * Hkv;
    for (int64_t i = threadIdx.x; i < n; i += kScanThreads)
      if (static_cast<uint8_t>(modes[i]) > 1u) bad |= kErrMode;
  }
  if (bad) atomicOr(&err, bad);
  __syncthreads();
  const int32_t tiles = block_exclusive_scan(tile_prefix, B, tmp);
  if (threadIdx.x == 0) {
    tile_prefix[B] = err ? 0 : tiles;
    meta[kMetaTiles] = err ? 0 : tiles;
    meta[kMetaXaRows] = 0;
    meta[kMetaError] = err;
    meta[kMetaStamp] = err ? 0 : stamp;
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

// Raw item x (part major, then KV head, sequence, and query tile from the
// last, most expensive tile down) and its banded sort key; the stable sort
// keeps this raw order inside a band.  With one
// part an item covers its head's routed mode; with two (dual-mode forward)
// part 0 covers every head's SA set and part 1 the rest of its causal blocks.
__global__ __launch_bounds__(256) void items_kernel(
    const int32_t* __restrict__ cu, const int8_t* __restrict__ modes, int32_t B, int32_t Hkv,
    int32_t BMq, int32_t parts, int32_t head_config, int32_t n_sink,
    const int32_t* __restrict__ meta, const int32_t* __restrict__ tile_prefix,
    const int32_t* __restrict__ seq_w, const int32_t* __restrict__ xa_cnt, int32_t xa_nqb,
    int32_t maxcost, int64_t max_items, Item* __restrict__ raw, uint32_t* __restrict__ keys) {
  const int64_t x = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (x >= max_items) return;
  const int32_t tiles = meta[kMetaTiles];
  const int64_t per_part = static_cast<int64_t>(tiles) * Hkv;
  if (x >= per_part * parts) {
    keys[x] = empty_key(maxcost);
    return;
  }
  const int part = static_cast<int>(x / per_part);
  const int64_t xi = x - part * per_part;
  const int kvh = static_cast<int>(xi / tiles);
  const int32_t rem = static_cast<int32_t>(xi - static_cast<int64_t>(kvh) * tiles);
  const int b = find_seq(tile_prefix, B, rem);
  const int qt = (tile_prefix[b + 1] - 1) - rem;
  const int L = cu[b + 1] - cu[b];
  const int p0 = qt * BMq, p1 = min(p0 + BMq, L) - 1;
  int mode;
  if (parts == 1) mode = computation_mode(head_config, modes[static_cast<int64_t>(b) * Hkv + kvh] != 0);
  else mode = part == 0 ? kModeSA : kModeMiddle;
  int cost;
  if (mode == kModeXA) {
    // the kept 128-blocks of the tile's XA query block, two 64-blocks each,
    // less the diagonal block's second half when the tile ends before it
    const int i = p0 / kXaBlock;
    const int cnt = xa_cnt[(static_cast<int64_t>(b) * Hkv + kvh) * xa_nqb + i];
    cost = 2 * cnt - (2 * i + 1 > p1 / kBlock ? 1 : 0);
  } else {
    cost = key_range(mode, p0 / kBlock, p1 / kBlock, n_sink, seq_w[b]).count();
  }
  Item it;
  it.b = b;
  it.kvh = kvh;
  it.qt = qt;
  it.cost = cost;
  it.mode = mode;
  raw[x] = it;
  keys[x] = cost_key(cost, maxcost);
}

// Stable counting sort by key, one workgroup of kSortWaves waves.  The n
// entries split into kSortWaves consecutive segments, one per wave:
//  1. each wave counts its segment's keys into its own LDS histogram;
//  2. an exclusive scan in (key, wave) order turns the histograms into the
//     first output slot of each (key, wave) run;
//  3. each wave walks its segment in steps of 64 entries; a lane's rank
//     among the equal keys of its step (lanes below it with the same key)
//     gives its slot, and the last lane of each key advances that key's slot.
// Equal keys thus keep their index order: within a step by lane, across steps
// by the walk, across segments by the scan order.
__global__ __launch_bounds__(kSortWaves * 64) void key_sort_kernel(const uint32_t* __restrict__ keys,
                                                                   int64_t n,
                                                                   int32_t* __restrict__ order) {
  __shared__ int32_t hist[kSortWaves][kSortBands];
  __shared__ int32_t tmp[kSortWaves + 1];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  for (int i = tid; i < kSortWaves * kSortBands; i += kSortWaves * 64) (&hist[0][0])[i] = 0;
  __syncthreads();
  const int64_t per = (n + kSortWaves - 1) / kSortWaves;
  const int64_t seg0 = min(n, per * wave), seg1 = min(n, seg0 + per);
  // (a step whose 64 keys are all equal, the common case in a band-sorted
  // list, adds its count with one atomic instead of 64 to the same word)
  for (int64_t base = seg0; base < seg1; base += 64) {
    const int64_t i = base + lane;
    const bool valid = i < seg1;
    const uint32_t k = valid ? min(keys[i], kSortBands - 1u) : 0xFFFFFFFFu;
    const uint32_t k0 = __builtin_amdgcn_readfirstlane(k);
    const uint64_t nval = __ballot(valid);
    if (__ballot(valid && k == k0) == nval) {
      if (lane == 0) atomicAdd(&hist[wave][k0], static_cast<int32_t>(__popcll(nval)));
    } else if (valid) {
      atomicAdd(&hist[wave][k], 1);
    }
  }
  __syncthreads();
  // thread t owns key t (kSortBands == kSortWaves * 64): its total over the
  // waves, scanned across keys, then split back over the waves
  static_assert(kSortBands == kSortWaves * 64, "one key per thread in the scan");
  int32_t tot = 0;
#pragma unroll
  for (int w = 0; w < kSortWaves; ++w) tot += hist[w][tid];
  int32_t x = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  if (tid == 0) {
    int32_t acc = 0;
    for (int w = 0; w < kSortWaves; ++w) {
      const int32_t t = tmp[w];
      tmp[w] = acc;
      acc += t;
    }
  }
  __syncthreads();
  int32_t slot = tmp[wave] + x - tot;
#pragma unroll
  for (int w = 0; w < kSortWaves; ++w) {
    const int32_t c = hist[w][tid];
    hist[w][tid] = slot;
    slot += c;
  }
  __syncthreads();
  for (int64_t base = seg0; base < seg1; base += 64) {
    const int64_t i = base + lane;
    const bool valid = i < seg1;
    const uint32_t k = valid ? min(keys[i], kSortBands - 1u) : 0xFFFFFFFFu;
    // lanes holding this lane's key: one ballot when the whole step shares
    // one key, else a pass over the lanes
    const uint32_t k0 = __builtin_amdgcn_readfirstlane(k);
    uint64_t same = __ballot(k == k0);
    if (same != ~uint64_t(0)) {
      same = 0;
      for (int j = 0; j < 64; ++j) {
        const uint32_t kj = __builtin_amdgcn_readlane(k, j);
        same |= static_cast<uint64_t>(kj == k) << j;
      }
    }
    const uint64_t below = (uint64_t(1) << lane) - 1;
    const int rank = __popcll(same & below);
    const int32_t first = valid ? hist[wave][k] : 0;
    if (valid) order[first + rank] = static_cast<int32_t>(i);
    // every lane has read its key's slot before the run's last lane moves it
    __builtin_amdgcn_wave_barrier();
    if (valid && (same >> lane) == 1u) hist[wave][k] = first + __popcll(same);
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

Workspace plan_workspace(const Shape& s) {
  auto align = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  Workspace w{};
  w.nbins = (s.max_seqlen + kBlock - 1) / kBlock + 1;
  w.max_items = static_cast<int64_t>(s.parts) * s.Hkv * ((s.T + s.BMq - 1) / s.BMq + s.B);
  size_t off = 0;
  w.meta = off;        off = align(off + sizeof(int32_t) * kMetaSlots);
  w.tile_prefix = off; off = align(off + sizeof(int32_t) * (s.B + 1));
  w.seq_w = off;       off = align(off + sizeof(int32_t) * s.B);
  w.keys = off;        off = align(off + sizeof(uint32_t) * w.max_items);
  w.order = off;       off = align(off + sizeof(int32_t) * w.max_items);
  w.items_raw = off;   off = align(off + sizeof(Item) * w.max_items);
  w.xa_nqb = (s.max_seqlen + kXaBlock - 1) / kXaBlock;
  w.xa_cnt = off;
  w.xa_list = off;
  w.xa_rows = off;
  w.xa_lse = off;
  if (s.xa) {
    const int64_t rows = static_cast<int64_t>(s.B) * s.Hkv;
    off = align(off + sizeof(int32_t) * rows * w.xa_nqb);
    w.xa_list = off;
    off = align(off + sizeof(int32_t) * rows * xa_row_offset(w.xa_nqb));
    w.xa_rows = off;
    off = align(off + sizeof(int32_t) * rows);
    w.xa_lse = off;
    off = align(off + sizeof(float) * kXaGroupsPerBlock * static_cast<int64_t>(s.B) * s.Hq *
                          xa_row_offset(w.xa_nqb));
  }
  w.total = off;
  return w;
}

hipError_t launch_setup(const Shape& s, const Geometry& g, const int8_t* modes, const int32_t* cu,
                        const Workspace& ws, char* base, hipStream_t st) {
  int32_t* meta = reinterpret_cast<int32_t*>(base + ws.meta);
  int32_t* tile_prefix = reinterpret_cast<int32_t*>(base + ws.tile_prefix);
  int32_t* seq_w = reinterpret_cast<int32_t*>(base + ws.seq_w);
  // (modes may be null: the dual-mode forward without the mixed output)
  hipLaunchKernelGGL(setup_kernel, dim3(1), dim3(kScanThreads), 0, st, cu, modes, s.B,
                     s.Hkv, s.T, s.max_seqlen, s.BMq, g.n_sink, g.window_blocks, g.keep_fraction,
                     plan_stamp(s), meta, tile_prefix, seq_w);
  return hipGetLastError();
}

hipError_t launch_items(const Shape& s, const Geometry& g, const int8_t* modes, const int32_t* cu,
                        const Workspace& ws, char* base, hipStream_t st) {
  int32_t* meta = reinterpret_cast<int32_t*>(base + ws.meta);
  int32_t* tile_prefix = reinterpret_cast<int32_t*>(base + ws.tile_prefix);
  int32_t* seq_w = reinterpret_cast<int32_t*>(base + ws.seq_w);
  uint32_t* keys = reinterpret_cast<uint32_t*>(base + ws.keys);
  int32_t* order = reinterpret_cast<int32_t*>(base + ws.order);
  Item* raw = reinterpret_cast<Item*>(base + ws.items_raw);
  const unsigned grid = static_cast<unsigned>((ws.max_items + 255) / 256);
  const int32_t* xa_cnt = s.xa ? reinterpret_cast<const int32_t*>(base + ws.xa_cnt) : nullptr;
  hipLaunchKernelGGL(items_kernel, dim3(grid), dim3(256), 0, st, cu, modes, s.B, s.Hkv, s.BMq,
                     s.parts, s.head_config, g.n_sink, meta, tile_prefix, seq_w, xa_cnt,
                     ws.xa_nqb, ws.nbins - 1, ws.max_items, raw, keys);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_key_sort(keys, ws.max_items, order, st);
}

hipError_t launch_key_sort(const uint32_t* keys, int64_t n, int32_t* order, hipStream_t st) {
  hipLaunchKernelGGL(key_sort_kernel, dim3(1), dim3(kSortWaves * 64), 0, st, keys, n, order);
  return hipGetLastError();
}

hipError_t launch_worklist(const Shape& s, const Geometry& g, const int8_t* modes,
                           const int32_t* cu, const Workspace& ws, char* base, hipStream_t st) {
  hipError_t e = launch_setup(s, g, modes, cu, ws, base, st);
  if (e != hipSuccess) return e;
  return launch_items(s, g, modes, cu, ws, base, st);
}

}  // namespace ea
