// Internal declarations shared by the HIP translation units of libea.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ea.h"

namespace ea {

// Query rows per attention work item: G query heads x (kTileRows / G) positions,
// 32 rows per wave of the attention kernel's workgroup.
constexpr int kTileRows = 256;
constexpr int kAttnWaves = kTileRows / 32;
// Consecutive work-list entries given to one XCD before moving to the next:
// one entry per CU of the XCD, so the workgroups that run together on an XCD
// take neighbouring entries (same KV head, adjacent query tiles) and share
// their K/V rows in that XCD's L2.
constexpr int kXcdChunk = 32;
constexpr int kNumXcd = 8;
// The work list is ordered by cost in bands of 2^kCostBandShift key blocks,
// so that entries within a band keep their head / sequence / tile order.
constexpr int kCostBandShift = 5;
// Key/value block of the sparse pattern and of the attention inner loop.
constexpr int kBlock = 64;
// Bins of the work lists' counting sort (one workgroup; its per-wave
// histograms take kSortWaves * kSortBands * 4 bytes of LDS).
constexpr int kSortBands = 1024;
constexpr int kSortWaves = 16;

// Sort key of a work item of `cost` (visible key blocks, or query blocks
// walked) when no item costs more than maxcost: 0 for the costliest band of
// 2^kCostBandShift blocks, growing as the cost falls; capped below
// kSortBands - 1 (only lists of sequences beyond two million tokens have more
// bands, and then their cheapest bands share the last bin).
__host__ __device__ inline uint32_t cost_key(int cost, int maxcost) {
  const int c = cost < maxcost ? cost : maxcost;
  const int k = (maxcost - c) >> kCostBandShift;
  return static_cast<uint32_t>(k < kSortBands - 2 ? k : kSortBands - 2);
}
// Sort key of the list's empty slots: after every real item.
__host__ __device__ inline uint32_t empty_key(int maxcost) {
  const int k = (maxcost >> kCostBandShift) + 1;
  return static_cast<uint32_t>(k < kSortBands - 1 ? k : kSortBands - 1);
}

// Key-block sets an attention work item can cover.
enum ItemMode : int32_t {
  kModeFA = 0,      // every causal key block
  kModeSA = 1,      // sink blocks and the local window
  kModeMiddle = 2,  // the causal blocks SA leaves out: FA = SA set + middle set
  kModeXA = 3       // the key blocks the XAttention selection kept (ea_xa.hip)
};

// XAttention (XA) mode: blocks of kXaBlock tokens are selected by the
// antidiagonal scores of position groups of kXaStride; one 128-token XA block
// spans two 64-token attention blocks.
constexpr int kXaBlock = 128;
constexpr int kXaStride = 8;
constexpr int kXaGroupsPerBlock = kXaBlock / kXaStride;

// Computation mode of router decision r (0 retrieval head, 1 sparse head)
// under an ea_head_config.
__host__ __device__ inline int computation_mode(int head_config, int r) {
  if (head_config == EA_HEADS_FA_XA) return r ? kModeXA : kModeFA;
  if (head_config == EA_HEADS_XA_SSA) return r ? kModeSA : kModeXA;
  return r ? kModeSA : kModeFA;
}

// Offset of query block i's list in the triangular per-(sequence, KV head)
// array of kept key blocks: row i holds at most i + 1 entries.
__host__ __device__ inline int64_t xa_row_offset(int64_t i) { return i * (i + 1) / 2; }

// One attention work item: a query tile of one KV-head group of one sequence,
// over one key-block set.
struct Item {
  int32_t b;     // sequence
  int32_t kvh;   // KV head
  int32_t qt;    // query tile: positions [qt * BMq, qt * BMq + BMq)
  int32_t cost;  // visible key blocks (scheduling key)
  int32_t mode;  // ItemMode
};

// Key blocks a query tile covering query blocks [qb0, qb1] visits in `mode`,
// in order: [0, r1_end) then [r2_beg, kend).  SA: the sinks below the first
// row's window, then the union of the rows' windows; middle: the blocks from
// the last sink to the last row's window start, exclusive.
struct KeyRange {
  int r1_end, r2_beg, kend;
  __host__ __device__ int count() const { return r1_end + (kend > r2_beg ? kend - r2_beg : 0); }
};

__host__ __device__ inline KeyRange key_range(int mode, int qb0, int qb1, int n_sink, int w) {
  KeyRange r{0, 0, qb1 + 1};
  if (mode == kModeSA) {
    const int ws = qb0 - w + 1 > 0 ? qb0 - w + 1 : 0;
    r.r1_end = n_sink < ws ? n_sink : ws;
    r.r2_beg = ws;
  } else if (mode == kModeMiddle) {
    r.r2_beg = n_sink;
    r.kend = qb1 - w + 1;
  }
  return r;
}

// Work-list position of workgroup wg.  The hardware hands workgroup wg to XCD
// wg mod 8; the j-th workgroup an XCD receives (j = wg / 8) takes entry
// j mod C of chunk 8 (j / C) + x of the list, C = kXcdChunk, with x = wg mod 8
// in even rounds j / C and 7 - wg mod 8 in odd ones.  Chunks are cost-sorted,
// so the snake keeps any XCD from taking the costlier chunk of every round.
__device__ inline int64_t list_position(int64_t wg) {
  const int64_t j = wg / kNumXcd, round = j / kXcdChunk;
  const int64_t x = (round & 1) ? (kNumXcd - 1 - wg % kNumXcd) : (wg % kNumXcd);
  return (round * kNumXcd + x) * kXcdChunk + j % kXcdChunk;
}

// Whether every row of a tile over query positions [p0, ...] (query blocks
// [qb0, qb1]) sees every key of block kb, so that the block needs no mask.
__device__ inline bool block_full(int mode, int kb, int p0, int qb0, int qb1, int ns, int w) {
  if (mode == kModeMiddle) return qb0 - kb >= w;
  return (kb * kBlock + kBlock - 1 <= p0) && (mode == kModeFA || kb < ns || qb1 - kb < w);
}

// Whether a row in query block qblk may see block kb at all (the causal test
// on single keys is applied on top; in the middle set it always holds, since
// kb <= qblk - w < qblk).
__device__ inline bool block_visible(int mode, int kb, int qblk, int ns, int w) {
  if (mode == kModeMiddle) return qblk - kb >= w;
  return mode == kModeFA || kb < ns || qblk - kb < w;
}

// Slots of the small int32 header at the start of the workspace.
enum Meta : int {
  kMetaTiles = 0,       // sum over sequences of ceil(L_b / BMq); items = tiles * Hkv
  kMetaStamp = 1,       // plan_stamp() of the sizes the list was built for
  kMetaXaRows = 2,      // XA mode: number of (sequence, KV head) rows in XA mode
  kMetaError = 3,       // MetaError bits of the device contents the planner found invalid
  kMetaSlots = 64
};

// Device-content checks of the planner (setup_kernel).  Any set bit makes the
// planner write stamp 0 and zero tiles, so that no later kernel of the call
// (XA selection, work list, attention, backward, merge) reads Q, K, V or
// writes an output.
enum MetaError : int32_t {
  kErrCuStart = 1,      // cu_seqlens[0] != 0
  kErrCuOrder = 2,      // cu_seqlens decreases somewhere
  kErrCuEnd = 4,        // cu_seqlens[B] != total_tokens
  kErrSeqLen = 8,       // a sequence is longer than max_seqlen
  kErrMode = 16         // a mode value outside {0, 1}
};

// Upper bound the host accepts for n_sink_blocks and window_blocks, so that
// block arithmetic on them (sums of a few blocks counts) stays in int32.
constexpr int32_t kMaxGeomBlocks = 1 << 24;

// Byte layout of the workspace, a pure function of the host-visible sizes.
struct Workspace {
  size_t meta, tile_prefix, seq_w, keys, order, items_raw;
  size_t total;
  int64_t max_items;   // bound on work items
  int32_t nbins;       // cost bins of the sort key
  // XA mode only (Shape.xa): per (sequence, KV head, query block) the number
  // of kept key blocks, and the triangular array of their list entries
  // (key block j | per-head mask << 16, ascending j)
  // (and, per XA query head and query block, each group row's log2-sum-exp2
  // over every key block: the selection's single-pass scratch)
  size_t xa_cnt, xa_list, xa_rows, xa_lse;
  int32_t xa_nqb;      // query blocks of kXaBlock per sequence (upper bound)
};

struct Shape {
  int32_t B;
  int64_t T;
  int32_t max_seqlen, Hq, Hkv, d, G, BMq;
  int32_t elem_bytes;
  // work items per query tile: 1 for the routed forward (the head's own mode),
  // 2 for the dual-mode forward (SA set and middle set of every head)
  int32_t parts = 1;
  // ea_head_config mapping router decisions to computation modes, and
  // whether the workspace holds the XA selection lists
  int32_t head_config = EA_HEADS_FA_SSA;
  int32_t xa = 0;
};

Workspace plan_workspace(const Shape& s);

// A 31-bit fingerprint of the sizes a work list is built for.  The planner
// writes it into the workspace header and the attention kernel does nothing
// unless it finds the fingerprint of its own sizes there, so a run over an
// unplanned (or differently planned) workspace never reads a stale list.
inline int32_t plan_stamp(const Shape& s) {
  uint64_t h = 0x9E3779B97F4A7C15ull;
  const int64_t v[9] = {s.B, s.T, s.Hq, s.Hkv, s.BMq, s.max_seqlen, s.parts, s.head_config, s.xa};
  for (int64_t x : v) {
    h ^= static_cast<uint64_t>(x) + 0x9E3779B97F4A7C15ull + (h << 6) + (h >> 2);
    h *= 0xBF58476D1CE4E5B9ull;
  }
  return static_cast<int32_t>((h >> 33) | 1u);
}

struct Geometry {
  int32_t n_sink;
  int32_t window_blocks;   // 0: per sequence from keep_fraction
  float keep_fraction;
  float scale_log2;        // softmax scale * log2(e)
  float scale;             // softmax scale
};

// Launchers (stream-ordered, no synchronisation).  Return hipSuccess or the
// launch error.
hipError_t launch_route(const void* K, bool bf16, const int32_t* cu, int32_t B, int32_t Hkv,
                        const ea_router_desc& r, int8_t* modes, float* logits, hipStream_t st);

hipError_t launch_worklist(const Shape& s, const Geometry& g, const int8_t* modes,
                           const int32_t* cu, const Workspace& ws, char* base, hipStream_t st);
// The two halves of launch_worklist: the per-sequence setup with its
// device-content checks, then the items and their cost order (the XA
// selection runs between the two).
hipError_t launch_setup(const Shape& s, const Geometry& g, const int8_t* modes, const int32_t* cu,
                        const Workspace& ws, char* base, hipStream_t st);
hipError_t launch_items(const Shape& s, const Geometry& g, const int8_t* modes, const int32_t* cu,
                        const Workspace& ws, char* base, hipStream_t st);

// Stable counting sort of n entries by key (each key < kSortBands): order
// receives the entry indices 0..n-1, ascending by key and, within a key, by
// index.  One workgroup; stream-ordered.
hipError_t launch_key_sort(const uint32_t* keys, int64_t n, int32_t* order, hipStream_t st);

// Outputs of an attention launch: items of mode FA or SA write O / lse,
// items of the middle set O_mid / lse_mid (dual-mode forward only).
struct AttnOut {
  void* O;
  float* lse;
  void* O_mid;
  float* lse_mid;
};

hipError_t launch_attention(const Shape& s, const Geometry& g, const void* Q, const void* K,
                            const void* V, const int32_t* cu, const AttnOut& out,
                            const Workspace& ws, char* base, hipStream_t st);

// XAttention selection (ea_xa.hip): dynamic LDS bytes of its kernel (0 if the
// sizes are not supported), and the launcher, which fills the workspace's
// XA counts and lists for every XA head (optionally also the block masses and
// keep flags, [B, Hq, nqb, nqb]).
size_t xa_plan_lds_bytes(const Shape& s);
hipError_t launch_xa_plan(const Shape& s, const Geometry& g, float tau, const void* Q,
                          const void* K, const int8_t* modes, const int32_t* cu,
                          const Workspace& ws, char* base, float* mass, uint8_t* keep,
                          hipStream_t st);

// Mode-aware KV cache (ea_decode.hip): the device view of a cache buffer.
struct CacheView {
  int32_t B, Hkv, d, max_len, n_sink, window_blocks;
  float keep_fraction;
  int64_t area_blocks;   // 64-token blocks the caller's buffer has room for
  int32_t* lengths;      // [B] tokens held per sequence
  int32_t* cap;          // [B * Hkv] slot capacity in blocks
  int32_t* ring;         // [B * Hkv] ring size in blocks past the sinks, 0 = no ring
  int64_t* base;         // [B * Hkv] first block of the slot
  int8_t* mode;          // [B * Hkv] 0 = FA, 1 = SA
  int32_t* valid;        // [1] 1 once the slot table fits the buffer
  uint16_t* K;           // block pb: K rows at K + pb * 2 * 64 * d, V rows 64 * d later
  uint16_t* V;           // = K + 64 * d
};

// Byte layout of a cache buffer: the header (a function of B and Hkv) and the
// blocks after it, each 64 K rows then 64 V rows of d bf16 values.
struct CacheLayout {
  size_t lengths, cap, ring, base, mode, valid, blocks;
};
CacheLayout cache_layout(int32_t B, int32_t Hkv);
// Slot capacity in blocks for a KV head of the given mode.
int32_t cache_slot_blocks(int mode, int32_t max_len, int32_t n_sink, int32_t window_blocks,
                          float keep_fraction);

// Arguments of one decode step (one query token per sequence).
struct DecodeArgs {
  const uint16_t* q;   // [B, Hq, d] bf16
  const uint16_t* k_new;  // [B, Hkv, d] bf16: the new token's K and V rows
  const uint16_t* v_new;
  uint16_t* O;         // [B, Hq, d] bf16
  float* lse;          // [B, Hq] or null
  float* o_part;       // [B, Hq, n_chunks, d] chunk partials (workspace)
  float* lse_part;     // [B, Hq, n_chunks]
  int32_t Hq, G, n_chunks, chunk_blocks;
  float scale;
};

// Key blocks per decode chunk (one workgroup of the split over the cache).
constexpr int kDecodeChunkBlocks = 16;

hipError_t launch_cache_init(const CacheView& c, const int8_t* modes, hipStream_t st);
hipError_t launch_cache_fill(const CacheView& c, const int32_t* cu, int64_t T, const void* K,
                             const void* V, hipStream_t st);
hipError_t launch_decode(const CacheView& c, const DecodeArgs& a, hipStream_t st);

// Arguments of the backward kernels (ea_backward.hip).
struct BwdArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  const uint16_t* O;
  const uint16_t* dO;
  const float* lse;     // [Hq, T] natural log, from the forward
  uint16_t* dQ;
  uint16_t* dK;
  uint16_t* dV;
  float* Dv;            // [Hq, T] rowsum(dO * O) (workspace)
  float* lse2;          // [Hq, T] LSE in log2 units (workspace)
  const int32_t* cu;
  const int8_t* modes;
  const int32_t* seq_w;
  const Item* items;
  const int32_t* order;
  const int32_t* meta;
  const int32_t* dkv_order;  // dK/dV items in cost order
  int64_t T, max_items, dkv_n;
  int32_t B, Hq, Hkv, G, BMq, n_sink, stamp, npair;
  float scale;
};

// Keys per workgroup of the dK/dV kernel (32 per pair of waves).
constexpr int kDkvWaves = 8;
constexpr int kDkvKeys = 16 * kDkvWaves;

// Cost-ordered list of the dK/dV kernel's items (sequence, KV head, key
// group), in its own workspace region.
struct DkvList {
  size_t keys, order, total;
  int64_t n;
  int32_t npair, maxcost;
};
DkvList dkv_list_layout(const Shape& s);

hipError_t launch_backward(const Shape& s, const Geometry& g, BwdArgs args, const DkvList& l,
                           char* list_base, hipStream_t st);

// Router-logit gradient through the straight-through estimator (ea_dual.hip):
// chunks of tokens per sequence for the partial sums, and the launcher.
int32_t logit_grad_chunks(int32_t max_seqlen);
hipError_t launch_logit_grad(const Shape& s, const int32_t* cu, const void* dO, const void* O_fa,
                             const void* O_sa, const float* r_soft, float tau, float* dz, float* dr,
                             float* part, hipStream_t st);

// Training-forward helpers (ea_dual.hip).
hipError_t launch_gumbel_route(const float* logits, const float* gumbel, float tau, int64_t n,
                               float* r_soft, int8_t* modes, hipStream_t st);
// O_fa / lse_fa hold the middle-set partial on entry and the FA result on
// exit; O (if not null) receives the straight-through mix selected by modes.
// Does nothing unless meta holds the plan stamp of s.
hipError_t launch_dual_merge(const Shape& s, const int32_t* cu, const int8_t* modes,
                             const void* O_sa, const float* lse_sa, void* O_fa, float* lse_fa,
                             void* O, const int32_t* meta, hipStream_t st);

// Matrix-core ceiling probe (ea_probe.hip) and its FLOP count.
hipError_t launch_mfma_probe(float* out, int32_t n_workgroups, int32_t iters, uint32_t seed,
                             hipStream_t st);
int64_t mfma_probe_flops(int32_t n_workgroups, int32_t iters);

}  // namespace ea
