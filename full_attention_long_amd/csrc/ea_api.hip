// C ABI of libea: argument validation and stream-ordered launches.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "ea_internal.h"

namespace {

thread_local std::string g_err;

ea_status fail(ea_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

ea_status ok() {
  g_err.clear();
  return EA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// EA_VALIDATE=1 (any value but empty or "0") makes every call that plans a
// work list, or runs one, wait for the planner's device-content checks and
// return their verdict; without it the checks still run on the device and
// keep every later kernel of the call from touching memory, but nothing
// waits for them (ea_workspace_status reads the verdict later).
// The variable is read at every call, so a process can switch it.
bool validate_on() {
  const char* e = getenv("EA_VALIDATE");
  return e && e[0] && strcmp(e, "0") != 0;
}

std::string describe_meta_error(int32_t err) {
  std::string m;
  auto add = [&](int32_t bit, const char* what) {
    if (err & bit) m += (m.empty() ? "" : "; ") + std::string(what);
  };
  add(ea::kErrCuStart, "cu_seqlens[0] != 0");
  add(ea::kErrCuOrder, "cu_seqlens decreases");
  add(ea::kErrCuEnd, "cu_seqlens[B] != total_tokens");
  add(ea::kErrSeqLen, "a sequence is longer than max_seqlen");
  add(ea::kErrMode, "a mode value is not 0 or 1");
  return m;
}

// Waits for `stream`, then reads the planner's verdict from the workspace
// header (the header sits at offset 0 of every planned workspace).
ea_status workspace_verdict(const void* workspace, void* stream) {
  int32_t err = 0;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(&err, static_cast<const char*>(workspace) + sizeof(int32_t) * ea::kMetaError,
                                sizeof(err), hipMemcpyDeviceToHost, hs);
  if (e == hipSuccess) e = hipStreamSynchronize(hs);
  if (e != hipSuccess) return fail(EA_ERR_HIP, "reading the workspace header failed: %s", hipGetErrorString(e));
  if (err != 0)
    return fail(EA_ERR_INVALID_ARG, "invalid device contents: %s", describe_meta_error(err).c_str());
  return EA_OK;
}

// Host-side checks of cu_seqlens for the calls that take no workspace
// (router, KV-cache fill), under EA_VALIDATE only: copies the B + 1 values.
// total_tokens < 0 skips the end check, max_len < 0 the length check.
ea_status host_check_cu(const int32_t* cu, int32_t B, int64_t total_tokens, int64_t max_len,
                        void* stream) {
  std::vector<int32_t> h(static_cast<size_t>(B) + 1);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(h.data(), cu, sizeof(int32_t) * h.size(), hipMemcpyDeviceToHost, hs);
  if (e == hipSuccess) e = hipStreamSynchronize(hs);
  if (e != hipSuccess) return fail(EA_ERR_HIP, "reading cu_seqlens failed: %s", hipGetErrorString(e));
  int32_t err = 0;
  if (h[0] != 0) err |= ea::kErrCuStart;
  if (total_tokens >= 0 && h[B] != total_tokens) err |= ea::kErrCuEnd;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t len = static_cast<int64_t>(h[b + 1]) - h[b];
    if (len < 0) err |= ea::kErrCuOrder;
    if (max_len >= 0 && len > max_len) err |= ea::kErrSeqLen;
  }
  if (err != 0)
    return fail(EA_ERR_INVALID_ARG, "invalid device contents: %s", describe_meta_error(err).c_str());
  return EA_OK;
}

// Validates the sizes shared by the workspace query and the prefill call.
ea_status check_shape(int32_t B, int64_t T, int32_t max_seqlen, int32_t Hq, int32_t Hkv,
                      int32_t d, ea_dtype dtype, ea::Shape* out) {
  if (B < 1) return fail(EA_ERR_INVALID_ARG, "B must be >= 1 (got %d)", B);
  if (T < 0 || T >= (int64_t(1) << 31))
    return fail(EA_ERR_INVALID_ARG, "total_tokens must be in [0, 2^31) (got %lld)", (long long)T);
  if (T > 0 && (max_seqlen < 1 || max_seqlen > T))
    return fail(EA_ERR_INVALID_ARG, "max_seqlen must be in [1, total_tokens] (got %d)", max_seqlen);
  if (Hq < 1 || Hkv < 1) return fail(EA_ERR_INVALID_ARG, "Hq and Hkv must be >= 1");
  if (Hq % Hkv != 0) return fail(EA_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  const int32_t G = Hq / Hkv;
  if (G > ea::kTileRows)
    return fail(EA_ERR_UNSUPPORTED, "Hq / Hkv must be <= %d (got %d)", ea::kTileRows, G);
  if (d != 64 && d != 128) return fail(EA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", d);
  if (dtype != EA_F32 && dtype != EA_BF16) return fail(EA_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  // Q, K and V rows of one sequence are addressed with 32-bit byte offsets
  if (static_cast<int64_t>(T > 0 ? max_seqlen : 1) * Hq * d >= (int64_t(1) << 31))
    return fail(EA_ERR_UNSUPPORTED, "max_seqlen * Hq * head_dim must be < 2^31 (got %lld)",
                (long long)max_seqlen * Hq * d);
  out->B = B;
  out->T = T;
  out->max_seqlen = T > 0 ? max_seqlen : 1;
  out->Hq = Hq;
  out->Hkv = Hkv;
  out->d = d;
  out->G = G;
  out->BMq = ea::kTileRows / G;
  out->elem_bytes = dtype == EA_BF16 ? 2 : 4;
  return EA_OK;
}

// Shared validation of the plan, run and one-shot prefill calls.
// parts: 1 for the routed forward (modes required), 2 for the dual-mode one.
ea_status check_prefill(int32_t B, int64_t T, int32_t max_seqlen, int32_t Hq, int32_t Hkv,
                        int32_t d, ea_dtype dtype, const ea_sparsity_params* p, const void* modes,
                        const void* cu_seqlens, const void* workspace, size_t workspace_bytes,
                        ea::Shape* s, ea::Workspace* ws, ea::Geometry* g, int parts = 1,
                        int head_config = EA_HEADS_FA_SSA, int xa = 0) {
  ea_status st = check_shape(B, T, max_seqlen, Hq, Hkv, d, dtype, s);
  if (st != EA_OK) return st;
  s->parts = parts;
  s->head_config = head_config;
  s->xa = xa;
  if (!p) return fail(EA_ERR_INVALID_ARG, "null sparsity params");
  if (p->block != ea::kBlock)
    return fail(EA_ERR_UNSUPPORTED, "sparsity block must be %d (got %d)", ea::kBlock, p->block);
  if (p->n_sink_blocks < 0 || p->n_sink_blocks > ea::kMaxGeomBlocks)
    return fail(EA_ERR_INVALID_ARG, "n_sink_blocks must be in [0, %d] (got %d)", ea::kMaxGeomBlocks,
                p->n_sink_blocks);
  if (p->window_blocks < 0 || p->window_blocks > ea::kMaxGeomBlocks)
    return fail(EA_ERR_INVALID_ARG, "window_blocks must be in [0, %d] (got %d)", ea::kMaxGeomBlocks,
                p->window_blocks);
  if (p->window_blocks == 0 && !(p->keep_fraction > 0.f && p->keep_fraction <= 1.f))
    return fail(EA_ERR_INVALID_ARG, "keep_fraction must be in (0, 1] (got %g)", (double)p->keep_fraction);
  if (!(p->softmax_scale >= 0.f) || isinf(p->softmax_scale))
    return fail(EA_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  if ((parts == 1 && !modes) || !cu_seqlens) return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  *ws = ea::plan_workspace(*s);
  if (!workspace || workspace_bytes < ws->total)
    return fail(EA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", ws->total,
                workspace ? workspace_bytes : (size_t)0);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(EA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  g->n_sink = p->n_sink_blocks;
  g->window_blocks = p->window_blocks;
  g->keep_fraction = p->keep_fraction;
  g->scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / sqrtf(static_cast<float>(d));
  g->scale_log2 = g->scale * 1.44269504088896340736f;
  return EA_OK;
}

ea_status check_tensors(const void* Q, const void* K, const void* V, const void* O) {
  if (!Q || !K || !V || !O) return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O))
    return fail(EA_ERR_INVALID_ARG, "Q, K, V and O must be 16-byte aligned");
  return EA_OK;
}

}  // namespace

extern "C" {

int32_t ea_abi_version(void) { return EA_ABI_VERSION; }

ea_status ea_workspace_status(const void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  if (workspace_bytes < sizeof(int32_t) * ea::kMetaSlots)
    return fail(EA_ERR_WORKSPACE, "workspace of at least %zu bytes expected (got %zu)",
                sizeof(int32_t) * ea::kMetaSlots, workspace_bytes);
  ea_status st = workspace_verdict(workspace, stream);
  return st != EA_OK ? st : ok();
}

const char* ea_last_error(void) { return g_err.c_str(); }

ea_status ea_route(const void* K, ea_dtype dtype, const int32_t* cu_seqlens, int32_t B,
                   int32_t Hkv, const ea_router_desc* r, int8_t* modes, float* logits,
                   void* stream) {
  if (!K || !cu_seqlens || !r || !modes) return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  if (dtype != EA_F32 && dtype != EA_BF16) return fail(EA_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (B < 1 || Hkv < 1) return fail(EA_ERR_INVALID_ARG, "B and Hkv must be >= 1");
  if ((int64_t)B * Hkv >= (int64_t(1) << 31)) return fail(EA_ERR_INVALID_ARG, "B * Hkv too large");
  if (r->head_dim < 1 || r->head_dim > 256)
    return fail(EA_ERR_UNSUPPORTED, "router head_dim must be in [1, 256] (got %d)", r->head_dim);
  if (r->task_hidden < 1 || r->task_hidden > 4096)
    return fail(EA_ERR_UNSUPPORTED, "task_hidden must be in [1, 4096] (got %d)", r->task_hidden);
  if (r->router_hidden < 1 || r->router_hidden > 1024)
    return fail(EA_ERR_UNSUPPORTED, "router_hidden must be in [1, 1024] (got %d)", r->router_hidden);
  if (r->pool_len < 1) return fail(EA_ERR_INVALID_ARG, "pool_len must be >= 1 (got %d)", r->pool_len);
  if (!r->w1 || !r->b1 || !r->w2 || !r->b2 || !r->w3 || !r->b3 || !r->w4 || !r->b4)
    return fail(EA_ERR_INVALID_ARG, "null router weight pointer");
  if (validate_on()) {
    ea_status v = host_check_cu(cu_seqlens, B, -1, -1, stream);
    if (v != EA_OK) return v;
  }
  hipError_t e = ea::launch_route(K, dtype == EA_BF16, cu_seqlens, B, Hkv, *r, modes, logits,
                                  static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(EA_ERR_HIP, "route launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t ea_hybrid_prefill_workspace_size(int32_t B, int64_t total_tokens, int32_t max_seqlen,
                                        int32_t Hq, int32_t Hkv, int32_t head_dim,
                                        ea_dtype dtype) {
  ea::Shape s;
  if (check_shape(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype, &s) != EA_OK) return 0;
  g_err.clear();
  return ea::plan_workspace(s).total;
}

ea_status ea_hybrid_prefill_plan_layout(int32_t B, int64_t total_tokens, int32_t max_seqlen,
                                        int32_t Hq, int32_t Hkv, int32_t head_dim, ea_dtype dtype,
                                        int64_t* items_offset, int64_t* keys_offset,
                                        int64_t* order_offset, int64_t* n_slots) {
  ea::Shape s;
  ea_status st = check_shape(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype, &s);
  if (st != EA_OK) return st;
  if (!items_offset || !keys_offset || !order_offset || !n_slots)
    return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  const ea::Workspace ws = ea::plan_workspace(s);
  *items_offset = static_cast<int64_t>(ws.items_raw);
  *keys_offset = static_cast<int64_t>(ws.keys);
  *order_offset = static_cast<int64_t>(ws.order);
  *n_slots = ws.max_items;
  return ok();
}

ea_status ea_hybrid_prefill_plan(const int8_t* modes, const int32_t* cu_seqlens, int32_t B,
                                 int64_t total_tokens, int32_t max_seqlen, int32_t Hq,
                                 int32_t Hkv, int32_t head_dim, ea_dtype dtype,
                                 const ea_sparsity_params* p, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  ea::Shape s;
  ea::Workspace ws;
  ea::Geometry g;
  ea_status st = check_prefill(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype, p, modes,
                               cu_seqlens, workspace, workspace_bytes, &s, &ws, &g);
  if (st != EA_OK) return st;
  if (total_tokens == 0) return ok();
  hipError_t e = ea::launch_worklist(s, g, modes, cu_seqlens, ws, static_cast<char*>(workspace),
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(EA_ERR_HIP, "work-list launch failed: %s", hipGetErrorString(e));
  if (validate_on() && (st = workspace_verdict(workspace, stream)) != EA_OK) return st;
  return ok();
}

ea_status ea_hybrid_prefill_run(const void* Q, const void* K, const void* V, ea_dtype dtype,
                                const int8_t* modes, const int32_t* cu_seqlens, int32_t B,
                                int64_t total_tokens, int32_t max_seqlen, int32_t Hq, int32_t Hkv,
                                int32_t head_dim, const ea_sparsity_params* p, void* O, float* lse,
                                const void* workspace, size_t workspace_bytes, void* stream) {
  ea::Shape s;
  ea::Workspace ws;
  ea::Geometry g;
  ea_status st = check_prefill(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype, p, modes,
                               cu_seqlens, workspace, workspace_bytes, &s, &ws, &g);
  if (st != EA_OK) return st;
  if ((st = check_tensors(Q, K, V, O)) != EA_OK) return st;
  if (total_tokens == 0) return ok();
  if (validate_on() && (st = workspace_verdict(workspace, stream)) != EA_OK) return st;
  hipError_t e = ea::launch_attention(s, g, Q, K, V, cu_seqlens, ea::AttnOut{O, lse, nullptr, nullptr},
                                      ws, static_cast<char*>(const_cast<void*>(workspace)),
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(EA_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

// The one-shot prefill; `validate` lets EA_VALIDATE make the call wait for
// the device-content checks (the allocation-free entry point never waits).
ea_status prefill_impl(const void* Q, const void* K, const void* V, ea_dtype dtype,
                       const int8_t* modes, const int32_t* cu_seqlens, int32_t B,
                       int64_t total_tokens, int32_t max_seqlen, int32_t Hq, int32_t Hkv,
                       int32_t head_dim, const ea_sparsity_params* p, void* O, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream, bool validate) {
  ea::Shape s;
  ea::Workspace ws;
  ea::Geometry g;
  ea_status st = check_prefill(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype, p, modes,
                               cu_seqlens, workspace, workspace_bytes, &s, &ws, &g);
  if (st != EA_OK) return st;
  if ((st = check_tensors(Q, K, V, O)) != EA_OK) return st;
  if (total_tokens == 0) return ok();
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(workspace);
  hipError_t e = ea::launch_worklist(s, g, modes, cu_seqlens, ws, base, hs);
  if (e != hipSuccess) return fail(EA_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
  if (validate && validate_on() && (st = workspace_verdict(workspace, stream)) != EA_OK) return st;
  e = ea::launch_attention(s, g, Q, K, V, cu_seqlens, ea::AttnOut{O, lse, nullptr, nullptr}, ws,
                           base, hs);
  if (e != hipSuccess) return fail(EA_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Workspace of the allocation-free prefill: one static array per GPU, held
// until the process ends.  In host code the array's name only stands for the
// device symbol; its device address comes from hipGetSymbolAddress, once per
// device (each GPU holds its own copy at its own address).
constexpr size_t kNoAllocBytes = size_t(4) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kNoAllocBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

ea_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(EA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(EA_ERR_UNSUPPORTED, "device index %d is beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(EA_ERR_HIP, "hipGetSymbolAddress of the static workspace failed: %s",
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return EA_OK;
}

}  // namespace

extern "C" {

ea_status ea_hybrid_prefill(const void* Q, const void* K, const void* V, ea_dtype dtype,
                            const int8_t* modes, const int32_t* cu_seqlens, int32_t B,
                            int64_t total_tokens, int32_t max_seqlen, int32_t Hq, int32_t Hkv,
                            int32_t head_dim, const ea_sparsity_params* p, void* O, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl(Q, K, V, dtype, modes, cu_seqlens, B, total_tokens, max_seqlen, Hq, Hkv,
                      head_dim, p, O, lse, workspace, workspace_bytes, stream, true);
}

size_t ea_hybrid_prefill_noalloc_max_workspace(void) { return kNoAllocBytes; }

ea_status ea_hybrid_prefill_noalloc(const void* Q, const void* K, const void* V, ea_dtype dtype,
                                    const int8_t* modes, const int32_t* cu_seqlens, int32_t B,
                                    int64_t total_tokens, int32_t max_seqlen, int32_t Hq,
                                    int32_t Hkv, int32_t head_dim, const ea_sparsity_params* p,
                                    void* O, float* lse, void* stream) {
  ea::Shape s;
  ea_status st = check_shape(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype, &s);
  if (st != EA_OK) return st;
  const size_t need = ea::plan_workspace(s).total;
  if (need > kNoAllocBytes)
    return fail(EA_ERR_WORKSPACE,
                "these sizes need %zu bytes of workspace; the static workspace of the "
                "allocation-free prefill holds %zu (use ea_hybrid_prefill with a workspace)",
                need, kNoAllocBytes);
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != EA_OK) return st;
  return prefill_impl(Q, K, V, dtype, modes, cu_seqlens, B, total_tokens, max_seqlen, Hq, Hkv,
                      head_dim, p, O, lse, ws, kNoAllocBytes, stream, false);
}

ea_status ea_gumbel_route(const float* logits, const float* gumbel, float tau, int32_t n,
                          float* r_soft, int8_t* modes, void* stream) {
  if (!logits || !modes) return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  if (n < 0) return fail(EA_ERR_INVALID_ARG, "n must be >= 0 (got %d)", n);
  if (!(tau > 0.f) || isinf(tau)) return fail(EA_ERR_INVALID_ARG, "tau must be finite and > 0");
  hipError_t e = ea::launch_gumbel_route(logits, gumbel, tau, n, r_soft, modes,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(EA_ERR_HIP, "routing launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t ea_dual_prefill_workspace_size(int32_t B, int64_t total_tokens, int32_t max_seqlen,
                                      int32_t Hq, int32_t Hkv, int32_t head_dim, ea_dtype dtype) {
  ea::Shape s;
  if (check_shape(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype, &s) != EA_OK) return 0;
  g_err.clear();
  s.parts = 2;
  return ea::plan_workspace(s).total;
}

ea_status ea_dual_prefill(const void* Q, const void* K, const void* V, ea_dtype dtype,
                          const int8_t* modes, const int32_t* cu_seqlens, int32_t B,
                          int64_t total_tokens, int32_t max_seqlen, int32_t Hq, int32_t Hkv,
                          int32_t head_dim, const ea_sparsity_params* p, void* O, void* O_fa,
                          void* O_sa, float* lse_fa, float* lse_sa, void* workspace,
                          size_t workspace_bytes, void* stream) {
  ea::Shape s;
  ea::Workspace ws;
  ea::Geometry g;
  ea_status st = check_prefill(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype, p, modes,
                               cu_seqlens, workspace, workspace_bytes, &s, &ws, &g, 2);
  if (st != EA_OK) return st;
  if ((st = check_tensors(Q, K, V, O_fa)) != EA_OK) return st;
  if (!O_sa || !lse_fa || !lse_sa) return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(O_sa) || (O && !aligned16(O)))
    return fail(EA_ERR_INVALID_ARG, "O, O_fa and O_sa must be 16-byte aligned");
  if (O && !modes) return fail(EA_ERR_INVALID_ARG, "modes is required when O is requested");
  if (O_fa == O_sa || (O && (O == O_fa || O == O_sa)) || lse_fa == lse_sa)
    return fail(EA_ERR_INVALID_ARG, "the outputs must not alias");
  if (total_tokens == 0) return ok();
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(workspace);
  hipError_t e = ea::launch_worklist(s, g, modes, cu_seqlens, ws, base, hs);
  if (e != hipSuccess) return fail(EA_ERR_HIP, "dual prefill launch failed: %s", hipGetErrorString(e));
  if (validate_on() && (st = workspace_verdict(workspace, stream)) != EA_OK) return st;
  e = ea::launch_attention(s, g, Q, K, V, cu_seqlens, ea::AttnOut{O_sa, lse_sa, O_fa, lse_fa}, ws,
                           base, hs);
  if (e == hipSuccess)
    e = ea::launch_dual_merge(s, cu_seqlens, modes, O_sa, lse_sa, O_fa, lse_fa, O,
                              reinterpret_cast<const int32_t*>(base + ws.meta), hs);
  if (e != hipSuccess) return fail(EA_ERR_HIP, "dual prefill launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t ea_xa_prefill_workspace_size(int32_t B, int64_t total_tokens, int32_t max_seqlen,
                                    int32_t Hq, int32_t Hkv, int32_t head_dim, ea_dtype dtype) {
  ea::Shape s;
  if (check_shape(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype, &s) != EA_OK) return 0;
  g_err.clear();
  s.xa = 1;
  return ea::plan_workspace(s).total;
}

}  // extern "C"

namespace {

// Validation shared by the XA prefill entry points.
ea_status check_xa(int32_t B, int64_t total_tokens, int32_t max_seqlen, int32_t Hq, int32_t Hkv,
                   int32_t head_dim, ea_dtype dtype, const ea_sparsity_params* p,
                   const ea_xa_params* xa, const void* modes, const void* cu_seqlens,
                   const void* workspace, size_t workspace_bytes, ea::Shape* s, ea::Workspace* ws,
                   ea::Geometry* g) {
  if (!xa) return fail(EA_ERR_INVALID_ARG, "null XA params");
  if (xa->block != ea::kXaBlock)
    return fail(EA_ERR_UNSUPPORTED, "XA block must be %d (got %d)", ea::kXaBlock, xa->block);
  if (xa->stride != ea::kXaStride)
    return fail(EA_ERR_UNSUPPORTED, "XA stride must be %d (got %d)", ea::kXaStride, xa->stride);
  if (!(xa->threshold >= 0.f && xa->threshold <= 1.f))
    return fail(EA_ERR_INVALID_ARG, "XA threshold must be in [0, 1] (got %g)", (double)xa->threshold);
  if (xa->head_config != EA_HEADS_FA_SSA && xa->head_config != EA_HEADS_FA_XA &&
      xa->head_config != EA_HEADS_XA_SSA)
    return fail(EA_ERR_INVALID_ARG, "unknown head configuration %d", xa->head_config);
  ea_status st = check_prefill(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype, p, modes,
                               cu_seqlens, workspace, workspace_bytes, s, ws, g, 1,
                               xa->head_config, 1);
  if (st != EA_OK) return st;
  if (dtype != EA_BF16) return fail(EA_ERR_UNSUPPORTED, "XA mode needs dtype EA_BF16");
  if (s->G < 2 || s->G > 16 || (s->G & (s->G - 1)) != 0)
    return fail(EA_ERR_UNSUPPORTED, "XA mode needs Hq / Hkv a power of two in [2, 16] (got %d)", s->G);
  if (ea::xa_plan_lds_bytes(*s) == 0)
    return fail(EA_ERR_UNSUPPORTED, "max_seqlen %d is too long for XA mode (at most %d blocks of %d)",
                max_seqlen, 4096, ea::kXaBlock);
  return EA_OK;
}

}  // namespace

extern "C" {

ea_status ea_xa_prefill_plan(const void* Q, const void* K, ea_dtype dtype, const int8_t* modes,
                             const int32_t* cu_seqlens, int32_t B, int64_t total_tokens,
                             int32_t max_seqlen, int32_t Hq, int32_t Hkv, int32_t head_dim,
                             const ea_sparsity_params* p, const ea_xa_params* xa,
                             float* xa_mass, uint8_t* xa_keep, void* workspace,
                             size_t workspace_bytes, void* stream) {
  ea::Shape s;
  ea::Workspace ws;
  ea::Geometry g;
  ea_status st = check_xa(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype, p, xa, modes,
                          cu_seqlens, workspace, workspace_bytes, &s, &ws, &g);
  if (st != EA_OK) return st;
  if (!Q || !K) return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(Q) || !aligned16(K)) return fail(EA_ERR_INVALID_ARG, "Q and K must be 16-byte aligned");
  if (total_tokens == 0) return ok();
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(workspace);
  // setup (with the device-content checks) first: the selection reads its verdict
  hipError_t e = ea::launch_setup(s, g, modes, cu_seqlens, ws, base, hs);
  if (e != hipSuccess) return fail(EA_ERR_HIP, "XA plan launch failed: %s", hipGetErrorString(e));
  if (validate_on() && (st = workspace_verdict(workspace, stream)) != EA_OK) return st;
  e = ea::launch_xa_plan(s, g, xa->threshold, Q, K, modes, cu_seqlens, ws, base, xa_mass, xa_keep, hs);
  if (e == hipSuccess) e = ea::launch_items(s, g, modes, cu_seqlens, ws, base, hs);
  if (e != hipSuccess) return fail(EA_ERR_HIP, "XA plan launch failed: %s", hipGetErrorString(e));
  return ok();
}

ea_status ea_xa_prefill_run(const void* Q, const void* K, const void* V, ea_dtype dtype,
                            const int8_t* modes, const int32_t* cu_seqlens, int32_t B,
                            int64_t total_tokens, int32_t max_seqlen, int32_t Hq, int32_t Hkv,
                            int32_t head_dim, const ea_sparsity_params* p, const ea_xa_params* xa,
                            void* O, float* lse, const void* workspace, size_t workspace_bytes,
                            void* stream) {
  ea::Shape s;
  ea::Workspace ws;
  ea::Geometry g;
  ea_status st = check_xa(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype, p, xa, modes,
                          cu_seqlens, workspace, workspace_bytes, &s, &ws, &g);
  if (st != EA_OK) return st;
  if ((st = check_tensors(Q, K, V, O)) != EA_OK) return st;
  if (total_tokens == 0) return ok();
  if (validate_on() && (st = workspace_verdict(workspace, stream)) != EA_OK) return st;
  hipError_t e = ea::launch_attention(s, g, Q, K, V, cu_seqlens, ea::AttnOut{O, lse, nullptr, nullptr},
                                      ws, static_cast<char*>(const_cast<void*>(workspace)),
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(EA_ERR_HIP, "XA attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

ea_status ea_xa_prefill(const void* Q, const void* K, const void* V, ea_dtype dtype,
                        const int8_t* modes, const int32_t* cu_seqlens, int32_t B,
                        int64_t total_tokens, int32_t max_seqlen, int32_t Hq, int32_t Hkv,
                        int32_t head_dim, const ea_sparsity_params* p, const ea_xa_params* xa,
                        void* O, float* lse, float* xa_mass, uint8_t* xa_keep, void* workspace,
                        size_t workspace_bytes, void* stream) {
  ea::Shape s;
  ea::Workspace ws;
  ea::Geometry g;
  ea_status st = check_xa(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype, p, xa, modes,
                          cu_seqlens, workspace, workspace_bytes, &s, &ws, &g);
  if (st != EA_OK) return st;
  if ((st = check_tensors(Q, K, V, O)) != EA_OK) return st;
  if (total_tokens == 0) return ok();
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(workspace);
  hipError_t e = ea::launch_setup(s, g, modes, cu_seqlens, ws, base, hs);
  if (e != hipSuccess) return fail(EA_ERR_HIP, "XA prefill launch failed: %s", hipGetErrorString(e));
  if (validate_on() && (st = workspace_verdict(workspace, stream)) != EA_OK) return st;
  e = ea::launch_xa_plan(s, g, xa->threshold, Q, K, modes, cu_seqlens, ws, base, xa_mass, xa_keep, hs);
  if (e == hipSuccess) e = ea::launch_items(s, g, modes, cu_seqlens, ws, base, hs);
  if (e == hipSuccess)
    e = ea::launch_attention(s, g, Q, K, V, cu_seqlens, ea::AttnOut{O, lse, nullptr, nullptr}, ws,
                             base, hs);
  if (e != hipSuccess) return fail(EA_ERR_HIP, "XA prefill launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

ea_status check_cache_desc(const ea_kvcache_desc* c) {
  if (!c) return fail(EA_ERR_INVALID_ARG, "null cache descriptor");
  if (c->B < 1 || c->Hkv < 1) return fail(EA_ERR_INVALID_ARG, "B and Hkv must be >= 1");
  if (static_cast<int64_t>(c->B) * c->Hkv > (1 << 24))
    return fail(EA_ERR_INVALID_ARG, "B * Hkv must be <= 2^24");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(EA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", c->head_dim);
  if (c->max_len < 1) return fail(EA_ERR_INVALID_ARG, "max_len must be >= 1");
  if (c->max_len > 2048 * ea::kDecodeChunkBlocks * ea::kBlock)
    return fail(EA_ERR_UNSUPPORTED, "max_len must be <= %d", 2048 * ea::kDecodeChunkBlocks * ea::kBlock);
  if (c->n_sink_blocks < 0 || c->window_blocks < 0 || c->n_sink_blocks > ea::kMaxGeomBlocks ||
      c->window_blocks > ea::kMaxGeomBlocks)
    return fail(EA_ERR_INVALID_ARG, "n_sink_blocks and window_blocks must be in [0, %d]",
                ea::kMaxGeomBlocks);
  if (c->window_blocks == 0 && !(c->keep_fraction > 0.f && c->keep_fraction <= 1.f))
    return fail(EA_ERR_INVALID_ARG, "keep_fraction must be in (0, 1]");
  return EA_OK;
}

ea::CacheView cache_view(const ea_kvcache_desc* d, void* cache, size_t bytes) {
  const ea::CacheLayout l = ea::cache_layout(d->B, d->Hkv);
  char* p = static_cast<char*>(cache);
  ea::CacheView v{};
  v.B = d->B;
  v.Hkv = d->Hkv;
  v.d = d->head_dim;
  v.max_len = d->max_len;
  v.n_sink = d->n_sink_blocks;
  v.window_blocks = d->window_blocks;
  v.keep_fraction = d->keep_fraction;
  const size_t blk = static_cast<size_t>(2) * ea::kBlock * d->head_dim * 2;
  v.area_blocks = bytes > l.blocks ? static_cast<int64_t>((bytes - l.blocks) / blk) : 0;
  v.lengths = reinterpret_cast<int32_t*>(p + l.lengths);
  v.cap = reinterpret_cast<int32_t*>(p + l.cap);
  v.ring = reinterpret_cast<int32_t*>(p + l.ring);
  v.base = reinterpret_cast<int64_t*>(p + l.base);
  v.mode = reinterpret_cast<int8_t*>(p + l.mode);
  v.valid = reinterpret_cast<int32_t*>(p + l.valid);
  v.K = reinterpret_cast<uint16_t*>(p + l.blocks);
  v.V = v.K + static_cast<size_t>(ea::kBlock) * d->head_dim;
  return v;
}

ea_status check_cache_buffer(const ea_kvcache_desc* d, const void* cache, size_t bytes) {
  if (!cache) return fail(EA_ERR_INVALID_ARG, "null cache");
  if ((reinterpret_cast<uintptr_t>(cache) & 255u) != 0)
    return fail(EA_ERR_INVALID_ARG, "cache must be 256-byte aligned");
  if (bytes < ea::cache_layout(d->B, d->Hkv).blocks)
    return fail(EA_ERR_WORKSPACE, "cache of %zu bytes is smaller than its header", bytes);
  return EA_OK;
}

}  // namespace

extern "C" {

size_t ea_kvcache_bytes(const ea_kvcache_desc* desc, const int8_t* modes_host) {
  if (check_cache_desc(desc) != EA_OK || !modes_host) return 0;
  g_err.clear();
  int64_t blocks = 0;
  const int64_t ns = static_cast<int64_t>(desc->B) * desc->Hkv;
  for (int64_t s = 0; s < ns; ++s)
    blocks += ea::cache_slot_blocks(modes_host[s], desc->max_len, desc->n_sink_blocks,
                                    desc->window_blocks, desc->keep_fraction);
  return ea::cache_layout(desc->B, desc->Hkv).blocks +
         static_cast<size_t>(blocks) * 2 * ea::kBlock * desc->head_dim * 2;
}

ea_status ea_kvcache_init(const ea_kvcache_desc* desc, const int8_t* modes, void* cache,
                          size_t bytes, void* stream) {
  ea_status st = check_cache_desc(desc);
  if (st != EA_OK) return st;
  if (!modes) return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  if ((st = check_cache_buffer(desc, cache, bytes)) != EA_OK) return st;
  hipError_t e = ea::launch_cache_init(cache_view(desc, cache, bytes), modes,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(EA_ERR_HIP, "cache init launch failed: %s", hipGetErrorString(e));
  return ok();
}

ea_status ea_kvcache_prefill(const ea_kvcache_desc* desc, void* cache, size_t bytes,
                             const void* K, const void* V, const int32_t* cu_seqlens,
                             int64_t total_tokens, void* stream) {
  ea_status st = check_cache_desc(desc);
  if (st != EA_OK) return st;
  if ((st = check_cache_buffer(desc, cache, bytes)) != EA_OK) return st;
  if (!K || !V || !cu_seqlens) return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(K) || !aligned16(V)) return fail(EA_ERR_INVALID_ARG, "K and V must be 16-byte aligned");
  if (total_tokens < 0 || total_tokens >= (int64_t(1) << 31))
    return fail(EA_ERR_INVALID_ARG, "total_tokens must be in [0, 2^31)");
  if (validate_on() && (st = host_check_cu(cu_seqlens, desc->B, total_tokens, desc->max_len, stream)) != EA_OK)
    return st;
  hipError_t e = ea::launch_cache_fill(cache_view(desc, cache, bytes), cu_seqlens, total_tokens,
                                       K, V, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(EA_ERR_HIP, "cache fill launch failed: %s", hipGetErrorString(e));
  return ok();
}

static int32_t decode_chunks(const ea_kvcache_desc* d) {
  const int32_t NB = (d->max_len + ea::kBlock - 1) / ea::kBlock;
  return (NB + ea::kDecodeChunkBlocks - 1) / ea::kDecodeChunkBlocks;
}

size_t ea_decode_workspace_size(const ea_kvcache_desc* desc, int32_t Hq) {
  if (check_cache_desc(desc) != EA_OK || Hq < 1) return 0;
  g_err.clear();
  const size_t rows = static_cast<size_t>(desc->B) * Hq * decode_chunks(desc);
  return ((rows * desc->head_dim * sizeof(float) + 255) & ~static_cast<size_t>(255)) +
         rows * sizeof(float);
}

ea_status ea_decode_step(const ea_kvcache_desc* desc, void* cache, size_t bytes, const void* q,
                         const void* k_new, const void* v_new, int32_t Hq, float softmax_scale,
                         void* O, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream) {
  ea_status st = check_cache_desc(desc);
  if (st != EA_OK) return st;
  if ((st = check_cache_buffer(desc, cache, bytes)) != EA_OK) return st;
  if (!q || !k_new || !v_new || !O) return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(O))
    return fail(EA_ERR_INVALID_ARG, "q, k_new, v_new and O must be 16-byte aligned");
  if (Hq < 1 || Hq % desc->Hkv != 0)
    return fail(EA_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, desc->Hkv);
  if (Hq / desc->Hkv > 16) return fail(EA_ERR_UNSUPPORTED, "Hq / Hkv must be <= 16 for decode");
  if (!(softmax_scale >= 0.f) || isinf(softmax_scale))
    return fail(EA_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  const size_t need = ea_decode_workspace_size(desc, Hq);
  if (!workspace || workspace_bytes < need)
    return fail(EA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(EA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  ea::DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.O = static_cast<uint16_t*>(O);
  a.lse = lse;
  a.Hq = Hq;
  a.G = Hq / desc->Hkv;
  a.n_chunks = decode_chunks(desc);
  a.chunk_blocks = ea::kDecodeChunkBlocks;
  a.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf(static_cast<float>(desc->head_dim));
  const size_t rows = static_cast<size_t>(desc->B) * Hq * a.n_chunks;
  a.o_part = static_cast<float*>(workspace);
  a.lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        ((rows * desc->head_dim * sizeof(float) + 255) & ~static_cast<size_t>(255)));
  hipError_t e = ea::launch_decode(cache_view(desc, cache, bytes), a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(EA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

static size_t bwd_row_bytes(const ea::Shape& s) {
  return (static_cast<size_t>(s.Hq) * s.T * sizeof(float) + 255) & ~static_cast<size_t>(255);
}
static size_t bwd_extra_bytes(const ea::Shape& s) {
  return 2 * bwd_row_bytes(s) + ea::dkv_list_layout(s).total;
}

size_t ea_hybrid_backward_workspace_size(int32_t B, int64_t total_tokens, int32_t max_seqlen,
                                         int32_t Hq, int32_t Hkv, int32_t head_dim,
                                         ea_dtype dtype) {
  ea::Shape s;
  if (check_shape(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype, &s) != EA_OK) return 0;
  g_err.clear();
  return ea::plan_workspace(s).total + bwd_extra_bytes(s);
}

ea_status ea_hybrid_backward(const void* Q, const void* K, const void* V, const void* O,
                             const void* dO, const float* lse, ea_dtype dtype,
                             const int8_t* modes, const int32_t* cu_seqlens, int32_t B,
                             int64_t total_tokens, int32_t max_seqlen, int32_t Hq, int32_t Hkv,
                             int32_t head_dim, const ea_sparsity_params* p, void* dQ, void* dK,
                             void* dV, void* workspace, size_t workspace_bytes, void* stream) {
  ea::Shape s;
  ea::Workspace ws;
  ea::Geometry g;
  if (dtype != EA_BF16) return fail(EA_ERR_UNSUPPORTED, "the backward is built for bf16 only");
  ea_status st = check_prefill(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype, p, modes,
                               cu_seqlens, workspace, workspace_bytes, &s, &ws, &g);
  if (st != EA_OK) return st;
  if ((st = check_tensors(Q, K, V, O)) != EA_OK) return st;
  if (!dO || !lse || !dQ || !dK || !dV) return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(dO) || !aligned16(dQ) || !aligned16(dK) || !aligned16(dV))
    return fail(EA_ERR_INVALID_ARG, "dO, dQ, dK and dV must be 16-byte aligned");
  const size_t need = ws.total + bwd_extra_bytes(s);
  if (workspace_bytes < need)
    return fail(EA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if (total_tokens == 0) return ok();
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(workspace);
  hipError_t e = ea::launch_worklist(s, g, modes, cu_seqlens, ws, base, hs);
  if (e != hipSuccess) return fail(EA_ERR_HIP, "work-list launch failed: %s", hipGetErrorString(e));
  if (validate_on() && (st = workspace_verdict(workspace, stream)) != EA_OK) return st;
  ea::BwdArgs a{};
  a.Q = static_cast<const uint16_t*>(Q);
  a.K = static_cast<const uint16_t*>(K);
  a.V = static_cast<const uint16_t*>(V);
  a.O = static_cast<const uint16_t*>(O);
  a.dO = static_cast<const uint16_t*>(dO);
  a.lse = lse;
  a.dQ = static_cast<uint16_t*>(dQ);
  a.dK = static_cast<uint16_t*>(dK);
  a.dV = static_cast<uint16_t*>(dV);
  const size_t rb = bwd_row_bytes(s);
  a.Dv = reinterpret_cast<float*>(base + ws.total);
  a.lse2 = reinterpret_cast<float*>(base + ws.total + rb);
  a.cu = cu_seqlens;
  a.modes = modes;
  a.seq_w = reinterpret_cast<const int32_t*>(base + ws.seq_w);
  a.items = reinterpret_cast<const ea::Item*>(base + ws.items_raw);
  a.order = reinterpret_cast<const int32_t*>(base + ws.order);
  a.meta = reinterpret_cast<const int32_t*>(base + ws.meta);
  a.T = s.T;
  a.max_items = ws.max_items;
  a.B = s.B;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.G = s.G;
  a.BMq = s.BMq;
  a.n_sink = g.n_sink;
  a.stamp = ea::plan_stamp(s);
  a.scale = g.scale;
  e = ea::launch_backward(s, g, a, ea::dkv_list_layout(s), base + ws.total + 2 * rb, hs);
  if (e != hipSuccess) return fail(EA_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t ea_router_logit_grad_workspace_size(int32_t B, int32_t max_seqlen, int32_t Hkv) {
  if (B < 1 || Hkv < 1 || max_seqlen < 1) return 0;
  g_err.clear();
  return static_cast<size_t>(B) * Hkv * ea::logit_grad_chunks(max_seqlen) * 2 * sizeof(float);
}

ea_status ea_router_logit_grad(const void* dO, const void* O_fa, const void* O_sa, ea_dtype dtype,
                               const int32_t* cu_seqlens, int32_t B, int64_t total_tokens,
                               int32_t max_seqlen, int32_t Hq, int32_t Hkv, int32_t head_dim,
                               const float* r_soft, float tau, float* dz, float* dr,
                               void* workspace, size_t workspace_bytes, void* stream) {
  ea::Shape s;
  ea_status st = check_shape(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype, &s);
  if (st != EA_OK) return st;
  if (!dO || !O_fa || !O_sa || !cu_seqlens || !r_soft || !dz)
    return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  if (!(tau > 0.f) || isinf(tau)) return fail(EA_ERR_INVALID_ARG, "tau must be finite and > 0");
  const size_t need = ea_router_logit_grad_workspace_size(B, s.max_seqlen, Hkv);
  if (!workspace || workspace_bytes < need)
    return fail(EA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  hipError_t e = ea::launch_logit_grad(s, cu_seqlens, dO, O_fa, O_sa, r_soft, tau, dz, dr,
                                       static_cast<float*>(workspace), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(EA_ERR_HIP, "logit gradient launch failed: %s", hipGetErrorString(e));
  return ok();
}

ea_status ea_mfma_probe(float* out, int32_t n_workgroups, int32_t iters, uint32_t seed,
                        int64_t* flops, void* stream) {
  if (!out) return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  if (n_workgroups < 1 || n_workgroups > (1 << 20))
    return fail(EA_ERR_INVALID_ARG, "n_workgroups must be in [1, 2^20] (got %d)", n_workgroups);
  if (iters < 1 || iters > (1 << 26))
    return fail(EA_ERR_INVALID_ARG, "iters must be in [1, 2^26] (got %d)", iters);
  if (!aligned16(out)) return fail(EA_ERR_INVALID_ARG, "out must be 16-byte aligned");
  if (flops) *flops = ea::mfma_probe_flops(n_workgroups, iters);
  hipError_t e = ea::launch_mfma_probe(out, n_workgroups, iters, seed, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(EA_ERR_HIP, "probe launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
