// Training-forward kernels: Gumbel-Softmax routing with straight-through hard
// decisions, and the merge that turns the dual-mode attention launch's two
// partial results per head into the FA output and the mixed layer output.
//
// Pages: the Gumbel-Softmax and straight-through-estimator paragraphs of the
// method section of "Elastic Attention: Test-time Adaptive Sparsity Ratios
// for Efficient Transformers" ("Technical Summary: Elastic Attention",
// Sec. 2.2): routing logits z go through a Gumbel-Softmax with an annealed
// temperature to r_soft, the hard decision is its argmax, and the forward pass
// uses the hard decision while gradients flow through r_soft.  During router
// training every head therefore needs both its FA and its SA output.
//
// The dual-mode attention launch covers each head's causal key blocks exactly
// once, split into the SA set (sinks + local window) and the rest: the SA
// items produce O_SA and LSE_SA directly, the others a partial (O_mid,
// LSE_mid) over the keys SA leaves out.  Since softmax attention over a union
// of disjoint key sets is the LSE-weighted mean of the attention over each,
//   LSE_FA = log(e^LSE_SA + e^LSE_mid),
//   O_FA   = e^(LSE_SA - LSE_FA) O_SA + e^(LSE_mid - LSE_FA) O_mid,
// the merge below needs nothing but those two partials, and the FA output
// costs no more matrix work than an FA-only forward.
#include "ea_internal.h"

#include <math.h>

namespace ea {
namespace {

__global__ __launch_bounds__(256) void gumbel_route_kernel(const float* __restrict__ logits,
                                                           const float* __restrict__ gumbel,
                                                           float tau, int64_t n,
                                                           float* __restrict__ r_soft,
                                                           int8_t* __restrict__ modes) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float y0 = logits[2 * i], y1 = logits[2 * i + 1];
  if (gumbel) {
    y0 += gumbel[2 * i];
    y1 += gumbel[2 * i + 1];
  }
  y0 /= tau;
  y1 /= tau;
  // two-way softmax, the larger exponent first for range
  const float m = fmaxf(y0, y1);
  const float e0 = expf(y0 - m), e1 = expf(y1 - m);
  const float inv = 1.0f / (e0 + e1);
  if (r_soft) {
    r_soft[2 * i] = e0 * inv;
    r_soft[2 * i + 1] = e1 * inv;
  }
  modes[i] = y1 > y0 ? 1 : 0;  // argmax, a tie to FA
}

__device__ __forceinline__ int find_seq(const int32_t* cu, int B, int64_t t) {
  int lo = 0, hi = B;  // invariant: cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

template <typename E, int VEC>
struct Vec {
  E v[VEC];
};

// One thread per VEC consecutive elements of a row (t, hq); the d / VEC
// threads of a row sit in one wave, so the row's LSE is read by all of them
// before any writes it back.
template <typename E, int VEC>
__global__ __launch_bounds__(256) void dual_merge_kernel(
    const int32_t* __restrict__ cu, int32_t B, const int8_t* __restrict__ modes, int32_t Hkv,
    int32_t G, int64_t T, int32_t Hq, int32_t d, const E* __restrict__ O_sa,
    const float* __restrict__ lse_sa, E* O_fa, float* lse_fa, E* __restrict__ O,
    const int32_t* __restrict__ meta, int32_t stamp) {
  if (meta[kMetaStamp] != stamp) return;  // the planner rejected the device contents
  const int cpr = d / VEC;
  const int64_t total = T * Hq * cpr;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = idx / cpr;
    const int c = static_cast<int>(idx - r * cpr);
    const int64_t t = r / Hq;
    const int hq = static_cast<int>(r - t * Hq);
    const int64_t li = static_cast<int64_t>(hq) * T + t;
    const float la = lse_sa[li], lb = lse_fa[li];
    const float m = fmaxf(la, lb);
    const float wa = expf(la - m), wb = expf(lb - m);  // wb = 0 when the middle set is empty
    const float sw = wa + wb;
    const float ca = wa / sw, cb = wb / sw;
    const int64_t off = r * d + static_cast<int64_t>(c) * VEC;
    const Vec<E, VEC> a = *reinterpret_cast<const Vec<E, VEC>*>(O_sa + off);
    const Vec<E, VEC> bm = *reinterpret_cast<const Vec<E, VEC>*>(O_fa + off);
    Vec<E, VEC> f;
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      f.v[e] = static_cast<E>(ca * static_cast<float>(a.v[e]) + cb * static_cast<float>(bm.v[e]));
    *reinterpret_cast<Vec<E, VEC>*>(O_fa + off) = f;
    if (c == 0) lse_fa[li] = m + logf(sw);
    if (O) {
      const int b = find_seq(cu, B, t);
      const bool sa = modes[static_cast<int64_t>(b) * Hkv + hq / G] != 0;
      *reinterpret_cast<Vec<E, VEC>*>(O + off) = sa ? a : f;
    }
  }
}

// Router-logit gradient, stage 1: per (sequence, KV head, chunk of
// kGradChunk tokens) the sums over its tokens and the G query heads of
// <dO, O_FA> and <dO, O_SA>; a workgroup reduces in a fixed order.
constexpr int kGradChunk = 256;

template <typename E>
__global__ __launch_bounds__(256) void logit_grad_partial_kernel(
    const int32_t* __restrict__ cu, int32_t B, int32_t Hkv, int32_t G, int32_t Hq, int32_t d,
    int32_t nchunk, const E* __restrict__ dO, const E* __restrict__ O_fa,
    const E* __restrict__ O_sa, float* __restrict__ part) {
  __shared__ float red[2][4];
  const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int t0 = cu[b] + chunk * kGradChunk, t1 = min(cu[b + 1], t0 + kGradChunk);
  const int row_elems = G * d;  // the group's heads are contiguous in a token row
  float a0 = 0.f, a1 = 0.f;
  for (int t = t0; t < t1; ++t) {
    const int64_t base = (static_cast<int64_t>(t) * Hq + static_cast<int64_t>(g) * G) * d;
    for (int e = tid; e < row_elems; e += 256) {
      const float x = static_cast<float>(dO[base + e]);
      a0 += x * static_cast<float>(O_fa[base + e]);
      a1 += x * static_cast<float>(O_sa[base + e]);
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    a0 += __shfl_xor(a0, off, 64);
    a1 += __shfl_xor(a1, off, 64);
  }
  if (tid % 64 == 0) {
    red[0][tid / 64] = a0;
    red[1][tid / 64] = a1;
  }
  __syncthreads();
  if (tid == 0) {
    const int64_t pi = ((static_cast<int64_t>(b) * Hkv + g) * nchunk + chunk) * 2;
    part[pi] = t0 < t1 ? (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]) : 0.f;
    part[pi + 1] = t0 < t1 ? (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]) : 0.f;
  }
}

// Stage 2: dr = the chunks' sums in order, then through the Gumbel-Softmax:
// dz = r_soft * (dr - <dr, r_soft>) / tau.
__global__ __launch_bounds__(256) void logit_grad_final_kernel(const float* __restrict__ part,
                                                               int64_t n, int32_t nchunk,
                                                               const float* __restrict__ r_soft,
                                                               float tau, float* __restrict__ dz,
                                                               float* __restrict__ dr) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float d0 = 0.f, d1 = 0.f;
  for (int c = 0; c < nchunk; ++c) {
    d0 += part[(i * nchunk + c) * 2];
    d1 += part[(i * nchunk + c) * 2 + 1];
  }
  const float r0 = r_soft[2 * i], r1 = r_soft[2 * i + 1];
  const float mean = d0 * r0 + d1 * r1;
  dz[2 * i] = r0 * (d0 - mean) / tau;
  dz[2 * i + 1] = r1 * (d1 - mean) / tau;
  if (dr) {
    dr[2 * i] = d0;
    dr[2 * i + 1] = d1;
  }
}

}  // namespace

int32_t logit_grad_chunks(int32_t max_seqlen) { return (max_seqlen + kGradChunk - 1) / kGradChunk; }

hipError_t launch_logit_grad(const Shape& s, const int32_t* cu, const void* dO, const void* O_fa,
                             const void* O_sa, const float* r_soft, float tau, float* dz, float* dr,
                             float* part, hipStream_t st) {
  const int32_t nchunk = logit_grad_chunks(s.max_seqlen);
  const dim3 grid(static_cast<unsigned>(nchunk), static_cast<unsigned>(s.Hkv), static_cast<unsigned>(s.B));
  if (s.elem_bytes == 2)
    hipLaunchKernelGGL((logit_grad_partial_kernel<__bf16>), grid, dim3(256), 0, st, cu, s.B, s.Hkv,
                       s.G, s.Hq, s.d, nchunk, static_cast<const __bf16*>(dO),
                       static_cast<const __bf16*>(O_fa), static_cast<const __bf16*>(O_sa), part);
  else
    hipLaunchKernelGGL((logit_grad_partial_kernel<float>), grid, dim3(256), 0, st, cu, s.B, s.Hkv,
                       s.G, s.Hq, s.d, nchunk, static_cast<const float*>(dO),
                       static_cast<const float*>(O_fa), static_cast<const float*>(O_sa), part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = static_cast<int64_t>(s.B) * s.Hkv;
  hipLaunchKernelGGL(logit_grad_final_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                     0, st, part, n, nchunk, r_soft, tau, dz, dr);
  return hipGetLastError();
}

hipError_t launch_gumbel_route(const float* logits, const float* gumbel, float tau, int64_t n,
                               float* r_soft, int8_t* modes, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>((n + 255) / 256);
  hipLaunchKernelGGL(gumbel_route_kernel, dim3(grid), dim3(256), 0, st, logits, gumbel, tau, n,
                     r_soft, modes);
  return hipGetLastError();
}

hipError_t launch_dual_merge(const Shape& s, const int32_t* cu, const int8_t* modes,
                             const void* O_sa, const float* lse_sa, void* O_fa, float* lse_fa,
                             void* O, const int32_t* meta, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  const int32_t stamp = plan_stamp(s);
  const int vec = s.elem_bytes == 2 ? 8 : 4;  // 16-byte accesses
  const int64_t threads = s.T * s.Hq * (s.d / vec);
  const unsigned grid = static_cast<unsigned>(threads / 256 + 1 < 65536 ? threads / 256 + 1 : 65536);
  if (s.elem_bytes == 2)
    hipLaunchKernelGGL((dual_merge_kernel<__bf16, 8>), dim3(grid), dim3(256), 0, st, cu, s.B,
                       modes, s.Hkv, s.G, s.T, s.Hq, s.d, static_cast<const __bf16*>(O_sa), lse_sa,
                       static_cast<__bf16*>(O_fa), lse_fa, static_cast<__bf16*>(O), meta, stamp);
  else
    hipLaunchKernelGGL((dual_merge_kernel<float, 4>), dim3(grid), dim3(256), 0, st, cu, s.B,
                       modes, s.Hkv, s.G, s.T, s.Hq, s.d, static_cast<const float*>(O_sa), lse_sa,
                       static_cast<float*>(O_fa), lse_fa, static_cast<float*>(O), meta, stamp);
  return hipGetLastError();
}

}  // namespace ea
