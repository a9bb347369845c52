// Attention router: boundary pooling of the Key states, task MLP, router MLP
// and the hard FA/SA argmax, one workgroup per (sequence, KV head).
//
// Pages: "Elastic Attention: Test-time Adaptive Sparsity Ratios for Efficient
// Transformers", router paragraph on Fig. 3(c) (pool x_K along the sequence to
// x'_K in R^{H x d'}, task MLP, router MLP, logits z in R^{H x 2}) and the
// boundary-pooling paragraph of the implementation details (first and last 100
// tokens); Fig. 3(b) paragraph for the 0 = FA / 1 = SA convention.
//
// The work is tiny (200 rows of K, ~0.14-0.27M weights) and latency bound:
// pooling reads coalesced rows of K; each matrix-vector product gives
// kRowsPerWave output rows per wave at a time, the lanes striding the
// contiguous input axis, so the loads of all those rows are in flight
// together, then one butterfly reduction across the wave per row.
#include "ea_internal.h"

namespace ea {
namespace {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kRowsPerWave = 8;

__device__ __forceinline__ float load_elem(const void* p, int64_t i, bool bf16) {
  if (bf16) {
    uint32_t u = static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16;
    return __uint_as_float(u);
  }
  return static_cast<const float*>(p)[i];
}

__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// out[r] = act(W[r, :] . x + bias[r]) for r < rows; x and out in LDS.
__device__ void matvec(const float* __restrict__ W, const float* __restrict__ bias,
                       const float* x, float* out, int rows, int cols, bool act) {
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  for (int r0 = wave * kRowsPerWave; r0 < rows; r0 += kRouteWaves * kRowsPerWave) {
    float acc[kRowsPerWave];
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) acc[j] = 0.f;
#pragma unroll 4
    for (int c = lane; c < cols; c += 64) {
      const float xv = x[c];
#pragma unroll
      for (int j = 0; j < kRowsPerWave; ++j)
        if (r0 + j < rows) acc[j] += W[static_cast<int64_t>(r0 + j) * cols + c] * xv;
    }
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) acc[j] = wave_sum(acc[j]);
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < kRowsPerWave; ++j) {
        if (r0 + j < rows) {
          const float y = acc[j] + bias[r0 + j];
          out[r0 + j] = act ? gelu_erf(y) : y;
        }
      }
    }
  }
}

__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const void* __restrict__ K, bool bf16, const int32_t* __restrict__ cu, int32_t Hkv,
    ea_router_desc r, int8_t* __restrict__ modes, float* __restrict__ logits) {
  extern __shared__ float smem[];
  const int d = r.head_dim;
  float* x = smem;                        // [d] pooled keys
  float* h1 = x + d;                      // [task_hidden]
  float* t = h1 + r.task_hidden;          // [d] task features
  float* h3 = t + d;                      // [router_hidden]
  float* z = h3 + r.router_hidden;        // [2]
  float* part = z + 2;                    // [kRouteThreads] partial sums

  const int b = blockIdx.x / Hkv, g = blockIdx.x % Hkv;
  const int s0 = cu[b];
  const int L = cu[b + 1] - s0;
  const int64_t out = static_cast<int64_t>(b) * Hkv + g;
  if (L <= 0) {
    if (threadIdx.x == 0) {
      modes[out] = 0;
      if (logits) {
        logits[2 * out] = 0.f;
        logits[2 * out + 1] = 0.f;
      }
    }
    return;
  }
  // Boundary rows: [0, head_end) and [tail_beg, L), disjoint by construction.
  const int head_end = min(r.pool_len, L);
  const int tail_beg = max(head_end, L - r.pool_len);
  const int n_rows = head_end + (L - tail_beg);

  // Thread (stripe, c) sums column c over rows stripe, stripe + n_stripes, ...
  const int n_stripes = kRouteThreads / d;
  const int c = threadIdx.x % d, stripe = threadIdx.x / d;
  float acc = 0.f;
  if (stripe < n_stripes) {
#pragma unroll 8
    for (int i = stripe; i < n_rows; i += n_stripes) {
      const int row = i < head_end ? i : tail_beg + (i - head_end);
      acc += load_elem(K, (static_cast<int64_t>(s0 + row) * Hkv + g) * d + c, bf16);
    }
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x < d) {
    float s = 0.f;
    for (int k = 0; k < n_stripes; ++k) s += part[k * d + threadIdx.x];
    x[threadIdx.x] = s / static_cast<float>(n_rows);
  }
  __syncthreads();
  matvec(r.w1, r.b1, x, h1, r.task_hidden, d, true);
  __syncthreads();
  matvec(r.w2, r.b2, h1, t, d, r.task_hidden, false);
  __syncthreads();
  matvec(r.w3, r.b3, t, h3, r.router_hidden, d, true);
  __syncthreads();
  matvec(r.w4, r.b4, h3, z, 2, r.router_hidden, false);
  __syncthreads();
  if (threadIdx.x == 0) {
    modes[out] = z[1] > z[0] ? 1 : 0;
    if (logits) {
      logits[2 * out] = z[0];
      logits[2 * out + 1] = z[1];
    }
  }
}

}  // namespace

hipError_t launch_route(const void* K, bool bf16, const int32_t* cu, int32_t B, int32_t Hkv,
                        const ea_router_desc& r, int8_t* modes, float* logits, hipStream_t st) {
  const size_t smem =
      sizeof(float) * (2 * r.head_dim + r.task_hidden + r.router_hidden + 2 + kRouteThreads);
  const unsigned grid = static_cast<unsigned>(B) * static_cast<unsigned>(Hkv);
  hipLaunchKernelGGL(route_kernel, dim3(grid), dim3(kRouteThreads), smem, st, K, bf16, cu, Hkv,
                     r, modes, logits);
  return hipGetLastError();
}

}  // namespace ea
