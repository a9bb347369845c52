// Matrix-core ceiling probe: back-to-back bf16 MFMAs on every CU with the
// attention kernel's instruction and waves per CU, and no memory traffic in
// the loop.  Its throughput is the practical bf16 peak at whatever clock the
// board holds under a pure matrix load, the figure the attention kernel's
// throughput is set against beside the 2.4 GHz data-sheet peak.
#include "ea_internal.h"

namespace ea {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int kProbeThreads = 512;   // 8 waves, as the attention kernel
constexpr int kProbeSets = 4;        // operand register sets cycled through
constexpr int kProbeChains = 4;      // independent accumulators per wave
// More LDS than half a CU's 160 KiB: one probe workgroup per CU.
constexpr int kProbeLdsBytes = 96 * 1024;

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  // integer finaliser of MurmurHash3
  x ^= x >> 16;
  x *= 0x85ebca6bu;
  x ^= x >> 13;
  x *= 0xc2b2ae35u;
  x ^= x >> 16;
  return x;
}

// A bf16 with random sign and mantissa and an exponent in [2^-2, 2^1]: full
// operand toggling with no overflow of the fp32 accumulators.
__device__ __forceinline__ unsigned short random_bf16(uint32_t r) {
  return static_cast<unsigned short>(((r >> 31) << 15) | ((125u + (r & 3u)) << 7) | ((r >> 2) & 0x7fu));
}

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(float* __restrict__ out,
                                                                   int32_t iters, uint32_t seed) {
  extern __shared__ float probe_lds[];
  const uint32_t gid = blockIdx.x * kProbeThreads + threadIdx.x;
  bf16x8 a[kProbeSets], b[kProbeSets];
#pragma unroll
  for (int s = 0; s < kProbeSets; ++s) {
    u16x8 ua, ub;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ua[e] = random_bf16(mix32(seed ^ mix32(gid * 64u + s * 16u + e)));
      ub[e] = random_bf16(mix32(~seed ^ mix32(gid * 64u + s * 16u + 8u + e)));
    }
    a[s] = __builtin_bit_cast(bf16x8, ua);
    b[s] = __builtin_bit_cast(bf16x8, ub);
  }
  f32x16 acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) acc[c] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int s = 0; s < kProbeSets; ++s)
#pragma unroll
      for (int c = 0; c < kProbeChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[(s + c) % kProbeSets], acc[c], 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += acc[c][e];
  if (threadIdx.x == 0) probe_lds[0] = 0.f;  // the LDS reservation is only for placement
  out[gid] = sum;
}

}  // namespace

hipError_t launch_mfma_probe(float* out, int32_t n_workgroups, int32_t iters, uint32_t seed,
                             hipStream_t st) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(n_workgroups), dim3(kProbeThreads), kProbeLdsBytes,
                     st, out, iters, seed);
  return hipGetLastError();
}

int64_t mfma_probe_flops(int32_t n_workgroups, int32_t iters) {
  // 2 * 32 * 32 * 16 FLOP per MFMA, kProbeSets * kProbeChains MFMAs per wave
  // per iteration, 8 waves per workgroup
  return static_cast<int64_t>(n_workgroups) * (kProbeThreads / 64) * iters * kProbeSets *
         kProbeChains * 2 * 32 * 32 * 16;
}

}  // namespace ea
