// Matrix-core throughput probe (measurement only; no part of the relation-KL path).
//
// The relation kernels' roofline is quoted against MI355X's published dense bf16 figure,
// 256 CUs x 4 SIMDs x 1024 flop/clk x 2.4 GHz.  Under a full matrix load the part does not
// hold 2.4 GHz, so the rate a perfect kernel could reach on the box is lower.  This probe
// measures it: every SIMD runs two waves (the relation backward's occupancy), each issuing
// independent v_mfma_f32_32x32x16_bf16 on four accumulator chains with operands in
// registers, cycled through eight pseudo-random fragments so that the matrix cores switch as
// they do on real data (the part is power-limited: constant operands would run faster).  With vector_work = 1 each group of four MFMAs also carries the vector work of
// one backward probability step per element (two FMAs, two exp2, a subtraction) for four
// elements, as in the backward's W tiles, so the figure includes the power drawn by that
// work beside the matrix cores.  The result is written to `sink` so that nothing is elided.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "lard.h"
#include "probe_internal.h"

namespace lard {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = LARD_PROBE_THREADS;           // 8 waves: two per SIMD
constexpr int kProbeGroups = LARD_PROBE_MFMA_PER_ITER / 4;  // groups of four MFMAs per iteration
constexpr int kProbeLdsFloats = 96 * 1024 / 4;
constexpr int kProbeFrags = 8;  // operand fragments cycled through

template <bool VEC>
__global__ __launch_bounds__(kProbeThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mfma_probe_kernel(float* sink, int iters, float c) {
  // more than half of a CU's LDS, so that one workgroup (two waves per SIMD) runs per CU
  __shared__ float occupancy[kProbeLdsFloats];
  const int lane = threadIdx.x & 63;
  occupancy[threadIdx.x] = c;
  // eight A and eight B fragments of pseudo-random N(0,1)-like bf16 values, cycled so that
  // consecutive MFMAs see different operands (the multipliers switch as with real data)
  bf16x8 a[kProbeFrags], b[kProbeFrags];
#pragma unroll
  for (int f = 0; f < kProbeFrags; ++f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t h = (uint32_t)(threadIdx.x * 131 + f * 17 + e) * 2654435761u;
      h ^= h >> 15;
      h *= 2246822519u;
      h ^= h >> 13;
      // sum of four uniform bytes, centred: roughly normal with unit variance
      const float u = (float)((h & 255) + ((h >> 8) & 255) + ((h >> 16) & 255) + (h >> 24));
      a[f][e] = (__bf16)((u - 510.0f) * (1.0f / 147.8f));
      h = h * 2654435761u + 12345u;
      h ^= h >> 16;
      const float w = (float)((h & 255) + ((h >> 8) & 255) + ((h >> 16) & 255) + (h >> 24));
      b[f][e] = (__bf16)((w - 510.0f) * (1.0f / 147.8f));
    }
  }
  f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
  float v[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = 0.01f * (float)(lane + r);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kProbeGroups; ++k) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(4 * k) % kProbeFrags], b[(4 * k + 1) % kProbeFrags], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(4 * k + 1) % kProbeFrags], b[(4 * k + 3) % kProbeFrags], acc1, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(4 * k + 2) % kProbeFrags], b[(4 * k + 5) % kProbeFrags], acc2, 0, 0, 0);
      acc3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(4 * k + 3) % kProbeFrags], b[(4 * k + 7) % kProbeFrags], acc3, 0, 0, 0);
      if constexpr (VEC) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = (4 * k + q) & 15;
          const float u0 = fmaf(v[r], c, -1.0f), u1 = fmaf(v[r], c, -2.0f);
          v[r] = __builtin_amdgcn_exp2f(u0) - __builtin_amdgcn_exp2f(u1);
        }
      }
    }
  }
  __syncthreads();
  float s = occupancy[(threadIdx.x + 64) % kProbeThreads];
#pragma unroll
  for (int r = 0; r < 16; ++r) s += v[r] + acc0[r] + acc1[r] + acc2[r] + acc3[r];
  sink[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

}  // namespace

int launch_probe_mfma(bool vector_work, int iters, int workgroups, float* sink, void* stream) {
  const char* inject = getenv("LARD_FAULT_INJECT");
  if (inject && inject[0] == '1') return (int)hipErrorLaunchFailure;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (vector_work)
    mfma_probe_kernel<true><<<workgroups, kProbeThreads, 0, s>>>(sink, iters, 0.5f);
  else
    mfma_probe_kernel<false><<<workgroups, kProbeThreads, 0, s>>>(sink, iters, 0.5f);
  return (int)hipGetLastError();
}

}  // namespace lard
