// Throughput probes for the units the attention kernels lean on: the hardware exp2
// (v_exp_f32, a transcendental), fp32 fused multiply-add on the vector ALU, and the
// bf16 matrix cores (32x32x8 and 32x32x16 shapes). Each probe runs independent
// dependency chains in every lane of a full grid so the measured rate is the unit's
// issue rate; the result is written to `sink` so the compiler keeps the work. The exp
// chains step x -> exp2(-|x|), which stays in [0.5, 1] and costs one v_exp_f32 with
// source modifiers (negate, absolute value) and no other instruction.
#include "gt_internal.h"

namespace gt {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kChains = 8;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(kProbeThreads) void probe_exp(float* sink, int iters) {
  float x[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) x[c] = -1.0f - 1e-3f * (threadIdx.x + c);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = __builtin_amdgcn_exp2f(-__builtin_fabsf(x[c]));
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += x[c];
  sink[blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kProbeThreads) void probe_fma(float* sink, int iters) {
  float x[kChains];
  const float a = 0.999f, b = 1e-4f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) x[c] = 1.0f + 1e-3f * (threadIdx.x + c);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = fmaf(x[c], a, b);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += x[c];
  sink[blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

// One exp plus four fma per chain step: shows whether transcendentals overlap with FMAs.
__global__ __launch_bounds__(kProbeThreads) void probe_exp_fma(float* sink, int iters) {
  float x[kChains], y[kChains];
  const float a = 0.999f, b = 1e-4f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
    x[c] = -1.0f - 1e-3f * (threadIdx.x + c);
    y[c] = 1.0f;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      x[c] = __builtin_amdgcn_exp2f(-__builtin_fabsf(x[c]));
      y[c] = fmaf(fmaf(fmaf(fmaf(y[c], a, b), a, b), a, b), a, b);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += x[c] + y[c];
  sink[blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kProbeThreads) void probe_mfma_x8(float* sink, int iters) {
  s16x4 a, b;
  for (int e = 0; e < 4; ++e) {
    a[e] = static_cast<short>(0x3C00 + threadIdx.x % 7);
    b[e] = static_cast<short>(0x3C00 + threadIdx.x % 5);
  }
  f32x16 acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
  for (int c = 0; c < 4; ++c)
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  sink[blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kProbeThreads) void probe_mfma_x16(float* sink, int iters) {
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(1.0f + 0.01f * (threadIdx.x % 7));
    b[e] = static_cast<__bf16>(1.0f + 0.01f * (threadIdx.x % 5));
  }
  f32x16 acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
  for (int c = 0; c < 4; ++c)
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  sink[blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

}  // namespace

// kind: 0 exp, 1 fma, 2 exp+4fma, 3 mfma 32x32x8 bf16, 4 mfma 32x32x16 bf16.
// Work per launch: blocks*256 lanes x iters x kChains (x 5 for kind 2) operations,
// or blocks*4 waves x iters x 4 matrix instructions for kinds 3 and 4.
hipError_t launch_probe(int kind, int blocks, int iters, float* sink, hipStream_t s) {
  switch (kind) {
    case 0: hipLaunchKernelGGL(probe_exp, dim3(blocks), dim3(kProbeThreads), 0, s, sink, iters); break;
    case 1: hipLaunchKernelGGL(probe_fma, dim3(blocks), dim3(kProbeThreads), 0, s, sink, iters); break;
    case 2: hipLaunchKernelGGL(probe_exp_fma, dim3(blocks), dim3(kProbeThreads), 0, s, sink, iters); break;
    case 3: hipLaunchKernelGGL(probe_mfma_x8, dim3(blocks), dim3(kProbeThreads), 0, s, sink, iters); break;
    default: hipLaunchKernelGGL(probe_mfma_x16, dim3(blocks), dim3(kProbeThreads), 0, s, sink, iters); break;
  }
  return hipGetLastError();
}

}  // namespace gt
