// Matrix-core peak probe: MFMAs issued back to back on register operands,
// with no memory traffic, so that the rate the chip sustains at its running
// clock can be set beside the grouped GEMMs' rates ([MoK clip] How-to item 1:
// profile first to see where the time goes). Each wavefront keeps 8
// independent accumulator chains, enough to cover the dependent-issue latency
// of one chain.
#include "mok_device.h"
#include "mok_launch.h"

namespace {

constexpr int kChains = 8;

__global__ __launch_bounds__(256) void probe_mfma_bf16_kernel(int iters, float* __restrict__ sink) {
  const int t = threadIdx.x;
  bf16x8_t a, b;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    a[u] = (__bf16)(1.0f + 0.001f * (float)((t + u) & 7));
    b[u] = (__bf16)(1.0f - 0.001f * (float)((t * 3 + u) & 7));
  }
  f32x16_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = (f32x16_t){};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int q = 0; q < 16; ++q) s += acc[c][q];
  sink[(int64_t)blockIdx.x * 256 + t] = s;
}

__global__ __launch_bounds__(256) void probe_mfma_f8_kernel(int iters, float* __restrict__ sink) {
  const int t = threadIdx.x;
  i32x8_t a, b;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    a[u] = 0x38383838 + ((t + u) & 3);        // E4M3 codes near 1.0
    b[u] = 0x38383838 + ((t * 3 + u) & 3);
  }
  f32x16_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = (f32x16_t){};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int q = 0; q < 16; ++q) s += acc[c][q];
  sink[(int64_t)blockIdx.x * 256 + t] = s;
}

}  // namespace

hipError_t mok_launch_probe_mfma(int kind, int workgroups, int iters, float* sink, hipStream_t st) {
  if (workgroups <= 0 || iters <= 0) return hipSuccess;
  if (kind == 0)
    hipLaunchKernelGGL(probe_mfma_bf16_kernel, dim3(workgroups), dim3(256), 0, st, iters, sink);
  else
    hipLaunchKernelGGL(probe_mfma_f8_kernel, dim3(workgroups), dim3(256), 0, st, iters, sink);
  return hipGetLastError();
}
