// Measurement aid, not part of the attention path: the bf16 MFMA rate the
// chip sustains under a plain loop of back-to-back v_mfma_f32_32x32x16_bf16
// on every SIMD, so that throughput figures can be stated against the rate
// measured in the same run as well as against the published dense peak.
//
// Each wave keeps four independent 32x32 accumulators and multiplies two
// register operands holding varied bf16 values (random mantissas and signs,
// magnitudes in [0.5, 1)), so the multipliers switch as they do on real data.
#include "common.h"
#include "kernels.h"

namespace wanattn {

namespace {

__global__ __launch_bounds__(256) void mfma_peak_kernel(float* __restrict__ sink, int iters) {
  uint32_t x = ((uint32_t)blockIdx.x * 256u + threadIdx.x) * 2654435761u + 0x9e3779b9u;
  u32x4 wa, wb;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    x = x * 1664525u + 1013904223u;
    wa[t] = 0x3f003f00u | (x & 0x807f807fu);
    x = x * 1664525u + 1013904223u;
    wb[t] = 0x3f003f00u | (x & 0x807f807fu);
  }
  const bf16x8 a = __builtin_bit_cast(bf16x8, wa);
  const bf16x8 b = __builtin_bit_cast(bf16x8, wb);
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = mfma32(a, b, acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_peak(float* sink, int workgroups, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream, sink, iters);
  return hipGetLastError();
}

}  // namespace wanattn
