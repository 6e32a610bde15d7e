// Exact merge of partial attention results over disjoint key sets (the key
// shards of Ring attention, the "outside" axis of the 2D context parallelism
// in the anthology note's Key takeaways, Attention dominates): with
// LSE = ln sum_r exp(LSE_r) and w_r = exp(LSE_r - LSE),
//   O = sum_r w_r O_r,
// since O_r = sum_{j in r} exp(s_j - LSE_r) v_j.  Shards with an empty key
// set (LSE_r = -inf) get weight 0; if every shard is empty, O = 0 and
// LSE = -inf.  HBM-bound: R + 1 reads/writes of a [B, L, H, 128] bf16 tensor.
#include "common.h"
#include "kernels.h"

namespace wanattn {

namespace {

// 16 threads per (b, n, h) row, one 8-element chunk each.
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeParams p) {
  const int64_t rows = (int64_t)p.B * p.L * p.H;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t tix = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; tix < rows * 16; tix += stride) {
    const int64_t row = tix >> 4;
    const int c = (int)(tix & 15);
    const int h = (int)(row % p.H);
    const int64_t bn = row / p.H;
    const int n = (int)(bn % p.L);
    const int b = (int)(bn / p.L);
    const int64_t si = ((int64_t)b * p.H + h) * p.L + n;
    float m = -INFINITY;
    for (int r = 0; r < p.R; ++r) m = fmaxf(m, p.lse[r][si]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float lse = -INFINITY;
    if (m > -INFINITY) {
      float sum = 0.f;
      for (int r = 0; r < p.R; ++r) sum += expf(p.lse[r][si] - m);
      lse = m + logf(sum);
      for (int r = 0; r < p.R; ++r) {
        const float w = expf(p.lse[r][si] - lse);
        const u32x4 x = *reinterpret_cast<const u32x4*>(p.o[r] + row * HD + c * 8);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          acc[2 * t] = fmaf(w, bf16_lo(x[t]), acc[2 * t]);
          acc[2 * t + 1] = fmaf(w, bf16_hi(x[t]), acc[2 * t + 1]);
        }
      }
    }
    u32x4 y;
#pragma unroll
    for (int t = 0; t < 4; ++t) y[t] = pack_bf16(acc[2 * t], acc[2 * t + 1]);
    *reinterpret_cast<u32x4*>(p.out + row * HD + c * 8) = y;
    if (c == 0 && p.out_lse != nullptr) p.out_lse[si] = lse;
  }
}

}  // namespace

hipError_t launch_lse_merge(const MergeParams& p, hipStream_t stream) {
  if (p.R < 1 || p.R > MERGE_MAX) return hipErrorInvalidValue;
  const int64_t threads = (int64_t)p.B * p.L * p.H * 16;
  if (threads == 0) return hipSuccess;
  int64_t blocks = (threads + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace wanattn
