// 3D RoPE: the cos/sin table and the standalone (pre-)rotation of a
// [B, L, H, 128] bf16 tensor.  Positions are the row-major (frame, row,
// column) indices of the post-patchify token grid (Wan2.1 reading notes,
// 2. Model Design: latent [1+T/4, H/8, W/8], (1,2,2) patch; DiT block
// paragraph: 3D RoPE over time, height and width).
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace wanattn {

namespace {

// One table entry per thread: angle p * theta^(-2j/d_a) in fp64, cos/sin in
// fp64 (device libm), rounded to fp32.
__global__ void rope_table_kernel(float2* table, int f, int h, int w, int nf, int nh, int nw, double theta) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nf_tot = (int64_t)f * nf;
  const int64_t nh_tot = (int64_t)h * nh;
  const int64_t nw_tot = (int64_t)w * nw;
  if (e >= nf_tot + nh_tot + nw_tot) return;
  int64_t local;
  int npairs;
  if (e < nf_tot) {
    local = e;
    npairs = nf;
  } else if (e < nf_tot + nh_tot) {
    local = e - nf_tot;
    npairs = nh;
  } else {
    local = e - nf_tot - nh_tot;
    npairs = nw;
  }
  const int64_t pos = local / npairs;
  const int j = (int)(local % npairs);
  const double omega = pow(theta, -2.0 * (double)j / (double)(2 * npairs));
  const double ang = (double)pos * omega;
  double s, c;
  sincos(ang, &s, &c);
  table[e] = make_float2((float)c, (float)s);
}

// One 16-byte chunk (8 elements, 4 pairs) per thread; memory-bound.
__global__ __launch_bounds__(256) void rope3d_kernel(const uint16_t* x, uint16_t* y, int64_t nchunks, int L, int H,
                                                     RopeDev rope, bool inverse) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t cidx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; cidx < nchunks; cidx += stride) {
    const int c = (int)(cidx & 15);
    const int64_t row = cidx >> 4;                 // (b, n, h) row index
    const int n = (int)((row / H) % L);
    const u32x4 v = *reinterpret_cast<const u32x4*>(x + cidx * 8);
    *reinterpret_cast<u32x4*>(y + cidx * 8) = rope_chunk(rope, token_pos(rope, n), c, v, inverse);
  }
}

}  // namespace

hipError_t launch_rope_table(float* table, int f, int h, int w, int d_f, int d_h, int d_w, double theta,
                             hipStream_t stream) {
  const int64_t total = (int64_t)f * (d_f / 2) + (int64_t)h * (d_h / 2) + (int64_t)w * (d_w / 2);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<float2*>(table), f, h, w, d_f / 2, d_h / 2, d_w / 2, theta);
  return hipGetLastError();
}

hipError_t launch_rope3d(const uint16_t* x, uint16_t* y, int B, int L, int H, const RopeDev& rope, bool inverse,
                         hipStream_t stream) {
  const int64_t nchunks = (int64_t)B * L * H * (HD / 8);
  if (nchunks == 0) return hipSuccess;
  int64_t blocks = (nchunks + 255) / 256;
  const int64_t cap = 256 * 64;                    // 64 blocks per CU; grid-stride beyond that
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(rope3d_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, y, nchunks, L, H, rope,
                     inverse);
  return hipGetLastError();
}

}  // namespace wanattn
