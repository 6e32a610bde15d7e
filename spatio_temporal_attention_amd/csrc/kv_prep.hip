// Key/value preparation for the self-attention forward: one pass over K and V
// that writes them in the forward's tile layout, so that its main loop stages
// each 64-key tile with plain contiguous copies (no row clamping or 64-bit
// address arithmetic per tile) and reads V without the LDS transpose.
//
// Per (b, h, tile t) of 64 keys k = 64t .. 64t+63 (keys >= L are zero):
//   kt  [64][128] bf16   RNE_bf16(R(p_k) k_k), the keys rotated by 3D RoPE
//                        (3D RoPE over the (frame, height, width) token grid,
//                        Wan2.1 reading notes, 2. Model Design) or copied
//                        unrotated without a table;
//   k8t [64][128] fp8    the same rotated keys (from fp32) as OCP e4m3,
//                        saturated, when requested;
//   vt  [128][64] bf16   V transposed: row d holds v_k[d] at position pos(k),
//                        pos = k with bits 2 and 3 swapped (the key order of
//                        the PV product's register fragments).
#include "common.h"
#include "kernels.h"

namespace wanattn {

namespace {

__global__ __launch_bounds__(256) void kv_tiles_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                       uint16_t* __restrict__ kt, uint8_t* __restrict__ k8t,
                                                       uint16_t* __restrict__ vt, int L, int H, int nt,
                                                       RopeDev rope) {
  __shared__ __attribute__((aligned(16))) uint16_t s[TILE_ROWS][HD + 8];
  const int tile = blockIdx.x % nt;
  const int bh = blockIdx.x / nt;
  const int h = bh % H;
  const int b = bh / H;
  const int tid = threadIdx.x;
  const int64_t tile_elems = (int64_t)blockIdx.x * TILE_ELEMS;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int c = tid + 256 * it;   // 64 keys x 16 chunks of 8 d
    const int key = c >> 4;
    const int ch = c & 15;
    const int gk = tile * TILE_ROWS + key;
    u32x4 kx = u32x4{0u, 0u, 0u, 0u};
    u32x4 vx = u32x4{0u, 0u, 0u, 0u};
    if (gk < L) {
      const int64_t off = (((int64_t)b * L + gk) * H + h) * HD + ch * 8;
      kx = *reinterpret_cast<const u32x4*>(k + off);
      vx = *reinterpret_cast<const u32x4*>(v + off);
    }
    float r[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      r[2 * t] = bf16_lo(kx[t]);
      r[2 * t + 1] = bf16_hi(kx[t]);
    }
    if (rope.table != nullptr && gk < L) {
      const TokenPos pos = token_pos(rope, gk);
#pragma unroll
      for (int t = 0; t < 4; ++t) rope_rotate(r[2 * t], r[2 * t + 1], rope_cs(rope, pos, 4 * ch + t), false);
    }
    u32x4 ko;
#pragma unroll
    for (int t = 0; t < 4; ++t) ko[t] = pack_bf16(r[2 * t], r[2 * t + 1]);
    const int64_t dst = tile_elems + key * HD + ch * 8;
    *reinterpret_cast<u32x4*>(kt + dst) = ko;
    if (k8t != nullptr) {
      u32x2 o8;
      o8[0] = pack_fp8x4(r[0], r[1], r[2], r[3]);
      o8[1] = pack_fp8x4(r[4], r[5], r[6], r[7]);
      *reinterpret_cast<u32x2*>(k8t + dst) = o8;
    }
    *reinterpret_cast<u32x4*>(&s[key][ch * 8]) = vx;
  }
  __syncthreads();
  uint16_t* out = vt + tile_elems;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int c = tid + 256 * it;   // 128 d rows x 8 chunks of 8 positions
    const int d = c >> 3;
    const int pc = c & 7;
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p0 = 8 * pc + 2 * e;
      const int k0 = (p0 & ~12) | ((p0 & 4) << 1) | ((p0 & 8) >> 1);   // bit 0 untouched: k0 + 1 is p0 + 1
      w[e] = (uint32_t)s[k0][d] | ((uint32_t)s[k0 + 1][d] << 16);
    }
    *reinterpret_cast<u32x4*>(out + d * 64 + pc * 8) = w;
  }
}

}  // namespace

hipError_t launch_kv_tiles(const uint16_t* k, const uint16_t* v, uint16_t* kt, uint8_t* k8t, uint16_t* vt, int B,
                           int L, int H, const RopeDev& rope, hipStream_t stream) {
  const int nt = (L + TILE_ROWS - 1) / TILE_ROWS;
  const int64_t total = (int64_t)B * H * nt;
  if (total <= 0 || total > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_tiles_kernel, dim3((unsigned)total), dim3(256), 0, stream, k, v, kt, k8t, vt, L, H, nt, rope);
  return hipGetLastError();
}

}  // namespace wanattn
