// Key/value preparation for the self-attention forward: one pass over K and V
// that writes them in the forward's tile layout, so that its main loop stages
// each 64-key tile with plain contiguous copies (no row clamping or 64-bit
// address arithmetic per tile) and reads V without the LDS transpose.
//
// Per (b, h, tile t) of 64 keys k = 64t .. 64t+63 (keys >= L are zero):
//   kt  [64][128]   without RoPE: the keys as given (bf16); with RoPE: the
//                   keys rotated by 3D RoPE over the (frame, height, width)
//                   token grid (Wan2.1 reading notes, 2. Model Design), in
//                   fp32, scaled by 2^-e_t and rounded to fp16, where e_t
//                   puts the tile's largest |element| in [2^14, 2^15);
//   kexp[t]         e_t (with RoPE);
//   vt  [128][64]   V transposed (bf16): row d holds v_k[d] at position
//                   pos(k), pos = k with bits 2 and 3 swapped (the key order
//                   of the PV product's register fragments).
#include "common.h"
#include "kernels.h"

namespace wanattn {

namespace {

template <bool F16>
__global__ __launch_bounds__(256) void kv_tiles_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                       uint16_t* __restrict__ kt, int* __restrict__ kexp,
                                                       uint16_t* __restrict__ vt, int L, int H, int nt,
                                                       RopeDev rope) {
  __shared__ __attribute__((aligned(16))) uint16_t s[TILE_ROWS][HD + 8];
  __shared__ float wmax[4];
  const int tile = blockIdx.x % nt;
  const int bh = blockIdx.x / nt;
  const int h = bh % H;
  const int b = bh / H;
  const int tid = threadIdx.x;
  const int64_t tile_elems = (int64_t)blockIdx.x * TILE_ELEMS;
  float r[4][8];      // keys of this thread's 4 chunks (rotated with F16)
  float mk = 0.f;
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
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      r[it][2 * t] = bf16_lo(kx[t]);
      r[it][2 * t + 1] = bf16_hi(kx[t]);
    }
    if (F16 && gk < L) {
      const TokenPos pos = token_pos(rope, gk);
#pragma unroll
      for (int t = 0; t < 4; ++t) rope_rotate(r[it][2 * t], r[it][2 * t + 1], rope_cs(rope, pos, 4 * ch + t), false);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) mk = fmaxf(mk, fabsf(r[it][e]));
    *reinterpret_cast<u32x4*>(&s[key][ch * 8]) = vx;
  }
  int et = 0;
  if (F16) {
    // tile max |k~| -> e_t
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mk = fmaxf(mk, __shfl_xor(mk, o));
    if ((tid & 63) == 0) wmax[tid >> 6] = mk;
  }
  __syncthreads();
  if (F16) {
    et = pow2_exponent_15(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])));
    if (tid == 0) kexp[blockIdx.x] = et;
  }
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int c = tid + 256 * it;
    const int key = c >> 4;
    const int ch = c & 15;
    u32x4 ko;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      ko[t] = F16 ? pack_f16(ldexpf(r[it][2 * t], -et), ldexpf(r[it][2 * t + 1], -et))
                  : pack_bf16(r[it][2 * t], r[it][2 * t + 1]);
    *reinterpret_cast<u32x4*>(kt + tile_elems + key * HD + ch * 8) = ko;
  }
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

hipError_t launch_kv_tiles(const uint16_t* k, const uint16_t* v, uint16_t* kt, int* kexp, uint16_t* vt, int B, int L,
                           int H, const RopeDev& rope, hipStream_t stream) {
  const int nt = (L + TILE_ROWS - 1) / TILE_ROWS;
  const int64_t total = (int64_t)B * H * nt;
  if (total <= 0 || total > 0x7fffffff) return hipErrorInvalidValue;
  const bool f16 = rope.table != nullptr;
  if (f16 != (kexp != nullptr)) return hipErrorInvalidValue;
  if (f16)
    hipLaunchKernelGGL(kv_tiles_kernel<true>, dim3((unsigned)total), dim3(256), 0, stream, k, v, kt, kexp, vt, L, H, nt,
                       rope);
  else
    hipLaunchKernelGGL(kv_tiles_kernel<false>, dim3((unsigned)total), dim3(256), 0, stream, k, v, kt, kexp, vt, L, H,
                       nt, rope);
  return hipGetLastError();
}

}  // namespace wanattn
