// Tile preparation passes.  The attention kernels stage 64-token tiles of
// one (b, h) with contiguous copies and read every MFMA operand with plain
// 16-byte LDS reads; these passes write the operands in that form, once:
//
//   row tile  [64][128]  token-major, as the [B, L, H, 128] input row order;
//   T tile    [128][64]  transposed: row d holds x_n[d] of the tile's tokens n
//                        at position pos(n), pos = n with bits 2 and 3
//                        swapped (the k order of the MFMA register fragments
//                        that feed the products contracting over tokens);
//   fp16 tile            a row tile of R(p) x * 2^-e, e chosen per tile so
//                        that the largest |R(p) x| lies in [2^14, 2^15), and
//                        the exponent e beside it.  R is the 3D RoPE over the
//                        (frame, height, width) token grid (Wan2.1 reading
//                        notes, 2. Model Design), or the identity.
// Tokens >= L are zero in every tile.
//
// Forward (kv_tiles_kernel): K as an fp16 tile with its exponent (with RoPE)
// or a bf16 row tile (without), V as a T tile.
// Backward (bwd_k_tiles_kernel, bwd_q_tiles_kernel): the fp16 tiles of K and
// Q with their exponents (bit-identical to what the forward multiplies, so
// the recomputed scores match the forward's LSE), T tiles of R(p)k, R(p)q
// and dO, row tiles of V and dO, and per query tile the row statistics
// LSE_i * log2(e) and -Delta_i, Delta_i = <dO_i, O_i>.
#include "common.h"
#include "kernels.h"

namespace wanattn {

namespace {

// Thread t (of 256) holds tile tokens n = t/16 + 16*it at 8-element chunk
// c = t%16, it = 0..3: each 16-lane group reads one 256-byte row.
struct TileFrag {
  float x[4][8];
};

__device__ __forceinline__ int frag_token(int tid, int it) { return (tid >> 4) + 16 * it; }
__device__ __forceinline__ int frag_chunk(int tid) { return tid & 15; }

// Tokens [64*tile, +64) of head (b, h) of a [B, L, H, 128] bf16 tensor as raw
// bf16 pairs (16 bytes per thread and row).  Tokens at or past `valid` (<= L)
// are zero.  The loads are only issued here: a kernel issues all of its loads
// before it uses any of them, so their latencies overlap.
struct TileRaw {
  u32x4 v[4];
};
__device__ __forceinline__ void load_raw(TileRaw& r, const uint16_t* __restrict__ x, int b, int h, int tile, int L,
                                         int H, int tid, int valid) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int n = tile * TILE_ROWS + frag_token(tid, it);
    r.v[it] = u32x4{0u, 0u, 0u, 0u};
    if (n < valid) r.v[it] = *reinterpret_cast<const u32x4*>(x + (((int64_t)b * L + n) * H + h) * HD + frag_chunk(tid) * 8);
  }
}

// The raw tile in fp32, optionally rotated; returns this thread's max |x|.
// `pos0` is the RoPE token index of row 0.
__device__ __forceinline__ float convert_tile(TileFrag& f, const TileRaw& r, int tile, const RopeDev& rope, bool rotate,
                                              int tid, int valid, int pos0) {
  float m = 0.f;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int n = tile * TILE_ROWS + frag_token(tid, it);
    const int ch = frag_chunk(tid);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f.x[it][2 * t] = bf16_lo(r.v[it][t]);
      f.x[it][2 * t + 1] = bf16_hi(r.v[it][t]);
    }
    if (rotate && n < valid) {
      const TokenPos pos = token_pos(rope, pos0 + n);
#pragma unroll
      for (int t = 0; t < 4; ++t) rope_rotate(f.x[it][2 * t], f.x[it][2 * t + 1], rope_cs(rope, pos, 4 * ch + t), false);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(f.x[it][e]));
  }
  return m;
}

// Max over the 256 threads (every thread gets it).  Ends with a barrier that
// orders LDS only: the global stores already issued stay in flight.
__device__ __forceinline__ float block_max(float m, float* wmax, int tid) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  lds_barrier();
  return fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
}

__device__ __forceinline__ void store_row_tile_f16(uint16_t* __restrict__ tile, const TileFrag& f, int e, int tid) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    u32x4 w;
#pragma unroll
    for (int t = 0; t < 4; ++t) w[t] = pack_f16(ldexpf(f.x[it][2 * t], -e), ldexpf(f.x[it][2 * t + 1], -e));
    *reinterpret_cast<u32x4*>(tile + frag_token(tid, it) * HD + frag_chunk(tid) * 8) = w;
  }
}

__device__ __forceinline__ void store_row_tile_bf16(uint16_t* __restrict__ tile, const TileFrag& f, int tid) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    u32x4 w;
#pragma unroll
    for (int t = 0; t < 4; ++t) w[t] = pack_bf16(f.x[it][2 * t], f.x[it][2 * t + 1]);
    *reinterpret_cast<u32x4*>(tile + frag_token(tid, it) * HD + frag_chunk(tid) * 8) = w;
  }
}

typedef uint16_t StageRows[TILE_ROWS][HD + 8];   // padded: column reads spread over banks

// bf16 of the fragment into the LDS staging rows (no barrier).
__device__ __forceinline__ void stage_bf16(StageRows& s, const TileFrag& f, int tid) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    u32x4 w;
#pragma unroll
    for (int t = 0; t < 4; ++t) w[t] = pack_bf16(f.x[it][2 * t], f.x[it][2 * t + 1]);
    *reinterpret_cast<u32x4*>(&s[frag_token(tid, it)][frag_chunk(tid) * 8]) = w;
  }
}

// T tile from the staged rows (call after a barrier).
__device__ __forceinline__ void store_t_tile(uint16_t* __restrict__ tile, const StageRows& s, int tid) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int c = tid + 256 * it;   // 128 d rows x 8 chunks of 8 positions
    const int d = c >> 3;
    const int pc = c & 7;
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p0 = 8 * pc + 2 * e;
      const int n0 = (p0 & ~12) | ((p0 & 4) << 1) | ((p0 & 8) >> 1);   // bit 0 untouched: n0 + 1 is p0 + 1
      w[e] = (uint32_t)s[n0][d] | ((uint32_t)s[n0 + 1][d] << 16);
    }
    *reinterpret_cast<u32x4*>(tile + d * 64 + pc * 8) = w;
  }
}

// Forward: K (fp16 tile + exponent with RoPE, bf16 row tile without) and V^T.
template <bool F16>
__global__ __launch_bounds__(256) void kv_tiles_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                       uint16_t* __restrict__ kt, int* __restrict__ kexp,
                                                       uint16_t* __restrict__ vt, int L, int H, int nt,
                                                       RopeDev rope, const int32_t* __restrict__ lens, int pos0) {
  __shared__ __attribute__((aligned(16))) StageRows s;
  __shared__ float wmax[4];
  const int tile = blockIdx.x % nt;
  const int bh = blockIdx.x / nt;
  const int h = bh % H;
  const int b = bh / H;
  const int tid = threadIdx.x;
  const int64_t off = (int64_t)blockIdx.x * TILE_ELEMS;
  const int valid = lens != nullptr ? min(max(lens[b], 0), L) : L;
  TileRaw rk, rv;
  load_raw(rk, k, b, h, tile, L, H, tid, valid);
  load_raw(rv, v, b, h, tile, L, H, tid, valid);
  TileFrag f;
  const float mk = convert_tile(f, rk, tile, rope, F16, tid, valid, pos0);
  if (F16) {
    const int e = pow2_exponent_15(block_max(mk, wmax, tid));
    if (tid == 0) kexp[blockIdx.x] = e;
    store_row_tile_f16(kt + off, f, e, tid);
  } else {
    store_row_tile_bf16(kt + off, f, tid);
  }
  convert_tile(f, rv, tile, rope, false, tid, valid, 0);
  stage_bf16(s, f, tid);
  lds_barrier();
  store_t_tile(vt + off, s, tid);
}

// Backward, key side: K fp16 tile + exponent (as the forward's), (R k)^T, V rows.
__global__ __launch_bounds__(256) void bwd_k_tiles_kernel(const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v, uint16_t* __restrict__ kf,
                                                          int* __restrict__ kexp, uint16_t* __restrict__ kt,
                                                          uint16_t* __restrict__ vr, int L, int H, int nt,
                                                          RopeDev rope, const int32_t* __restrict__ lens) {
  __shared__ __attribute__((aligned(16))) StageRows s;
  __shared__ float wmax[4];
  const int tile = blockIdx.x % nt;
  const int bh = blockIdx.x / nt;
  const int h = bh % H;
  const int b = bh / H;
  const int tid = threadIdx.x;
  const int64_t off = (int64_t)blockIdx.x * TILE_ELEMS;
  const int valid = lens != nullptr ? min(max(lens[b], 0), L) : L;
  TileRaw rk, rv;
  load_raw(rk, k, b, h, tile, L, H, tid, valid);
  load_raw(rv, v, b, h, tile, L, H, tid, valid);
  TileFrag f;
  const float mk = convert_tile(f, rk, tile, rope, rope.table != nullptr, tid, valid, 0);
  const int e = pow2_exponent_15(block_max(mk, wmax, tid));
  if (tid == 0) kexp[blockIdx.x] = e;
  store_row_tile_f16(kf + off, f, e, tid);
  stage_bf16(s, f, tid);
  lds_barrier();
  store_t_tile(kt + off, s, tid);
  convert_tile(f, rv, tile, rope, false, tid, valid, 0);
  store_row_tile_bf16(vr + off, f, tid);
}

// Backward, query side: Q fp16 tile + exponent, (R q)^T, dO rows, dO^T, and the tile's row
// statistics: LSE * log2(e) (+inf for a row past L or without a valid key: P = 0) and -Delta
// (0 past L) in the order the backward's accumulators hold their rows, then the tile's exponent.
// Entry x = 16 hf + j (x < 32) holds rows r and 32 + r, r = 8 (j / 4) + 4 hf + j % 4: the row of
// register j of a 32x32 accumulator block in lane half hf, as {LSE log2 e (r), -Delta (r),
// LSE log2 e (32 + r), -Delta (32 + r)}.
__global__ __launch_bounds__(256) void bwd_q_tiles_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ dout,
                                                          const uint16_t* __restrict__ o,
                                                          const float* __restrict__ lse, uint16_t* __restrict__ qf,
                                                          int* __restrict__ qexp, uint16_t* __restrict__ qt,
                                                          uint16_t* __restrict__ dor, uint16_t* __restrict__ dot,
                                                          float* __restrict__ qstat, int L, int H, int nt,
                                                          RopeDev rope) {
  __shared__ __attribute__((aligned(16))) StageRows s;
  __shared__ float wmax[4];
  __shared__ float ndelta_s[TILE_ROWS];
  const int tile = blockIdx.x % nt;
  const int bh = blockIdx.x / nt;
  const int h = bh % H;
  const int b = bh / H;
  const int tid = threadIdx.x;
  const int64_t off = (int64_t)blockIdx.x * TILE_ELEMS;
  TileRaw rq, rd, ro;
  load_raw(rq, q, b, h, tile, L, H, tid, L);
  load_raw(rd, dout, b, h, tile, L, H, tid, L);
  load_raw(ro, o, b, h, tile, L, H, tid, L);
  TileFrag f;
  const float mq = convert_tile(f, rq, tile, rope, rope.table != nullptr, tid, L, 0);
  const int e = pow2_exponent_15(block_max(mq, wmax, tid));
  if (tid == 0) qexp[blockIdx.x] = e;
  store_row_tile_f16(qf + off, f, e, tid);
  stage_bf16(s, f, tid);
  lds_barrier();
  store_t_tile(qt + off, s, tid);
  lds_barrier();   // the staging rows are reused below

  // dO: row tile, T tile, and Delta = <dO, O> per token (16 lanes per row).
  convert_tile(f, rd, tile, rope, false, tid, L, 0);
  store_row_tile_bf16(dor + off, f, tid);
  stage_bf16(s, f, tid);
  TileFrag g;
  convert_tile(g, ro, tile, rope, false, tid, L, 0);
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    float d = 0.f;
#pragma unroll
    for (int e2 = 0; e2 < 8; ++e2) d = fmaf(f.x[it][e2], g.x[it][e2], d);
    d += __shfl_xor(d, 8, 16);
    d += __shfl_xor(d, 4, 16);
    d += __shfl_xor(d, 2, 16);
    d += __shfl_xor(d, 1, 16);
    const int n = tile * TILE_ROWS + frag_token(tid, it);
    if (frag_chunk(tid) == 0) ndelta_s[frag_token(tid, it)] = (n < L) ? -d : 0.f;
  }
  lds_barrier();
  store_t_tile(dot + off, s, tid);
  // The tile's statistics by row: LSE_i log2 e in floats [0, 64), -Delta_i in
  // [64, 128), the exponent at 128 (four consecutive rows of one statistic
  // are one 16-byte read).
  float* st = qstat + (int64_t)blockIdx.x * QSTAT_FLOATS;
  if (tid < TILE_ROWS) {
    const int n = tile * TILE_ROWS + tid;
    const float x = (n < L) ? lse[((int64_t)b * H + h) * L + n] : -INFINITY;
    st[tid] = (x > -INFINITY) ? x * 1.4426950408889634f : INFINITY;
  } else if (tid < 2 * TILE_ROWS) {
    st[tid] = ndelta_s[tid - TILE_ROWS];
  } else {
    st[tid] = (tid == 2 * TILE_ROWS) ? __int_as_float(e) : 0.f;
  }
}

hipError_t grid_of_tiles(int B, int L, int H, int& nt, dim3& grid) {
  nt = (L + TILE_ROWS - 1) / TILE_ROWS;
  const int64_t total = (int64_t)B * H * nt;
  if (total <= 0 || total > 0x7fffffff) return hipErrorInvalidValue;
  grid = dim3((unsigned)total);
  return hipSuccess;
}

}  // namespace

hipError_t launch_kv_tiles(const uint16_t* k, const uint16_t* v, uint16_t* kt, int* kexp, uint16_t* vt, int B, int L,
                           int H, const RopeDev& rope, const int32_t* lens, int pos0, hipStream_t stream) {
  int nt;
  dim3 grid;
  if (grid_of_tiles(B, L, H, nt, grid) != hipSuccess) return hipErrorInvalidValue;
  const bool f16 = rope.table != nullptr;
  if (f16 != (kexp != nullptr)) return hipErrorInvalidValue;
  if (f16)
    hipLaunchKernelGGL(kv_tiles_kernel<true>, grid, dim3(256), 0, stream, k, v, kt, kexp, vt, L, H, nt, rope, lens,
                       pos0);
  else
    hipLaunchKernelGGL(kv_tiles_kernel<false>, grid, dim3(256), 0, stream, k, v, kt, kexp, vt, L, H, nt, rope, lens,
                       pos0);
  return hipGetLastError();
}

hipError_t launch_bwd_k_tiles(const uint16_t* k, const uint16_t* v, uint16_t* kf, int* kexp, uint16_t* kt,
                              uint16_t* vr, int B, int L, int H, const RopeDev& rope, const int32_t* lens,
                              hipStream_t stream) {
  int nt;
  dim3 grid;
  if (grid_of_tiles(B, L, H, nt, grid) != hipSuccess) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_k_tiles_kernel, grid, dim3(256), 0, stream, k, v, kf, kexp, kt, vr, L, H, nt, rope, lens);
  return hipGetLastError();
}

hipError_t launch_bwd_q_tiles(const uint16_t* q, const uint16_t* dout, const uint16_t* o, const float* lse,
                              uint16_t* qf, int* qexp, uint16_t* qt, uint16_t* dor, uint16_t* dot, float* qstat, int B,
                              int L, int H, const RopeDev& rope, hipStream_t stream) {
  int nt;
  dim3 grid;
  if (grid_of_tiles(B, L, H, nt, grid) != hipSuccess) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_q_tiles_kernel, grid, dim3(256), 0, stream, q, dout, o, lse, qf, qexp, qt, dor, dot, qstat, L,
                     H, nt, rope);
  return hipGetLastError();
}

}  // namespace wanattn
