// Self-attention backward for gfx950, as two deterministic passes plus a
// row-statistics pre-pass.  The formulas are the calculus of the forward
// (full spatio-temporal attention with 3D RoPE; "Wan Team, Alibaba (2025)",
// Key takeaways, Backbone; training in bf16 per the Wan2.1 reading notes,
// 3. Training):
//   Delta_i = <dO_i, O_i>
//   P_ij    = exp(scale <q~_i, k~_j> - LSE_i)           (recomputed, never stored)
//   dV_j    = sum_i P_ij dO_i
//   dS_ij   = P_ij (<dO_i, v_j> - Delta_i)
//   dq~_i   = scale sum_j dS_ij k~_j,   dk~_j = scale sum_i dS_ij q~_i
//   dq_i    = R(p_i)^T dq~_i,           dk_j  = R(p_j)^T dk~_j
// q~ and k~ arrive pre-rotated (q~ as a bf16 hi + lo pair, exactly as the
// forward used it, so the recomputed P matches the forward's LSE); the inverse
// rotation is fused into the dQ and dK stores.  Tiles move global -> LDS by
// direct loads (global_load_lds), double-buffered.
//
//  * bwd_delta: Delta per row (memory-bound).
//  * bwd_dkdv:  workgroup = 128 keys (4 waves x 32), loop over 64-query tiles.
//               S = Q~ K~^T and dP = dO V^T with the wave's K~/V rows held in
//               registers as MFMA B operands (lane owns key column j);
//               dV^T += dO^T P and dK~^T += Q~^T dS read Q~/dO through the LDS
//               transpose read and take P/dS from the accumulators.
//  * bwd_dq:    workgroup = 128 queries, loop over 64-key tiles; S^T = K~ Q~^T,
//               dP^T = V dO^T (lane owns query row i), dQ~^T += K~^T dS^T.
#include "common.h"
#include "kernels.h"

namespace wanattn {

namespace {

constexpr float LOG2E = 1.4426950408889634f;

// Delta_i = <dO_i, O_i>; 16 lanes per row (one 16-byte chunk each).
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdParams p) {
  const int64_t rows = (int64_t)p.B * p.L * p.H;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t tix = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; tix < rows * 16; tix += stride) {
    const int64_t row = tix >> 4;
    const int c = (int)(tix & 15);
    const u32x4 a = *reinterpret_cast<const u32x4*>(p.dout + row * HD + c * 8);
    const u32x4 o = *reinterpret_cast<const u32x4*>(p.o + row * HD + c * 8);
    float s = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      s = fmaf(bf16_lo(a[t]), bf16_lo(o[t]), s);
      s = fmaf(bf16_hi(a[t]), bf16_hi(o[t]), s);
    }
    s += __shfl_xor(s, 8, 16);
    s += __shfl_xor(s, 4, 16);
    s += __shfl_xor(s, 2, 16);
    s += __shfl_xor(s, 1, 16);
    if (c == 0) {
      const int h = (int)(row % p.H);
      const int64_t bn = row / p.H;
      const int n = (int)(bn % p.L);
      const int b = (int)(bn / p.L);
      p.delta[((int64_t)b * p.H + h) * p.L + n] = s;
    }
  }
}

// Store 4 consecutive head-dim elements [d0, d0+4) of token n (two rotary
// pairs), optionally rotated back by minus the angle, as bf16.
__device__ __forceinline__ void store_grad4(uint16_t* row_ptr, const RopeDev& rope, const TokenPos& pos, int d0,
                                            float g0, float g1, float g2, float g3) {
  if (rope.table != nullptr) {
    rope_rotate(g0, g1, rope_cs(rope, pos, d0 / 2), true);
    rope_rotate(g2, g3, rope_cs(rope, pos, d0 / 2 + 1), true);
  }
  u32x2 w;
  w[0] = pack_bf16(g0, g1);
  w[1] = pack_bf16(g2, g3);
  *reinterpret_cast<u32x2*>(row_ptr + d0) = w;
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup owns 128 keys; loop over query tiles of 64.
// SPLIT: rotated queries come as bf16 hi + lo; S takes both (as the forward did).
// ---------------------------------------------------------------------------
template <bool SPLIT>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdParams p) {
  constexpr int NT = SPLIT ? 3 : 2;                                           // Q~ hi, [Q~ lo], dO
  __shared__ __attribute__((aligned(16))) uint16_t tiles[2][NT][TILE_ELEMS];
  __shared__ float lse2_s[2][TILE_ROWS];                                      // LSE * log2 e (+inf: no row)
  __shared__ float delta_s[2][TILE_ROWS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int kt = logical % p.n_tiles;
  const int bh = logical / p.n_tiles;
  const int h = bh % p.H;
  const int b = bh / p.H;

  const int64_t rs = (int64_t)p.H * HD;
  const int64_t head_off = ((int64_t)b * p.L * p.H + h) * HD;
  const uint16_t* qbase = p.q + head_off;
  const uint16_t* qlbase = SPLIT ? p.q_lo + head_off : nullptr;
  const uint16_t* dobase = p.dout + head_off;
  const float* lse_row = p.lse + ((int64_t)b * p.H + h) * p.L;
  const float* delta_row = p.delta + ((int64_t)b * p.H + h) * p.L;

  // This lane's key row j as B-operand fragments of K~ and V.
  const int j = kt * 128 + wave * 32 + col;
  const bool key_ok = j < p.L;
  bf16x8 kf[8], vf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    u32x4 xk = u32x4{0u, 0u, 0u, 0u}, xv = u32x4{0u, 0u, 0u, 0u};
    if (key_ok) {
      xk = *reinterpret_cast<const u32x4*>(p.k + head_off + (int64_t)j * rs + (2 * s + half) * 8);
      xv = *reinterpret_cast<const u32x4*>(p.v + head_off + (int64_t)j * rs + (2 * s + half) * 8);
    }
    kf[s] = __builtin_bit_cast(bf16x8, xk);
    vf[s] = __builtin_bit_cast(bf16x8, xv);
  }

  f32x16 dk_acc[4], dv_acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    dk_acc[d] = f32x16{};
    dv_acc[d] = f32x16{};
  }
  const float c2 = p.scale_log2;
  const int n_qt = (p.L + TILE_ROWS - 1) / TILE_ROWS;

  auto stage = [&](int buf, int row0) {
    tile_dma(tiles[buf][0], qbase, rs, row0, p.L, wv, lane);
    if (SPLIT) tile_dma(tiles[buf][1], qlbase, rs, row0, p.L, wv, lane);
    tile_dma(tiles[buf][NT - 1], dobase, rs, row0, p.L, wv, lane);
    if (tid < TILE_ROWS) {
      const int i = row0 + tid;
      lse2_s[buf][tid] = (i < p.L) ? lse_row[i] * LOG2E : INFINITY;
    } else if (tid < 2 * TILE_ROWS) {
      const int i = row0 + tid - TILE_ROWS;
      delta_s[buf][tid - TILE_ROWS] = (i < p.L) ? delta_row[i] : 0.f;
    }
  };

  stage(0, 0);
  wait_vmem();
  __syncthreads();

  for (int t = 0; t < n_qt; ++t) {
    const int buf = t & 1;
    const bool has_next = t + 1 < n_qt;
    if (has_next) stage(buf ^ 1, (t + 1) * TILE_ROWS);
    const uint16_t* qs = tiles[buf][0];
    const uint16_t* qls = tiles[buf][SPLIT ? 1 : 0];
    const uint16_t* ds_ = tiles[buf][NT - 1];

    bf16x8 pf[4], dsf[4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 s_acc = f32x16{}, dp_acc = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        s_acc = mfma32(lds_row_frag(qs, qb * 32 + col, 2 * s + half), kf[s], s_acc);
        if (SPLIT) s_acc = mfma32(lds_row_frag(qls, qb * 32 + col, 2 * s + half), kf[s], s_acc);
        dp_acc = mfma32(lds_row_frag(ds_, qb * 32 + col, 2 * s + half), vf[s], dp_acc);
      }
      float pv[16], dsv[16];
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int r = qb * 32 + 8 * (jj >> 2) + 4 * half + (jj & 3);   // query row in the tile
        const float pe = __builtin_amdgcn_exp2f(fmaf(s_acc[jj], c2, -lse2_s[buf][r]));
        pv[jj] = pe;
        dsv[jj] = pe * (dp_acc[jj] - delta_s[buf][r]);
      }
      pf[2 * qb] = pack_acc8(pv);
      pf[2 * qb + 1] = pack_acc8(pv + 8);
      dsf[2 * qb] = pack_acc8(dsv);
      dsf[2 * qb + 1] = pack_acc8(dsv + 8);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int qg = 0; qg < 4; ++qg) {
        dv_acc[d] = mfma32(lds_col_frag(ds_, qg * 16, d * 32, lane), pf[qg], dv_acc[d]);
        dk_acc[d] = mfma32(lds_col_frag(qs, qg * 16, d * 32, lane), dsf[qg], dk_acc[d]);
      }
    }

    if (has_next) wait_vmem();
    __syncthreads();
  }

  if (key_ok) {
    TokenPos pos{0, 0, 0};
    if (p.rope.table != nullptr) pos = token_pos(p.rope, j);
    uint16_t* dkrow = p.dk + head_off + (int64_t)j * rs;
    uint16_t* dvrow = p.dv + head_off + (int64_t)j * rs;
    RopeDev none = p.rope;
    none.table = nullptr;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int d0 = d * 32 + 8 * jq + 4 * half;
        store_grad4(dkrow, p.rope, pos, d0, dk_acc[d][4 * jq] * p.scale, dk_acc[d][4 * jq + 1] * p.scale,
                    dk_acc[d][4 * jq + 2] * p.scale, dk_acc[d][4 * jq + 3] * p.scale);
        store_grad4(dvrow, none, pos, d0, dv_acc[d][4 * jq], dv_acc[d][4 * jq + 1], dv_acc[d][4 * jq + 2],
                    dv_acc[d][4 * jq + 3]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: workgroup owns 128 queries; loop over key tiles of 64.
// ---------------------------------------------------------------------------
template <bool SPLIT>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t tiles[2][2][TILE_ELEMS];   // [buffer][K~ | V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = logical % p.n_tiles;
  const int bh = logical / p.n_tiles;
  const int h = bh % p.H;
  const int b = bh / p.H;

  const int64_t rs = (int64_t)p.H * HD;
  const int64_t head_off = ((int64_t)b * p.L * p.H + h) * HD;
  const uint16_t* kbase = p.k + head_off;
  const uint16_t* vbase = p.v + head_off;

  const int i = qt * 128 + wave * 32 + col;
  const bool row_ok = i < p.L;
  bf16x8 qf[8], dof[8];
  bf16x8 ql[SPLIT ? 8 : 1];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    u32x4 xq = u32x4{0u, 0u, 0u, 0u}, xd = u32x4{0u, 0u, 0u, 0u}, xl = u32x4{0u, 0u, 0u, 0u};
    if (row_ok) {
      const int64_t off = head_off + (int64_t)i * rs + (2 * s + half) * 8;
      xq = *reinterpret_cast<const u32x4*>(p.q + off);
      xd = *reinterpret_cast<const u32x4*>(p.dout + off);
      if (SPLIT) xl = *reinterpret_cast<const u32x4*>(p.q_lo + off);
    }
    qf[s] = __builtin_bit_cast(bf16x8, xq);
    dof[s] = __builtin_bit_cast(bf16x8, xd);
    if (SPLIT) ql[s] = __builtin_bit_cast(bf16x8, xl);
  }
  const int64_t stat = ((int64_t)b * p.H + h) * p.L + i;
  const float lse2 = row_ok ? p.lse[stat] * LOG2E : INFINITY;
  const float delta = row_ok ? p.delta[stat] : 0.f;
  const float c2 = p.scale_log2;

  f32x16 dq_acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) dq_acc[d] = f32x16{};
  const int n_kt = (p.L + TILE_ROWS - 1) / TILE_ROWS;

  tile_dma(tiles[0][0], kbase, rs, 0, p.L, wv, lane);
  tile_dma(tiles[0][1], vbase, rs, 0, p.L, wv, lane);
  wait_vmem();
  __syncthreads();

  for (int t = 0; t < n_kt; ++t) {
    const int buf = t & 1;
    const bool has_next = t + 1 < n_kt;
    if (has_next) {
      tile_dma(tiles[buf ^ 1][0], kbase, rs, (t + 1) * TILE_ROWS, p.L, wv, lane);
      tile_dma(tiles[buf ^ 1][1], vbase, rs, (t + 1) * TILE_ROWS, p.L, wv, lane);
    }
    const uint16_t* ks = tiles[buf][0];
    const uint16_t* vs = tiles[buf][1];
    const int key0 = t * TILE_ROWS;
    const bool partial = key0 + TILE_ROWS > p.L;

    bf16x8 dsf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s_acc = f32x16{}, dp_acc = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 a = lds_row_frag(ks, kb * 32 + col, 2 * s + half);
        s_acc = mfma32(a, qf[s], s_acc);
        if (SPLIT) s_acc = mfma32(a, ql[s], s_acc);
        dp_acc = mfma32(lds_row_frag(vs, kb * 32 + col, 2 * s + half), dof[s], dp_acc);
      }
      float dsv[16];
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        float pe = __builtin_amdgcn_exp2f(fmaf(s_acc[jj], c2, -lse2));
        if (partial) {
          const int key = key0 + kb * 32 + 8 * (jj >> 2) + 4 * half + (jj & 3);
          if (key >= p.L) pe = 0.f;
        }
        dsv[jj] = pe * (dp_acc[jj] - delta);
      }
      dsf[2 * kb] = pack_acc8(dsv);
      dsf[2 * kb + 1] = pack_acc8(dsv + 8);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int kg = 0; kg < 4; ++kg) {
        dq_acc[d] = mfma32(lds_col_frag(ks, kg * 16, d * 32, lane), dsf[kg], dq_acc[d]);
      }
    }

    if (has_next) wait_vmem();
    __syncthreads();
  }

  if (row_ok) {
    TokenPos pos{0, 0, 0};
    if (p.rope.table != nullptr) pos = token_pos(p.rope, i);
    uint16_t* dqrow = p.dq + head_off + (int64_t)i * rs;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        store_grad4(dqrow, p.rope, pos, d * 32 + 8 * jq + 4 * half, dq_acc[d][4 * jq] * p.scale,
                    dq_acc[d][4 * jq + 1] * p.scale, dq_acc[d][4 * jq + 2] * p.scale,
                    dq_acc[d][4 * jq + 3] * p.scale);
      }
    }
  }
}

}  // namespace

hipError_t launch_bwd_delta(const BwdParams& p, hipStream_t stream) {
  const int64_t threads = (int64_t)p.B * p.L * p.H * 16;
  int64_t blocks = (threads + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdParams& p, hipStream_t stream) {
  BwdParams q = p;
  q.n_tiles = (p.L + 127) / 128;
  const int64_t total = (int64_t)q.n_tiles * p.H * p.B;
  if (total <= 0 || total > 0x7fffffff) return hipErrorInvalidValue;
  if (p.q_lo != nullptr) hipLaunchKernelGGL(bwd_dkdv_kernel<true>, dim3((unsigned)total), dim3(256), 0, stream, q);
  else hipLaunchKernelGGL(bwd_dkdv_kernel<false>, dim3((unsigned)total), dim3(256), 0, stream, q);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdParams& p, hipStream_t stream) {
  BwdParams q = p;
  q.n_tiles = (p.L + 127) / 128;
  const int64_t total = (int64_t)q.n_tiles * p.H * p.B;
  if (total <= 0 || total > 0x7fffffff) return hipErrorInvalidValue;
  if (p.q_lo != nullptr) hipLaunchKernelGGL(bwd_dq_kernel<true>, dim3((unsigned)total), dim3(256), 0, stream, q);
  else hipLaunchKernelGGL(bwd_dq_kernel<false>, dim3((unsigned)total), dim3(256), 0, stream, q);
  return hipGetLastError();
}

}  // namespace wanattn
