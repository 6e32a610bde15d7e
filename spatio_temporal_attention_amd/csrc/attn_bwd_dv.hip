// Backward dV pass for gfx950 (the formulas and the tile layouts are those of
// attn_bwd.hip, whose other passes share bwd_common.h).  Its own file so that
// it can be built with the iterative ILP machine scheduler: with it the
// compiler keeps more fragment reads in flight here (720p: 100.5 -> 94.4 ms),
// while the register-bound dK and dQ passes spill or slow down under it.
#include <algorithm>
#include <type_traits>

#include "bwd_common.h"

namespace wanattn {

namespace {

using namespace bwd;

// dV_j = sum_i P_ij dO_i.  Workgroup = 256 keys (8 waves, one workgroup per
// CU: each query tile crosses from L2 once per CU, not once per 128 keys);
// query tiles staged as Q fp16 rows and dO^T.  S = Q K^T from the
// wave's K rows in registers, dV^T += dO^T P with P from the accumulators.
template <bool KMASK, bool TAIL>
__global__ __launch_bounds__(64 * DV_WAVES, 1) void bwd_dv_kernel(BwdParams p) {
  // Double-buffered tiles as separate objects, named statically in the
  // two-way unrolled loop (LDS reads do not wait for copies in flight).
  __shared__ __attribute__((aligned(16))) uint16_t q_lds0[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t q_lds1[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t dot_lds0[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t dot_lds1[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) float lse2_s0[TILE_ROWS];   // LSE * log2 e (+inf: no row)
  __shared__ __attribute__((aligned(16))) float lse2_s1[TILE_ROWS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const KeySide ks = key_side<DV_WAVES, KMASK, TAIL>(p, wv, col);

  bf16x8 kf[8];   // K fp16 (bit patterns): B operand of S
  load_row_frags(kf, p.kf + (ks.ktile0 + (ks.tile_ok ? ks.ktile : 0)) * TILE_ELEMS, 32 * (wave & 1) + col, half,
                 ks.tile_ok);
  const int e_k = ks.tile_ok ? p.kexp[ks.ktile0 + ks.ktile] : 0;

  f32x16 dv_acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) dv_acc[d] = f32x16{};
  const float* lse_row = p.lse + ((int64_t)ks.b * p.H + ks.h) * p.Lq;

  constexpr int NCP = 16 / DV_WAVES;   // 1 KB copies per wave and tile
  uint32_t roff[NCP], toff[NCP];
#pragma unroll
  for (int i = 0; i < NCP; ++i) {
    roff[i] = rowtile_lane_off<DV_WAVES>(wv, i, lane);
    toff[i] = ttile_lane_off<DV_WAVES>(wv, i, lane);
  }
  const uint32_t bytes = (uint32_t)ks.nt * (TILE_ELEMS * 2);   // < 2^32, checked by the launcher
  const __amdgpu_buffer_rsrc_t qfr = tile_rsrc(p.qf + ks.tile0 * TILE_ELEMS, bytes);
  const __amdgpu_buffer_rsrc_t dotr = tile_rsrc(p.dot + ks.tile0 * TILE_ELEMS, bytes);
  const_i32* qexp = const_ptr(p.qexp + ks.tile0);   // scalar loads

  struct Buf {
    uint16_t* q;
    uint16_t* dOt;
    float* lse2;
  };
  const Buf buf0{q_lds0, dot_lds0, lse2_s0};
  const Buf buf1{q_lds1, dot_lds1, lse2_s1};
  auto stage = [&](const Buf& dst, int t) {
    const uint32_t soff = (uint32_t)t * (TILE_ELEMS * 2);
#pragma unroll
    for (int i = 0; i < NCP; ++i) {
      buf_dma16(qfr, roff[i], soff, tile_lds_block<DV_WAVES>(dst.q, wv, i));
      buf_dma16(dotr, toff[i], soff, tile_lds_block<DV_WAVES>(dst.dOt, wv, i));
    }
  };
  // LSE of query tile t: threads 0..63, into a register, published to LDS
  // once loaded (rows past Lq, and rows with no valid key, get +inf: P = 0).
  auto load_stats = [&](int t) {
    float x = -INFINITY;
    if (tid < TILE_ROWS) {
      const int i = t * TILE_ROWS + tid;
      if (i < p.Lq) x = lse_row[i];
    }
    return x;
  };
  auto store_stats = [&](const Buf& dst, float x) {
    if (tid < TILE_ROWS) dst.lse2[tid] = (x > -INFINITY) ? x * LOG2E : INFINITY;
  };

  // A query split can be empty (rounding of the split size): it writes zero partials.
  if (ks.t0 < ks.t1) {
    int e_q;
    {
      const float st = load_stats(ks.t0);
      stage(buf0, ks.t0);
      e_q = qexp[ks.t0];
      wait_vmem();
      store_stats(buf0, st);
    }
    __syncthreads();

    auto iteration = [&](auto parity, int t) {
      constexpr int P = decltype(parity)::value;
      const Buf& cur = P ? buf1 : buf0;
      const Buf& nxt = P ? buf0 : buf1;
      const bool has_next = t + 1 < ks.t1;
      int e_q_next = 0;
      float st = 0.f;
      if (has_next) {
        st = load_stats(t + 1);
        stage(nxt, t + 1);
        e_q_next = qexp[t + 1];
      }
      const float g = ldexpf(p.scale_log2, e_q + e_k);
      bf16x8 pf[4];
  #pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x16 s_acc = f32x16{};
  #pragma unroll
        for (int s = 0; s < 8; ++s) s_acc = mfma32_f16(lds_row_frag(cur.q, qb * 32 + col, 2 * s + half), kf[s], s_acc);
        float pv[16];
  #pragma unroll
        for (int m = 0; m < 4; ++m) {
          // rows qb*32 + 8m + 4*half + (0..3) of this tile: the accumulator's row order
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(cur.lse2 + qb * 32 + 8 * m + 4 * half);
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            float pe = __builtin_amdgcn_exp2f(fmaf(s_acc[4 * m + e], g, -l4[e]));
            if (KMASK && !ks.key_live) pe = 0.f;
            pv[4 * m + e] = pe;
          }
        }
        pf[2 * qb] = pack_acc8(pv);
        pf[2 * qb + 1] = pack_acc8(pv + 8);
      }
  #pragma unroll
      for (int d = 0; d < 4; ++d) {
  #pragma unroll
        for (int qg = 0; qg < 4; ++qg) dv_acc[d] = mfma32(lds_vt_frag(cur.dOt, d * 32 + col, qg, half), pf[qg], dv_acc[d]);
      }
      if (has_next) {
        wait_vmem();
        store_stats(nxt, st);
      }
      __syncthreads();
      e_q = e_q_next;
    };
    int t = ks.t0;
    for (; t + 1 < ks.t1; t += 2) {
      iteration(std::integral_constant<int, 0>{}, t);
      iteration(std::integral_constant<int, 1>{}, t + 1);
    }
    if (t < ks.t1) iteration(std::integral_constant<int, 0>{}, t);
  }

  if (TAIL) {
    // fp32 partial over this query range, rows of the workgroup's 256 keys, after the dK~ partials
    const int64_t region = (int64_t)gridDim.x * (32 * DV_WAVES) * HD;
    float* row = p.kv_part + region + ((int64_t)blockIdx.x * (32 * DV_WAVES) + wave * 32 + col) * HD;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int jq = 0; jq < 4; ++jq)
        *reinterpret_cast<f32x4*>(row + d * 32 + 8 * jq + 4 * half) =
            f32x4{dv_acc[d][4 * jq], dv_acc[d][4 * jq + 1], dv_acc[d][4 * jq + 2], dv_acc[d][4 * jq + 3]};
    }
  } else if (ks.key_ok && p.q_split > 1) {
    // fp32 partial over this split's query tiles, summed by bwd_kv_reduce_kernel
    const int64_t part = (int64_t)p.q_split * p.B * p.H * p.Lk * HD;   // dV follows dK~
    float* row = p.part + part + ((((int64_t)ks.split * p.B + ks.b) * p.H + ks.h) * p.Lk + ks.j) * HD;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int jq = 0; jq < 4; ++jq)
        *reinterpret_cast<f32x4*>(row + d * 32 + 8 * jq + 4 * half) =
            f32x4{dv_acc[d][4 * jq], dv_acc[d][4 * jq + 1], dv_acc[d][4 * jq + 2], dv_acc[d][4 * jq + 3]};
    }
  } else if (ks.key_ok) {
    uint16_t* dvrow = p.dv + ((int64_t)ks.b * p.Lk * p.H + ks.h) * HD + (int64_t)ks.j * p.H * HD;
    RopeDev none = p.rope;
    none.table = nullptr;
    const TokenPos pos{0, 0, 0};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int jq = 0; jq < 4; ++jq)
        store_grad4(dvrow, none, pos, d * 32 + 8 * jq + 4 * half, dv_acc[d][4 * jq], dv_acc[d][4 * jq + 1],
                    dv_acc[d][4 * jq + 2], dv_acc[d][4 * jq + 3]);
    }
  }
}

}  // namespace

hipError_t launch_bwd_dv(const BwdParams& q, int n_main, int n_tail, hipStream_t stream) {
  // q.n_tiles: key blocks of 32 * DV_WAVES keys; the main grid is blocks x q_split x H x B less the
  // tail's blocks, which run as n_tail = tail x kv_split workgroups.
  const int64_t total = (int64_t)q.n_tiles * q.q_split * q.H * q.B;
  if (total <= 0 || total > 0x7fffffff || n_main < 0 || n_tail < 0) return hipErrorInvalidValue;
  if (n_main > 0) {
    if (q.k_lens != nullptr)
      hipLaunchKernelGGL((bwd_dv_kernel<true, false>), dim3((unsigned)n_main), dim3(64 * DV_WAVES), 0, stream, q);
    else
      hipLaunchKernelGGL((bwd_dv_kernel<false, false>), dim3((unsigned)n_main), dim3(64 * DV_WAVES), 0, stream, q);
  }
  if (n_tail > 0) {
    if (q.k_lens != nullptr)
      hipLaunchKernelGGL((bwd_dv_kernel<true, true>), dim3((unsigned)n_tail), dim3(64 * DV_WAVES), 0, stream, q);
    else
      hipLaunchKernelGGL((bwd_dv_kernel<false, true>), dim3((unsigned)n_tail), dim3(64 * DV_WAVES), 0, stream, q);
  }
  return hipSuccess;
}

}  // namespace wanattn
