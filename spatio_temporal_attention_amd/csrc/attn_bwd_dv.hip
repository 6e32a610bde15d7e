// Backward dV pass for gfx950 (the formulas and the tile layouts are those of
// attn_bwd.hip, whose other passes share bwd_common.h).  Its own file so that
// it can be built with the iterative ILP machine scheduler: with it the
// compiler keeps more fragment reads in flight here (720p: 100.5 -> 94.4 ms),
// while the register-bound dK and dQ passes spill or slow down under it.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "bwd_common.h"

namespace wanattn {

namespace {

using namespace bwd;

// dV_j = sum_i P_ij dO_i.  Workgroup = 256 keys (8 waves, one workgroup per
// CU, two waves per SIMD); query tiles staged as Q fp16 rows, dO^T and the
// row statistics.  S = Q K^T from the wave's K rows in registers, dV^T +=
// dO^T P with P from the accumulators.  The same ping-pong as the dK pass
// (attn_bwd.hip): M(u) = dV of query tile u-1, then S of tile u; V(u) = P of
// tile u, its LSE read by row from the tile statistics (four 16-byte LDS
// broadcast reads per 32-row block); waves 4..7 one phase behind; Q(u+1), dO^T(u)
// and the statistics of u+1 copied in interval 2u and waited for before
// barrier 2u+1.
constexpr uint32_t DV_Q = 0;         // Q row tile at + 16384 * slot
constexpr uint32_t DV_DOT = 32768;   // dO^T at + 16384 * slot
constexpr uint32_t DV_ST = 65536;    // statistics at + 1024 * (tile & 3)
constexpr uint32_t DV_LDS = DV_ST + 4 * 1024;

template <bool KMASK, bool TAIL>
__global__ __launch_bounds__(64 * DV_WAVES, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dv_kernel(
    BwdParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[DV_LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const bool late = wv >= DV_WAVES / 2;   // waves 4..7: one phase behind
  const KeySide ks = key_side<DV_WAVES, KMASK, TAIL>(p, wv, col);

  bf16x8 kf[8];   // K fp16 (bit patterns): B operand of S
  load_row_frags(kf, p.kf + (ks.ktile0 + (ks.tile_ok ? ks.ktile : 0)) * TILE_ELEMS, 32 * (wave & 1) + col, half,
                 ks.tile_ok);
  const int e_k = ks.tile_ok ? p.kexp[ks.ktile0 + ks.ktile] : 0;

  f32x16 dv_acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) dv_acc[d] = f32x16{};

  // This lane's LDS byte offsets (slot, row block and matrix are immediates).
  uint32_t rf[8], tf[4];
#pragma unroll
  for (int s = 0; s < 8; ++s) rf[s] = DV_Q + col * 256 + (((2 * s + half) ^ swz(col)) << 4);
#pragma unroll
  for (int kg = 0; kg < 4; ++kg) tf[kg] = DV_DOT + col * 128 + (((2 * kg + half) ^ swz8(col)) << 4);
  // LSE log2 e of this lane's rows of value group jg in row block qb: rows
  // 32 qb + 8 jg + 4 half + 0..3, one 16-byte read shared by the lanes of the
  // half (an LDS broadcast).
  const uint32_t sf = DV_ST + 16 * half;
  auto frag = [&](uint32_t off) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(smem + off);
  };

  uint32_t roff[2], toff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    roff[i] = rowtile_lane_off<DV_WAVES>(wv, i, lane);
    toff[i] = ttile_lane_off<DV_WAVES>(wv, i, lane);
  }
  const uint32_t bytes = (uint32_t)ks.nt * (TILE_ELEMS * 2);   // < 2^32, checked by the launcher
  const __amdgpu_buffer_rsrc_t qfr = tile_rsrc(p.qf + ks.tile0 * TILE_ELEMS, bytes);
  const __amdgpu_buffer_rsrc_t dotr = tile_rsrc(p.dot + ks.tile0 * TILE_ELEMS, bytes);
  const __amdgpu_buffer_rsrc_t str = tile_rsrc(p.qstat + ks.tile0 * QSTAT_FLOATS, (uint32_t)ks.nt * 1024u);
  auto copy_q = [&](int slot, int t) __attribute__((always_inline)) {
    const uint32_t soff = (uint32_t)t * (TILE_ELEMS * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) buf_dma16(qfr, roff[i], soff, smem + DV_Q + 16384 * slot + 2048 * wv + 1024 * i);
  };
  auto copy_dot = [&](int slot, int t) __attribute__((always_inline)) {
    const uint32_t soff = (uint32_t)t * (TILE_ELEMS * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) buf_dma16(dotr, toff[i], soff, smem + DV_DOT + 16384 * slot + 2048 * wv + 1024 * i);
  };
  auto copy_stats = [&](int t) __attribute__((always_inline)) {
    if (wv == 0) buf_dma16(str, 16 * lane, (uint32_t)t * 1024u, smem + DV_ST + 1024 * (t & 3));
  };

  // A query split can be empty (rounding of the split size): it writes zero partials.
  const int n = ks.t1 - ks.t0;
  if (n > 0) {
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    // The copies of interval 2u: Q(u+1) into slot (u+1) & 1, dO^T(u) into slot u & 1, statistics(u+1).
    auto copies = [&](auto parity, int u) __attribute__((always_inline)) {
      constexpr int P = decltype(parity)::value;   // u & 1
      if (u + 1 < n) {
        copy_q(P ^ 1, ks.t0 + u + 1);
        copy_stats(ks.t0 + u + 1);
      }
      copy_dot(P, ks.t0 + u);
    };
    copy_q(0, ks.t0);
    copy_stats(ks.t0);
    wait_vmem();
    __syncthreads();
    if (late) {
      copies(P0{}, 0);   // interval 0: the late waves' "V(-1)"
      dma_barrier();     // the early waves run M(0) meanwhile
    }

    f32x16 s_acc[2];
    bf16x8 pf[4];
    auto phase_end = [&](bool vmem) __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      if (vmem) wait_vmem();
      dma_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    // M(u), parity P = u & 1: dV of tile u-1 (GRAD: u > 0), then S of tile u (SDP: u < n).
    auto m_phase = [&](auto parity, auto grad_tag, auto sdp_tag, int u) __attribute__((always_inline)) {
      constexpr int P = decltype(parity)::value;
      constexpr bool GRAD = decltype(grad_tag)::value;
      constexpr bool SDP = decltype(sdp_tag)::value;
      if (SDP && !late) copies(parity, u);
      if (!KMASK || ks.wave_live) {
        if (GRAD) {
#pragma unroll
          for (int kg = 0; kg < 4; ++kg)
#pragma unroll
            for (int d = 0; d < 4; ++d)
              dv_acc[d] = mfma32(frag(tf[kg] + 16384 * (P ^ 1) + 4096 * d), pf[kg], dv_acc[d]);
        }
        if (SDP) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) s_acc[qb] = f32x16{};
#pragma unroll
          for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              s_acc[qb] = mfma32_f16(frag(rf[s] + 16384 * P + 8192 * qb), kf[s], s_acc[qb]);
        }
        // Keep six fragment reads in flight ahead of the MFMAs (registers allow it here).
        constexpr int n_mfma = (GRAD ? 16 : 0) + (SDP ? 16 : 0);
        constexpr int AHEAD = 6;
        __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
        for (int k = 0; k < n_mfma - AHEAD; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
      }
      phase_end(late);
    };
    // V(u): P = exp2(S g - LSE log2 e), packed to bf16 for the next M.
    auto v_phase = [&](auto parity, int u) __attribute__((always_inline)) {
      const int t = ks.t0 + u;
      if (late && u + 1 < n) copies(std::integral_constant<int, decltype(parity)::value ^ 1>{}, u + 1);
      if (!KMASK || ks.wave_live) {
        // LSE log2 e of the tile's 64 rows, then -Delta, then the tile exponent
        const int e_q = *reinterpret_cast<const int*>(smem + DV_ST + 1024 * (t & 3) + 512);
        const float g = ldexpf(p.scale_log2, e_q + e_k);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          float l2[16], pv[16];
#pragma unroll
          for (int jg = 0; jg < 4; ++jg) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(smem + sf + 1024 * (t & 3) + 4 * (32 * qb + 8 * jg));
#pragma unroll
            for (int i = 0; i < 4; ++i) l2[4 * jg + i] = x[i];
          }
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            float pe = __builtin_amdgcn_exp2f(fmaf(s_acc[qb][j], g, -l2[j]));
            if (KMASK && !ks.key_live) pe = 0.f;
            pv[j] = pe;
          }
          pf[2 * qb] = pack_acc8(pv);
          pf[2 * qb + 1] = pack_acc8(pv + 8);
        }
        // P is complete here: the code sinking passes must not move its
        // arithmetic past the barrier into the next products phase.
#pragma unroll
        for (int i = 0; i < 4; ++i) pin_vgprs(pf[i]);
      }
      phase_end(!late);
    };
    m_phase(P0{}, std::false_type{}, std::true_type{}, 0);
    v_phase(P0{}, 0);
    int u = 1;
    for (; u + 1 < n; u += 2) {
      m_phase(P1{}, std::true_type{}, std::true_type{}, u);
      v_phase(P1{}, u);
      m_phase(P0{}, std::true_type{}, std::true_type{}, u + 1);
      v_phase(P0{}, u + 1);
    }
    if (u < n) {
      m_phase(P1{}, std::true_type{}, std::true_type{}, u);
      v_phase(P1{}, u);
    }
    // M(n): the last tile's dV product
    if (n & 1) m_phase(P1{}, std::true_type{}, std::false_type{}, n);
    else m_phase(P0{}, std::true_type{}, std::false_type{}, n);
    if (!late) dma_barrier();   // matches the late waves' barrier before their M(0)
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
