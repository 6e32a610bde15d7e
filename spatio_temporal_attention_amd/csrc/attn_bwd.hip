// Self-attention backward for gfx950: two deterministic passes over the
// tiles the prep passes write (kv_prep.hip).  The formulas are the calculus
// of the forward (full spatio-temporal attention with 3D RoPE; "Wan Team,
// Alibaba (2025)", Key takeaways, Backbone; training in bf16 per the Wan2.1
// reading notes, 3. Training):
//   Delta_i = <dO_i, O_i>                                  (prep pass)
//   P_ij    = exp(scale <q~_i, k~_j> - LSE_i)              (recomputed, never stored)
//   dV_j    = sum_i P_ij dO_i
//   dS_ij   = P_ij (<dO_i, v_j> - Delta_i)
//   dq~_i   = scale sum_j dS_ij k~_j,   dk~_j = scale sum_i dS_ij q~_i
//   dq_i    = R(p_i)^T dq~_i,           dk_j  = R(p_j)^T dk~_j
// The scores are recomputed from the same fp16 operands the forward used
// (q~ and k~ per 64-token tile scaled by 2^-e and rounded to fp16), so P
// matches the forward's LSE; s * log2(e) = scale*log2(e) * 2^(e_q + e_k) * S.
// The gradient products take bf16 operands (P, dS, dO, V, q~^T, k~^T).
// Every MFMA operand comes from a plain 16-byte LDS read or from registers:
// operands contracted over tokens come from T tiles (token-position order
// matching the accumulator registers), so no LDS transpose read is needed.
// The inverse rotation is fused into the dQ and dK stores.
//
//  * bwd_dv (attn_bwd_dv.hip):   workgroup = 256 keys (8 waves x 32, one workgroup per CU),
//    loop over 64-query tiles staged as Q fp16 rows and dO^T.  S = Q K^T
//    (lane owns key j), dV^T += dO^T P with P from the accumulators.
//  * bwd_dk:   workgroup = 256 keys (8 waves x 32, one workgroup per CU),
//    query tiles staged as Q fp16 rows, dO rows and (R q)^T.  S = Q K^T,
//    dP - Delta = dO V^T - Delta, dK~^T += (R q)^T dS.  (One kernel for both
//    would hold K, V and both accumulators per wave: one wave per SIMD.)
//  * bwd_dq:   workgroup = 256 queries (8 waves, two per SIMD), loop over
//    64-key tiles staged as K fp16 rows, (R k)^T, V rows.  S^T = K Q^T,
//    dP^T = V dO^T (lane owns query i), dQ~^T += (R k)^T dS^T.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "bwd_common.h"
#include "validate.h"

namespace wanattn {

namespace {

using namespace bwd;

// dk~_j = scale sum_i dS_ij q~_i, dS_ij = P_ij (<dO_i, v_j> - Delta_i).
// Workgroup = 256 keys (8 waves, one workgroup per CU, two waves per SIMD);
// query tiles staged as Q fp16 rows, dO rows, (R q)^T and the row
// statistics.  A wave holds the K and V rows of its 32 keys in registers (the
// B operands of S = Q K^T and of dP - Delta = dO V^T - Delta, whose
// accumulator starts at -Delta) and accumulates dK~^T += (R q)^T dS with dS
// taken from the accumulators.  A lane holds 16 query rows of each 32-row
// block, in four runs of 4 consecutive rows shared by its half of the wave;
// the statistics are stored by row, so each run's LSE or -Delta is one
// 16-byte LDS read that the half's lanes share (a broadcast).
//
// Ping-pong, as in the forward: each wave alternates a products phase M(u)
// (MFMA: dK~ += (R q)^T dS of query tile u-1, then S and dP of tile u) and a
// softmax phase V(u) (VALU: P and dS of tile u); waves 4..7 run one phase
// behind waves 0..3 and all eight meet at a barrier after every phase, so on
// each SIMD (waves w and w + 4) one wave feeds the matrix cores while the
// other computes its dS.
//
// Interval k lies between barriers k-1 and k; the early waves run phase k
// (M(u) = 2u, V(u) = 2u+1) in interval k, the late waves in interval k+1.
// Q/dO of tile u are read in intervals 2u..2u+1, its statistics in
// 2u..2u+2, its (R q)^T in 2u+2..2u+3 (double buffers; statistics in a ring
// of four).  In interval 2u every wave copies its share of Q/dO(u+1) and
// (R q)^T(u), wave 0 the statistics of u+1 (the early waves at the start of
// M(u), the late ones at the start of V(u-1)), into slots last read in
// interval 2u-1 or before; each wave waits for its copies before barrier
// 2u+1, and they are first read in interval 2u+2: two intervals of latency.
constexpr uint32_t DK_QD = 0;        // Q row tile at + 32768 * slot, dO row tile at + 16384
constexpr uint32_t DK_QT = 65536;    // (R q)^T at + 16384 * slot
constexpr uint32_t DK_ST = 98304;    // statistics at + 1024 * (tile & 3)
constexpr uint32_t DK_LDS = DK_ST + 4 * 1024;
static_assert(QSTAT_FLOATS * 4 == 1024, "one 1 KB copy per statistics tile");

template <bool KMASK, bool TAIL>
__global__ __launch_bounds__(64 * DK_WAVES, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dk_kernel(
    BwdParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[DK_LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const bool late = wv >= DK_WAVES / 2;   // waves 4..7: one phase behind
  const KeySide ks = key_side<DK_WAVES, KMASK, TAIL>(p, wv, col);

  bf16x8 kf[8], vf[8];   // K fp16 (bit patterns), V bf16: B operands of S and dP
  const int64_t ktile = ks.ktile0 + (ks.tile_ok ? ks.ktile : 0);
  load_row_frags(kf, p.kf + ktile * TILE_ELEMS, 32 * (wave & 1) + col, half, ks.tile_ok);
  load_row_frags(vf, p.vr + ktile * TILE_ELEMS, 32 * (wave & 1) + col, half, ks.tile_ok);
  const int e_k = ks.tile_ok ? p.kexp[ks.ktile0 + ks.ktile] : 0;

  f32x16 dk_acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) dk_acc[d] = f32x16{};

  // This lane's LDS byte offsets; the slot, the 32-row block and the matrix
  // are immediates.  Row fragments (Q, dO): row col, chunk 2s + half
  // (tile_off's swizzle); (R q)^T fragments: row col, chunk 2kg + half
  // (tile8_off's); statistics: entry 16 half + lane % 16.
  uint32_t rf[8], tf[4];
#pragma unroll
  for (int s = 0; s < 8; ++s) rf[s] = DK_QD + col * 256 + (((2 * s + half) ^ swz(col)) << 4);
#pragma unroll
  for (int kg = 0; kg < 4; ++kg) tf[kg] = DK_QT + col * 128 + (((2 * kg + half) ^ swz8(col)) << 4);
  // Statistics (LSE log2 e, then -Delta, by row): this lane's rows of value
  // group jg in row block qb are 32 qb + 8 jg + 4 half + 0..3, one 16-byte
  // read that every lane of the half shares (an LDS broadcast).
  const uint32_t sf = DK_ST + 16 * half;
  auto frag = [&](uint32_t off) __attribute__((always_inline)) { return *reinterpret_cast<const bf16x8*>(smem + off); };
  auto stat4 = [&](uint32_t off) __attribute__((always_inline)) { return *reinterpret_cast<const f32x4*>(smem + off); };

  uint32_t roff[2], toff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    roff[i] = rowtile_lane_off<DK_WAVES>(wv, i, lane);
    toff[i] = ttile_lane_off<DK_WAVES>(wv, i, lane);
  }
  const uint32_t bytes = (uint32_t)ks.nt * (TILE_ELEMS * 2);   // < 2^32, checked by the launcher
  const __amdgpu_buffer_rsrc_t qfr = tile_rsrc(p.qf + ks.tile0 * TILE_ELEMS, bytes);
  const __amdgpu_buffer_rsrc_t dor = tile_rsrc(p.dor + ks.tile0 * TILE_ELEMS, bytes);
  const __amdgpu_buffer_rsrc_t qtr = tile_rsrc(p.qt + ks.tile0 * TILE_ELEMS, bytes);
  const __amdgpu_buffer_rsrc_t str = tile_rsrc(p.qstat + ks.tile0 * QSTAT_FLOATS, (uint32_t)ks.nt * 1024u);
  auto copy_qd = [&](int slot, int t) __attribute__((always_inline)) {
    const uint32_t soff = (uint32_t)t * (TILE_ELEMS * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      buf_dma16(qfr, roff[i], soff, smem + DK_QD + 32768 * slot + 2048 * wv + 1024 * i);
      buf_dma16(dor, roff[i], soff, smem + DK_QD + 32768 * slot + 16384 + 2048 * wv + 1024 * i);
    }
  };
  auto copy_qt = [&](int slot, int t) __attribute__((always_inline)) {
    const uint32_t soff = (uint32_t)t * (TILE_ELEMS * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) buf_dma16(qtr, toff[i], soff, smem + DK_QT + 16384 * slot + 2048 * wv + 1024 * i);
  };
  auto copy_stats = [&](int t) __attribute__((always_inline)) {
    if (wv == 0) buf_dma16(str, 16 * lane, (uint32_t)t * 1024u, smem + DK_ST + 1024 * (t & 3));
  };

  // A query split can be empty (rounding of the split size): it writes zero partials.
  const int n = ks.t1 - ks.t0;
  if (n > 0) {
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    // The copies of interval 2u (tile u = index within the range): Q/dO(u+1) into slot
    // (u+1) & 1, (R q)^T(u) into slot u & 1, statistics(u+1).
    auto copies = [&](auto parity, int u) __attribute__((always_inline)) {
      constexpr int P = decltype(parity)::value;   // u & 1
      if (u + 1 < n) {
        copy_qd(P ^ 1, ks.t0 + u + 1);
        copy_stats(ks.t0 + u + 1);
      }
      copy_qt(P, ks.t0 + u);
    };
    copy_qd(0, ks.t0);
    copy_stats(ks.t0);
    wait_vmem();
    __syncthreads();
    if (late) {
      copies(P0{}, 0);   // interval 0: the late waves' "V(-1)"
      dma_barrier();     // the early waves run M(0) meanwhile
    }

    f32x16 s_acc[2], dp_acc[2];
    bf16x8 dsf[4];
    // The end of a phase (VMEM: wait for this wave's copies first).  No
    // instruction moves across it: each phase keeps to its own pipe.
    auto phase_end = [&](bool vmem) __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      if (vmem) wait_vmem();
      dma_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    // M(u), parity P = u & 1: dK~ of tile u-1 (GRAD: u > 0), then S and dP of tile u (SDP: u < n).
    auto m_phase = [&](auto parity, auto grad_tag, auto sdp_tag, int u) __attribute__((always_inline)) {
      constexpr int P = decltype(parity)::value;
      constexpr bool GRAD = decltype(grad_tag)::value;
      constexpr bool SDP = decltype(sdp_tag)::value;
      const int t = ks.t0 + u;
      if (SDP && !late) copies(parity, u);
      if (!KMASK || ks.wave_live) {
        // -Delta of the accumulator's rows, read first, so that its wait does not drain the fragment reads
        // queued behind it
        f32x4 nd[2][4];
        if (SDP) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int jg = 0; jg < 4; ++jg) nd[qb][jg] = stat4(sf + 1024 * (t & 3) + 256 + 4 * (32 * qb + 8 * jg));
          __builtin_amdgcn_sched_barrier(0);
        }
        if (GRAD) {
#pragma unroll
          for (int kg = 0; kg < 4; ++kg)
#pragma unroll
            for (int d = 0; d < 4; ++d)
              dk_acc[d] = mfma32(frag(tf[kg] + 16384 * (P ^ 1) + 4096 * d), dsf[kg], dk_acc[d]);
        }
        if (SDP) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            s_acc[qb] = f32x16{};
#pragma unroll
            for (int j = 0; j < 16; ++j) dp_acc[qb][j] = nd[qb][j >> 2][j & 3];
          }
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int s = 0; s < 8; ++s) {
              s_acc[qb] = mfma32_f16(frag(rf[s] + 32768 * P + 8192 * qb), kf[s], s_acc[qb]);
              dp_acc[qb] = mfma32(frag(rf[s] + 32768 * P + 16384 + 8192 * qb), vf[s], dp_acc[qb]);
            }
        }
        // Keep four fragment reads in flight ahead of the MFMAs.
        constexpr int n_mfma = (GRAD ? 16 : 0) + (SDP ? 32 : 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int k = 0; k < n_mfma - 4; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
      phase_end(late);
    };
    // V(u): P = exp2(S g - LSE log2 e), dS = P (dP - Delta), packed to bf16 for the next M.
    auto v_phase = [&](auto parity, int u) __attribute__((always_inline)) {
      const int t = ks.t0 + u;
      if (late && u + 1 < n) copies(std::integral_constant<int, decltype(parity)::value ^ 1>{}, u + 1);
      if (!KMASK || ks.wave_live) {
        const int e_q = *reinterpret_cast<const int*>(smem + DK_ST + 1024 * (t & 3) + 512);
        const float g = ldexpf(p.scale_log2, e_q + e_k);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          float l2[16], dsv[16];
#pragma unroll
          for (int jg = 0; jg < 4; ++jg) {
            const f32x4 x = stat4(sf + 1024 * (t & 3) + 4 * (32 * qb + 8 * jg));
#pragma unroll
            for (int i = 0; i < 4; ++i) l2[4 * jg + i] = x[i];
          }
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            float pe = __builtin_amdgcn_exp2f(fmaf(s_acc[qb][j], g, -l2[j]));
            if (KMASK && !ks.key_live) pe = 0.f;
            dsv[j] = pe * dp_acc[qb][j];
          }
          dsf[2 * qb] = pack_acc8(dsv);
          dsf[2 * qb + 1] = pack_acc8(dsv + 8);
          __builtin_amdgcn_sched_barrier(0);   // one 32-row half at a time (registers)
        }
        // dS is complete here: the code sinking passes must not move its
        // arithmetic past the barrier into the next products phase.
#pragma unroll
        for (int i = 0; i < 4; ++i) pin_vgprs(dsf[i]);
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
    // M(n): the last tile's dK~ product
    if (n & 1) m_phase(P1{}, std::true_type{}, std::false_type{}, n);
    else m_phase(P0{}, std::true_type{}, std::false_type{}, n);
    if (!late) dma_barrier();   // matches the late waves' barrier before their M(0)
  }

  if (TAIL) {
    // fp32 partial (unscaled, unrotated) over this query range, rows of the workgroup's 256 keys
    float* row = p.kv_part + ((int64_t)blockIdx.x * (32 * DK_WAVES) + wave * 32 + col) * HD;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int jq = 0; jq < 4; ++jq)
        *reinterpret_cast<f32x4*>(row + d * 32 + 8 * jq + 4 * half) =
            f32x4{dk_acc[d][4 * jq], dk_acc[d][4 * jq + 1], dk_acc[d][4 * jq + 2], dk_acc[d][4 * jq + 3]};
    }
  } else if (ks.key_ok && p.q_split > 1) {
    // fp32 partial (unscaled, unrotated) over this split's query tiles
    float* row = p.part + ((((int64_t)ks.split * p.B + ks.b) * p.H + ks.h) * p.Lk + ks.j) * HD;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int jq = 0; jq < 4; ++jq)
        *reinterpret_cast<f32x4*>(row + d * 32 + 8 * jq + 4 * half) =
            f32x4{dk_acc[d][4 * jq], dk_acc[d][4 * jq + 1], dk_acc[d][4 * jq + 2], dk_acc[d][4 * jq + 3]};
    }
  } else if (ks.key_ok) {
    TokenPos pos{0, 0, 0};
    if (p.rope.table != nullptr) pos = token_pos(p.rope, ks.j);
    uint16_t* dkrow = p.dk + ((int64_t)ks.b * p.Lk * p.H + ks.h) * HD + (int64_t)ks.j * p.H * HD;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int jq = 0; jq < 4; ++jq)
        store_grad4(dkrow, p.rope, pos, d * 32 + 8 * jq + 4 * half, dk_acc[d][4 * jq] * p.scale,
                    dk_acc[d][4 * jq + 1] * p.scale, dk_acc[d][4 * jq + 2] * p.scale, dk_acc[d][4 * jq + 3] * p.scale);
    }
  }
}

// Sum of the q_split partial dK~ and dV of every key (fixed order: deterministic),
// then dk = R(p_j)^T scale dK~ and dv, in bf16.  One thread per 4 elements.
__global__ __launch_bounds__(256) void bwd_kv_reduce_kernel(BwdParams p) {
  const int64_t n4 = (int64_t)p.B * p.H * p.Lk * (HD / 4);
  const int64_t part = (int64_t)p.q_split * p.B * p.H * p.Lk * HD;
  const int64_t stride_s = (int64_t)p.B * p.H * p.Lk * HD;
  RopeDev none = p.rope;
  none.table = nullptr;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    const int d0 = 4 * (int)(i % (HD / 4));
    const int64_t r = i / (HD / 4);   // ((b * H) + h) * Lk + j
    const int j = (int)(r % p.Lk);
    const int64_t bh = r / p.Lk;
    const int h = (int)(bh % p.H);
    const int b = (int)(bh / p.H);
    f32x4 sk = f32x4{0.f, 0.f, 0.f, 0.f}, sv = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < p.q_split; ++s) {
      sk += *reinterpret_cast<const f32x4*>(p.part + s * stride_s + r * HD + d0);
      sv += *reinterpret_cast<const f32x4*>(p.part + part + s * stride_s + r * HD + d0);
    }
    TokenPos pos{0, 0, 0};
    if (p.rope.table != nullptr) pos = token_pos(p.rope, j);
    const int64_t off = (((int64_t)b * p.Lk + j) * p.H + h) * HD;
    store_grad4(p.dk + off, p.rope, pos, d0, sk[0] * p.scale, sk[1] * p.scale, sk[2] * p.scale, sk[3] * p.scale);
    store_grad4(p.dv + off, none, pos, d0, sv[0], sv[1], sv[2], sv[3]);
  }
}

// Sum of the dK/dV tail split's partials (fixed order over the query ranges), then
// dk = R(p_j)^T scale dK~ and dv in bf16.  One thread per key and four head-dim columns.
__global__ __launch_bounds__(256) void bwd_kv_tail_reduce_kernel(BwdParams p, int tail) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int c4 = (int)(idx & 31);
  const int64_t rr = idx >> 5;
  const int rl = (int)(rr % 256);
  const int ti = (int)(rr / 256);
  if (ti >= tail) return;
  const int logical = p.kv_base + ti;
  const int kb = logical % p.n_tiles;
  const int bh = logical / p.n_tiles;
  const int b = bh % p.B;
  const int h = bh / p.B;
  const int j = kb * 256 + rl;
  if (j >= p.Lk) return;
  const int64_t region = (int64_t)tail * p.kv_split * 256 * HD;   // dV partials follow dK~
  const float* src = p.kv_part + ((int64_t)ti * p.kv_split * 256 + rl) * HD + 4 * c4;
  f32x4 sk = f32x4{0.f, 0.f, 0.f, 0.f}, sv = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < p.kv_split; ++s) {
    sk += *reinterpret_cast<const f32x4*>(src + (int64_t)s * 256 * HD);
    sv += *reinterpret_cast<const f32x4*>(src + region + (int64_t)s * 256 * HD);
  }
  TokenPos pos{0, 0, 0};
  if (p.rope.table != nullptr) pos = token_pos(p.rope, j);
  RopeDev none = p.rope;
  none.table = nullptr;
  const int64_t off = (((int64_t)b * p.Lk + j) * p.H + h) * HD;
  store_grad4(p.dk + off, p.rope, pos, 4 * c4, sk[0] * p.scale, sk[1] * p.scale, sk[2] * p.scale, sk[3] * p.scale);
  store_grad4(p.dv + off, none, pos, 4 * c4, sv[0], sv[1], sv[2], sv[3]);
}

// ---------------------------------------------------------------------------
// dQ: workgroup owns 256 queries (query tiles 4qb .. 4qb+3); loop over 64-key tiles.
// ---------------------------------------------------------------------------
// A wave holds the fp16 Q rows and the dO rows of its 32 queries (B operands
// of S^T = K Q^T and dP^T = V dO^T; the lane owns query i, so its LSE and
// Delta are two registers) and accumulates dq~^T += (R k)^T dS^T.  The same
// ping-pong as the dK pass: M(u) = dq~ of key tile u-1, then S^T and dP^T of
// tile u; V(u) = P and dS of tile u; waves 4..7 one phase behind.  K/V rows of
// tile u are read in intervals 2u..2u+1, its (R k)^T in 2u+2..2u+3 (double
// buffers); in interval 2u every wave copies its share of K/V(u+1) and
// (R k)^T(u) and waits for them before barrier 2u+1.
constexpr uint32_t DQ_KV = 0;        // K fp16 row tile at + 32768 * slot, V row tile at + 16384
constexpr uint32_t DQ_KT = 65536;    // (R k)^T at + 16384 * slot
constexpr uint32_t DQ_LDS = DQ_KT + 2 * 16384;

// SPLIT: the tail launch (one key range of a query block, fp32 partial of dq~ out).
template <bool SPLIT>
__global__ __launch_bounds__(64 * DQ_WAVES, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(
    BwdParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[DQ_LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const bool late = wv >= DQ_WAVES / 2;   // waves 4..7: one phase behind

  int logical, split = 0;
  if (SPLIT) {
    logical = p.dq_base + (int)blockIdx.x / p.dq_split;
    split = (int)blockIdx.x % p.dq_split;
  } else {
    logical = xcd_remap(blockIdx.x, gridDim.x);
  }
  const int qb = logical % p.n_tiles;
  const int bh = logical / p.n_tiles;
  const int b = bh % p.B;   // batch innermost: every XCD gets the same heads of every item
  const int h = bh / p.B;
  const int nt = (p.Lq + TILE_ROWS - 1) / TILE_ROWS;     // query tiles
  const int ntk = (p.Lk + TILE_ROWS - 1) / TILE_ROWS;    // key tiles
  const int64_t tile0 = (int64_t)(b * p.H + h) * nt;
  const int64_t ktile0 = (int64_t)(b * p.H + h) * ntk;
  const int n_keys = p.k_lens != nullptr ? min(max(p.k_lens[b], 0), p.Lk) : p.Lk;
  const int nkt = (n_keys + TILE_ROWS - 1) / TILE_ROWS;  // key tiles of valid keys
  // Key tiles [t0, t1): all of them, or one of p.dq_split ranges.
  int t0 = 0, t1 = nkt;
  if (SPLIT) {
    const int chunk = (nkt + p.dq_split - 1) / p.dq_split;
    t0 = min(nkt, split * chunk);
    t1 = min(nkt, t0 + chunk);
  }

  // This lane's query i: row 32*(wave%2) + col of query tile 4qb + wave/2.
  const int qtile = 4 * qb + (wv >> 1);
  const int i = qb * 256 + wave * 32 + col;
  const bool row_ok = i < p.Lq;
  const bool tile_ok = qtile < nt;
  bf16x8 qf[8], dof[8];   // Q fp16 (bit patterns), dO bf16: B operands of S^T and dP^T
  load_row_frags(qf, p.qf + (tile0 + (tile_ok ? qtile : 0)) * TILE_ELEMS, 32 * (wave & 1) + col, half, tile_ok);
  load_row_frags(dof, p.dor + (tile0 + (tile_ok ? qtile : 0)) * TILE_ELEMS, 32 * (wave & 1) + col, half, tile_ok);
  const int e_q = tile_ok ? p.qexp[tile0 + qtile] : 0;
  // LSE_i log2 e (+inf past Lq or with no valid key: P = 0) and -Delta_i of row r = 32 (wave % 2) + col of
  // the tile, from the query prep pass (floats r and 64 + r of the tile's statistics)
  const float* st = p.qstat + (tile0 + (tile_ok ? qtile : 0)) * QSTAT_FLOATS + 32 * (wave & 1) + col;
  const float lse2 = tile_ok ? st[0] : INFINITY;
  const float ndelta = tile_ok ? st[TILE_ROWS] : 0.f;

  f32x16 dq_acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) dq_acc[d] = f32x16{};

  // This lane's LDS byte offsets (slot, 32-key block and matrix are immediates):
  // row fragments (K, V): row col, chunk 2s + half; (R k)^T: row col, chunk 2kg + half.
  uint32_t rf[8], tf[4];
#pragma unroll
  for (int s = 0; s < 8; ++s) rf[s] = DQ_KV + col * 256 + (((2 * s + half) ^ swz(col)) << 4);
#pragma unroll
  for (int kg = 0; kg < 4; ++kg) tf[kg] = DQ_KT + col * 128 + (((2 * kg + half) ^ swz8(col)) << 4);
  auto frag = [&](uint32_t off) __attribute__((always_inline)) { return *reinterpret_cast<const bf16x8*>(smem + off); };

  uint32_t roff[2], toff[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    roff[c] = rowtile_lane_off<DQ_WAVES>(wv, c, lane);
    toff[c] = ttile_lane_off<DQ_WAVES>(wv, c, lane);
  }
  const uint32_t bytes = (uint32_t)ntk * (TILE_ELEMS * 2);   // < 2^32, checked by the launcher
  const __amdgpu_buffer_rsrc_t kfr = tile_rsrc(p.kf + ktile0 * TILE_ELEMS, bytes);
  const __amdgpu_buffer_rsrc_t ktr = tile_rsrc(p.kt + ktile0 * TILE_ELEMS, bytes);
  const __amdgpu_buffer_rsrc_t vrr = tile_rsrc(p.vr + ktile0 * TILE_ELEMS, bytes);
  const_i32* kexp = const_ptr(p.kexp + ktile0);   // scalar loads
  auto copy_kv = [&](int slot, int t) __attribute__((always_inline)) {
    const uint32_t soff = (uint32_t)t * (TILE_ELEMS * 2);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      buf_dma16(kfr, roff[c], soff, smem + DQ_KV + 32768 * slot + 2048 * wv + 1024 * c);
      buf_dma16(vrr, roff[c], soff, smem + DQ_KV + 32768 * slot + 16384 + 2048 * wv + 1024 * c);
    }
  };
  auto copy_kt = [&](int slot, int t) __attribute__((always_inline)) {
    const uint32_t soff = (uint32_t)t * (TILE_ELEMS * 2);
#pragma unroll
    for (int c = 0; c < 2; ++c) buf_dma16(ktr, toff[c], soff, smem + DQ_KT + 16384 * slot + 2048 * wv + 1024 * c);
  };

  // The full key tiles [t0, t0 + n) run as ping-pong phases; a partial last tile (keys past
  // n_keys get P = 0; only the range that holds it) runs after them in one step.
  const bool partial_last = t1 > t0 && t1 == nkt && n_keys % TILE_ROWS != 0;
  const int n = t1 - t0 - (partial_last ? 1 : 0);
  f32x16 s_acc[2], dp_acc[2];
  bf16x8 dsf[4];
  // S^T and dP^T of the tile in K/V slot P; dq~ from (R k)^T slot P (MFMA only).
  auto sdp = [&](auto parity) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s_acc[kb] = f32x16{};
      dp_acc[kb] = f32x16{};
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        s_acc[kb] = mfma32_f16(frag(rf[s] + 32768 * P + 8192 * kb), qf[s], s_acc[kb]);
        dp_acc[kb] = mfma32(frag(rf[s] + 32768 * P + 16384 + 8192 * kb), dof[s], dp_acc[kb]);
      }
  };
  auto grad = [&](auto parity) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
#pragma unroll
    for (int kg = 0; kg < 4; ++kg)
#pragma unroll
      for (int d = 0; d < 4; ++d) dq_acc[d] = mfma32(frag(tf[kg] + 16384 * P + 4096 * d), dsf[kg], dq_acc[d]);
  };
  // P = exp2(S g - LSE log2 e), dS = P (dP - Delta) into dsf; MASK: keys past n_keys get P = 0.
  auto softmax = [&](auto mask_tag, int t, int e_k) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const float g = ldexpf(p.scale_log2, e_q + e_k);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float dsv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float pe = __builtin_amdgcn_exp2f(fmaf(s_acc[kb][j], g, -lse2));
        if (MASK) {
          const int key = t * TILE_ROWS + kb * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
          if (key >= n_keys) pe = 0.f;
        }
        dsv[j] = pe * (dp_acc[kb][j] + ndelta);
      }
      dsf[2 * kb] = pack_acc8(dsv);
      dsf[2 * kb + 1] = pack_acc8(dsv + 8);
      __builtin_amdgcn_sched_barrier(0);   // one 32-key half at a time (registers)
    }
  };
  if (n > 0) {
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    // The copies of interval 2u: K/V(u+1) into slot (u+1) & 1, (R k)^T(u) into slot u & 1.
    auto copies = [&](auto parity, int u) __attribute__((always_inline)) {
      constexpr int P = decltype(parity)::value;   // u & 1
      if (u + 1 < n) copy_kv(P ^ 1, t0 + u + 1);
      copy_kt(P, t0 + u);
    };
    copy_kv(0, t0);
    int e_k = kexp[t0];   // exponent of the tile whose softmax comes next
    wait_vmem();
    __syncthreads();
    if (late) {
      copies(P0{}, 0);   // interval 0: the late waves' "V(-1)"
      dma_barrier();     // the early waves run M(0) meanwhile
    }
    auto phase_end = [&](bool vmem) __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      if (vmem) wait_vmem();
      dma_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    // M(u), parity P = u & 1: dq~ of tile u-1 (GRAD: u > 0), then S^T and dP^T of tile u (SDP: u < n).
    auto m_phase = [&](auto parity, auto grad_tag, auto sdp_tag, int u) __attribute__((always_inline)) {
      constexpr int P = decltype(parity)::value;
      constexpr bool GRAD = decltype(grad_tag)::value;
      constexpr bool SDP = decltype(sdp_tag)::value;
      if (SDP && !late) copies(parity, u);
      if (GRAD) grad(std::integral_constant<int, P ^ 1>{});
      if (SDP) sdp(parity);
      // Keep four fragment reads in flight ahead of the MFMAs.
      constexpr int n_mfma = (GRAD ? 16 : 0) + (SDP ? 32 : 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int k = 0; k < n_mfma - 4; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      phase_end(late);
    };
    // V(u): the softmax of tile u; the late waves copy for interval 2u+2 first.
    auto v_phase = [&](auto parity, int u) __attribute__((always_inline)) {
      const int t = t0 + u;
      if (late && u + 1 < n) copies(std::integral_constant<int, decltype(parity)::value ^ 1>{}, u + 1);
      const int e_t = e_k;
      if (u + 1 < n) e_k = kexp[t + 1];   // scalar load, waited for at the barrier
      softmax(std::false_type{}, t, e_t);
      // dS is complete here: the code sinking passes must not move its
      // arithmetic past the barrier into the next products phase.
#pragma unroll
      for (int k = 0; k < 4; ++k) pin_vgprs(dsf[k]);
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
    // M(n): the last full tile's dq~ product
    if (n & 1) m_phase(P1{}, std::true_type{}, std::false_type{}, n);
    else m_phase(P0{}, std::true_type{}, std::false_type{}, n);
    if (!late) dma_barrier();   // matches the late waves' barrier before their M(0)
  }
  if (partial_last) {
    // Every wave has left the slots (the last barrier above, or none used).
    const int t = t1 - 1;
    copy_kv(0, t);
    copy_kt(0, t);
    wait_vmem();
    __syncthreads();
    sdp(std::integral_constant<int, 0>{});
    softmax(std::true_type{}, t, kexp[t]);
    grad(std::integral_constant<int, 0>{});
  }

  if (SPLIT) {
    // Partial dq~ of this key range (unscaled, unrotated): rows of 128 fp32.
    float* dst = p.dq_part + ((int64_t)blockIdx.x * 256 + wave * 32 + col) * HD;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq)
        *reinterpret_cast<f32x4*>(dst + d * 32 + 8 * jq + 4 * half) =
            f32x4{dq_acc[d][4 * jq], dq_acc[d][4 * jq + 1], dq_acc[d][4 * jq + 2], dq_acc[d][4 * jq + 3]};
    return;
  }
  if (row_ok) {
    TokenPos pos{0, 0, 0};
    if (p.rope.table != nullptr) pos = token_pos(p.rope, i);
    const int64_t rs = (int64_t)p.H * HD;
    uint16_t* dqrow = p.dq + ((int64_t)b * p.Lq * p.H + h) * HD + (int64_t)i * rs;
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

// Sum of the dQ tail split's partials (fixed order over the key ranges), then
// dq = R(p_i)^T scale dq~ in bf16.  One thread per row and four head-dim columns.
__global__ __launch_bounds__(256) void bwd_dq_reduce_kernel(BwdParams p, int tail) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int c4 = (int)(idx & 31);
  const int64_t rr = idx >> 5;
  const int rl = (int)(rr % 256);
  const int ti = (int)(rr / 256);
  if (ti >= tail) return;
  const int logical = p.dq_base + ti;
  const int qb = logical % p.n_tiles;
  const int bh = logical / p.n_tiles;
  const int b = bh % p.B;
  const int h = bh / p.B;
  const int i = qb * 256 + rl;
  if (i >= p.Lq) return;
  const float* src = p.dq_part + ((int64_t)ti * p.dq_split * 256 + rl) * HD + 4 * c4;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < p.dq_split; ++s) acc += *reinterpret_cast<const f32x4*>(src + (int64_t)s * 256 * HD);
  TokenPos pos{0, 0, 0};
  if (p.rope.table != nullptr) pos = token_pos(p.rope, i);
  uint16_t* dqrow = p.dq + (((int64_t)b * p.Lq + i) * p.H + h) * HD;
  store_grad4(dqrow, p.rope, pos, 4 * c4, acc[0] * p.scale, acc[1] * p.scale, acc[2] * p.scale, acc[3] * p.scale);
}

// The tiles of one (b, h) are addressed through buffer resources of 32-bit extent.
bool tiles_addressable(int L) {
  return (int64_t)((L + TILE_ROWS - 1) / TILE_ROWS) * (TILE_ELEMS * 2) <= (int64_t)0xffffffff;
}

}  // namespace

hipError_t launch_bwd_dkdv(const BwdParams& p, hipStream_t stream) {
  if (!tiles_addressable(p.Lq) || !tiles_addressable(p.Lk)) return hipErrorInvalidValue;
  if (p.q_split < 1 || (p.q_split > 1 && p.part == nullptr)) return hipErrorInvalidValue;
  static_assert(32 * DK_WAVES == 256 && 32 * DV_WAVES == 256, "key blocks of 256 (the tail split's rows)");
  BwdParams q = p;
  q.n_tiles = (p.Lk + 255) / 256;
  const int64_t total = (int64_t)q.n_tiles * p.q_split * p.H * p.B;
  if (total <= 0 || total > 0x7fffffff) return hipErrorInvalidValue;
  // Tail split by the rule the workspace was sized by (no query split only).
  FwdSplit sp{(int)total, (int)total, 0, 1};
  if (p.kv_part != nullptr) {
    if (p.q_split != 1) return hipErrorInvalidValue;
    sp = fwd_tail_split(p.B, p.Lk, p.H);
  }
  if (sp.n != total) return hipErrorInvalidValue;
  q.kv_base = sp.n_main;
  q.kv_split = sp.S;
  if (launch_bwd_dv(q, sp.n_main, sp.tail * sp.S, stream) != hipSuccess) return hipErrorInvalidValue;
  if (sp.n_main > 0) {
    if (p.k_lens != nullptr)
      hipLaunchKernelGGL((bwd_dk_kernel<true, false>), dim3((unsigned)sp.n_main), dim3(64 * DK_WAVES), 0, stream, q);
    else
      hipLaunchKernelGGL((bwd_dk_kernel<false, false>), dim3((unsigned)sp.n_main), dim3(64 * DK_WAVES), 0, stream, q);
  }
  if (sp.tail > 0) {
    const dim3 g((unsigned)(sp.tail * sp.S));
    if (p.k_lens != nullptr)
      hipLaunchKernelGGL((bwd_dk_kernel<true, true>), g, dim3(64 * DK_WAVES), 0, stream, q);
    else
      hipLaunchKernelGGL((bwd_dk_kernel<false, true>), g, dim3(64 * DK_WAVES), 0, stream, q);
    hipLaunchKernelGGL(bwd_kv_tail_reduce_kernel, dim3((unsigned)(sp.tail * 32)), dim3(256), 0, stream, q, sp.tail);
  }
  if (p.q_split > 1) {
    const int64_t n4 = (int64_t)p.B * p.H * p.Lk * (HD / 4);
    const unsigned blocks = (unsigned)std::min<int64_t>((n4 + 255) / 256, 65536);
    hipLaunchKernelGGL(bwd_kv_reduce_kernel, dim3(blocks), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdParams& p, hipStream_t stream) {
  if (!tiles_addressable(p.Lq) || !tiles_addressable(p.Lk)) return hipErrorInvalidValue;
  BwdParams q = p;
  q.n_tiles = (p.Lq + 255) / 256;
  const int64_t total = (int64_t)q.n_tiles * p.H * p.B;
  if (total <= 0 || total > 0x7fffffff) return hipErrorInvalidValue;
  // Tail split by the rule the workspace was sized by (256-row query blocks, as the forward's).
  FwdSplit sp{(int)total, (int)total, 0, 1};
  if (p.dq_part != nullptr) sp = fwd_tail_split(p.B, p.Lq, p.H);
  if (sp.n != total) return hipErrorInvalidValue;
  if (sp.n_main > 0)
    hipLaunchKernelGGL(bwd_dq_kernel<false>, dim3((unsigned)sp.n_main), dim3(64 * DQ_WAVES), 0, stream, q);
  if (sp.tail > 0) {
    q.dq_base = sp.n_main;
    q.dq_split = sp.S;
    hipLaunchKernelGGL(bwd_dq_kernel<true>, dim3((unsigned)(sp.tail * sp.S)), dim3(64 * DQ_WAVES), 0, stream, q);
    hipLaunchKernelGGL(bwd_dq_reduce_kernel, dim3((unsigned)(sp.tail * 32)), dim3(256), 0, stream, q, sp.tail);
  }
  return hipGetLastError();
}

}  // namespace wanattn
