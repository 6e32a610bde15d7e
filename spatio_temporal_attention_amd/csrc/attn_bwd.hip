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

#include "bwd_common.h"
#include "validate.h"

namespace wanattn {

namespace {

using namespace bwd;

// dk~_j = scale sum_i dS_ij q~_i, dS_ij = P_ij (<dO_i, v_j> - Delta_i).
// Workgroup = 256 keys (8 waves, one workgroup per CU); query tiles staged
// as Q fp16 rows, dO rows and (R q)^T.  S = Q K^T and dP - Delta = dO V^T -
// Delta (the accumulator starts at -Delta of its rows) from the wave's K
// and V rows in registers; dK~^T += (R q)^T dS with dS from the accumulators.
template <bool KMASK, bool TAIL>
__global__ __launch_bounds__(64 * DK_WAVES, 1) void bwd_dk_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t q_lds0[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t q_lds1[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t do_lds0[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t do_lds1[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t qt_lds0[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t qt_lds1[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) float lse2_s0[TILE_ROWS];   // LSE * log2 e (+inf: no row)
  __shared__ __attribute__((aligned(16))) float lse2_s1[TILE_ROWS];
  __shared__ __attribute__((aligned(16))) float ndelta_s0[TILE_ROWS];   // -Delta
  __shared__ __attribute__((aligned(16))) float ndelta_s1[TILE_ROWS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const KeySide ks = key_side<DK_WAVES, KMASK, TAIL>(p, wv, col);

  bf16x8 kf[8], vf[8];   // K fp16 (bit patterns), V bf16: B operands of S and dP
  const int64_t ktile = ks.ktile0 + (ks.tile_ok ? ks.ktile : 0);
  load_row_frags(kf, p.kf + ktile * TILE_ELEMS, 32 * (wave & 1) + col, half, ks.tile_ok);
  load_row_frags(vf, p.vr + ktile * TILE_ELEMS, 32 * (wave & 1) + col, half, ks.tile_ok);
  const int e_k = ks.tile_ok ? p.kexp[ks.ktile0 + ks.ktile] : 0;

  f32x16 dk_acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) dk_acc[d] = f32x16{};
  const float* lse_row = p.lse + ((int64_t)ks.b * p.H + ks.h) * p.Lq;
  const float* delta_row = p.delta + ((int64_t)ks.b * p.H + ks.h) * p.Lq;

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
  const_i32* qexp = const_ptr(p.qexp + ks.tile0);   // scalar loads

  struct Buf {
    uint16_t* q;
    uint16_t* dO;
    uint16_t* qt;
    float* lse2;
    float* ndelta;
  };
  const Buf buf0{q_lds0, do_lds0, qt_lds0, lse2_s0, ndelta_s0};
  const Buf buf1{q_lds1, do_lds1, qt_lds1, lse2_s1, ndelta_s1};
  auto stage = [&](const Buf& dst, int t) {
    const uint32_t soff = (uint32_t)t * (TILE_ELEMS * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      buf_dma16(qfr, roff[i], soff, tile_lds_block<DK_WAVES>(dst.q, wv, i));
      buf_dma16(dor, roff[i], soff, tile_lds_block<DK_WAVES>(dst.dO, wv, i));
      buf_dma16(qtr, toff[i], soff, tile_lds_block<DK_WAVES>(dst.qt, wv, i));
    }
  };
  // Row statistics of query tile t: threads 0..63 read LSE, 64..127 Delta,
  // into a register, published to LDS once loaded.
  auto load_stats = [&](int t) {
    float x = 0.f;
    if (tid < TILE_ROWS) {
      const int i = t * TILE_ROWS + tid;
      x = (i < p.Lq) ? lse_row[i] : -INFINITY;
    } else if (tid < 2 * TILE_ROWS) {
      const int i = t * TILE_ROWS + tid - TILE_ROWS;
      x = (i < p.Lq) ? delta_row[i] : 0.f;
    }
    return x;
  };
  auto store_stats = [&](const Buf& dst, float x) {
    // rows past Lq, and rows with no valid key (LSE = -inf), contribute nothing
    if (tid < TILE_ROWS) dst.lse2[tid] = (x > -INFINITY) ? x * LOG2E : INFINITY;
    else if (tid < 2 * TILE_ROWS) dst.ndelta[tid - TILE_ROWS] = -x;
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
      // With a key mask, a wave whose 32 keys are all padding skips the products
      // (its gradients stay zero) but still copies its share and meets every barrier.
      if (!KMASK || ks.wave_live) {
      const float g = ldexpf(p.scale_log2, e_q + e_k);
      bf16x8 dsf[4];
  #pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        // rows qb*32 + 8m + 4*half + (0..3) of this tile: the accumulator's row order
        f32x16 s_acc = f32x16{}, dp_acc;
  #pragma unroll
        for (int m = 0; m < 4; ++m) {
          const f32x4 nd = *reinterpret_cast<const f32x4*>(cur.ndelta + qb * 32 + 8 * m + 4 * half);
  #pragma unroll
          for (int e = 0; e < 4; ++e) dp_acc[4 * m + e] = nd[e];
        }
  #pragma unroll
        for (int s = 0; s < 8; ++s) {
          s_acc = mfma32_f16(lds_row_frag(cur.q, qb * 32 + col, 2 * s + half), kf[s], s_acc);
          dp_acc = mfma32(lds_row_frag(cur.dO, qb * 32 + col, 2 * s + half), vf[s], dp_acc);
        }
        float dsv[16];
  #pragma unroll
        for (int m = 0; m < 4; ++m) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(cur.lse2 + qb * 32 + 8 * m + 4 * half);
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            float pe = __builtin_amdgcn_exp2f(fmaf(s_acc[4 * m + e], g, -l4[e]));
            if (KMASK && !ks.key_live) pe = 0.f;
            dsv[4 * m + e] = pe * dp_acc[4 * m + e];
          }
        }
        dsf[2 * qb] = pack_acc8(dsv);
        dsf[2 * qb + 1] = pack_acc8(dsv + 8);
      }
  #pragma unroll
      for (int d = 0; d < 4; ++d) {
  #pragma unroll
        for (int qg = 0; qg < 4; ++qg) dk_acc[d] = mfma32(lds_vt_frag(cur.qt, d * 32 + col, qg, half), dsf[qg], dk_acc[d]);
      }
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
// SPLIT: the tail launch (one key range of a query block, fp32 partial of dq~ out).
template <bool SPLIT>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t tiles[2][3][TILE_ELEMS];   // [buf][K fp16 | (Rk)^T | V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(wave);

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
  const int64_t stat = ((int64_t)b * p.H + h) * p.Lq + i;
  const float lse_i = row_ok ? p.lse[stat] : -INFINITY;
  const float lse2 = (lse_i > -INFINITY) ? lse_i * LOG2E : INFINITY;   // no valid key: P = 0
  const float delta = row_ok ? p.delta[stat] : 0.f;

  f32x16 dq_acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) dq_acc[d] = f32x16{};

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

  auto stage = [&](int buf, int t) {
    const uint32_t soff = (uint32_t)t * (TILE_ELEMS * 2);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      buf_dma16(kfr, roff[c], soff, tile_lds_block<DQ_WAVES>(tiles[buf][0], wv, c));
      buf_dma16(ktr, toff[c], soff, tile_lds_block<DQ_WAVES>(tiles[buf][1], wv, c));
      buf_dma16(vrr, roff[c], soff, tile_lds_block<DQ_WAVES>(tiles[buf][2], wv, c));
    }
  };

  int e_k = 0;
  if (t1 > t0) {
    stage(0, t0);
    e_k = kexp[t0];
  }
  wait_vmem();
  __syncthreads();

  // One 64-key tile; MASK: the last tile when L % 64 != 0 (keys >= L get P = 0).
  auto key_tile = [&](auto mask_tag, int t, int buf) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const uint16_t* ks = tiles[buf][0];
    const uint16_t* kts = tiles[buf][1];
    const uint16_t* vs = tiles[buf][2];
    const float g = ldexpf(p.scale_log2, e_q + e_k);
    bf16x8 dsf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s_acc = f32x16{}, dp_acc = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        s_acc = mfma32_f16(lds_row_frag(ks, kb * 32 + col, 2 * s + half), qf[s], s_acc);
        dp_acc = mfma32(lds_row_frag(vs, kb * 32 + col, 2 * s + half), dof[s], dp_acc);
      }
      float dsv[16];
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        float pe = __builtin_amdgcn_exp2f(fmaf(s_acc[jj], g, -lse2));
        if (MASK) {
          const int key = t * TILE_ROWS + kb * 32 + 8 * (jj >> 2) + 4 * half + (jj & 3);
          if (key >= n_keys) pe = 0.f;
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
        dq_acc[d] = mfma32(lds_vt_frag(kts, d * 32 + col, kg, half), dsf[kg], dq_acc[d]);
      }
    }
  };

  // Full tiles in the loop; a partial last tile is peeled off after it (only by the range that holds it:
  // an empty range, t0 == t1 == nkt, has n_full == t1).
  const int n_full = max(t0, min(n_keys / TILE_ROWS, t1));
  for (int t = t0; t < n_full; ++t) {
    const int buf = (t - t0) & 1;
    const bool has_next = t + 1 < t1;
    int e_k_next = 0;
    if (has_next) {
      stage(buf ^ 1, t + 1);
      e_k_next = kexp[t + 1];
    }
    key_tile(std::false_type{}, t, buf);
    if (has_next) wait_vmem();
    __syncthreads();
    e_k = e_k_next;
  }
  if (n_full < t1) key_tile(std::true_type{}, n_full, (n_full - t0) & 1);

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
