// Self-attention forward for gfx950 over the tiles the K/V prep pass writes
// (kv_prep.hip): full spatio-temporal attention with 3D RoPE, the rotation
// applied to the queries on load (keys arrive rotated).
//
// Computes, per (batch b, head h, query i), over the valid keys j < n_keys:
//   s_ij = scale <q~_i, k~_j>,  O_i = sum_j softmax_j(s_ij) v_j,  LSE_i = ln sum_j exp(s_ij)
// -- full spatio-temporal attention over latent patches ("Wan Team, Alibaba
// (2025)", Key takeaways, Backbone) with positions entering through 3D RoPE
// (Wan2.1 reading notes, 2. Model Design, DiT block paragraph).  The same
// kernel serves variable lengths (q_lens, k_lens) and key/query shards at
// token offsets (q_pos0, k_pos0: RoPE at global positions).
//
// Design (one workgroup = 8 waves = 256 query rows of one (b, h), one
// workgroup per CU, two waves per SIMD):
//  * each wave keeps its 32 rotated query rows in registers as the B operand
//    of S^T = K Q^T (MFMA 32x32x16), so every lane owns one query row;
//  * with RoPE the score product runs in fp16 (3 more mantissa bits than
//    bf16, same MFMA rate).  Each 64-row tile of rotated queries is scaled by
//    2^-e_q so that its largest |element| lies in [2^14, 2^15) and rounded to
//    fp16; the key prep pass does the same per 64-key tile (exponent e_t);
//    the softmax applies s = scale * 2^(e_q + e_t) * S.  The backward's prep
//    passes reproduce these fp16 operands bit for bit.  (Rounding the rotated
//    query to bf16 instead would move LSE by up to ~1.2e-3 at 720p: a query's
//    rounding error shifts all its scores coherently.)  Without RoPE the bf16
//    inputs are used as given;
//  * K tiles (64 keys, row-major) and V^T tiles (token order matching the
//    accumulator registers) go global -> LDS by buffer_load ... lds,
//    double-buffered; O^T += V^T P^T takes P straight from the S^T
//    accumulators (bf16, RNE) with plain 16-byte LDS reads of V^T;
//  * online softmax in fp32, log2 domain, with lazy rescaling that takes no
//    per-tile max (m moves only when a row's partial sum of P would exceed
//    2^16);
//  * ping-pong: each wave alternates a softmax phase (VALU) and a products
//    phase (MFMA: O += P(t) V(t), then the scores of tile t+1); waves 4..7
//    run one phase behind waves 0..3 and all eight meet at a barrier after
//    every phase, so on each SIMD (waves w and w + 4) one wave feeds the
//    matrix cores while the other runs its softmax;
//  * the main launches take their query tiles from a work counter in the
//    workspace, head-major with the batch item innermost: the XCDs of a chip
//    run at unequal speeds, and the faster ones take more tiles (common.h);
//    without a counter (the split's own launch) workgroups are ordered
//    XCD-aware, so the resident workgroups of one XCD walk the same head's
//    K/V tiles through its L2;
//  * fixed lengths: the last query tiles run as key ranges at the end of the
//    main launch, whose fp32 partials a merge pass combines exactly.
// Built with the iterative ILP machine scheduler (build flags of this file):
// with the default one the products phase reads each LDS fragment just before
// its MFMA.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "validate.h"

namespace wanattn {

namespace {

constexpr int FWD_BC = TILE_ROWS;         // keys per tile
constexpr float PSUM_LIMIT = 65536.0f;    // largest partial row sum of P kept without a rescale

// Phase schedule:
//   barrier k:  waves 0..3 have finished their phase k, waves 4..7 phase k-1
//   (phase 2t = softmax(t), phase 2t+1 = products(t)).
// K(t+1) and V(t) are read during products(t) (between barriers 2t and 2t+2
// over both groups).  K(t+2) and V(t+1) go into the buffers K(t) and V(t-1)
// leave, 1/8 of each tile per wave, all issued after barrier 2t: the early
// waves at the start of their products phase, the late waves at the start
// of their softmax phase (the shorter phase); each wave waits for its own
// copies before the barrier that ends its products phase (2t+1 and 2t+2),
// before anyone reads them (products(t+1), after barrier 2t+2).  Both groups
// run the same code; the late waves add a barrier before their first phase,
// the early ones one after their last.
constexpr int PP_WAVES = 8;
constexpr int PP_BR = 32 * PP_WAVES;   // query rows per workgroup
static_assert(PP_BR == FWD_ROWS, "the tail split and its workspace assume 256-row workgroups");

// SPLIT: the tail launch (one key range of a query tile, fp32 partial out).
// The main launch with fixed lengths and 8 waves (UNI below) also runs the
// pieces itself, as its workgroups from p.n_main_wg on, after the whole tiles.
// VARLEN: the main launch with variable lengths, where a workgroup whose query
// tile lies wholly past its item's length leaves at once (an instantiation of
// its own, so the fixed-length code is unaffected).
// NW: waves per workgroup.  8: the ping-pong pairs above, one workgroup per
// CU.  4 (short key sequences such as the text context, 128 query rows): no
// phase offset inside the workgroup; two workgroups share each CU, so one
// loads its queries or stores its output while the other computes.
template <bool POS_SCALE, bool F16, bool SPLIT, bool VARLEN, int NW = PP_WAVES>
// Two waves per SIMD by design; without the explicit target the compiler aims
// for four (the LDS would allow more) and schedules for register pressure
// instead of latency.
__global__ __launch_bounds__(64 * NW, 8 / NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_pp_kernel(
    FwdParams p) {
  static_assert(NW == 8 || NW == 4, "8 ping-pong waves or 4 plain ones");
  constexpr int BR = 32 * NW;          // query rows per workgroup
  constexpr int NCP = 16 / NW;         // 1 KB copies per wave of every K and V tile
  __shared__ __attribute__((aligned(16))) uint16_t k_lds0[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t k_lds1[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds0[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds1[TILE_ELEMS];
  __shared__ float qmax_s[NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const bool late = NW == 8 && wv >= NW / 2;   // waves 4..7: one phase behind

  constexpr bool UNI = !SPLIT && !VARLEN && NW == 8;
  // With p.work (the main launches, fixed or variable lengths) the workgroup
  // takes its item from that counter (take_work_item), below p.n_items: items
  // below p.n_main_wg are whole query tiles (logical order), item
  // p.n_main_wg + k is piece k (fixed lengths only).
  int item = (int)blockIdx.x;
  const bool counted = !SPLIT && NW == 8 && p.work != nullptr;
  if (counted) {
    item = take_work_item(p.work);
    if (item >= p.n_items) return;   // the whole workgroup: item is uniform
  }
  int logical, split = 0, piece_idx = 0;
  bool piece = SPLIT;
  if (SPLIT) {
    piece_idx = item;
    logical = p.qt_base + piece_idx / p.n_split;
    split = piece_idx % p.n_split;
  } else if (UNI && item >= p.n_main_wg) {
    piece = true;
    piece_idx = item - p.n_main_wg;
    logical = p.qt_base + piece_idx / p.n_split;
    split = piece_idx % p.n_split;
  } else {
    logical = counted ? item : xcd_remap(item, UNI ? p.n_main_wg : (int)gridDim.x);
  }
  const int qt = logical % p.n_qtiles;
  const int bh = logical / p.n_qtiles;
  const int b = bh % p.B;   // batch innermost: every XCD gets the same heads of every item
  const int h = bh / p.B;

  int n_keys = p.Lk;
  if (p.k_lens != nullptr) n_keys = min(max(p.k_lens[b], 0), p.Lk);
  const int64_t q_row_stride = (int64_t)p.H * HD;
  const uint16_t* qbase = p.q + ((int64_t)b * p.Lq * p.H + h) * HD;
  const int nkt = (p.Lk + FWD_BC - 1) / FWD_BC;
  const int64_t tile0 = (int64_t)(b * p.H + h) * nkt;

  const int i = qt * BR + wave * 32 + col;
  int n_q = p.Lq;
  if (p.q_lens != nullptr) n_q = min(max(p.q_lens[b], 0), p.Lq);
  const bool row_ok = i < n_q;
  if (VARLEN && qt * BR >= n_q) return;   // uniform over the workgroup; nothing to compute or store
  bf16x8 qf[8];
  float g_q = p.scale_log2;
  {
    TokenPos pos{0, 0, 0};
    if (p.rope.table != nullptr && row_ok) pos = token_pos(p.rope, p.q_pos0 + i);
    if (F16) {
      float y[8][8];
      float mq = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int c = 2 * s + half;
        u32x4 x = u32x4{0u, 0u, 0u, 0u};
        if (row_ok) x = *reinterpret_cast<const u32x4*>(qbase + (int64_t)i * q_row_stride + c * 8);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float y0 = bf16_lo(x[t]);
          float y1 = bf16_hi(x[t]);
          if (row_ok) rope_rotate(y0, y1, rope_cs(p.rope, pos, 4 * c + t), false);
          y[s][2 * t] = y0;
          y[s][2 * t + 1] = y1;
          mq = fmaxf(mq, fmaxf(fabsf(y0), fabsf(y1)));
        }
      }
      // One exponent per 64-row query tile (waves 2u and 2u+1).
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) mq = fmaxf(mq, __shfl_xor(mq, o));
      if (lane == 0) qmax_s[wave] = mq;
      __syncthreads();
      const int e_q = pow2_exponent_15(fmaxf(qmax_s[wave & ~1], qmax_s[wave | 1]));
      g_q = ldexpf(p.scale_log2, e_q);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        u32x4 w;
#pragma unroll
        for (int t = 0; t < 4; ++t) w[t] = pack_f16(ldexpf(y[s][2 * t], -e_q), ldexpf(y[s][2 * t + 1], -e_q));
        qf[s] = __builtin_bit_cast(bf16x8, w);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        u32x4 x = u32x4{0u, 0u, 0u, 0u};
        const int c = 2 * s + half;
        if (row_ok) {
          x = *reinterpret_cast<const u32x4*>(qbase + (int64_t)i * q_row_stride + c * 8);
          if (p.rope.table != nullptr) x = rope_chunk(p.rope, pos, c, x, false);
        }
        qf[s] = __builtin_bit_cast(bf16x8, x);
      }
    }
  }

  f32x16 o_acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o_acc[d] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const_i32* kexp = F16 ? const_ptr(p.kexp + tile0) : nullptr;   // scalar loads
  const int n_tiles = (n_keys + FWD_BC - 1) / FWD_BC;
  // Key tiles [t_begin, t_end): all of them, or one of p.n_split ranges.
  int t_begin = 0, t_end = n_tiles;
  if (piece) {
    const int chunk = (n_tiles + p.n_split - 1) / p.n_split;
    t_begin = min(n_tiles, split * chunk);
    t_end = min(n_tiles, t_begin + chunk);
  }

  if (t_end > t_begin) {
    // Each wave copies 1/NW of every K and V tile (NCP x 1 KB each).
    uint32_t koff[NCP], voff[NCP];
#pragma unroll
    for (int c = 0; c < NCP; ++c) {
      koff[c] = rowtile_lane_off<NW>(wv, c, lane);
      voff[c] = ttile_lane_off<NW>(wv, c, lane);
    }
    const uint32_t bytes = (uint32_t)nkt * (TILE_ELEMS * 2);   // < 2^32, checked by the launcher
    const __amdgpu_buffer_rsrc_t krs = tile_rsrc(p.kt + tile0 * TILE_ELEMS, bytes);
    const __amdgpu_buffer_rsrc_t vrs = tile_rsrc(p.vt + tile0 * TILE_ELEMS, bytes);
    auto stage_k = [&](uint16_t* dst, int t) {
#pragma unroll
      for (int c = 0; c < NCP; ++c)
        buf_dma16(krs, koff[c], (uint32_t)t * (TILE_ELEMS * 2), tile_lds_block<NW>(dst, wv, c));
    };
    auto stage_v = [&](uint16_t* dst, int t) {
#pragma unroll
      for (int c = 0; c < NCP; ++c)
        buf_dma16(vrs, voff[c], (uint32_t)t * (TILE_ELEMS * 2), tile_lds_block<NW>(dst, wv, c));
    };

    f32x16 s_acc[2];
    auto scores = [&](const uint16_t* ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s_acc[kb] = f32x16{};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const bf16x8 a = lds_row_frag(ks, kb * 32 + col, 2 * s + half);
          s_acc[kb] = F16 ? mfma32_f16(a, qf[s], s_acc[kb]) : mfma32(a, qf[s], s_acc[kb]);
        }
      }
    };

    // Softmax of tile t (VALU phase): P into pf.  MASK: the partial last tile.
    bf16x8 pf[4];
    auto softmax = [&](auto mask_tag, int t, int e_t) {
      constexpr bool MASK = decltype(mask_tag)::value;
      const float g = F16 ? ldexpf(g_q, e_t) : g_q;
      float sv[2][16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          float x = POS_SCALE ? s_acc[kb][j] : s_acc[kb][j] * g;
          if (MASK) {
            const int key = t * FWD_BC + kb * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
            if (key >= n_keys) x = -INFINITY;
          }
          sv[kb][j] = x;
        }
      }
      float psum;
      auto exps = [&]() {
        float part[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          float pv[16];
          part[kb] = 0.f;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            if (POS_SCALE) pv[j] = __builtin_amdgcn_exp2f(fmaf(sv[kb][j], g, -m_run));
            else pv[j] = __builtin_amdgcn_exp2f(sv[kb][j] - m_run);
            part[kb] += pv[j];
          }
          pf[2 * kb] = pack_acc8(pv);
          pf[2 * kb + 1] = pack_acc8(pv + 8);
        }
        psum = part[0] + part[1];
      };
      exps();
      // Lazy rescaling without a per-tile max: while every row's partial
      // sum (32 of its P) stays <= PSUM_LIMIT, so does every P, and the tile
      // is kept (scores up to m + 11 in log2 units always are); otherwise (a
      // larger score, the first tile with m = -inf, a non-finite sum) m moves
      // up to the exact tile max, O and l are rescaled and P is recomputed.
      // Exact either way: O / l and LSE = m + log2 l use the m applied.
      if (__any(!(psum <= PSUM_LIMIT))) {
        float mx = sv[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sv[kb][j]);
        mx = xor32_max(mx);
        if (POS_SCALE) mx *= g;
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < 4; ++d) o_acc[d] *= alpha;
        exps();
      }
      l_run += psum;
    };

    // O^T += V^T P^T (MFMA phase, first half).
    auto pv_product = [&](const uint16_t* vs) {
#pragma unroll
      for (int hd = 0; hd < 2; ++hd) {
        bf16x8 a[2][4];
#pragma unroll
        for (int d = 0; d < 2; ++d)
#pragma unroll
          for (int kg = 0; kg < 4; ++kg) a[d][kg] = lds_vt_frag(vs, (2 * hd + d) * 32 + col, kg, half);
#pragma unroll
        for (int kg = 0; kg < 4; ++kg)
#pragma unroll
          for (int d = 0; d < 2; ++d) o_acc[2 * hd + d] = mfma32(a[d][kg], pf[kg], o_acc[2 * hd + d]);
      }
    };

    // Prologue: K(0), V(0), K(1) staged; S(0) by every wave.
    stage_k(k_lds0, t_begin);
    stage_v(v_lds0, t_begin);
    if (t_begin + 1 < t_end) stage_k(k_lds1, t_begin + 1);
    int e_nxt = F16 ? kexp[t_begin] : 0;   // exponent of the next tile to take its softmax
    wait_vmem();
    __syncthreads();
    scores(k_lds0);
    const int last = t_end - 1;
    const bool partial = n_keys % FWD_BC != 0 && t_end == n_tiles;   // only the last key tile is partial
    if (late) __syncthreads();   // the early waves run softmax(0) meanwhile

    // Tile t with parity P = t & 1: K(t+1) in K buffer 1-P, V(t) in V buffer
    // P; K(t+2) is copied into K buffer P, V(t+1) into V buffer 1-P.
    auto tile = [&](auto parity, int t) {
      constexpr int P = decltype(parity)::value;
      uint16_t* const k_fill = P ? k_lds1 : k_lds0;
      const uint16_t* const k_next = P ? k_lds0 : k_lds1;
      const uint16_t* const v_cur = P ? v_lds1 : v_lds0;
      uint16_t* const v_fill = P ? v_lds0 : v_lds1;
      // The late waves issue their copies in this softmax phase (after
      // barrier 2t), the early ones in their products phase; each waits for
      // its own before the barrier that ends its products phase.
      if (late) {
        if (t + 2 < t_end) stage_k(k_fill, t + 2);
        if (t + 1 < t_end) stage_v(v_fill, t + 1);
      }
      // Tile t's exponent was loaded one tile earlier; load tile t+1's now
      // (scalar load, needed after two barriers).
      const int e_t = e_nxt;
      if (F16 && t + 1 < t_end) e_nxt = kexp[t + 1];
      if constexpr (POS_SCALE) {
        // The partial last tile: keys past n_keys get a score of -inf in
        // place (exact under the positive factor), so one softmax serves
        // every tile (a second, masked copy costs ~50 VGPRs).
        if (partial && t == last) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int key = t * FWD_BC + kb * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
              if (key >= n_keys) s_acc[kb][j] = -INFINITY;
            }
        }
        softmax(std::false_type{}, t, e_t);
      } else {
        if (partial && t == last) softmax(std::true_type{}, t, e_t);
        else softmax(std::false_type{}, t, e_t);
      }
      __syncthreads();   // barrier 2t (early waves), 2t+1 (late waves)
      if (!late) {
        if (t + 2 < t_end) stage_k(k_fill, t + 2);
        if (t + 1 < t_end) stage_v(v_fill, t + 1);
      }
      pv_product(v_cur);
      if (t < last) {
        scores(k_next);
        // Keep four fragment reads in flight ahead of the MFMAs.
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int k = 0; k < 28; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        wait_vmem();
        __syncthreads();   // barrier 2t+1 (early), 2t+2 (late)
      }
    };
    int t = t_begin;
    for (; t + 1 < t_end; t += 2) {
      tile(std::integral_constant<int, 0>{}, t);
      tile(std::integral_constant<int, 1>{}, t + 1);
    }
    if (t < t_end) tile(std::integral_constant<int, 0>{}, t);
    if (!late) __syncthreads();   // matches the late waves' barrier before their last products phase
  }

  const float l_tot = xor32_sum(l_run);
  if (piece) {
    // Partial of this key range: O unnormalized, the running max m (log2
    // units; -inf for an empty range) and l = sum of P against it.
    float* dst = p.part + ((int64_t)piece_idx * BR + wave * 32 + col) * FWD_PART_FLOATS;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq)
        *reinterpret_cast<f32x4*>(dst + d * 32 + 8 * jq + 4 * half) =
            f32x4{o_acc[d][4 * jq], o_acc[d][4 * jq + 1], o_acc[d][4 * jq + 2], o_acc[d][4 * jq + 3]};
    if (half == 0) {
      dst[128] = m_run;
      dst[129] = l_tot;
    }
  } else if (row_ok) {
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    uint16_t* orow = p.o + ((int64_t)b * p.Lq * p.H + h) * HD + (int64_t)i * q_row_stride;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        u32x2 w;
        w[0] = pack_bf16(o_acc[d][4 * jq] * inv, o_acc[d][4 * jq + 1] * inv);
        w[1] = pack_bf16(o_acc[d][4 * jq + 2] * inv, o_acc[d][4 * jq + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d * 32 + 8 * jq + 4 * half) = w;
      }
    }
    if (p.lse != nullptr && half == 0) {
      const float lse = (l_tot > 0.f) ? (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f : -INFINITY;
      p.lse[((int64_t)b * p.H + h) * p.Lq + i] = lse;
    }
  }
}

// Merge of the tail split's partials: per query row, m = max over the key
// ranges of m_s, l = sum_s l_s 2^(m_s - m), O = sum_s O_s 2^(m_s - m) / l and
// LSE = ln 2 (m + log2 l) (fixed order over s).  One thread per row and four
// head-dim columns.
__global__ __launch_bounds__(256) void fwd_split_merge_kernel(FwdParams p, int tail) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int c4 = (int)(idx & 31);
  const int64_t rr = idx >> 5;
  const int rl = (int)(rr % PP_BR);
  const int ti = (int)(rr / PP_BR);
  if (ti >= tail) return;
  const int logical = p.qt_base + ti;
  const int qt = logical % p.n_qtiles;
  const int bh = logical / p.n_qtiles;
  const int b = bh % p.B;
  const int h = bh / p.B;
  int n_q = p.Lq;
  if (p.q_lens != nullptr) n_q = min(max(p.q_lens[b], 0), p.Lq);
  const int i = qt * PP_BR + rl;
  if (i >= n_q) return;
  const int64_t stride = (int64_t)PP_BR * FWD_PART_FLOATS;
  const float* base = p.part + ((int64_t)ti * p.n_split * PP_BR + rl) * FWD_PART_FLOATS;
  float m = -INFINITY;
  for (int s = 0; s < p.n_split; ++s) m = fmaxf(m, base[s * stride + 128]);
  float l = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  if (m > -INFINITY) {
    for (int s = 0; s < p.n_split; ++s) {
      const float w = __builtin_amdgcn_exp2f(base[s * stride + 128] - m);   // 0 for an empty range
      l += base[s * stride + 129] * w;
      const f32x4 o4 = *reinterpret_cast<const f32x4*>(base + s * stride + 4 * c4);
      acc += o4 * w;
    }
  }
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  u32x2 w2;
  w2[0] = pack_bf16(acc[0] * inv, acc[1] * inv);
  w2[1] = pack_bf16(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<u32x2*>(p.o + (((int64_t)b * p.Lq + i) * p.H + h) * HD + 4 * c4) = w2;
  if (c4 == 0 && p.lse != nullptr)
    p.lse[((int64_t)b * p.H + h) * p.Lq + i] = (l > 0.f) ? (m + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

hipError_t launch_attn_fwd_tiled(const FwdParams& p, hipStream_t stream) {
  if (p.kt == nullptr || p.vt == nullptr) return hipErrorInvalidValue;
  // The tiles of one (b, h) are addressed through a buffer resource of 32-bit extent.
  if ((int64_t)((p.Lk + FWD_BC - 1) / FWD_BC) * (TILE_ELEMS * 2) > (int64_t)0xffffffff) return hipErrorInvalidValue;
  const bool f16 = p.rope.table != nullptr;   // fp16 scores against the fp16 key tiles
  if (f16 && p.kexp == nullptr) return hipErrorInvalidValue;
  FwdParams r = p;
  // Short key sequences (at most 8 tiles: the text context), without a tail split or variable query
  // lengths: 4-wave workgroups of 128 query rows, two per CU.
  const bool short_keys = p.part == nullptr && p.q_lens == nullptr && !f16 && (p.Lk + FWD_BC - 1) / FWD_BC <= 8;
  if (short_keys) {
    r.n_qtiles = (p.Lq + 127) / 128;
    const int64_t n4 = (int64_t)r.n_qtiles * p.H * p.B;
    if (n4 <= 0 || n4 > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)n4);
    if (p.scale_log2 > 0.f) hipLaunchKernelGGL((attn_fwd_pp_kernel<true, false, false, false, 4>), grid, dim3(256), 0, stream, r);
    else hipLaunchKernelGGL((attn_fwd_pp_kernel<false, false, false, false, 4>), grid, dim3(256), 0, stream, r);
    return hipGetLastError();
  }
  r.n_qtiles = (p.Lq + PP_BR - 1) / PP_BR;
  const int64_t n = (int64_t)r.n_qtiles * p.H * p.B;
  if (n <= 0 || n > 0x7fffffff) return hipErrorInvalidValue;
  // Fixed lengths: one launch, whose last workgroups run the split pieces
  // (fwd_split, the rule the workspace was sized by).  Variable lengths: a
  // main launch, then the pieces of fwd_tail_split's tail in a launch of
  // their own.
  const bool uni = p.q_lens == nullptr;
  FwdSplit sp{(int)n, (int)n, 0, 1};
  if (p.part != nullptr) sp = uni ? fwd_split(p.B, p.Lq, p.H) : fwd_tail_split(p.B, p.Lq, p.H);
  if (sp.n != n) return hipErrorInvalidValue;
  r.n_main_wg = sp.n_main;
  r.qt_base = sp.n_main;
  r.n_split = sp.S;
  const bool pos = p.scale_log2 > 0.f;
  const dim3 block(64 * PP_WAVES);
  if (uni) {
    const int64_t total = (int64_t)sp.n_main + (int64_t)sp.tail * sp.S;
    if (total > 0x7fffffff) return hipErrorInvalidValue;
    r.n_items = (int)total;
    int64_t wgs = total;
    if (r.work != nullptr) {
      if (!work_fits(total)) return hipErrorInvalidValue;
      wgs = work_grid(total);
      hipLaunchKernelGGL(work_reset_kernel, dim3(1), dim3(1), 0, stream, r.work);
    }
    const dim3 grid((unsigned)wgs);
    if (pos) {
      if (f16) hipLaunchKernelGGL((attn_fwd_pp_kernel<true, true, false, false>), grid, block, 0, stream, r);
      else hipLaunchKernelGGL((attn_fwd_pp_kernel<true, false, false, false>), grid, block, 0, stream, r);
    } else {
      if (f16) hipLaunchKernelGGL((attn_fwd_pp_kernel<false, true, false, false>), grid, block, 0, stream, r);
      else hipLaunchKernelGGL((attn_fwd_pp_kernel<false, false, false, false>), grid, block, 0, stream, r);
    }
  } else {
    if (sp.n_main > 0) {
      FwdParams m = r;
      m.n_items = sp.n_main;
      int64_t wgs = sp.n_main;
      if (m.work != nullptr) {
        if (!work_fits(sp.n_main)) return hipErrorInvalidValue;
        wgs = work_grid(sp.n_main);
        hipLaunchKernelGGL(work_reset_kernel, dim3(1), dim3(1), 0, stream, m.work);
      }
      const dim3 grid((unsigned)wgs);
      if (pos) {
        if (f16) hipLaunchKernelGGL((attn_fwd_pp_kernel<true, true, false, true>), grid, block, 0, stream, m);
        else hipLaunchKernelGGL((attn_fwd_pp_kernel<true, false, false, true>), grid, block, 0, stream, m);
      } else {
        if (f16) hipLaunchKernelGGL((attn_fwd_pp_kernel<false, true, false, true>), grid, block, 0, stream, m);
        else hipLaunchKernelGGL((attn_fwd_pp_kernel<false, false, false, true>), grid, block, 0, stream, m);
      }
    }
    if (sp.tail > 0) {
      const dim3 grid((unsigned)(sp.tail * sp.S));
      if (pos) {
        if (f16) hipLaunchKernelGGL((attn_fwd_pp_kernel<true, true, true, false>), grid, block, 0, stream, r);
        else hipLaunchKernelGGL((attn_fwd_pp_kernel<true, false, true, false>), grid, block, 0, stream, r);
      } else {
        if (f16) hipLaunchKernelGGL((attn_fwd_pp_kernel<false, true, true, false>), grid, block, 0, stream, r);
        else hipLaunchKernelGGL((attn_fwd_pp_kernel<false, false, true, false>), grid, block, 0, stream, r);
      }
    }
  }
  if (sp.tail > 0)
    hipLaunchKernelGGL(fwd_split_merge_kernel, dim3((unsigned)(sp.tail * (PP_BR * 32 / 256))), dim3(256), 0, stream,
                       r, sp.tail);
  return hipGetLastError();
}

}  // namespace wanattn
