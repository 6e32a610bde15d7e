// Attention forward for gfx950: full self-attention with 3D RoPE on the query
// load (keys arrive already rotated), and masked cross-attention, sharing one
// kernel.
//
// Computes, per (batch b, head h, query i), over the valid keys j < n_keys:
//   s_ij = scale <q~_i, k~_j>,  O_i = sum_j softmax_j(s_ij) v_j,  LSE_i = ln sum_j exp(s_ij)
// -- full spatio-temporal attention over latent patches ("Wan Team, Alibaba
// (2025)", Key takeaways, Backbone) with positions entering through 3D RoPE
// (Wan2.1 reading notes, 2. Model Design, DiT block paragraph).
//
// Design (one workgroup = 4 waves = 128 query rows of one (b, h)):
//  * each wave keeps its 32 rotated query rows in registers as the B operand
//    of S^T = K Q^T (bf16 MFMA 32x32x16), so every lane owns one query row and
//    the softmax needs one cross-lane step (lane l <-> l^32) per tile;
//  * F16 (with RoPE): the score product runs in fp16 (3 more mantissa bits
//    than bf16, same MFMA rate).  Each 64-row tile of rotated queries is
//    scaled by 2^-e_q so that its largest |element| lies in [2^14, 2^15) and
//    rounded to fp16; the key pre-pass does the same per 64-key tile
//    (exponent e_t); the softmax applies s = scale * 2^(e_q + e_t) * S.  The
//    backward's prep passes reproduce these fp16 operands bit for bit.  Rounding the rotated
//    query to bf16 instead would move LSE by up to ~1.2e-3 at 720p: a query's
//    rounding error shifts all its scores coherently; in fp16 it is 8x
//    smaller.  Without RoPE the inputs are used as given (bf16, exact);
//  * K and V tiles of 64 keys go global -> LDS directly (global_load_lds,
//    row-major, swizzled), double-buffered: the next tile's loads are in
//    flight while the current one is multiplied;
//  * O^T += V^T P^T takes P straight from the S^T accumulator registers
//    (bf16, RNE).  Self-attention reads V from V^T tiles written by a
//    pre-pass (v_tiles_kernel), one plain 16-byte LDS read per fragment; the
//    LDS transpose read (ds_read_b64_tr_b16) moves under half as many bytes
//    per clock and would make the loop LDS-bound.  Cross-attention (a short
//    text context, no workspace) keeps the transpose read;
//  * online softmax in fp32 in the log2 domain (scale * log2 e folded in),
//    with lazy rescaling of O and l: no per-tile max, m moves only when a
//    row's partial sum of P would exceed 2^16;
//  * workgroups are ordered head-major and XCD-aware so that the resident
//    workgroups of one XCD walk the same head's K/V through its L2.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace wanattn {

namespace {

constexpr int FWD_WAVES = 4;
constexpr int FWD_BR = 32 * FWD_WAVES;   // query rows per workgroup
constexpr int FWD_BC = TILE_ROWS;         // keys per tile
constexpr float PSUM_LIMIT = 65536.0f;    // largest partial row sum of P kept without a rescale

template <bool POS_SCALE, bool F16, bool TILED>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(FwdParams p) {
  // Two K and two V buffers as four separate objects: every access in the
  // (two-way unrolled) loop names its buffer statically, which lets the
  // compiler see that the ds_reads of one buffer do not depend on the DMA
  // copies in flight into another (otherwise each LDS read would wait for
  // all of them).
  __shared__ __attribute__((aligned(16))) uint16_t k_lds0[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t k_lds1[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds0[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds1[TILE_ELEMS];
  __shared__ float qmax_s[FWD_WAVES];                                        // F16: max |q~| per wave

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;       // which 32-lane half
  const int col = lane & 31;        // query row of this lane within the wave

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = logical % p.n_qtiles;
  const int bh = logical / p.n_qtiles;
  const int b = bh % p.B;   // batch innermost: every XCD gets the same heads of every item
  const int h = bh / p.B;

  int n_keys = p.Lk;
  if (p.k_lens != nullptr) n_keys = min(max(p.k_lens[b], 0), p.Lk);

  const int64_t q_row_stride = (int64_t)p.H * HD;
  const uint16_t* qbase = p.q + ((int64_t)b * p.Lq * p.H + h) * HD;
  const uint16_t* kbase = p.k + ((int64_t)b * p.Lk * p.H + h) * HD;
  const uint16_t* vbase = p.v + ((int64_t)b * p.Lk * p.H + h) * HD;
  // Tiled keys/values (self-attention): tile t of (b, h) is contiguous.
  const int nkt = (p.Lk + FWD_BC - 1) / FWD_BC;
  const int64_t tile0 = (int64_t)(b * p.H + h) * nkt;

  // ---- query fragments (B operand of S^T = K Q^T): lane holds row i, d in [16s + 8*half, +8)
  const int i = qt * FWD_BR + wave * 32 + col;
  int n_q = p.Lq;
  if (p.q_lens != nullptr) n_q = min(max(p.q_lens[b], 0), p.Lq);
  const bool row_ok = i < n_q;
  bf16x8 qf[8];       // F16: fp16 bit patterns
  float g_q = p.scale_log2;   // score factor of this wave: s * log2(e) = g_q * 2^e_t * S
  {
    TokenPos pos{0, 0, 0};
    if (p.rope.table != nullptr && row_ok) pos = token_pos(p.rope, p.q_pos0 + i);
    if (F16) {
      float y[8][8];   // rotated query, fp32
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
      // One exponent per 64-row query tile (waves 2u and 2u+1): the largest
      // |q~| of the tile goes to [2^14, 2^15).
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
  float m_run = -INFINITY;   // running max of scale*log2e*s (this lane's row)
  float l_run = 0.f;         // this lane's partial exp-sum (the other half holds the rest)
  // e_t of each key tile (scalar loads)
  const_i32* kexp = F16 ? const_ptr(p.kexp + tile0) : nullptr;

  const int n_tiles = (n_keys + FWD_BC - 1) / FWD_BC;

  // S^T of one 64-key tile (64 keys x 32 queries) as two 32x32 blocks.
  auto scores = [&](const uint16_t* ks, f32x16 (&s_acc)[2]) {
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

  // Online softmax of tile t's scores and O += P V.  MASK: the last tile,
  // whose keys past n_keys get -inf (full tiles carry no masking code).
  // NEXT: also compute the next tile's scores (from next_ks into s_nxt) in
  // the same basic block as this tile's exponentials (after the rescale
  // branch), so the scheduler can interleave them: one wave issues in
  // order, and the MFMAs only overlap VALU work placed between them.
  auto softmax_pv = [&](auto mask_tag, auto next_tag, f32x16 (&s_acc)[2], const uint16_t* vs, int t, int e_t,
                        const uint16_t* next_ks, f32x16 (&s_nxt)[2]) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool NEXT = decltype(next_tag)::value;
    // log2-domain factor of this tile's raw scores
    const float g = F16 ? ldexpf(g_q, e_t) : g_q;

    // Scores: raw for a positive scale, otherwise already scaled to the log2 domain.
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

    if (NEXT) scores(next_ks, s_nxt);

    // P = 2^(s - m) against the running max m, in fp32 (l sums these; P is
    // rounded to bf16, RNE, only for the P V product: summing the rounded
    // values instead would move LSE by up to ~2^-9 when few keys dominate).
    bf16x8 pf[4];
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

    // Lazy rescaling without a per-tile max: m only has to keep P finite
    // and bounded.  While every row's partial sum (32 of its P) stays <=
    // PSUM_LIMIT = 2^16, so does every P, and the tile is kept as computed;
    // scores up to m + 11 (log2 units) always stay on this path.  Otherwise
    // (a larger score, the first tile with m = -inf, or a non-finite sum)
    // the exact tile max is taken, m moves up to it, O and l are rescaled
    // and P is recomputed.  Exact either way: the final O / l and
    // LSE = m + log2 l use the m that was applied.
    if (__any(!(psum <= PSUM_LIMIT))) {
      float mx = sv[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sv[kb][j]);
      mx = xor32_max(mx);
      if (POS_SCALE) mx *= g;   // max(s) * g == max(s * g) for g > 0
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 while m was -inf
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < 4; ++d) o_acc[d] *= alpha;
      exps();
    }
    l_run += psum;

    // O^T (128 d x 32 queries) += V^T P^T over the 4 groups of 16 keys.
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int kg = 0; kg < 4; ++kg) {
        const bf16x8 a = TILED ? lds_vt_frag(vs, d * 32 + col, kg, half) : lds_col_frag(vs, kg * 16, d * 32, lane);
        o_acc[d] = mfma32(a, pf[kg], o_acc[d]);
      }
    }
  };

  if (n_tiles > 0) {
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    uint32_t koff[4], voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      koff[i] = rowtile_lane_off<FWD_WAVES>(wv, i, lane);
      voff[i] = ttile_lane_off<FWD_WAVES>(wv, i, lane);
    }
    const uint32_t bytes = (uint32_t)nkt * (TILE_ELEMS * 2);   // < 2^32, checked by the launcher
    const __amdgpu_buffer_rsrc_t krs = tile_rsrc(TILED ? p.kt + tile0 * TILE_ELEMS : p.k, bytes);
    const __amdgpu_buffer_rsrc_t vrs = tile_rsrc(TILED ? p.vt + tile0 * TILE_ELEMS : p.v, bytes);
    // Stage tile t of K (V) into the LDS buffer `dst`.
    auto stage_k = [&](uint16_t* dst, int t) {
      if (TILED) {
        const uint32_t soff = (uint32_t)t * (TILE_ELEMS * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) buf_dma16(krs, koff[i], soff, tile_lds_block<FWD_WAVES>(dst, wv, i));
      } else {
        tile_dma(dst, kbase, q_row_stride, t * FWD_BC, n_keys, wv, lane);
      }
    };
    auto stage_v = [&](uint16_t* dst, int t) {
      if (TILED) {
        const uint32_t soff = (uint32_t)t * (TILE_ELEMS * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) buf_dma16(vrs, voff[i], soff, tile_lds_block<FWD_WAVES>(dst, wv, i));
      } else {
        tile_dma(dst, vbase, q_row_stride, t * FWD_BC, n_keys, wv, lane);
      }
    };
    // Software pipeline: iteration t computes the scores of tile t+1 (MFMA)
    // while the softmax of tile t (VALU) runs, then O += P(t) V(t).  K runs
    // one tile ahead of V: iteration t copies K(t+2) and V(t+1) into the
    // buffers K(t) and V(t-1) have left.  A tile's exponent is loaded with
    // its copies, so the wait that ends the previous iteration covers it.
    stage_k(k_lds0, 0);
    stage_v(v_lds0, 0);
    int e_cur = F16 ? kexp[0] : 0;
    int e_nxt = 0;
    if (n_tiles > 1) {
      stage_k(k_lds1, 1);
      if (F16) e_nxt = kexp[1];
    }
    wait_vmem();
    __syncthreads();
    f32x16 s_a[2], s_b[2];
    scores(k_lds0, s_a);
    __syncthreads();   // K buffer 0 is refilled in iteration 0
    const int last = n_tiles - 1;
    // Iteration t (parity P = t & 1): scores of tile t are in s_in, K(t+1)
    // is in K buffer 1-P, V(t) in V buffer P; K(t+2) goes into K buffer P
    // and V(t+1) into V buffer 1-P.
    auto iteration = [&](auto parity, int t, f32x16 (&s_in)[2], f32x16 (&s_out)[2]) {
      const int P = parity;
      uint16_t* const k_fill = P ? k_lds1 : k_lds0;
      const uint16_t* const k_next = P ? k_lds0 : k_lds1;
      const uint16_t* const v_cur = P ? v_lds1 : v_lds0;
      uint16_t* const v_fill = P ? v_lds0 : v_lds1;
      int e_nxt2 = 0;
      if (t + 2 < n_tiles) {
        stage_k(k_fill, t + 2);
        if (F16) e_nxt2 = kexp[t + 2];
      }
      stage_v(v_fill, t + 1);
      softmax_pv(std::false_type{}, std::true_type{}, s_in, v_cur, t, e_cur, k_next, s_out);
      e_cur = e_nxt;
      e_nxt = e_nxt2;
      wait_vmem();
      __syncthreads();
    };
    // Only the last tile can be partial.
    auto finish = [&](f32x16 (&s)[2], const uint16_t* vs) {
      if (n_keys % FWD_BC != 0)
        softmax_pv(std::true_type{}, std::false_type{}, s, vs, last, e_cur, nullptr, s);
      else
        softmax_pv(std::false_type{}, std::false_type{}, s, vs, last, e_cur, nullptr, s);
    };
    if constexpr (TILED) {
      // Unrolled by two: the buffer parity is a compile-time constant.
      int t = 0;
      for (; t + 1 < last; t += 2) {
        iteration(std::integral_constant<int, 0>{}, t, s_a, s_b);
        iteration(std::integral_constant<int, 1>{}, t + 1, s_b, s_a);
      }
      if (t < last) {
        iteration(std::integral_constant<int, 0>{}, t, s_a, s_b);
        finish(s_b, v_lds1);
      } else {
        finish(s_a, v_lds0);
      }
    } else {
      // Short key sets (text context): a plain loop with the parity at run
      // time (the per-lane addressing of the row-major copies leaves no
      // registers for a second copy of the body).
      for (int t = 0; t < last; ++t) {
        iteration(t & 1, t, s_a, s_b);
        s_a[0] = s_b[0];
        s_a[1] = s_b[1];
      }
      finish(s_a, (last & 1) ? v_lds1 : v_lds0);
    }
  }

  // ---- epilogue: O = O / l (bf16), LSE = ln sum exp(s) = ln2 * (m + log2 l)
  const float l_tot = xor32_sum(l_run);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (row_ok) {
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
      const float lse = (l_tot > 0.f) ? (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f
                                      : -INFINITY;
      p.lse[((int64_t)b * p.H + h) * p.Lq + i] = lse;
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd(const FwdParams& p, hipStream_t stream) {
  FwdParams q = p;
  q.n_qtiles = (p.Lq + FWD_BR - 1) / FWD_BR;
  const int64_t total = (int64_t)q.n_qtiles * p.H * p.B;
  if (total <= 0 || total > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)total), block(256);
  // With RoPE the scores run in fp16 (see F16) against the fp16 key tiles
  // and their exponents (self-attention only).
  const bool f16 = p.rope.table != nullptr;
  const bool vt = p.kt != nullptr;
  if (vt && p.vt == nullptr) return hipErrorInvalidValue;
  // The tiles of one (b, h) are addressed through a buffer resource of 32-bit extent.
  if (vt && (int64_t)((p.Lk + FWD_BC - 1) / FWD_BC) * (TILE_ELEMS * 2) > (int64_t)0xffffffff)
    return hipErrorInvalidValue;
  if (f16 && (p.kexp == nullptr || !vt)) return hipErrorInvalidValue;
  if (p.scale_log2 > 0.f) {
    if (f16) hipLaunchKernelGGL((attn_fwd_kernel<true, true, true>), grid, block, 0, stream, q);
    else if (vt) hipLaunchKernelGGL((attn_fwd_kernel<true, false, true>), grid, block, 0, stream, q);
    else hipLaunchKernelGGL((attn_fwd_kernel<true, false, false>), grid, block, 0, stream, q);
  } else {
    if (f16) hipLaunchKernelGGL((attn_fwd_kernel<false, true, true>), grid, block, 0, stream, q);
    else if (vt) hipLaunchKernelGGL((attn_fwd_kernel<false, false, true>), grid, block, 0, stream, q);
    else hipLaunchKernelGGL((attn_fwd_kernel<false, false, false>), grid, block, 0, stream, q);
  }
  return hipGetLastError();
}

}  // namespace wanattn
