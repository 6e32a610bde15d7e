// Cross-attention forward for gfx950: video-token queries attend to a short
// text context with key padding (one valid length per batch item), reading
// q, k and v as given (bf16, row-major, no workspace).  Self-attention over
// the prep pass's tiles is attn_fwd_pp.hip; launch_attn_fwd dispatches.
//
// Computes, per (batch b, head h, query i), over the valid keys j < n_keys:
//   s_ij = scale <q_i, k_j>,  O_i = sum_j softmax_j(s_ij) v_j,  LSE_i = ln sum_j exp(s_ij)
// -- the cross-attention to umT5 text embeddings in every DiT block ("Wan
// Team, Alibaba (2025)", Key takeaways, Backbone); an empty key set gives
// O = 0 and LSE = -inf.
//
// Design (one workgroup = 4 waves = 128 query rows of one (b, h), two
// workgroups per CU):
//  * each wave keeps its 32 query rows in registers as the B operand of
//    S^T = K Q^T (bf16 MFMA 32x32x16), so every lane owns one query row;
//  * K and V tiles of 64 keys go global -> LDS directly (global_load_lds,
//    row-major, swizzled, rows past n_keys clamped to the last valid key and
//    masked), double-buffered; O^T += V^T P^T takes P straight from the S^T
//    accumulators (bf16, RNE) and V through the LDS transpose read;
//  * online softmax in fp32, log2 domain, lazy rescaling without a per-tile
//    max (as in attn_fwd_pp.hip);
//  * software pipeline: the next tile's score MFMAs are issued in the same
//    basic block as this tile's exponentials.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace wanattn {

namespace {

constexpr int FWD_WAVES = 4;
constexpr int FWD_BR = 32 * FWD_WAVES;   // query rows per workgroup
constexpr int FWD_BC = TILE_ROWS;         // keys per tile
constexpr float PSUM_LIMIT = 65536.0f;    // largest partial row sum of P kept without a rescale

template <bool POS_SCALE>
__global__ __launch_bounds__(256, 2) void cross_fwd_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds0[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t k_lds1[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds0[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds1[TILE_ELEMS];

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

  // query fragments (B operand of S^T = K Q^T): lane holds row i, d in [16s + 8*half, +8)
  const int i = qt * FWD_BR + wave * 32 + col;
  int n_q = p.Lq;
  if (p.q_lens != nullptr) n_q = min(max(p.q_lens[b], 0), p.Lq);
  const bool row_ok = i < n_q;
  if (qt * FWD_BR >= n_q) return;   // query tile wholly past its item's length: nothing to do
  bf16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    u32x4 x = u32x4{0u, 0u, 0u, 0u};
    if (row_ok) x = *reinterpret_cast<const u32x4*>(qbase + (int64_t)i * q_row_stride + (2 * s + half) * 8);
    qf[s] = __builtin_bit_cast(bf16x8, x);
  }
  const float g = p.scale_log2;   // s * log2(e) = g * S

  f32x16 o_acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o_acc[d] = f32x16{};
  float m_run = -INFINITY;   // running max of scale*log2e*s (this lane's row)
  float l_run = 0.f;         // this lane's partial exp-sum (the other half holds the rest)
  const int n_tiles = (n_keys + FWD_BC - 1) / FWD_BC;

  // S^T of one 64-key tile (64 keys x 32 queries) as two 32x32 blocks.
  auto scores = [&](const uint16_t* ks, f32x16 (&s_acc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s_acc[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) s_acc[kb] = mfma32(lds_row_frag(ks, kb * 32 + col, 2 * s + half), qf[s], s_acc[kb]);
    }
  };

  // Online softmax of tile t's scores and O += P V.  MASK: the last tile,
  // whose keys past n_keys get -inf.  NEXT: also compute the next tile's
  // scores (from next_ks into s_nxt) in the same basic block as this tile's
  // exponentials.
  auto softmax_pv = [&](auto mask_tag, auto next_tag, f32x16 (&s_acc)[2], const uint16_t* vs, int t,
                        const uint16_t* next_ks, f32x16 (&s_nxt)[2]) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool NEXT = decltype(next_tag)::value;
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
    // rounded to bf16, RNE, only for the P V product).
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
    // Lazy rescaling without a per-tile max: while every row's partial sum
    // (32 of its P) stays <= PSUM_LIMIT, so does every P and the tile is kept;
    // otherwise (a larger score, the first tile with m = -inf, a non-finite
    // sum) m moves up to the exact tile max, O and l are rescaled and P is
    // recomputed.  Exact either way: O / l and LSE = m + log2 l use the m
    // that was applied.
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
      for (int kg = 0; kg < 4; ++kg) o_acc[d] = mfma32(lds_col_frag(vs, kg * 16, d * 32, lane), pf[kg], o_acc[d]);
    }
  };

  if (n_tiles > 0) {
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    auto stage_k = [&](uint16_t* dst, int t) { tile_dma(dst, kbase, q_row_stride, t * FWD_BC, n_keys, wv, lane); };
    auto stage_v = [&](uint16_t* dst, int t) { tile_dma(dst, vbase, q_row_stride, t * FWD_BC, n_keys, wv, lane); };
    // Software pipeline: iteration t computes the scores of tile t+1 while
    // the softmax of tile t runs, then O += P(t) V(t).  K runs one tile ahead
    // of V: iteration t copies K(t+2) and V(t+1) into the buffers K(t) and
    // V(t-1) have left.
    stage_k(k_lds0, 0);
    stage_v(v_lds0, 0);
    if (n_tiles > 1) stage_k(k_lds1, 1);
    wait_vmem();
    __syncthreads();
    f32x16 s_cur[2], s_nxt[2];
    scores(k_lds0, s_cur);
    __syncthreads();   // K buffer 0 is refilled in iteration 0
    const int last = n_tiles - 1;
    for (int t = 0; t < last; ++t) {
      const bool odd = t & 1;
      if (t + 2 < n_tiles) stage_k(odd ? k_lds1 : k_lds0, t + 2);
      stage_v(odd ? v_lds0 : v_lds1, t + 1);
      softmax_pv(std::false_type{}, std::true_type{}, s_cur, odd ? v_lds1 : v_lds0, t, odd ? k_lds0 : k_lds1, s_nxt);
      s_cur[0] = s_nxt[0];
      s_cur[1] = s_nxt[1];
      wait_vmem();
      __syncthreads();
    }
    // Only the last tile can be partial.
    const uint16_t* v_last = (last & 1) ? v_lds1 : v_lds0;
    if (n_keys % FWD_BC != 0)
      softmax_pv(std::true_type{}, std::false_type{}, s_cur, v_last, last, nullptr, s_cur);
    else
      softmax_pv(std::false_type{}, std::false_type{}, s_cur, v_last, last, nullptr, s_cur);
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
  // Self-attention over the prep pass's tiles.
  if (p.kt != nullptr) return launch_attn_fwd_tiled(p, stream);
  // Row-major K/V (cross-attention): no RoPE on this path.
  if (p.rope.table != nullptr || p.vt != nullptr) return hipErrorInvalidValue;
  FwdParams q = p;
  q.n_qtiles = (p.Lq + FWD_BR - 1) / FWD_BR;
  const int64_t total = (int64_t)q.n_qtiles * p.H * p.B;
  if (total <= 0 || total > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)total), block(64 * FWD_WAVES);
  if (p.scale_log2 > 0.f) hipLaunchKernelGGL(cross_fwd_kernel<true>, grid, block, 0, stream, q);
  else hipLaunchKernelGGL(cross_fwd_kernel<false>, grid, block, 0, stream, q);
  return hipGetLastError();
}

}  // namespace wanattn
