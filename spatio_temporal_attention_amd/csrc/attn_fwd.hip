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
// Design (persistent: two workgroups of 4 waves per CU, each walking a
// contiguous range of 128-row query tiles, batch item innermost, so the
// workgroups of one XCD share a head's text keys through its L2):
//  * each wave keeps its 32 query rows in registers as the B operand of
//    S^T = K Q^T (bf16 MFMA 32x32x16), so every lane owns one query row;
//    the next query tile's rows are loaded at the current tile's last pair,
//    once the current rows have served their last score product;
//  * K and V tiles of 64 keys go global -> LDS directly (buffer_load ... lds
//    from the row-major tensors, swizzled; rows past n_keys fall outside the
//    copy's resource, read as zero and are masked), double-buffered, as one
//    stream over every (query tile, key tile) pair of the workgroup, so no
//    query tile starts on an empty pipeline (each pair's copies are issued
//    one pair ahead);
//  * O^T += V^T P^T takes P straight from the S^T accumulators (bf16, RNE)
//    and V through the LDS transpose read;
//  * online softmax in fp32, log2 domain, lazy rescaling without a per-tile
//    max (as in attn_fwd_pp.hip);
//  * no software pipelining of the next pair's scores inside a wave (its
//    accumulators do not fit beside the persistent state); the two
//    workgroups of a CU overlap each other's softmax and products instead;
//  * query loads and O / LSE stores go through buffer resources bounded to
//    the tile's valid rows (no per-lane branches).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace wanattn {

namespace {

constexpr int FWD_WAVES = 4;
constexpr int FWD_BR = 32 * FWD_WAVES;   // query rows per query tile
constexpr int FWD_BC = TILE_ROWS;         // keys per tile
constexpr float PSUM_LIMIT = 65536.0f;    // largest partial row sum of P kept without a rescale
constexpr int CROSS_WG_PER_CU = 2;
constexpr int CROSS_CUS = 256;

// Buffer resource over the rows [row0, row0 + n) of head (b, h) of a
// [B, L, H, 128] bf16 tensor (row r at byte r * H * 256): accesses at rows
// >= n fall outside it (loads return 0, stores are dropped).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* t, int64_t row_stride_bytes, int64_t base_off,
                                                            int n) {
  const uint32_t bytes = n > 0 ? (uint32_t)((int64_t)(n - 1) * row_stride_bytes + HD * 2) : 0u;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(t + base_off), (short)0, (int)bytes, 0x00020000);
}

template <bool POS_SCALE>
__global__ __launch_bounds__(256, CROSS_WG_PER_CU) void cross_fwd_kernel(FwdParams p, int n_units) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds0[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t k_lds1[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds0[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds1[TILE_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;       // which 32-lane half
  const int col = lane & 31;        // query row of this lane within the wave
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  // This workgroup's query tiles [j_begin, j_end), ordered ((head, batch), tile).
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int per = n_units / (int)gridDim.x;
  const int rem = n_units % (int)gridDim.x;
  const int j_begin = wg * per + min(wg, rem);
  const int j_end = j_begin + per + (wg < rem ? 1 : 0);

  const int64_t row_stride = (int64_t)p.H * HD;     // elements
  const int64_t row_bytes = row_stride * 2;
  const_i32* klens = p.k_lens != nullptr ? const_ptr(p.k_lens) : nullptr;
  struct Tile {
    int b, h, qt, n_keys, n_t;
  };
  auto tile_of = [&](int j) __attribute__((always_inline)) {
    Tile t;
    t.qt = j % p.n_qtiles;
    const int bh = j / p.n_qtiles;
    t.b = bh % p.B;
    t.h = bh / p.B;
    t.n_keys = klens != nullptr ? min(max(klens[t.b], 0), p.Lk) : p.Lk;
    t.n_t = (t.n_keys + FWD_BC - 1) / FWD_BC;
    return t;
  };
  auto q_rows = [&](const Tile& t) __attribute__((always_inline)) { return min(FWD_BR, p.Lq - t.qt * FWD_BR); };
  auto head_off = [&](const Tile& t, int L) __attribute__((always_inline)) { return ((int64_t)t.b * L * p.H + t.h) * HD; };
  const int wrow = wave * 32 + col;   // this lane's row within a query tile

  // 32 rows' query fragments (lane: row wrow, d in [16s + 8*half, +8)); rows past Lq read as 0.
  auto load_q = [&](const Tile& t, bf16x8 (&dst)[8]) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r =
        rows_rsrc(p.q, row_bytes, head_off(t, p.Lq) + (int64_t)t.qt * FWD_BR * row_stride, q_rows(t));
    const uint32_t off = (uint32_t)(wrow * row_bytes) + (uint32_t)half * 16;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      dst[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off + s * 32, 0, 0));
  };

  // Query tiles without a valid key: O = 0, LSE = -inf.
  for (int j = j_begin; j < j_end; ++j) {
    const Tile t = tile_of(j);
    if (t.n_t > 0) continue;
    const int i = t.qt * FWD_BR + wrow;
    if (i < p.Lq) {
      uint16_t* orow = p.o + head_off(t, p.Lq) + (int64_t)i * row_stride;
#pragma unroll
      for (int c = 0; c < 8; ++c)
        *reinterpret_cast<u32x2*>(orow + 64 * half + 8 * c) = u32x2{0u, 0u},
        *reinterpret_cast<u32x2*>(orow + 64 * half + 8 * c + 4) = u32x2{0u, 0u};
      if (p.lse != nullptr && half == 0) p.lse[((int64_t)t.b * p.H + t.h) * p.Lq + i] = -INFINITY;
    }
  }
  // The stream of (query tile, key tile) pairs over the tiles with keys.
  auto next_j = [&](int j) __attribute__((always_inline)) {
    do {
      ++j;
    } while (j < j_end && tile_of(j).n_t == 0);
    return j;
  };
  int jc = j_begin;
  if (jc < j_end && tile_of(jc).n_t == 0) jc = next_j(jc);
  if (jc >= j_end) return;

  // Cursor of a pair: query tile j (its Tile cached), key tile t.
  struct Cur {
    int j, t;
    Tile tl;
  };
  auto advance = [&](Cur& c) __attribute__((always_inline)) {
    if (++c.t >= c.tl.n_t) {
      c.t = 0;
      c.j = next_j(c.j);
      if (c.j < j_end) c.tl = tile_of(c.j);
    }
  };
  // K and V tiles: 64 rows of the pair's (b, h) through a resource bounded to
  // its valid keys, so rows past n_keys read as zero and padding is never
  // read; this wave copies rows 16 wv .. 16 wv + 15.
  uint32_t kv_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) kv_off[i] = rows_lane_off(wv, i, lane, (uint32_t)row_bytes);
  auto stage = [&](const uint16_t* src, uint16_t* dst, const Cur& c) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = rows_rsrc(src, row_bytes, head_off(c.tl, p.Lk), c.tl.n_keys);
    const uint32_t soff = (uint32_t)(c.t * FWD_BC) * (uint32_t)row_bytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) buf_dma16(r, kv_off[i], soff, tile_lds_block<FWD_WAVES>(dst, wv, i));
  };
  auto stage_k = [&](uint16_t* dst, const Cur& c) __attribute__((always_inline)) { stage(p.k, dst, c); };
  auto stage_v = [&](uint16_t* dst, const Cur& c) __attribute__((always_inline)) { stage(p.v, dst, c); };

  // Byte offsets of this lane's transposed V reads inside a tile (rows 16 kg + ... add kg * 4096):
  // lds_col_frag's rows and columns for d-block d, the +0 and +8 row halves.
  uint32_t vt_off[4][2];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int row = 4 * (lane >> 5) + ((lane & 15) >> 2) + 8 * hh;
      const int cc = d * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      vt_off[d][hh] = (uint32_t)tile_off(row, cc) * 2;
    }

  const float g = p.scale_log2;   // s * log2(e) = g * S
  bf16x8 qf[8];
  f32x16 o_acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o_acc[d] = f32x16{};
  float m_run = -INFINITY;   // running max of scale*log2e*s (this lane's row)
  float l_run = 0.f;         // this lane's partial exp-sum (the other half holds the rest)

  // S^T of one 64-key tile (64 keys x 32 queries) as two 32x32 blocks.
  auto scores = [&](const uint16_t* ks, f32x16 (&s_acc)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s_acc[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) s_acc[kb] = mfma32(lds_row_frag(ks, kb * 32 + col, 2 * s + half), qf[s], s_acc[kb]);
    }
  };

  // Online softmax of a pair's scores and O += P V.  MASK: keys at or past
  // n_keys get -inf (only the last key tile of a query tile can be partial).
  auto softmax_pv = [&](auto mask_tag, f32x16 (&s_acc)[2], const uint16_t* vs, int t, int n_keys)
                        __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
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

    // P = 2^(s - m) against the running max m, in fp32 (l sums these; P is
    // rounded to bf16, RNE, only for the P V product).
    bf16x8 pf[4];
    float psum;
    auto exps = [&]() __attribute__((always_inline)) {
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

    // O^T (128 d x 32 queries) += V^T P^T over the 4 groups of 16 keys, V
    // through the LDS transpose read (the fragments of lds_col_frag, from
    // the per-lane offsets computed once).
    const uint8_t* vb = reinterpret_cast<const uint8_t*>(vs);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int kg = 0; kg < 4; ++kg) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + vt_off[d][0] + kg * 4096));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + vt_off[d][1] + kg * 4096));
        const u32x2 a = __builtin_bit_cast(u32x2, lo);
        const u32x2 b = __builtin_bit_cast(u32x2, hi);
        o_acc[d] = mfma32(__builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]}), pf[kg], o_acc[d]);
      }
    }
  };

  // O = O / l (bf16) and LSE = ln sum exp(s) = ln2 * (m + log2 l) of a query
  // tile at its last pair, then a fresh accumulator.  The stores go through
  // resources bounded to the tile's rows (and, for LSE, the lower half-wave).
  auto finish_tile = [&](const Tile& t) __attribute__((always_inline)) {
    const float l_tot = xor32_sum(l_run);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    const __amdgpu_buffer_rsrc_t ro =
        rows_rsrc(p.o, row_bytes, head_off(t, p.Lq) + (int64_t)t.qt * FWD_BR * row_stride, q_rows(t));
    const uint32_t off = (uint32_t)(wrow * row_bytes) + (uint32_t)half * 8;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        u32x2 w;
        w[0] = pack_bf16(o_acc[d][4 * jq] * inv, o_acc[d][4 * jq + 1] * inv);
        w[1] = pack_bf16(o_acc[d][4 * jq + 2] * inv, o_acc[d][4 * jq + 3] * inv);
        __builtin_amdgcn_raw_buffer_store_b64(w, ro, off + (uint32_t)(d * 64 + 16 * jq), 0, 0);
      }
    }
    if (p.lse != nullptr) {
      const float lse = (l_tot > 0.f) ? (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f : -INFINITY;
      const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
          p.lse + ((int64_t)t.b * p.H + t.h) * p.Lq + (int64_t)t.qt * FWD_BR, (short)0, q_rows(t) * 4, 0x00020000);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rl, half ? 0x80000000u : (uint32_t)wrow * 4, 0, 0);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) o_acc[d] = f32x16{};
    m_run = -INFINITY;
    l_run = 0.f;
  };

  // Rows past n_keys in a partial tile are zero-filled by the copies; the
  // buffers also start at zero, so no LDS row ever holds a non-finite value
  // (a masked key's P = 0 multiplies its V row).
#pragma unroll
  for (int c = 0; c < TILE_ELEMS * 2 / 16 / 256; ++c) {
    const int e = (c * 256 + tid) * 8;
    *reinterpret_cast<u32x4*>(k_lds0 + e) = u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(k_lds1 + e) = u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(v_lds0 + e) = u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(v_lds1 + e) = u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();

  // Prologue: the first pair's K and V and the first query tile's rows.
  Cur cur{jc, 0, tile_of(jc)};
  load_q(cur.tl, qf);
  stage_k(k_lds0, cur);
  stage_v(v_lds0, cur);
  wait_vmem();
  __syncthreads();

  // Pair with parity P = (pair index) & 1: its K and V in buffers P; the
  // copies of the next pair fill buffers 1-P, which the previous pair left.
  f32x16 s_acc[2];
  for (int P = 0;; P ^= 1) {
    uint16_t* const k_cur = P ? k_lds1 : k_lds0;
    uint16_t* const v_cur = P ? v_lds1 : v_lds0;
    uint16_t* const k_fill = P ? k_lds0 : k_lds1;
    uint16_t* const v_fill = P ? v_lds0 : v_lds1;
    Cur nx = cur;
    advance(nx);
    const bool has_next = nx.j < j_end;
    const bool last_of_tile = cur.t + 1 == cur.tl.n_t;
    if (has_next) {
      stage_k(k_fill, nx);
      stage_v(v_fill, nx);
    }
    scores(k_cur, s_acc);
    __builtin_amdgcn_sched_barrier(0);
    // This pair's scores were the last use of qf when it ends a query tile:
    // the next tile's rows load while its softmax and products run.
    if (has_next && last_of_tile) load_q(nx.tl, qf);
    if (last_of_tile && (cur.tl.n_keys % FWD_BC) != 0) {
      if (POS_SCALE) {
        // the partial last tile: keys past n_keys get a score of -inf in place
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = cur.t * FWD_BC + kb * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
            if (key >= cur.tl.n_keys) s_acc[kb][j] = -INFINITY;
          }
        softmax_pv(std::false_type{}, s_acc, v_cur, cur.t, cur.tl.n_keys);
      } else {
        softmax_pv(std::true_type{}, s_acc, v_cur, cur.t, cur.tl.n_keys);
      }
    } else {
      softmax_pv(std::false_type{}, s_acc, v_cur, cur.t, cur.tl.n_keys);
    }
    if (last_of_tile) finish_tile(cur.tl);
    cur = nx;
    wait_vmem();
    lds_barrier();
    if (!has_next) break;
  }
}

}  // namespace

hipError_t launch_attn_fwd(const FwdParams& p, hipStream_t stream) {
  // Self-attention over the prep pass's tiles.
  if (p.kt != nullptr) return launch_attn_fwd_tiled(p, stream);
  // Row-major K/V (cross-attention): no RoPE on this path.
  if (p.rope.table != nullptr || p.vt != nullptr) return hipErrorInvalidValue;
  if (p.q_lens != nullptr) return hipErrorInvalidValue;
  FwdParams q = p;
  q.n_qtiles = (p.Lq + FWD_BR - 1) / FWD_BR;
  const int64_t total = (int64_t)q.n_qtiles * p.H * p.B;
  if (total <= 0 || total > 0x7fffffff) return hipErrorInvalidValue;
  // 32-bit buffer offsets span one query tile: 127 rows of H * 256 bytes.
  if ((int64_t)(FWD_BR - 1) * p.H * HD * 2 + HD * 2 > (int64_t)0x7fffffff) return hipErrorInvalidValue;
  const int64_t wgs = std::min<int64_t>(total, (int64_t)CROSS_CUS * CROSS_WG_PER_CU);
  const dim3 grid((unsigned)wgs), block(64 * FWD_WAVES);
  if (p.scale_log2 > 0.f) hipLaunchKernelGGL(cross_fwd_kernel<true>, grid, block, 0, stream, q, (int)total);
  else hipLaunchKernelGGL(cross_fwd_kernel<false>, grid, block, 0, stream, q, (int)total);
  return hipGetLastError();
}

}  // namespace wanattn
