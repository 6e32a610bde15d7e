// FP8 self-attention forward for gfx950 (the pages name FP8 attention work
// without a recipe: "Wan Team, Alibaba (2025)" Tags, FP8 attention; anthology
// note, FP8 quantization).  The recipe here:
//  * q~ = R(p) q, k~ = R(p) k and v are quantized to OCP fp8 e4m3 (RNE,
//    saturating) per 64-token tile of each (b, h) after scaling by 2^-e, e
//    chosen so that the tile's largest |element| lies in [128, 256);
//  * both products run on the scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4
//    (fp8 x fp8, twice the bf16 rate), whose E8M0 scale operands undo the
//    tiles' powers of two exactly: S^T = 2^(e_k + e_q) K8 Q8^T and
//    O^T += 2^e_v V8^T P8^T;
//  * the softmax is fp32 as in the bf16 path; P is rounded to e4m3 for PV
//    (lazy rescaling keeps P <= 2^8, inside e4m3's range of 448), while the
//    row sums and LSE use the fp32 P.
// Everything else (layouts, online softmax, software pipeline, XCD-aware
// order) follows attn_fwd.hip.
//
// Register layout of the fp8 MFMA (32x32x64, lane l, wave64): A[32 x 64]:
// lane holds A[l%32][32*(l/32) + t], B[64 x 32]: B[32*(l/32) + t][l%32],
// t = 0..31 (one byte each); C as for 32x32x16.
//  * S^T (keys x queries): A = K rows (d chunk 64*k2 + 32*half), B = q row;
//  * O^T (d x queries) += V^T P^T over one 64-key tile per MFMA: the S^T
//    accumulators of lane half h hold keys {8g + 4h + e : g = 0..7, e = 0..3}
//    (two 32x32 blocks); they are the B operand's k = 32h + 4g + e, in
//    register order, so V^T tiles store key n at position
//    kappa(n) = 32*((n>>2)&1) + 4*(n>>3) + (n&3).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace wanattn {

namespace {

constexpr int F8_WAVES = 4;
constexpr int F8_BR = 32 * F8_WAVES;       // query rows per workgroup
constexpr int F8_BC = TILE_ROWS;           // keys per tile
constexpr int F8_TILE_BYTES = TILE_ELEMS;  // 64 x 128 fp8
constexpr float F8_PSUM_LIMIT = 256.0f;   // largest partial row sum of P kept without a rescale

// Four P values (each in [0, 256] on the path that uses them: see the
// partial-sum check) to e4m3, RNE, without the clamp of pack_fp8x4: values
// that could overflow (P = +inf or NaN while m = -inf) are recomputed before
// the product reads them.
__device__ __forceinline__ uint32_t pack_p8x4(float a, float b, float c, float d) {
  const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)w, true);
}

// e with x * 2^-e in [128, 256) (0 for x == 0).
__device__ __forceinline__ int pow2_exponent_8(float x) {
  if (!(x > 0.f)) return 0;
  int ex;
  frexpf(x, &ex);
  return ex - 8;
}

// K tile (64 rows x 128 B): 16-byte chunk c of row r at c ^ swz8(r).
__device__ __forceinline__ int k8_off(int row, int chunk) { return row * 128 + ((chunk ^ swz8(row)) << 4); }
// V^T tile (128 rows x 64 B): chunk c (of 4) of row r at c ^ ((r >> 2) & 3); the 16
// rows a 16-lane pass reads land on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int v8_off(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); }

__device__ __forceinline__ i32x8 join8(u32x4 lo, u32x4 hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// ---------------------------------------------------------------------------
// Prep: K (rotated) as fp8 row tiles and V as fp8 V^T tiles in kappa order,
// each with its exponent.  One workgroup per (b, h, 64-token tile).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kv8_tiles_kernel(const uint16_t* __restrict__ k,
                                                        const uint16_t* __restrict__ v, uint8_t* __restrict__ k8,
                                                        int* __restrict__ kexp, uint8_t* __restrict__ v8,
                                                        int* __restrict__ vexp, int L, int H, int nt, RopeDev rope) {
  __shared__ __attribute__((aligned(16))) uint8_t vs[TILE_ROWS][HD + 16];
  __shared__ float wmax[2][4];
  const int tile = blockIdx.x % nt;
  const int bh = blockIdx.x / nt;
  const int h = bh % H;
  const int b = bh / H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  float kx[4][8], vx[4][8];
  float mk = 0.f, mv = 0.f;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = (tid >> 4) + 16 * it;   // token in the tile
    const int ch = tid & 15;
    const int n = tile * TILE_ROWS + r;
    u32x4 a = u32x4{0u, 0u, 0u, 0u}, c = u32x4{0u, 0u, 0u, 0u};
    if (n < L) {
      const int64_t off = (((int64_t)b * L + n) * H + h) * HD + ch * 8;
      a = *reinterpret_cast<const u32x4*>(k + off);
      c = *reinterpret_cast<const u32x4*>(v + off);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      kx[it][2 * t] = bf16_lo(a[t]);
      kx[it][2 * t + 1] = bf16_hi(a[t]);
      vx[it][2 * t] = bf16_lo(c[t]);
      vx[it][2 * t + 1] = bf16_hi(c[t]);
    }
    if (rope.table != nullptr && n < L) {
      const TokenPos pos = token_pos(rope, n);
#pragma unroll
      for (int t = 0; t < 4; ++t) rope_rotate(kx[it][2 * t], kx[it][2 * t + 1], rope_cs(rope, pos, 4 * ch + t), false);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mk = fmaxf(mk, fabsf(kx[it][e]));
      mv = fmaxf(mv, fabsf(vx[it][e]));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mk = fmaxf(mk, __shfl_xor(mk, o));
    mv = fmaxf(mv, __shfl_xor(mv, o));
  }
  if (lane == 0) {
    wmax[0][tid >> 6] = mk;
    wmax[1][tid >> 6] = mv;
  }
  __syncthreads();
  const int ek = pow2_exponent_8(fmaxf(fmaxf(wmax[0][0], wmax[0][1]), fmaxf(wmax[0][2], wmax[0][3])));
  const int ev = pow2_exponent_8(fmaxf(fmaxf(wmax[1][0], wmax[1][1]), fmaxf(wmax[1][2], wmax[1][3])));
  if (tid == 0) {
    kexp[blockIdx.x] = ek;
    vexp[blockIdx.x] = ev;
  }
  const int64_t off = (int64_t)blockIdx.x * F8_TILE_BYTES;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = (tid >> 4) + 16 * it;
    const int ch = tid & 15;
    u32x2 w;
    w[0] = pack_fp8x4(ldexpf(kx[it][0], -ek), ldexpf(kx[it][1], -ek), ldexpf(kx[it][2], -ek), ldexpf(kx[it][3], -ek));
    w[1] = pack_fp8x4(ldexpf(kx[it][4], -ek), ldexpf(kx[it][5], -ek), ldexpf(kx[it][6], -ek), ldexpf(kx[it][7], -ek));
    *reinterpret_cast<u32x2*>(k8 + off + r * HD + ch * 8) = w;
    u32x2 y;
    y[0] = pack_fp8x4(ldexpf(vx[it][0], -ev), ldexpf(vx[it][1], -ev), ldexpf(vx[it][2], -ev), ldexpf(vx[it][3], -ev));
    y[1] = pack_fp8x4(ldexpf(vx[it][4], -ev), ldexpf(vx[it][5], -ev), ldexpf(vx[it][6], -ev), ldexpf(vx[it][7], -ev));
    *reinterpret_cast<u32x2*>(&vs[r][ch * 8]) = y;
  }
  __syncthreads();
  // V^T row d, position kappa holds token n(kappa) = 8*((kappa>>2)&7) + 4*(kappa>>5) + (kappa&3).
  const int d = tid >> 1;                  // 128 rows, 2 threads per row (32 positions each)
  const int k0 = 32 * (tid & 1);
  uint32_t wd[8];
#pragma unroll
  for (int w4 = 0; w4 < 8; ++w4) {
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int kap = k0 + 4 * w4 + e;
      const int n = 8 * ((kap >> 2) & 7) + 4 * (kap >> 5) + (kap & 3);
      word |= (uint32_t)vs[n][d] << (8 * e);
    }
    wd[w4] = word;
  }
  uint8_t* vrow = v8 + off + d * 64 + k0;
  *reinterpret_cast<u32x4*>(vrow) = u32x4{wd[0], wd[1], wd[2], wd[3]};
  *reinterpret_cast<u32x4*>(vrow + 16) = u32x4{wd[4], wd[5], wd[6], wd[7]};
}

// ---------------------------------------------------------------------------
// Forward over the fp8 tiles.
// ---------------------------------------------------------------------------
template <bool POS_SCALE>
__global__ __launch_bounds__(256, 2) void attn_fwd_fp8_kernel(FwdParams p, const uint8_t* __restrict__ k8,
                                                              const int* __restrict__ kexp_all,
                                                              const uint8_t* __restrict__ v8,
                                                              const int* __restrict__ vexp_all) {
  // Two K and two V^T buffers as separate objects, each named statically in
  // the unrolled loop, so LDS reads do not wait for the copies in flight
  // into the other buffers.
  __shared__ __attribute__((aligned(16))) uint8_t k_lds0[F8_TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t k_lds1[F8_TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds0[F8_TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds1[F8_TILE_BYTES];
  __shared__ float qmax_s[F8_WAVES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;

  // The workgroup's query tile: from the work counter (common.h), or blockIdx.x remapped.
  int logical;
  if (p.work != nullptr) {
    logical = take_work_item(p.work);
    if (logical >= p.n_items) return;   // the whole workgroup: the value is uniform
  } else {
    logical = xcd_remap(blockIdx.x, gridDim.x);
  }
  const int qt = logical % p.n_qtiles;
  const int bh = logical / p.n_qtiles;
  const int b = bh % p.B;   // batch innermost: every XCD gets the same heads of every item
  const int h = bh / p.B;
  const int n_keys = p.Lk;
  const int64_t q_row_stride = (int64_t)p.H * HD;
  const uint16_t* qbase = p.q + ((int64_t)b * p.Lq * p.H + h) * HD;
  const int nkt = (p.Lk + F8_BC - 1) / F8_BC;
  const int64_t tile0 = (int64_t)(b * p.H + h) * nkt;
  const_i32* kexp = const_ptr(kexp_all + tile0);   // scalar loads
  const_i32* vexp = const_ptr(vexp_all + tile0);

  // ---- queries: rotate, one exponent per 64-row tile, fp8 in the B layout of 32x32x64
  const int i = qt * F8_BR + wave * 32 + col;
  const bool row_ok = i < p.Lq;
  i32x8 qf8[2];
  int e_q;
  {
    TokenPos pos{0, 0, 0};
    if (p.rope.table != nullptr && row_ok) pos = token_pos(p.rope, i);
    float y[2][32];   // head dims 64*k2 + 32*half + t
    float mq = 0.f;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int c = 8 * k2 + 4 * half + cc;   // 8-element chunk
        u32x4 x = u32x4{0u, 0u, 0u, 0u};
        if (row_ok) x = *reinterpret_cast<const u32x4*>(qbase + (int64_t)i * q_row_stride + c * 8);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float y0 = bf16_lo(x[t]);
          float y1 = bf16_hi(x[t]);
          if (p.rope.table != nullptr && row_ok) rope_rotate(y0, y1, rope_cs(p.rope, pos, 4 * c + t), false);
          y[k2][8 * cc + 2 * t] = y0;
          y[k2][8 * cc + 2 * t + 1] = y1;
          mq = fmaxf(mq, fmaxf(fabsf(y0), fabsf(y1)));
        }
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mq = fmaxf(mq, __shfl_xor(mq, o));
    if (lane == 0) qmax_s[wave] = mq;
    __syncthreads();
    e_q = pow2_exponent_8(fmaxf(qmax_s[wave & ~1], qmax_s[wave | 1]));
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int w = 0; w < 8; ++w)
        qf8[k2][w] = (int)pack_fp8x4(ldexpf(y[k2][4 * w], -e_q), ldexpf(y[k2][4 * w + 1], -e_q),
                                     ldexpf(y[k2][4 * w + 2], -e_q), ldexpf(y[k2][4 * w + 3], -e_q));
  }
  const int scale_q = 127 + e_q;

  f32x16 o_acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o_acc[d] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c2 = p.scale_log2;
  const int n_tiles = nkt;

  auto scores = [&](const uint8_t* ks, int e_k, f32x16 (&s_acc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s_acc[kb] = f32x16{};
      const int row = kb * 32 + col;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const i32x8 a = join8(*reinterpret_cast<const u32x4*>(ks + k8_off(row, 4 * k2 + 2 * half)),
                              *reinterpret_cast<const u32x4*>(ks + k8_off(row, 4 * k2 + 2 * half + 1)));
        s_acc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf8[k2], s_acc[kb], 0, 0, 0, 127 + e_k, 0,
                                                                   scale_q);
      }
    }
  };

  auto softmax_pv = [&](auto mask_tag, auto next_tag, f32x16 (&s_acc)[2], const uint8_t* vs, int t, int e_v,
                        const uint8_t* next_ks, int e_k_next, f32x16 (&s_nxt)[2]) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool NEXT = decltype(next_tag)::value;
    float sv[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float x = POS_SCALE ? s_acc[kb][j] : s_acc[kb][j] * c2;
        if (MASK) {
          const int key = t * F8_BC + kb * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
          if (key >= n_keys) x = -INFINITY;
        }
        sv[kb][j] = x;
      }
    }
    if (NEXT) scores(next_ks, e_k_next, s_nxt);
    // P: fp32 for the row sum, e4m3 for PV (B operand: this lane's 32 keys in register order)
    float psum;
    i32x8 p8;
    auto exps = [&]() {
      float part[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float pv[16];
        part[kb] = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (POS_SCALE) pv[j] = __builtin_amdgcn_exp2f(fmaf(sv[kb][j], c2, -m_run));
          else pv[j] = __builtin_amdgcn_exp2f(sv[kb][j] - m_run);
          part[kb] += pv[j];
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) p8[4 * kb + w] = (int)pack_p8x4(pv[4 * w], pv[4 * w + 1], pv[4 * w + 2], pv[4 * w + 3]);
      }
      psum = part[0] + part[1];
    };
    exps();
    // Lazy rescaling without a per-tile max: while every row's partial sum
    // (32 of its P) stays <= F8_PSUM_LIMIT = 256, every P is <= 256, inside
    // e4m3's range, and the tile is kept; otherwise (a larger score, the
    // first tile with m = -inf, or a non-finite sum) m moves up to the exact
    // tile max, O and l are rescaled and P is recomputed.
    if (__any(!(psum <= F8_PSUM_LIMIT))) {
      float mx = sv[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sv[kb][j]);
      mx = xor32_max(mx);
      if (POS_SCALE) mx *= c2;
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 while m was -inf
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < 4; ++d) o_acc[d] *= alpha;
      exps();
    }
    l_run += psum;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int row = d * 32 + col;
      const i32x8 a = join8(*reinterpret_cast<const u32x4*>(vs + v8_off(row, 2 * half)),
                            *reinterpret_cast<const u32x4*>(vs + v8_off(row, 2 * half + 1)));
      o_acc[d] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, p8, o_acc[d], 0, 0, 0, 127 + e_v, 0, 127);
    }
  };

  if (n_tiles > 0) {
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    // Lane offsets (bytes) of the copies: K tile rows of 128 B (8 rows per 1 KB copy, 2 per wave),
    // V^T rows of 64 B (16 rows per copy, 2 per wave).
    uint32_t koff[2], voff[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int kr = 16 * wv + 8 * c + (lane >> 3);
      koff[c] = (uint32_t)(kr * 128 + (((lane & 7) ^ swz8(kr)) << 4));
      const int vr = 32 * wv + 16 * c + (lane >> 2);
      voff[c] = (uint32_t)(vr * 64 + (((lane & 3) ^ ((vr >> 2) & 3)) << 4));
    }
    const uint32_t bytes = (uint32_t)nkt * F8_TILE_BYTES;
    const __amdgpu_buffer_rsrc_t krs = tile_rsrc(k8 + tile0 * F8_TILE_BYTES, bytes);
    const __amdgpu_buffer_rsrc_t vrs = tile_rsrc(v8 + tile0 * F8_TILE_BYTES, bytes);
    auto stage_k = [&](uint8_t* dst, int t) {
#pragma unroll
      for (int c = 0; c < 2; ++c) buf_dma16(krs, koff[c], (uint32_t)t * F8_TILE_BYTES, dst + 2048 * wv + 1024 * c);
    };
    auto stage_v = [&](uint8_t* dst, int t) {
#pragma unroll
      for (int c = 0; c < 2; ++c) buf_dma16(vrs, voff[c], (uint32_t)t * F8_TILE_BYTES, dst + 2048 * wv + 1024 * c);
    };
    // Software pipeline as in attn_fwd.hip: scores of tile t+1 with the softmax of tile t.
    stage_k(k_lds0, 0);
    stage_v(v_lds0, 0);
    int ek_cur = kexp[0], ev_cur = vexp[0];
    int ek_nxt = 0, ev_nxt = 0;
    if (n_tiles > 1) {
      stage_k(k_lds1, 1);
      ek_nxt = kexp[1];
      ev_nxt = vexp[1];
    }
    wait_vmem();
    __syncthreads();
    f32x16 s_a[2], s_b[2];
    scores(k_lds0, ek_cur, s_a);
    __syncthreads();
    const int last = n_tiles - 1;
    // Iteration t (parity P = t & 1): K(t+1) in K buffer 1-P, V(t) in V
    // buffer P; K(t+2) goes into K buffer P, V(t+1) into V buffer 1-P.
    auto iteration = [&](auto parity, int t, f32x16 (&s_in)[2], f32x16 (&s_out)[2]) {
      constexpr int P = decltype(parity)::value;
      uint8_t* const k_fill = P ? k_lds1 : k_lds0;
      const uint8_t* const k_next = P ? k_lds0 : k_lds1;
      const uint8_t* const v_cur = P ? v_lds1 : v_lds0;
      uint8_t* const v_fill = P ? v_lds0 : v_lds1;
      int ek_nxt2 = 0, ev_nxt2 = 0;
      if (t + 2 < n_tiles) {
        stage_k(k_fill, t + 2);
        ek_nxt2 = kexp[t + 2];
        ev_nxt2 = vexp[t + 2];
      }
      stage_v(v_fill, t + 1);
      softmax_pv(std::false_type{}, std::true_type{}, s_in, v_cur, t, ev_cur, k_next, ek_nxt, s_out);
      ek_cur = ek_nxt;
      ev_cur = ev_nxt;
      ek_nxt = ek_nxt2;
      ev_nxt = ev_nxt2;
      wait_vmem();
      __syncthreads();
    };
    auto finish = [&](f32x16 (&sc)[2], const uint8_t* vbuf) {
      if (n_keys % F8_BC != 0)
        softmax_pv(std::true_type{}, std::false_type{}, sc, vbuf, last, ev_cur, nullptr, 0, sc);
      else
        softmax_pv(std::false_type{}, std::false_type{}, sc, vbuf, last, ev_cur, nullptr, 0, sc);
    };
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
  }

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
      const float lse = (l_tot > 0.f) ? (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f : -INFINITY;
      p.lse[((int64_t)b * p.H + h) * p.Lq + i] = lse;
    }
  }
}

}  // namespace

hipError_t launch_kv8_tiles(const uint16_t* k, const uint16_t* v, uint8_t* k8, int* kexp, uint8_t* v8, int* vexp,
                            int B, int L, int H, const RopeDev& rope, hipStream_t stream) {
  const int nt = (L + TILE_ROWS - 1) / TILE_ROWS;
  const int64_t total = (int64_t)B * H * nt;
  if (total <= 0 || total > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv8_tiles_kernel, dim3((unsigned)total), dim3(256), 0, stream, k, v, k8, kexp, v8, vexp, L, H,
                     nt, rope);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_fp8(const FwdParams& p, const uint8_t* k8, const int* kexp, const uint8_t* v8,
                               const int* vexp, hipStream_t stream) {
  FwdParams q = p;
  q.n_qtiles = (p.Lq + F8_BR - 1) / F8_BR;
  const int64_t total = (int64_t)q.n_qtiles * p.H * p.B;
  if (total <= 0 || total > 0x7fffffff || p.Lq != p.Lk) return hipErrorInvalidValue;
  if ((int64_t)((p.Lk + F8_BC - 1) / F8_BC) * F8_TILE_BYTES > (int64_t)0xffffffff) return hipErrorInvalidValue;
  q.n_items = (int)total;
  int64_t wgs = total;
  if (q.work != nullptr) {
    if (!work_fits(total)) return hipErrorInvalidValue;
    wgs = work_grid(total);
    hipLaunchKernelGGL(work_reset_kernel, dim3(1), dim3(1), 0, stream, q.work);
  }
  if (p.scale_log2 > 0.f)
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<true>), dim3((unsigned)wgs), dim3(256), 0, stream, q, k8, kexp, v8,
                       vexp);
  else
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<false>), dim3((unsigned)wgs), dim3(256), 0, stream, q, k8, kexp, v8,
                       vexp);
  return hipGetLastError();
}

}  // namespace wanattn
