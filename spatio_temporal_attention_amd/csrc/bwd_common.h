// Pieces shared by the backward passes (attn_bwd.hip: dK, dQ, the split
// reduction; attn_bwd_dv.hip: dV, built with another machine scheduler):
// constants, the gradient store with the inverse rotation, register
// fragments of a row tile, and the key-side setup of the dK and dV passes.
#pragma once

#include <utility>

#include "common.h"
#include "kernels.h"

namespace wanattn {
namespace bwd {

constexpr float LOG2E = 1.4426950408889634f;
constexpr int DV_WAVES = 8;
constexpr int DK_WAVES = 8;
constexpr int DQ_WAVES = 8;

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

// Row `r` of a row tile in global memory as the 8 register fragments of the
// 32x32x16 operand layout (lane half `half` holds chunks 2s + half).
__device__ __forceinline__ void load_row_frags(bf16x8 (&f)[8], const uint16_t* tile, int r, int half, bool ok) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    u32x4 x = u32x4{0u, 0u, 0u, 0u};
    if (ok) x = *reinterpret_cast<const u32x4*>(tile + r * HD + (2 * s + half) * 8);
    f[s] = __builtin_bit_cast(bf16x8, x);
  }
}

// ---------------------------------------------------------------------------
// dV and dK: one kernel each, so that either fits two waves per SIMD (a wave
// holding the K and V rows of its keys and both accumulators would need the
// whole register file: one wave per SIMD, nothing to hide LDS latency or
// overlap the softmax with the MFMAs).  The scores are recomputed in both.
// A wave owns 32 keys (lane owns key j); the loop runs over 64-query tiles.
// KMASK: keys j >= k_lens[b] get P = 0 (cross-attention key padding).
// ---------------------------------------------------------------------------

// Per-wave key setup shared by both kernels.
struct KeySide {
  int b, h, nt, j;
  int split, t0, t1;   // this workgroup's share [t0, t1) of the query tiles
  int64_t tile0;     // first query tile of (b, h)
  int64_t ktile0;    // first key tile of (b, h)
  int ktile;         // key tile holding this wave's keys
  bool key_ok, key_live, tile_ok;
  bool wave_live;   // some key of this wave's 32 is valid (all are without a key mask)
};

// TAIL: the tail launch of a pass without a query split; workgroup x is query range
// x % kv_split of key block kv_base + x / kv_split.
template <int NW, bool KMASK, bool TAIL>
__device__ __forceinline__ KeySide key_side(const BwdParams& p, int wave, int col) {
  KeySide k;
  int kb, bh, n_split;
  if (TAIL) {
    const int logical = p.kv_base + (int)blockIdx.x / p.kv_split;
    k.split = (int)blockIdx.x % p.kv_split;
    n_split = p.kv_split;
    kb = logical % p.n_tiles;
    bh = logical / p.n_tiles;
  } else {
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    kb = logical % p.n_tiles;
    const int rest = logical / p.n_tiles;
    k.split = rest % p.q_split;
    n_split = p.q_split;
    bh = rest / p.q_split;
  }
  k.b = bh % p.B;   // batch innermost: every XCD gets the same heads of every item
  k.h = bh / p.B;
  k.nt = (p.Lq + TILE_ROWS - 1) / TILE_ROWS;
  const int chunk = (k.nt + n_split - 1) / n_split;
  k.t0 = min(k.nt, k.split * chunk);
  k.t1 = min(k.nt, k.t0 + chunk);
  const int ntk = (p.Lk + TILE_ROWS - 1) / TILE_ROWS;
  k.tile0 = (int64_t)(k.b * p.H + k.h) * k.nt;
  k.ktile0 = (int64_t)(k.b * p.H + k.h) * ntk;
  // wave w: row 32*(w%2) + col of key tile (32 NW kb + 32 w) / 64
  k.ktile = (NW / 2) * kb + (wave >> 1);
  k.j = kb * 32 * NW + wave * 32 + col;
  k.key_ok = k.j < p.Lk;
  k.key_live = !KMASK || k.j < min(max(p.k_lens[k.b], 0), p.Lk);
  k.wave_live = !KMASK || kb * 32 * NW + wave * 32 < min(max(p.k_lens[k.b], 0), p.Lk);
  k.tile_ok = k.ktile < ntk;
  return k;
}

}  // namespace bwd
}  // namespace wanattn
