// Kernel parameter blocks and launchers (internal to libwanattn).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace wanattn {

// Attention forward (self or cross).  q/o: [B, Lq, H, 128], k/v: [B, Lk, H, 128] bf16.
struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;               // [B, H, Lq] or nullptr
  const int32_t* k_lens;    // [B] valid key counts or nullptr (all Lk)
  // Self-attention: k and v in the tile layout of launch_kv_tiles (then k/v
  // above are unused), [B, H, ceil(Lk/64)] tiles; nullptr: read k/v directly.
  const uint16_t* kt;       // keys, tiles of [64][128]: bf16, or with RoPE fp16 of R(p) k * 2^-e_t
  const int* kexp;          // with RoPE: e_t of every tile, else nullptr
  const uint16_t* vt;       // V^T, tiles of [128][64] bf16
  RopeDev rope;             // rope.table == nullptr: queries are not rotated
  int B, Lq, Lk, H;
  float scale_log2;         // softmax scale * log2(e)
  int n_qtiles;             // set by the launcher
};

// Self-attention backward.  All [B, L, H, 128] bf16 except lse/delta [B, H, L] fp32.
struct BwdParams {
  const uint16_t* q;        // rotated queries (bf16 hi part when q_lo != nullptr)
  const uint16_t* q_lo;     // rotated queries, lo part (q - hi rounded to bf16), or nullptr
  const uint16_t* k;        // rotated keys
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  float* delta;             // workspace [B, H, L]
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  RopeDev rope;             // rope.table != nullptr: rotate dq/dk back by minus the angle
  int B, L, H;
  float scale;
  float scale_log2;
  int n_tiles;              // set by the launchers
};

hipError_t launch_rope_table(float* table, int f, int h, int w, int d_f, int d_h, int d_w, double theta,
                             hipStream_t stream);
hipError_t launch_rope3d(const uint16_t* x, uint16_t* y, int B, int L, int H, const RopeDev& rope,
                         bool inverse, hipStream_t stream);
hipError_t launch_rope3d_split(const uint16_t* x, uint16_t* hi, uint16_t* lo, int B, int L, int H,
                               const RopeDev& rope, hipStream_t stream);
hipError_t launch_kv_tiles(const uint16_t* k, const uint16_t* v, uint16_t* kt, int* kexp, uint16_t* vt, int B, int L,
                           int H, const RopeDev& rope, hipStream_t stream);
hipError_t launch_attn_fwd(const FwdParams& p, hipStream_t stream);
hipError_t launch_bwd_delta(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdParams& p, hipStream_t stream);

}  // namespace wanattn
