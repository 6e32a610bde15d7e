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
  const int32_t* q_lens;    // [B] valid query counts or nullptr (all Lq); rows past it are not written
  int q_pos0, k_pos0;       // RoPE token index of query row 0 and key row 0 (shards of a longer sequence)
  // k and v in the tile layout of launch_kv_tiles (k/v above are then
  // unused), [B, H, ceil(Lk/64)] tiles.
  const uint16_t* kt;       // keys, tiles of [64][128]: bf16, or with RoPE fp16 of R(p) k * 2^-e_t
  const int* kexp;          // with RoPE: e_t of every tile, else nullptr
  const uint16_t* vt;       // V^T, tiles of [128][64] bf16
  RopeDev rope;             // rope.table == nullptr: queries are not rotated
  int B, Lq, Lk, H;
  float scale_log2;         // softmax scale * log2(e)
  int n_qtiles;             // set by the launcher
  // Tail split (self-attention only): fp32 partials of the last query tiles'
  // key ranges (nullptr: no split); qt_base and n_split are set by the launcher.
  float* part;
  int qt_base, n_split;
  // The main launch with its split pieces at the end (set by the launcher):
  // workgroups [0, n_main_wg) take whole query tiles, the rest the pieces.
  int n_main_wg;
  // Main launch with fixed lengths: a work counter, zero at launch, from which
  // workgroups take their items, and the number of items (n_main_wg whole
  // tiles, then the pieces); work == nullptr: workgroup x takes item x.
  int* work;
  int n_items;
};

// Self-attention backward over the prep passes' tiles: [B, H, ceil(L/64)]
// tiles of 16 KB each (row tiles [64][128], T tiles [128][64]).
struct BwdParams {
  const uint16_t* qf;       // Q row tiles, fp16 of R(p) q * 2^-e
  const int* qexp;          // e of every Q tile
  const uint16_t* qt;       // (R q)^T T tiles, bf16
  const uint16_t* dor;      // dO row tiles, bf16
  const uint16_t* dot;      // dO^T T tiles, bf16
  const uint16_t* kf;       // K row tiles, fp16 of R(p) k * 2^-e
  const int* kexp;          // e of every K tile
  const uint16_t* kt;       // (R k)^T T tiles, bf16
  const uint16_t* vr;       // V row tiles, bf16
  const float* lse;         // [B, H, L]
  const float* qstat;       // per query tile [B, H, nt][QSTAT_FLOATS]: LSE_i * log2(e), then -Delta_i
  uint16_t* dq;             // [B, L, H, 128] bf16 outputs
  uint16_t* dk;
  uint16_t* dv;
  const int32_t* k_lens;    // [B] valid key counts (keys past them get P = 0 and zero gradients) or nullptr
  RopeDev rope;             // rope.table != nullptr: rotate dq/dk back by minus the angle
  int B, Lq, Lk, H;         // q-side tensors [B, Lq, H, 128], k-side [B, Lk, H, 128]
  float scale;
  float scale_log2;
  int q_split;              // dK/dV: query range split over this many workgroups per key block (>= 1)
  float* part;              // q_split > 1: fp32 partial dK~ then dV, [q_split][B][H][Lk][128] each
  // Tail split of the dQ pass: fp32 partials of dq~ (nullptr: none); dq_base and
  // dq_split are set by the launcher.
  float* dq_part;
  int dq_base, dq_split;
  // Tail split of the dK/dV passes (q_split == 1 only): fp32 partials of dK~ then dV (nullptr: none);
  // kv_base and kv_split are set by the launcher.
  float* kv_part;
  int kv_base, kv_split;
  int n_tiles;              // set by the launchers
};

hipError_t launch_rope_table(float* table, int f, int h, int w, int d_f, int d_h, int d_w, double theta,
                             hipStream_t stream);
hipError_t launch_rope3d(const uint16_t* x, uint16_t* y, int B, int L, int H, const RopeDev& rope,
                         bool inverse, hipStream_t stream);
// lens: [B] valid token counts (tokens past them are treated as zero) or nullptr;
// pos0: RoPE token index of row 0.
hipError_t launch_kv_tiles(const uint16_t* k, const uint16_t* v, uint16_t* kt, int* kexp, uint16_t* vt, int B, int L,
                           int H, const RopeDev& rope, const int32_t* lens, int pos0, hipStream_t stream);
// O = sum_r exp(LSE_r - LSE) O_r, LSE = ln sum_r exp(LSE_r) over R <= MERGE_MAX partial results.
constexpr int MERGE_MAX = 16;
struct MergeParams {
  const uint16_t* o[MERGE_MAX];   // [B, L, H, 128] bf16
  const float* lse[MERGE_MAX];    // [B, H, L]
  uint16_t* out;
  float* out_lse;                 // or nullptr
  int R, B, L, H;
};
hipError_t launch_lse_merge(const MergeParams& p, hipStream_t stream);
// Attention over the prep pass's tiles (p.kt, p.vt, and p.kexp with RoPE): self-attention, its shards
// and variable lengths, and cross-attention (Lq != Lk, p.k_lens, no RoPE).
hipError_t launch_attn_fwd_tiled(const FwdParams& p, hipStream_t stream);
// FP8 forward: K as e4m3 row tiles [64][128] and V as e4m3 V^T tiles [128][64]
// (8 KB each, key order kappa), with int32 exponents per tile.
hipError_t launch_kv8_tiles(const uint16_t* k, const uint16_t* v, uint8_t* k8, int* kexp, uint8_t* v8, int* vexp,
                            int B, int L, int H, const RopeDev& rope, hipStream_t stream);
hipError_t launch_attn_fwd_fp8(const FwdParams& p, const uint8_t* k8, const int* kexp, const uint8_t* v8,
                               const int* vexp, hipStream_t stream);
hipError_t launch_bwd_k_tiles(const uint16_t* k, const uint16_t* v, uint16_t* kf, int* kexp, uint16_t* kt,
                              uint16_t* vr, int B, int L, int H, const RopeDev& rope, const int32_t* lens,
                              hipStream_t stream);
hipError_t launch_bwd_q_tiles(const uint16_t* q, const uint16_t* dout, const uint16_t* o, const float* lse,
                              uint16_t* qf, int* qexp, uint16_t* qt, uint16_t* dor, uint16_t* dot, float* qstat, int B,
                              int L, int H, const RopeDev& rope, hipStream_t stream);
// The dV pass alone (attn_bwd_dv.hip), p.n_tiles = key blocks of 256; called by launch_bwd_dkdv
// with the workgroup counts of the main launch and of the tail split's launch (0: none).
hipError_t launch_bwd_dv(const BwdParams& p, int n_main, int n_tail, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdParams& p, hipStream_t stream);
// Measurement aid (mfma_peak.hip): workgroups x 4 waves, each iters x 4 back-to-back bf16 MFMAs.
hipError_t launch_mfma_peak(float* sink, int workgroups, int iters, hipStream_t stream);

}  // namespace wanattn
