// Host-side argument checks of the wanattn C interface.  Pure C++ (no HIP),
// so the rules can be read and tested apart from the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/wanattn.h"

namespace wanattn {

// Largest element count of one [B, L, H, D] tensor the kernels index (64-bit
// offsets are used throughout; this bounds grids and int32 row counts).
constexpr int64_t MAX_TENSOR_ELEMS = (int64_t)1 << 40;

int check_dims(int B, int L, int H, int D);
int check_grid_rope(wanattn_grid g, wanattn_rope r, int L, int D);
int check_rope_only(wanattn_grid g, wanattn_rope r, int D);
int check_scale(float scale);
bool aligned(const void* p, size_t a);
int64_t rope_table_entries(wanattn_grid g, wanattn_rope r);   // (cos, sin) pairs; -1 if invalid

// Tail split of the self-attention forward.  Its workgroups take 256 query
// rows each, FWD_ROUND of them run at once (one per CU of an MI355X); when
// there are at least four rounds and the count n is not a multiple of the
// round, the last tail = n % FWD_ROUND query tiles would run alone on a few
// CUs.  They run instead as S = FWD_ROUND / tail (at most 8) key ranges each,
// whose fp32 partials a merge pass combines exactly.  S < 2: no split.
// (fwd_tail_split; the backward's dQ and dK/dV passes split their tails by it.)
// The self-attention forward itself (fwd_split) runs its pieces at the end of
// the main launch, after the whole query tiles, and from eight rounds on it
// also splits one more round, 4 key ranges per tile: over tens of rounds the
// CUs drift apart by about a round, and those that finish their last whole
// tile early take the pieces instead of idling until the last one finishes.
constexpr int FWD_ROUND = 256;
constexpr int FWD_ROWS = 256;          // query rows per forward workgroup
constexpr int FWD_PART_FLOATS = 132;   // per partial row: O (128, unnormalized), m (log2), l, 2 pad (16-byte rows)
struct FwdSplit {
  int n;        // workgroups of the whole forward
  int n_main;   // workgroups of the main launch (the first n_main query tiles)
  int tail;     // query tiles of the split launch (0: no split)
  int S;        // key ranges per tail tile
};
FwdSplit fwd_tail_split(int B, int Lq, int H);
FwdSplit fwd_split(int B, int Lq, int H);

// Forward workspace, in 64-key tiles of every (b, h): K (bf16, or with RoPE
// the rotated keys in fp16 with a power-of-two exponent per tile), V^T
// (bf16), then with RoPE the tile exponents (int32), then the main launch's
// work counter (256 bytes), then (self-attention with a tail split only) the
// fp32 partials [tail * S][FWD_ROWS][132]; each part starts on a 256-byte
// boundary.
struct FwdWsLayout {
  size_t kt, vt, kexp, part, work, total;   // byte offsets of the parts and the total size (part: 0 if none)
};
FwdWsLayout self_fwd_ws_layout(int B, int L, int H, int D, int with_rope);
size_t self_fwd_ws_bytes(int B, int L, int H, int D, int with_rope);
// The key/value tiles alone (the shard forward, whose query and key lengths differ, takes no split).
size_t fwd_tiles_ws_bytes(int B, int L, int H, int D, int with_rope);
// FP8 forward workspace: K and V^T e4m3 tiles ([B, H, ceil(L/64)] x 8 KB each), then
// their int32 exponents, then the work counter (256 bytes); each part on a 256-byte boundary.
struct Fp8WsLayout {
  size_t k8, v8, kexp, vexp, work, total;
};
Fp8WsLayout self_fwd_fp8_ws_layout(int B, int L, int H, int D);
// Backward workspace: the row statistics of every query tile (fp32
// [B, H, ceil(L/64)][256]: LSE * log2 e, -Delta, the tile exponent), then the prep passes' tiles
// (each [B, H, ceil(L/64)] x 16 KB), the two exponent arrays (int32 per
// tile) and, when the dK/dV passes split the query range (q_split > 1), their
// fp32 partials (2 x q_split x [B, H, Lk, D]); each part starts on a 256-byte
// boundary.
struct BwdWsLayout {
  size_t qstat, qf, qt, dor, dot, kf, kt, vr, qexp, kexp, part, kv_part, dq_part, total;
  int q_split;
  FwdSplit kv_split;   // tail split of the dK/dV passes (256-key blocks; only without a query split)
  FwdSplit dq_split;   // tail split of the dQ pass (256-row query blocks, the forward's rule)
};
// Query-side parts (qstat, qf, qt, dor, dot, qexp) over Lq tokens, key-side
// parts (kf, kt, vr, kexp) over Lk.
// Query-range split of the dK/dV passes: 1 while the key blocks alone give at
// least 256 workgroups, else enough splits for ~512 (each >= 8 query tiles, at
// most 32); their fp32 partials live in the backward workspace.
int bwd_q_split(int B, int Lq, int Lk, int H);
BwdWsLayout bwd_ws_layout(int B, int Lq, int Lk, int H, int D);
size_t self_bwd_ws_bytes(int B, int L, int H, int D, int with_rope);
size_t cross_bwd_ws_bytes(int B, int Lq, int Lk, int H, int D);

int validate_rope3d(const void* x, const void* y, int B, int L, int H, int D, wanattn_grid g, wanattn_rope r,
                    const float* table);
// Every check of validate_self_fwd except the workspace's.
int validate_self_fwd_args(const void* q, const void* k, const void* v, const void* o, const float* lse, int B,
                           int L, int H, int D, wanattn_grid g, wanattn_rope r, const float* table, float scale);
int validate_self_fwd(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int L,
                      int H, int D, wanattn_grid g, wanattn_rope r, const float* table, float scale,
                      const void* ws, size_t ws_bytes);
int validate_self_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, const void* dq, const void* dk, const void* dv, int B, int L, int H,
                      int D, wanattn_grid g, wanattn_rope r, const float* table, float scale, const void* ws,
                      size_t ws_bytes);
int validate_self_fwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const int32_t* seq_lens, int B, int L, int H, int D, wanattn_grid g, wanattn_rope r,
                             const float* table, float scale, const void* ws, size_t ws_bytes);
int validate_partial_fwd(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int Lq,
                         int Lk, int H, int D, wanattn_grid g, wanattn_rope r, const float* table, int q_offset,
                         int k_offset, float scale, const void* ws, size_t ws_bytes);
int validate_lse_merge(const void* const* o_parts, const float* const* lse_parts, int R, const void* o,
                       const float* lse, int B, int L, int H, int D);
int validate_cross_bwd(const void* q, const void* k, const void* v, const int32_t* k_lens, const void* o,
                       const float* lse, const void* dout, const void* dq, const void* dk, const void* dv, int B,
                       int Lq, int Lk, int H, int D, float scale, const void* ws, size_t ws_bytes);
int validate_cross_fwd(const void* q, const void* k, const void* v, const int32_t* k_lens, const void* o,
                       const float* lse, int B, int Lq, int Lk, int H, int D, float scale, const void* ws,
                       size_t ws_bytes);

}  // namespace wanattn
