// Host-side argument checks of the wanattn C interface (see validate.h).
#include <algorithm>
#include "validate.h"

#include <math.h>

namespace wanattn {

int check_dims(int B, int L, int H, int D) {
  if (B <= 0 || L <= 0 || H <= 0) return WANATTN_ERR_SHAPE;
  if (D != WANATTN_HEAD_DIM) return WANATTN_ERR_UNSUPPORTED;
  const int64_t elems = (int64_t)B * L * H * D;
  if (elems > MAX_TENSOR_ELEMS) return WANATTN_ERR_SHAPE;
  // workgroups of 128 rows per (b, h) must fit a 1-D grid
  if ((int64_t)B * H * ((L + 127) / 128) > 0x7fffffff) return WANATTN_ERR_SHAPE;
  return WANATTN_OK;
}

int check_rope_only(wanattn_grid g, wanattn_rope r, int D) {
  if (g.f <= 0 || g.h <= 0 || g.w <= 0) return WANATTN_ERR_SHAPE;
  if (r.d_f < 0 || r.d_h < 0 || r.d_w < 0) return WANATTN_ERR_UNSUPPORTED;
  if ((r.d_f | r.d_h | r.d_w) & 1) return WANATTN_ERR_UNSUPPORTED;
  if ((int64_t)r.d_f + r.d_h + r.d_w != D) return WANATTN_ERR_UNSUPPORTED;
  if (!(r.theta > 0.f) || !isfinite(r.theta)) return WANATTN_ERR_UNSUPPORTED;
  return WANATTN_OK;
}

int check_grid_rope(wanattn_grid g, wanattn_rope r, int L, int D) {
  const int rc = check_rope_only(g, r, D);
  if (rc != WANATTN_OK) return rc;
  if ((int64_t)g.f * g.h * g.w != (int64_t)L) return WANATTN_ERR_SHAPE;
  return WANATTN_OK;
}

int check_scale(float scale) { return isfinite(scale) ? WANATTN_OK : WANATTN_ERR_UNSUPPORTED; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int64_t rope_table_entries(wanattn_grid g, wanattn_rope r) {
  if (check_rope_only(g, r, r.d_f + r.d_h + r.d_w) != WANATTN_OK) return -1;
  if (r.d_f + r.d_h + r.d_w <= 0) return -1;
  return (int64_t)g.f * (r.d_f / 2) + (int64_t)g.h * (r.d_h / 2) + (int64_t)g.w * (r.d_w / 2);
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

FwdSplit fwd_tail_split(int B, int Lq, int H) {
  const int64_t n64 = (int64_t)B * H * (((int64_t)Lq + FWD_ROWS - 1) / FWD_ROWS);
  const int n = (int)std::min<int64_t>(n64, 0x7fffffff);
  FwdSplit sp{n, n, 0, 1};
  if (n64 < 4 * FWD_ROUND || n % FWD_ROUND == 0) return sp;
  const int tail = n % FWD_ROUND;
  const int S = std::min(8, FWD_ROUND / tail);
  if (S < 2) return sp;
  sp.n_main = n - tail;
  sp.tail = tail;
  sp.S = S;
  return sp;
}

FwdSplit fwd_split(int B, int Lq, int H) {
  FwdSplit sp = fwd_tail_split(B, Lq, H);
  if ((int64_t)sp.n < 8 * FWD_ROUND) return sp;
  const int tail = sp.n % FWD_ROUND + FWD_ROUND;
  sp.n_main = sp.n - tail;
  sp.tail = tail;
  sp.S = 4;
  return sp;
}

static FwdWsLayout fwd_tiles_layout(int B, int L, int H, int D, int with_rope) {
  FwdWsLayout w{0, 0, 0, 0, 0, 0};
  if (check_dims(B, L, H, D) != WANATTN_OK) return w;
  const size_t tiles = (size_t)B * H * (((size_t)L + 63) / 64);
  const size_t tile_elems = tiles * 64 * (size_t)D;
  w.kt = 0;                                   // K tiles [B, H, tile, 64, D], bf16 or fp16
  w.vt = align256(tile_elems * 2);            // V^T tiles [B, H, tile, D, 64] bf16
  w.total = align256(w.vt + tile_elems * 2);
  if (with_rope) {
    w.kexp = w.total;                         // exponent of every K tile, int32 [B, H, tile]
    w.total = w.kexp + tiles * 4;
  }
  // The main launch's work counter (one int, on 256 bytes of its own).
  w.work = align256(w.total);
  w.total = w.work + 256;
  return w;
}

FwdWsLayout self_fwd_ws_layout(int B, int L, int H, int D, int with_rope) {
  FwdWsLayout w = fwd_tiles_layout(B, L, H, D, with_rope);
  if (w.total == 0) return w;
  const FwdSplit sp = fwd_split(B, L, H);   // covers fwd_tail_split's tail too
  if (sp.tail > 0) {
    w.part = align256(w.total);
    w.total = w.part + (size_t)sp.tail * sp.S * FWD_ROWS * FWD_PART_FLOATS * 4;
  }
  return w;
}

size_t self_fwd_ws_bytes(int B, int L, int H, int D, int with_rope) {
  return self_fwd_ws_layout(B, L, H, D, with_rope).total;
}

size_t fwd_tiles_ws_bytes(int B, int L, int H, int D, int with_rope) {
  return fwd_tiles_layout(B, L, H, D, with_rope).total;
}

Fp8WsLayout self_fwd_fp8_ws_layout(int B, int L, int H, int D) {
  Fp8WsLayout w{};
  if (check_dims(B, L, H, D) != WANATTN_OK) return w;
  const size_t tiles = (size_t)B * H * (((size_t)L + 63) / 64);
  w.k8 = 0;
  w.v8 = align256(tiles * 64 * (size_t)D);
  w.kexp = align256(w.v8 + tiles * 64 * (size_t)D);
  w.vexp = align256(w.kexp + tiles * 4);
  w.work = align256(w.vexp + tiles * 4);   // the work counter (one int, on 256 bytes of its own)
  w.total = w.work + 256;
  return w;
}

int bwd_q_split(int B, int Lq, int Lk, int H) {
  const int64_t key_blocks = ((int64_t)Lk + 255) / 256 * H * B;   // dK workgroups without a split
  if (key_blocks <= 0 || key_blocks >= 256) return 1;
  const int64_t nt = ((int64_t)Lq + 63) / 64;
  // At least two rounds of 256 workgroups, at most 32 ranges of >= 8 query tiles each; among those, the
  // split whose last round is fullest (the smallest on a tie): a third round of 48 workgroups would leave
  // four fifths of the chip idle for a third of the pass.
  const int64_t lo = (512 + key_blocks - 1) / key_blocks;
  const int64_t hi = std::max<int64_t>(1, std::min<int64_t>(32, nt / 8));
  if (lo >= hi) return (int)hi;
  int64_t best = lo;
  double best_fill = 0.0;
  for (int64_t s = lo; s <= hi; ++s) {
    const int64_t n = key_blocks * s;
    const double fill = (double)n / (double)(256 * ((n + 255) / 256));
    if (fill > best_fill + 1e-9) {
      best_fill = fill;
      best = s;
    }
  }
  return (int)best;
}

BwdWsLayout bwd_ws_layout(int B, int Lq, int Lk, int H, int D) {
  BwdWsLayout w{};
  if (check_dims(B, Lq, H, D) != WANATTN_OK || check_dims(B, Lk, H, D) != WANATTN_OK) return w;
  const size_t qtiles = (size_t)B * H * (((size_t)Lq + 63) / 64);
  const size_t ktiles = (size_t)B * H * (((size_t)Lk + 63) / 64);
  const size_t qbytes = qtiles * 64 * (size_t)D * 2;
  const size_t kbytes = ktiles * 64 * (size_t)D * 2;
  size_t at = 0;
  w.qstat = at;
  at = align256(at + qtiles * 1024);
  size_t* qparts[] = {&w.qf, &w.qt, &w.dor, &w.dot};
  for (size_t* part : qparts) {
    *part = at;
    at = align256(at + qbytes);
  }
  size_t* kparts[] = {&w.kf, &w.kt, &w.vr};
  for (size_t* part : kparts) {
    *part = at;
    at = align256(at + kbytes);
  }
  w.qexp = at;
  at = align256(at + qtiles * 4);
  w.kexp = at;
  at += ktiles * 4;
  w.q_split = bwd_q_split(B, Lq, Lk, H);
  w.part = 0;
  if (w.q_split > 1) {
    w.part = align256(at);
    at = w.part + 2 * (size_t)w.q_split * B * H * Lk * (size_t)D * 4;
  }
  // dK/dV passes without a query split: the last key blocks as query ranges, fp32 partials of dK~ then
  // dV, [tail * S][256 keys][D] each.
  w.kv_split = FwdSplit{0, 0, 0, 1};
  if (w.q_split == 1) w.kv_split = fwd_tail_split(B, Lk, H);
  w.kv_part = 0;
  if (w.kv_split.tail > 0) {
    w.kv_part = align256(at);
    at = w.kv_part + 2 * (size_t)w.kv_split.tail * w.kv_split.S * FWD_ROWS * (size_t)D * 4;
  }
  // dQ pass: the last query blocks as key ranges, fp32 partials of dq~ [tail * S][256 rows][D].
  w.dq_split = fwd_tail_split(B, Lq, H);
  w.dq_part = 0;
  if (w.dq_split.tail > 0) {
    w.dq_part = align256(at);
    at = w.dq_part + (size_t)w.dq_split.tail * w.dq_split.S * FWD_ROWS * (size_t)D * 4;
  }
  w.total = at;
  return w;
}

size_t self_bwd_ws_bytes(int B, int L, int H, int D, int with_rope) {
  (void)with_rope;   // the same tiles serve both
  return bwd_ws_layout(B, L, L, H, D).total;
}

size_t cross_bwd_ws_bytes(int B, int Lq, int Lk, int H, int D) { return bwd_ws_layout(B, Lq, Lk, H, D).total; }

static int check_bf16(const void* p) {
  if (p == nullptr) return WANATTN_ERR_NULL;
  return aligned(p, 16) ? WANATTN_OK : WANATTN_ERR_ALIGN;
}

#define WANATTN_TRY(expr)          \
  do {                             \
    const int rc_ = (expr);        \
    if (rc_ != WANATTN_OK) return rc_; \
  } while (0)

int validate_rope3d(const void* x, const void* y, int B, int L, int H, int D, wanattn_grid g, wanattn_rope r,
                    const float* table) {
  if (x == nullptr || y == nullptr || table == nullptr) return WANATTN_ERR_NULL;
  WANATTN_TRY(check_dims(B, L, H, D));
  WANATTN_TRY(check_grid_rope(g, r, L, D));
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(table, 16)) return WANATTN_ERR_ALIGN;
  return WANATTN_OK;
}

int validate_self_fwd_args(const void* q, const void* k, const void* v, const void* o, const float* lse, int B,
                           int L, int H, int D, wanattn_grid g, wanattn_rope r, const float* table, float scale) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return WANATTN_ERR_NULL;
  WANATTN_TRY(check_dims(B, L, H, D));
  if (table != nullptr) WANATTN_TRY(check_grid_rope(g, r, L, D));
  WANATTN_TRY(check_scale(scale));
  WANATTN_TRY(check_bf16(q));
  WANATTN_TRY(check_bf16(k));
  WANATTN_TRY(check_bf16(v));
  WANATTN_TRY(check_bf16(o));
  if (lse != nullptr && !aligned(lse, 4)) return WANATTN_ERR_ALIGN;
  if (table != nullptr && !aligned(table, 16)) return WANATTN_ERR_ALIGN;
  return WANATTN_OK;
}

int validate_self_fwd(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int L,
                      int H, int D, wanattn_grid g, wanattn_rope r, const float* table, float scale,
                      const void* ws, size_t ws_bytes) {
  WANATTN_TRY(validate_self_fwd_args(q, k, v, o, lse, B, L, H, D, g, r, table, scale));
  if (ws == nullptr || ws_bytes < self_fwd_ws_bytes(B, L, H, D, table != nullptr)) return WANATTN_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return WANATTN_ERR_ALIGN;
  return WANATTN_OK;
}

int validate_self_fwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const int32_t* seq_lens, int B, int L, int H, int D, wanattn_grid g, wanattn_rope r,
                             const float* table, float scale, const void* ws, size_t ws_bytes) {
  if (seq_lens == nullptr) return WANATTN_ERR_NULL;
  WANATTN_TRY(validate_self_fwd(q, k, v, o, lse, B, L, H, D, g, r, table, scale, ws, ws_bytes));
  return aligned(seq_lens, 4) ? WANATTN_OK : WANATTN_ERR_ALIGN;
}

int validate_partial_fwd(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int Lq,
                         int Lk, int H, int D, wanattn_grid g, wanattn_rope r, const float* table, int q_offset,
                         int k_offset, float scale, const void* ws, size_t ws_bytes) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return WANATTN_ERR_NULL;
  WANATTN_TRY(check_dims(B, Lq, H, D));
  WANATTN_TRY(check_dims(B, Lk, H, D));
  if (q_offset < 0 || k_offset < 0) return WANATTN_ERR_SHAPE;
  if (table != nullptr) {
    WANATTN_TRY(check_rope_only(g, r, D));
    const int64_t total = (int64_t)g.f * g.h * g.w;
    if ((int64_t)q_offset + Lq > total || (int64_t)k_offset + Lk > total) return WANATTN_ERR_SHAPE;
    if (!aligned(table, 16)) return WANATTN_ERR_ALIGN;
  }
  WANATTN_TRY(check_scale(scale));
  const void* bufs[] = {q, k, v, o};
  for (const void* p : bufs) WANATTN_TRY(check_bf16(p));
  if (lse != nullptr && !aligned(lse, 4)) return WANATTN_ERR_ALIGN;
  if (ws == nullptr || ws_bytes < fwd_tiles_ws_bytes(B, Lk, H, D, table != nullptr)) return WANATTN_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return WANATTN_ERR_ALIGN;
  return WANATTN_OK;
}

int validate_lse_merge(const void* const* o_parts, const float* const* lse_parts, int R, const void* o,
                       const float* lse, int B, int L, int H, int D) {
  if (o_parts == nullptr || lse_parts == nullptr || o == nullptr) return WANATTN_ERR_NULL;
  if (R < 1 || R > 16) return WANATTN_ERR_SHAPE;
  WANATTN_TRY(check_dims(B, L, H, D));
  for (int r = 0; r < R; ++r) {
    if (o_parts[r] == nullptr || lse_parts[r] == nullptr) return WANATTN_ERR_NULL;
    WANATTN_TRY(check_bf16(o_parts[r]));
    if (!aligned(lse_parts[r], 4)) return WANATTN_ERR_ALIGN;
  }
  WANATTN_TRY(check_bf16(o));
  if (lse != nullptr && !aligned(lse, 4)) return WANATTN_ERR_ALIGN;
  return WANATTN_OK;
}

int validate_self_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, const void* dq, const void* dk, const void* dv, int B, int L, int H,
                      int D, wanattn_grid g, wanattn_rope r, const float* table, float scale, const void* ws,
                      size_t ws_bytes) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr || dout == nullptr ||
      dq == nullptr || dk == nullptr || dv == nullptr)
    return WANATTN_ERR_NULL;
  WANATTN_TRY(check_dims(B, L, H, D));
  if (table != nullptr) WANATTN_TRY(check_grid_rope(g, r, L, D));
  WANATTN_TRY(check_scale(scale));
  const void* bufs[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : bufs) WANATTN_TRY(check_bf16(p));
  if (!aligned(lse, 4)) return WANATTN_ERR_ALIGN;
  if (table != nullptr && !aligned(table, 16)) return WANATTN_ERR_ALIGN;
  if (ws == nullptr || ws_bytes < self_bwd_ws_bytes(B, L, H, D, table != nullptr)) return WANATTN_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return WANATTN_ERR_ALIGN;
  return WANATTN_OK;
}

int validate_cross_bwd(const void* q, const void* k, const void* v, const int32_t* k_lens, const void* o,
                       const float* lse, const void* dout, const void* dq, const void* dk, const void* dv, int B,
                       int Lq, int Lk, int H, int D, float scale, const void* ws, size_t ws_bytes) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr || dout == nullptr ||
      dq == nullptr || dk == nullptr || dv == nullptr)
    return WANATTN_ERR_NULL;
  WANATTN_TRY(check_dims(B, Lq, H, D));
  WANATTN_TRY(check_dims(B, Lk, H, D));
  WANATTN_TRY(check_scale(scale));
  const void* bufs[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : bufs) WANATTN_TRY(check_bf16(p));
  if (!aligned(lse, 4)) return WANATTN_ERR_ALIGN;
  if (k_lens != nullptr && !aligned(k_lens, 4)) return WANATTN_ERR_ALIGN;
  if (ws == nullptr || ws_bytes < cross_bwd_ws_bytes(B, Lq, Lk, H, D)) return WANATTN_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return WANATTN_ERR_ALIGN;
  return WANATTN_OK;
}

int validate_cross_fwd(const void* q, const void* k, const void* v, const int32_t* k_lens, const void* o,
                       const float* lse, int B, int Lq, int Lk, int H, int D, float scale, const void* ws,
                       size_t ws_bytes) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return WANATTN_ERR_NULL;
  WANATTN_TRY(check_dims(B, Lq, H, D));
  WANATTN_TRY(check_dims(B, Lk, H, D));
  WANATTN_TRY(check_scale(scale));
  WANATTN_TRY(check_bf16(q));
  WANATTN_TRY(check_bf16(k));
  WANATTN_TRY(check_bf16(v));
  WANATTN_TRY(check_bf16(o));
  if (lse != nullptr && !aligned(lse, 4)) return WANATTN_ERR_ALIGN;
  if (k_lens != nullptr && !aligned(k_lens, 4)) return WANATTN_ERR_ALIGN;
  if (ws == nullptr || ws_bytes < fwd_tiles_ws_bytes(B, Lk, H, D, 0)) return WANATTN_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return WANATTN_ERR_ALIGN;
  return WANATTN_OK;
}

}  // namespace wanattn
