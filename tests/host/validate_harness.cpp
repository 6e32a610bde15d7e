// Host-only harness over the library's argument checks
// (spatio_temporal_attention_amd/csrc/validate.cpp, pure C++), built with plain
// g++ and no HIP by tests/test_validate_host.py.  Each entry point forwards to
// one check with C linkage so the test can call it through ctypes.
#include "../../spatio_temporal_attention_amd/csrc/validate.h"

using namespace wanattn;

#define H_API extern "C" __attribute__((visibility("default")))

H_API int h_check_dims(int B, int L, int H, int D) { return check_dims(B, L, H, D); }
H_API int h_check_grid_rope(wanattn_grid g, wanattn_rope r, int L, int D) { return check_grid_rope(g, r, L, D); }
H_API int h_check_scale(float s) { return check_scale(s); }
H_API long long h_rope_table_entries(wanattn_grid g, wanattn_rope r) { return (long long)rope_table_entries(g, r); }
H_API void h_fwd_tail_split(int B, int Lq, int H, int* out) {
  const FwdSplit s = fwd_tail_split(B, Lq, H);
  out[0] = s.n;
  out[1] = s.n_main;
  out[2] = s.tail;
  out[3] = s.S;
}
H_API void h_fwd_split(int B, int Lq, int H, int* out) {
  const FwdSplit s = fwd_split(B, Lq, H);
  out[0] = s.n;
  out[1] = s.n_main;
  out[2] = s.tail;
  out[3] = s.S;
}
H_API int h_bwd_q_split(int B, int Lq, int Lk, int H) { return bwd_q_split(B, Lq, Lk, H); }
H_API size_t h_self_fwd_ws_bytes(int B, int L, int H, int D, int rope) { return self_fwd_ws_bytes(B, L, H, D, rope); }
H_API size_t h_fwd_tiles_ws_bytes(int B, int L, int H, int D, int rope) { return fwd_tiles_ws_bytes(B, L, H, D, rope); }
H_API size_t h_self_bwd_ws_bytes(int B, int L, int H, int D, int rope) { return self_bwd_ws_bytes(B, L, H, D, rope); }
H_API size_t h_cross_bwd_ws_bytes(int B, int Lq, int Lk, int H, int D) { return cross_bwd_ws_bytes(B, Lq, Lk, H, D); }

H_API int h_validate_rope3d(const void* x, const void* y, int B, int L, int H, int D, wanattn_grid g, wanattn_rope r,
                            const float* table) {
  return validate_rope3d(x, y, B, L, H, D, g, r, table);
}
H_API int h_validate_self_fwd(const void* q, const void* k, const void* v, const void* o, const float* lse, int B,
                              int L, int H, int D, wanattn_grid g, wanattn_rope r, const float* table, float scale,
                              const void* ws, size_t ws_bytes) {
  return validate_self_fwd(q, k, v, o, lse, B, L, H, D, g, r, table, scale, ws, ws_bytes);
}
H_API int h_validate_self_fwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                     const int32_t* seq_lens, int B, int L, int H, int D, wanattn_grid g,
                                     wanattn_rope r, const float* table, float scale, const void* ws,
                                     size_t ws_bytes) {
  return validate_self_fwd_varlen(q, k, v, o, lse, seq_lens, B, L, H, D, g, r, table, scale, ws, ws_bytes);
}
H_API int h_validate_partial_fwd(const void* q, const void* k, const void* v, const void* o, const float* lse, int B,
                                 int Lq, int Lk, int H, int D, wanattn_grid g, wanattn_rope r, const float* table,
                                 int q_offset, int k_offset, float scale, const void* ws, size_t ws_bytes) {
  return validate_partial_fwd(q, k, v, o, lse, B, Lq, Lk, H, D, g, r, table, q_offset, k_offset, scale, ws, ws_bytes);
}
H_API int h_validate_lse_merge(const void* const* o_parts, const float* const* lse_parts, int R, const void* o,
                               const float* lse, int B, int L, int H, int D) {
  return validate_lse_merge(o_parts, lse_parts, R, o, lse, B, L, H, D);
}
H_API int h_validate_self_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, const void* dq, const void* dk, const void* dv, int B, int L, int H,
                              int D, wanattn_grid g, wanattn_rope r, const float* table, float scale, const void* ws,
                              size_t ws_bytes) {
  return validate_self_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, L, H, D, g, r, table, scale, ws, ws_bytes);
}
H_API int h_validate_cross_bwd(const void* q, const void* k, const void* v, const int32_t* k_lens, const void* o,
                               const float* lse, const void* dout, const void* dq, const void* dk, const void* dv,
                               int B, int Lq, int Lk, int H, int D, float scale, const void* ws, size_t ws_bytes) {
  return validate_cross_bwd(q, k, v, k_lens, o, lse, dout, dq, dk, dv, B, Lq, Lk, H, D, scale, ws, ws_bytes);
}
H_API int h_validate_cross_fwd(const void* q, const void* k, const void* v, const int32_t* k_lens, const void* o,
                               const float* lse, int B, int Lq, int Lk, int H, int D, float scale, const void* ws,
                               size_t ws_bytes) {
  return validate_cross_fwd(q, k, v, k_lens, o, lse, B, Lq, Lk, H, D, scale, ws, ws_bytes);
}
