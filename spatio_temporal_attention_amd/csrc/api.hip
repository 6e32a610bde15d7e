// The exported C interface of libwanattn (declared in include/wanattn.h):
// argument validation on the host, then launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/wanattn.h"
#include "kernels.h"
#include "validate.h"

#define WANATTN_API extern "C" __attribute__((visibility("default")))

namespace wanattn {
namespace {

constexpr float LOG2E_F = 1.4426950408889634f;

RopeDev make_rope(wanattn_grid g, wanattn_rope r, const float* table) {
  RopeDev d{};
  d.table = reinterpret_cast<const float2*>(table);
  if (table != nullptr) {
    d.gh = g.h;
    d.gw = g.w;
    d.nf = r.d_f / 2;
    d.nh = r.d_h / 2;
    d.nw = r.d_w / 2;
    d.off_h = g.f * d.nf;
    d.off_w = d.off_h + g.h * d.nh;
  } else {
    d.gh = 1;
    d.gw = 1;
  }
  return d;
}

int hip_status(hipError_t e) { return e == hipSuccess ? WANATTN_OK : WANATTN_ERR_HIP; }

}  // namespace
}  // namespace wanattn

using namespace wanattn;

WANATTN_API const char* wanattn_strerror(int status) {
  switch (status) {
    case WANATTN_OK: return "wanattn: success";
    case WANATTN_ERR_NULL: return "wanattn: a required pointer is NULL";
    case WANATTN_ERR_SHAPE: return "wanattn: invalid shape (size <= 0, too large, or grid f*h*w != L)";
    case WANATTN_ERR_UNSUPPORTED:
      return "wanattn: unsupported argument (head dim must be 128; rotary split must be even widths summing to "
             "128; theta > 0; finite scale)";
    case WANATTN_ERR_ALIGN: return "wanattn: misaligned buffer (bf16/table/workspace need 16 bytes, fp32/int32 4)";
    case WANATTN_ERR_WORKSPACE:
      return "wanattn: workspace missing or too small (wanattn_self_fwd_noalloc: the problem needs more than its "
             "256 MiB static scratch)";
    case WANATTN_ERR_HIP: return "wanattn: HIP launch failed";
    default: return "wanattn: unknown status";
  }
}

WANATTN_API size_t wanattn_rope_table_bytes(wanattn_grid g, wanattn_rope r) {
  const int64_t n = rope_table_entries(g, r);
  return n < 0 ? 0 : (size_t)n * 2 * sizeof(float);
}

WANATTN_API int wanattn_rope_table_init(float* table, wanattn_grid g, wanattn_rope r, void* stream) {
  if (table == nullptr) return WANATTN_ERR_NULL;
  if (rope_table_entries(g, r) < 0) return WANATTN_ERR_SHAPE;
  if (!aligned(table, 16)) return WANATTN_ERR_ALIGN;
  return hip_status(launch_rope_table(table, g.f, g.h, g.w, r.d_f, r.d_h, r.d_w, (double)r.theta,
                                      (hipStream_t)stream));
}

WANATTN_API int wanattn_rope3d(const void* x, void* y, int B, int L, int H, int D, wanattn_grid g, wanattn_rope r,
                               const float* table, int inverse, void* stream) {
  const int rc = validate_rope3d(x, y, B, L, H, D, g, r, table);
  if (rc != WANATTN_OK) return rc;
  return hip_status(launch_rope3d((const uint16_t*)x, (uint16_t*)y, B, L, H, make_rope(g, r, table), inverse != 0,
                                  (hipStream_t)stream));
}

WANATTN_API size_t wanattn_self_fwd_workspace_bytes(int B, int L, int H, int D, int with_rope) {
  return self_fwd_ws_bytes(B, L, H, D, with_rope);
}

namespace wanattn {
namespace {

// Self-attention forward over (possibly sharded or length-limited) tokens:
// prep pass into the workspace, then the attention kernel.  lens: [B] valid
// token counts (queries and keys) or nullptr; q_pos0 / k_pos0: RoPE token
// index of the first query / key row.
int run_self_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Lq, int Lk, int H,
                 int D, wanattn_grid g, wanattn_rope r, const float* table, float scale, void* ws,
                 const int32_t* lens, int q_pos0, int k_pos0, bool tail_split, hipStream_t s) {
  const RopeDev rope = make_rope(g, r, table);
  // K (with RoPE rotated once, instead of on every query tile's visit, and
  // stored in fp16 with a power-of-two exponent per tile) and V are rewritten
  // in the forward's 64-key tile layout in one pass; queries are rotated on
  // load.
  // The tail split (self-attention, Lq == Lk) keeps its partials after the tiles.
  const FwdWsLayout wl = self_fwd_ws_layout(B, Lk, H, D, table != nullptr);
  uint16_t* kt = (uint16_t*)((uint8_t*)ws + wl.kt);
  uint16_t* vt = (uint16_t*)((uint8_t*)ws + wl.vt);
  int* kexp = table != nullptr ? (int*)((uint8_t*)ws + wl.kexp) : nullptr;
  const int e = hip_status(
      launch_kv_tiles((const uint16_t*)k, (const uint16_t*)v, kt, kexp, vt, B, Lk, H, rope, lens, k_pos0, s));
  if (e != WANATTN_OK) return e;
  FwdParams p{};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)o;
  p.lse = lse;
  p.k_lens = lens;
  p.q_lens = lens;
  p.q_pos0 = q_pos0;
  p.k_pos0 = k_pos0;
  p.kt = kt;
  p.kexp = kexp;
  p.vt = vt;
  p.rope = rope;
  p.B = B;
  p.Lq = Lq;
  p.Lk = Lk;
  p.H = H;
  p.scale_log2 = scale * LOG2E_F;
  p.part = (tail_split && wl.part != 0) ? (float*)((uint8_t*)ws + wl.part) : nullptr;
  p.work = (int*)((uint8_t*)ws + wl.work);   // right after the tiles in every forward workspace layout
  return hip_status(launch_attn_fwd_tiled(p, s));
}

}  // namespace
}  // namespace wanattn

WANATTN_API int wanattn_self_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int L,
                                 int H, int D, wanattn_grid g, wanattn_rope r, const float* table, float scale,
                                 void* ws, size_t ws_bytes, void* stream) {
  const int rc = validate_self_fwd(q, k, v, o, lse, B, L, H, D, g, r, table, scale, ws, ws_bytes);
  if (rc != WANATTN_OK) return rc;
  return run_self_fwd(q, k, v, o, lse, B, L, L, H, D, g, r, table, scale, ws, nullptr, 0, 0, true, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// Allocation-free self-attention forward.  For callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc): the forward's workspace (the K/V tiles and the tail
// split's partials) lives in one static device array per GPU instead of a
// caller buffer.
// ---------------------------------------------------------------------------
namespace wanattn {

constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)256 << 20;   // 256 MiB per GPU, held until the process ends
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_dev[MAX_DEVICES];   // device address of each GPU's copy of `scratch`, looked up once

// In host code `scratch` names a host-side stand-in, not device memory: the
// device address of the current GPU's copy comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// ever passed to a kernel.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return WANATTN_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return WANATTN_ERR_HIP;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return WANATTN_OK;
}

}  // namespace
}  // namespace wanattn

WANATTN_API int wanattn_self_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                         int L, int H, int D, wanattn_grid g, wanattn_rope r, const float* table,
                                         float scale, void* stream) {
  const int rc = validate_self_fwd_args(q, k, v, o, lse, B, L, H, D, g, r, table, scale);
  if (rc != WANATTN_OK) return rc;
  if (self_fwd_ws_bytes(B, L, H, D, table != nullptr) > NOALLOC_SCRATCH_BYTES) return WANATTN_ERR_WORKSPACE;
  void* ws = nullptr;
  const int e = scratch_address(&ws);
  if (e != WANATTN_OK) return e;
  // The same launches as wanattn_self_fwd; every byte of the scratch they read
  // is written earlier in the same call, so nothing needs clearing.
  return run_self_fwd(q, k, v, o, lse, B, L, L, H, D, g, r, table, scale, ws, nullptr, 0, 0, true, (hipStream_t)stream);
}

WANATTN_API size_t wanattn_self_fwd_fp8_workspace_bytes(int B, int L, int H, int D) {
  return self_fwd_fp8_ws_layout(B, L, H, D).total;
}

WANATTN_API int wanattn_self_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int L,
                                     int H, int D, wanattn_grid g, wanattn_rope r, const float* table, float scale,
                                     void* ws, size_t ws_bytes, void* stream) {
  // Same arguments as wanattn_self_fwd; only the workspace size differs.
  const size_t need = self_fwd_fp8_ws_layout(B, L, H, D).total;
  const int rc = validate_self_fwd(q, k, v, o, lse, B, L, H, D, g, r, table, scale, ws, (size_t)-1);
  if (rc != WANATTN_OK) return rc;
  if (need == 0 || ws_bytes < need) return WANATTN_ERR_WORKSPACE;
  const hipStream_t s = (hipStream_t)stream;
  const RopeDev rope = make_rope(g, r, table);
  const Fp8WsLayout w = self_fwd_fp8_ws_layout(B, L, H, D);
  uint8_t* base = (uint8_t*)ws;
  int e = hip_status(launch_kv8_tiles((const uint16_t*)k, (const uint16_t*)v, base + w.k8, (int*)(base + w.kexp),
                                      base + w.v8, (int*)(base + w.vexp), B, L, H, rope, s));
  if (e != WANATTN_OK) return e;
  FwdParams p{};
  p.q = (const uint16_t*)q;
  p.o = (uint16_t*)o;
  p.lse = lse;
  p.rope = rope;
  p.B = B;
  p.Lq = L;
  p.Lk = L;
  p.H = H;
  p.scale_log2 = scale * LOG2E_F;
  p.work = (int*)(base + w.work);
  return hip_status(launch_attn_fwd_fp8(p, base + w.k8, (const int*)(base + w.kexp), base + w.v8,
                                        (const int*)(base + w.vexp), s));
}

WANATTN_API int wanattn_self_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                                        const int32_t* seq_lens, int B, int L, int H, int D, wanattn_grid g,
                                        wanattn_rope r, const float* table, float scale, void* ws, size_t ws_bytes,
                                        void* stream) {
  const int rc = validate_self_fwd_varlen(q, k, v, o, lse, seq_lens, B, L, H, D, g, r, table, scale, ws, ws_bytes);
  if (rc != WANATTN_OK) return rc;
  return run_self_fwd(q, k, v, o, lse, B, L, L, H, D, g, r, table, scale, ws, seq_lens, 0, 0, true, (hipStream_t)stream);
}

WANATTN_API size_t wanattn_partial_fwd_workspace_bytes(int B, int Lk, int H, int D, int with_rope) {
  return fwd_tiles_ws_bytes(B, Lk, H, D, with_rope);
}

WANATTN_API int wanattn_partial_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Lq,
                                    int Lk, int H, int D, wanattn_grid g, wanattn_rope r, const float* table,
                                    int q_offset, int k_offset, float scale, void* ws, size_t ws_bytes,
                                    void* stream) {
  const int rc =
      validate_partial_fwd(q, k, v, o, lse, B, Lq, Lk, H, D, g, r, table, q_offset, k_offset, scale, ws, ws_bytes);
  if (rc != WANATTN_OK) return rc;
  return run_self_fwd(q, k, v, o, lse, B, Lq, Lk, H, D, g, r, table, scale, ws, nullptr, q_offset, k_offset, false,
                      (hipStream_t)stream);
}

WANATTN_API int wanattn_lse_merge(const void* const* o_parts, const float* const* lse_parts, int R, void* o,
                                  float* lse, int B, int L, int H, int D, void* stream) {
  const int rc = validate_lse_merge(o_parts, lse_parts, R, o, lse, B, L, H, D);
  if (rc != WANATTN_OK) return rc;
  MergeParams p{};
  for (int i = 0; i < R; ++i) {
    p.o[i] = (const uint16_t*)o_parts[i];
    p.lse[i] = lse_parts[i];
  }
  p.out = (uint16_t*)o;
  p.out_lse = lse;
  p.R = R;
  p.B = B;
  p.L = L;
  p.H = H;
  return hip_status(launch_lse_merge(p, (hipStream_t)stream));
}

WANATTN_API size_t wanattn_self_bwd_workspace_bytes(int B, int L, int H, int D, int with_rope) {
  return self_bwd_ws_bytes(B, L, H, D, with_rope);
}

namespace wanattn {
namespace {

// Backward over q-side [B, Lq, H, D] and k-side [B, Lk, H, D] tensors: prep
// passes (Q and K, rotated with a table, as fp16 tiles with the forward's
// power-of-two exponents, their bf16 transposes, dO and V tiles, the row
// statistics LSE * log2 e and -Delta), then
// the dK/dV and dQ passes over those tiles.  k_lens: key padding or nullptr.
int run_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
            void* dk, void* dv, const int32_t* k_lens, int B, int Lq, int Lk, int H, int D, const RopeDev& rope,
            float scale, void* ws, hipStream_t s) {
  const BwdWsLayout w = bwd_ws_layout(B, Lq, Lk, H, D);
  uint8_t* base = (uint8_t*)ws;
  BwdParams p{};
  p.qf = (const uint16_t*)(base + w.qf);
  p.qexp = (const int*)(base + w.qexp);
  p.qt = (const uint16_t*)(base + w.qt);
  p.dor = (const uint16_t*)(base + w.dor);
  p.dot = (const uint16_t*)(base + w.dot);
  p.kf = (const uint16_t*)(base + w.kf);
  p.kexp = (const int*)(base + w.kexp);
  p.kt = (const uint16_t*)(base + w.kt);
  p.vr = (const uint16_t*)(base + w.vr);
  p.lse = lse;
  p.qstat = (const float*)(base + w.qstat);
  p.dq = (uint16_t*)dq;
  p.dk = (uint16_t*)dk;
  p.dv = (uint16_t*)dv;
  p.k_lens = k_lens;
  p.rope = rope;
  p.B = B;
  p.Lq = Lq;
  p.Lk = Lk;
  p.H = H;
  p.scale = scale;
  p.scale_log2 = scale * LOG2E_F;
  p.q_split = w.q_split;
  p.part = (float*)(base + w.part);
  p.dq_part = w.dq_part != 0 ? (float*)(base + w.dq_part) : nullptr;
  p.kv_part = w.kv_part != 0 ? (float*)(base + w.kv_part) : nullptr;
  int e = hip_status(launch_bwd_k_tiles((const uint16_t*)k, (const uint16_t*)v, (uint16_t*)(base + w.kf),
                                        (int*)(base + w.kexp), (uint16_t*)(base + w.kt), (uint16_t*)(base + w.vr), B,
                                        Lk, H, rope, k_lens, s));
  if (e != WANATTN_OK) return e;
  e = hip_status(launch_bwd_q_tiles((const uint16_t*)q, (const uint16_t*)dout, (const uint16_t*)o, lse,
                                    (uint16_t*)(base + w.qf), (int*)(base + w.qexp), (uint16_t*)(base + w.qt),
                                    (uint16_t*)(base + w.dor), (uint16_t*)(base + w.dot), (float*)(base + w.qstat), B,
                                    Lq, H, rope, s));
  if (e != WANATTN_OK) return e;
  e = hip_status(launch_bwd_dkdv(p, s));
  if (e != WANATTN_OK) return e;
  return hip_status(launch_bwd_dq(p, s));
}

}  // namespace
}  // namespace wanattn

WANATTN_API int wanattn_self_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                 const void* dout, void* dq, void* dk, void* dv, int B, int L, int H, int D,
                                 wanattn_grid g, wanattn_rope r, const float* table, float scale, void* ws,
                                 size_t ws_bytes, void* stream) {
  const int rc = validate_self_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, L, H, D, g, r, table, scale, ws, ws_bytes);
  if (rc != WANATTN_OK) return rc;
  return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, nullptr, B, L, L, H, D, make_rope(g, r, table), scale, ws,
                 (hipStream_t)stream);
}

WANATTN_API size_t wanattn_cross_bwd_workspace_bytes(int B, int Lq, int Lk, int H, int D) {
  return cross_bwd_ws_bytes(B, Lq, Lk, H, D);
}

WANATTN_API int wanattn_cross_bwd(const void* q, const void* k, const void* v, const int32_t* k_lens, const void* o,
                                  const float* lse, const void* dout, void* dq, void* dk, void* dv, int B, int Lq,
                                  int Lk, int H, int D, float scale, void* ws, size_t ws_bytes, void* stream) {
  const int rc =
      validate_cross_bwd(q, k, v, k_lens, o, lse, dout, dq, dk, dv, B, Lq, Lk, H, D, scale, ws, ws_bytes);
  if (rc != WANATTN_OK) return rc;
  return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, k_lens, B, Lq, Lk, H, D, make_rope({1, 1, 1}, {0, 0, 0, 1.f}, nullptr),
                 scale, ws, (hipStream_t)stream);
}

WANATTN_API size_t wanattn_cross_fwd_workspace_bytes(int B, int Lk, int H, int D) {
  return fwd_tiles_ws_bytes(B, Lk, H, D, 0);
}

WANATTN_API int wanattn_cross_fwd(const void* q, const void* k, const void* v, const int32_t* k_lens, void* o,
                                  float* lse, int B, int Lq, int Lk, int H, int D, float scale, void* ws,
                                  size_t ws_bytes, void* stream) {
  const int rc = validate_cross_fwd(q, k, v, k_lens, o, lse, B, Lq, Lk, H, D, scale, ws, ws_bytes);
  if (rc != WANATTN_OK) return rc;
  // The text keys and values rewritten once into the forward's 64-key tiles
  // (bf16 K, transposed V; keys past k_lens[b] zero and never read), then the
  // self-attention kernel over them with Lq != Lk, the key mask and no RoPE.
  const RopeDev rope = make_rope(wanattn_grid{1, 1, 1}, wanattn_rope{0, 0, 0, 1.f}, nullptr);
  const FwdWsLayout wl = self_fwd_ws_layout(B, Lk, H, D, 0);
  uint16_t* kt = (uint16_t*)((uint8_t*)ws + wl.kt);
  uint16_t* vt = (uint16_t*)((uint8_t*)ws + wl.vt);
  const int e = hip_status(launch_kv_tiles((const uint16_t*)k, (const uint16_t*)v, kt, nullptr, vt, B, Lk, H, rope,
                                           k_lens, 0, (hipStream_t)stream));
  if (e != WANATTN_OK) return e;
  FwdParams p{};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)o;
  p.lse = lse;
  p.k_lens = k_lens;
  p.kt = kt;
  p.vt = vt;
  p.rope = rope;
  p.B = B;
  p.Lq = Lq;
  p.Lk = Lk;
  p.H = H;
  p.scale_log2 = scale * LOG2E_F;
  p.work = (int*)((uint8_t*)ws + wl.work);   // taken by the 8-wave path (more than 8 key tiles)
  return hip_status(launch_attn_fwd_tiled(p, (hipStream_t)stream));
}

WANATTN_API int wanattn_measure_mfma_peak(float* sink, int workgroups, int iters, void* stream) {
  if (sink == nullptr) return WANATTN_ERR_NULL;
  if (workgroups <= 0 || workgroups > (1 << 20) || iters <= 0) return WANATTN_ERR_SHAPE;
  if (!aligned(sink, 4)) return WANATTN_ERR_ALIGN;
  return hip_status(launch_mfma_peak(sink, workgroups, iters, (hipStream_t)stream));
}
