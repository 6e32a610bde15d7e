/*
 * wanattn -- spatio-temporal attention with 3D RoPE for Wan-style video DiTs,
 * on AMD Instinct MI355X (gfx950).  Plain C interface.
 *
 * Sources (page title, section):
 *   [notes]  "Wan -- Open and Advanced Large-Scale Video Generative Models (Wan2.1)"
 *            reading notes (gojay.top): "2. Model Design" (Wan-VAE paragraph:
 *            latent grid [1+T/4, H/8, W/8]; DiT backbone paragraph: (1,2,2)
 *            patch, L = (1+T/4)*H/16*W/16; DiT block paragraph: 3D RoPE on the
 *            code side), the code-notes config table ("1.3B vs 14B": dim
 *            1536/5120, 12/40 heads, so head dim 128; umT5 with 512 tokens),
 *            "3. Training" (bf16).
 *   [lit619] "Wan Team, Alibaba (2025) -- ARXIV-2503.20314", "Key takeaways":
 *            full spatio-temporal self-attention over latent patches plus
 *            cross-attention to umT5 text embeddings (Backbone); attention
 *            dominates at long sequence lengths and is split across GPUs by
 *            Ring (outside) x Ulysses (inside) context parallelism.
 *
 * Conventions shared by every call
 * --------------------------------
 *  Tensors.  q, k, v, o, dout, dq, dk, dv are contiguous [B, L, H, D] bf16
 *    (D innermost; passed as void*).  lse is contiguous [B, H, L] fp32, the
 *    natural-log log-sum-exp of each query row's scaled scores.  Cross-attention
 *    uses [B, Lq, H, D] for q/o and [B, Lk, H, D] for k/v.  D must be 128.
 *  Tokens and positions.  Token n of a self-attention sequence sits at grid
 *    position (f, h, w) = (n / (gh*gw), (n / gw) % gh, n % gw): row-major over
 *    the post-patchify grid wanattn_grid {f, h, w}, so f*h*w == L.
 *  3D RoPE.  The head dim splits into a time segment [0, d_f), a height
 *    segment [d_f, d_f+d_h) and a width segment [d_f+d_h, D).  Pair j of a
 *    segment of width d_a (elements o_a+2j, o_a+2j+1) turns by the angle
 *    p_a * theta^(-2j/d_a), p_a being the token's position on that axis:
 *      y[2j]   = x[2j] cos - x[2j+1] sin,   y[2j+1] = x[2j] sin + x[2j+1] cos.
 *    Each width must be even and >= 0, d_f + d_h + d_w == D, theta > 0.
 *  Rounding.  All arithmetic is fp32 (MFMA accumulates in fp32); every
 *    fp32 -> bf16 or fp16 rounding is round-to-nearest-even.  With RoPE the
 *    score product runs in fp16: each 64-token tile of rotated queries and
 *    each 64-token tile of rotated keys (of one batch item and head) is
 *    scaled by a power of two that puts its largest |element| in
 *    [2^14, 2^15) and rounded to fp16 (exact rescaling, any
 *    finite input); the forward undoes the powers of two in fp32.  Without
 *    RoPE the bf16 inputs enter the products unrounded.  P is rounded to bf16
 *    for the PV product; the softmax sums use the unrounded fp32 values.
 *  Memory.  Every pointer is device memory owned by the caller, which keeps it
 *    alive until the stream's work has finished.  bf16 buffers, the rope table
 *    and workspaces must be 16-byte aligned; fp32 and int32 buffers 4-byte
 *    aligned.  Outputs must not alias inputs (except x == y in wanattn_rope3d).
 *    The library allocates no device memory, keeps no global state, never
 *    synchronizes and never prints.
 *  Streams.  `stream` is a hipStream_t (NULL: the default stream).  All work
 *    is enqueued asynchronously on it; calls from several host threads on
 *    different streams are safe.
 *  Errors.  Arguments are validated on the host before anything is enqueued;
 *    on failure the call returns a nonzero WANATTN_ERR_* code and touches no
 *    memory.  WANATTN_ERR_HIP reports a launch failure (hipGetLastError).
 *    Faults inside kernels surface at the caller's next stream synchronization.
 */
#ifndef WANATTN_H
#define WANATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WANATTN_HEAD_DIM 128

enum wanattn_status {
  WANATTN_OK = 0,
  WANATTN_ERR_NULL = 1,         /* a required pointer is NULL */
  WANATTN_ERR_SHAPE = 2,        /* a size is <= 0 or too large, or f*h*w != L */
  WANATTN_ERR_UNSUPPORTED = 3,  /* D != 128, bad rotary split or theta, non-finite scale */
  WANATTN_ERR_ALIGN = 4,        /* a buffer is not aligned as documented above */
  WANATTN_ERR_WORKSPACE = 5,    /* workspace missing or smaller than the *_workspace_bytes value */
  WANATTN_ERR_HIP = 6           /* the HIP runtime rejected a launch */
};

/* Post-patchify token grid (frames, rows, columns): [1+T/4, H/16, W/16] for a
 * 1+T frame H x W clip ([notes] 2. Model Design). */
typedef struct wanattn_grid {
  int32_t f, h, w;
} wanattn_grid;

/* Head-dim split between the time/height/width axes and the rotary base
 * (the pages name 3D RoPE without its constants; the workloads use 48/40/40
 * and theta = 10000). */
typedef struct wanattn_rope {
  int32_t d_f, d_h, d_w;
  float theta;
} wanattn_rope;

/* Human-readable text of a status code (static storage; never NULL). */
const char* wanattn_strerror(int status);

/* ---------------------------------------------------------------------------
 * 3D RoPE table ([notes] 2. Model Design, DiT block paragraph: 3D RoPE over
 * time, height, width).
 *
 * Layout: three consecutive blocks, time then height then width.  Block a
 * holds size_a * (d_a/2) entries; entry (p, j) of block a is the float pair
 * (cos, sin) of p * theta^(-2j/d_a), computed in fp64 and rounded to fp32.
 * wanattn_rope_table_bytes returns 8 * (f*d_f/2 + h*d_h/2 + w*d_w/2), or 0 if
 * the grid or split is invalid.
 * ------------------------------------------------------------------------- */
size_t wanattn_rope_table_bytes(wanattn_grid g, wanattn_rope r);

/* Fill `table` (device, wanattn_rope_table_bytes(g, r) bytes) on `stream`. */
int wanattn_rope_table_init(float* table, wanattn_grid g, wanattn_rope r, void* stream);

/* y = R(p) x for every token (inverse != 0: y = R(p)^T x, the rotation by
 * minus the angle).  x, y: [B, L, H, D] bf16; x == y is allowed (in place).
 * Requires g.f*g.h*g.w == L and a table built for (g, r). */
int wanattn_rope3d(const void* x, void* y, int B, int L, int H, int D,
                   wanattn_grid g, wanattn_rope r, const float* table,
                   int inverse, void* stream);

/* ---------------------------------------------------------------------------
 * Self-attention forward: full (non-causal) softmax attention of every token
 * over every token of the same sequence and head ([lit619] Key takeaways,
 * Backbone; [notes] 1. Introduction), with 3D RoPE on q and k:
 *   s_ij = scale * <R(p_i) q_i, R(p_j) k_j>,  LSE_i = ln sum_j exp(s_ij),
 *   O_i  = sum_j exp(s_ij - LSE_i) v_j.
 * table == NULL: no rotation (g and r are then ignored).
 * lse may be NULL (not written).  scale: any finite value (1/sqrt(D) usual).
 * Workspace (required, 16-byte aligned): wanattn_self_fwd_workspace_bytes(B, L,
 * H, D, table != NULL) bytes.  It receives K and V rewritten in 64-key tiles
 * of every (b, h), zero-padded: K as [B, H, ceil(L/64), 64, D] (bf16, or with
 * a table the rotated keys in fp16 with one power-of-two exponent per tile,
 * the exponents following as int32 [B, H, ceil(L/64)]) and V transposed as
 * [B, H, ceil(L/64), D, 64] bf16 (the PV product's operand layout); each
 * part starts on a 256-byte boundary.  Then 256 bytes hold a counter from
 * which the workgroups take their query tiles.  Large problems add one more
 * part: the kernel runs 256-row query tiles, 256 at a time (one per compute
 * unit), and the last ones of n = B*H*ceil(L/256) run as S key ranges each,
 * whose fp32 partials ([tiles*S][256 rows][132 floats]) a merge pass combines
 * exactly: for n >= 2048 the last n % 256 + 256 tiles with S = 4; for
 * 1024 <= n < 2048 the last t = n % 256 with S = min(8, 256/t) (none if t = 0
 * or S < 2).  The size function accounts for all of it.  Its contents on
 * return are unspecified.
 * ------------------------------------------------------------------------- */
size_t wanattn_self_fwd_workspace_bytes(int B, int L, int H, int D, int with_rope);

int wanattn_self_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int L, int H, int D,
                     wanattn_grid g, wanattn_rope r, const float* table, float scale,
                     void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * FP8 self-attention forward: the operation of wanattn_self_fwd (same
 * arguments) computed with OCP fp8 e4m3 products at twice the bf16 MFMA rate
 * (FP8 attention is named without a recipe in [lit619] Tags; the recipe is
 * this library's).  The rotated queries, rotated keys and values are scaled
 * per 64-token tile of each (b, h) by the power of two that puts the tile's
 * largest |element| in [128, 256) and rounded to e4m3 (RNE, saturating at
 * +-448); both products run on fp8 MFMAs whose scale operands undo the powers
 * of two exactly; P is rounded to e4m3 for P.V, while the softmax statistics
 * and LSE use fp32 P.  Accuracy: O is the attention of the dequantized inputs
 * up to P's e4m3 rounding (relative L2 of a few 1e-2 on flat rows); LSE to
 * ~1e-4.  Workspace (required, 16-byte aligned):
 * wanattn_self_fwd_fp8_workspace_bytes(B, L, H, D): e4m3 K and V^T tiles
 * ([B, H, ceil(L/64)] x 8 KB each), their int32 exponents and a 256-byte
 * counter from which the workgroups take their query tiles.
 * ------------------------------------------------------------------------- */
size_t wanattn_self_fwd_fp8_workspace_bytes(int B, int L, int H, int D);

int wanattn_self_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int L, int H, int D,
                         wanattn_grid g, wanattn_rope r, const float* table, float scale,
                         void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Self-attention backward (training, [notes] 3. Training: bf16; the formulas
 * are the calculus of the forward above).  Given o and lse from
 * wanattn_self_fwd and the output gradient dout:
 *   Delta_i = <dout_i, o_i>;  P_ij = exp(s_ij - LSE_i);  dV_j = sum_i P_ij dout_i;
 *   dS_ij = P_ij (<dout_i, v_j> - Delta_i);
 *   dq_i = R(p_i)^T scale sum_j dS_ij R(p_j) k_j;  dk_j = R(p_j)^T scale sum_i dS_ij R(p_i) q_i.
 * Gradients are with respect to the unrotated q and k.  table == NULL: no RoPE.
 * Workspace (required, 16-byte aligned): wanattn_self_bwd_workspace_bytes bytes
 * (the same with or without a table).  It receives, per 64-token query tile
 * of every (b, h), the row statistics LSE_i * log2(e) and -Delta_i (fp32,
 * 1 KB a tile) and 64-token tiles of every (b, h): q and k (rotated with a table) in fp16 with
 * the forward's per-tile powers of two, their bf16 transposes, dout (rows and
 * transposed) and v, so that P is recomputed from exactly the operands the
 * forward multiplied; when few key blocks would leave the GPU idle (a short
 * key side: fewer than 256 blocks of 256 keys over B and H), the dK/dV passes
 * split the query range and the workspace also holds their fp32 partial sums
 * (reduced in a fixed order: results stay deterministic).  Each pass runs
 * blocks of 256 keys (dK, dV) or 256 queries (dQ), 256 at a time; for a block
 * count n that the forward's rule above would split (n >= 1024, t = n % 256,
 * S = min(8, 256/t) >= 2), the last t blocks run as S ranges of the other
 * side, and the workspace holds their fp32 partials too ([t*S][256][D] for
 * dK and for dV when the dK/dV passes have no query split of their own, then
 * [t*S][256][D] for dQ), also summed in a fixed order.  Its contents on
 * return are unspecified.
 * ------------------------------------------------------------------------- */
size_t wanattn_self_bwd_workspace_bytes(int B, int L, int H, int D, int with_rope);

int wanattn_self_bwd(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout,
                     void* dq, void* dk, void* dv,
                     int B, int L, int H, int D,
                     wanattn_grid g, wanattn_rope r, const float* table, float scale,
                     void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Variable-length self-attention forward: batch item b holds seq_lens[b]
 * valid tokens, the first ones of the [B, L, H, D] rows, and attends only
 * among them ([notes] code notes, WanModel forward and the sampler both take
 * a seq_len; [notes] 3. Training: joint image + video batches mix 1-frame and
 * many-frame latents).  seq_lens: device int32 [B], each clamped to [0, L].
 * Query rows i >= seq_lens[b] of o and lse are not written; keys
 * j >= seq_lens[b] are never used (their contents may be anything).  RoPE
 * positions follow the grid g of the padded length L (f*h*w == L), so a
 * prefix of whole frames has the positions it would have in a sequence of
 * its own.  Equal, item by item, to wanattn_self_fwd on the valid prefix.
 * Workspace: wanattn_self_fwd_workspace_bytes(B, L, H, D, table != NULL).
 * ------------------------------------------------------------------------- */
int wanattn_self_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* seq_lens, int B, int L, int H, int D,
                            wanattn_grid g, wanattn_rope r, const float* table, float scale,
                            void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Partial self-attention of one query shard over one key/value shard: the
 * per-hop step of Ring attention, the key-sharded ("outside") half of the 2D
 * context parallelism ([lit619] Key takeaways, attention dominates).  q holds
 * tokens [q_offset, q_offset + Lq) and k, v tokens [k_offset, k_offset + Lk)
 * of one sequence whose token grid is g (f*h*w >= both ends; RoPE positions
 * are those of the global token indices).  o ([B, Lq, H, D]) and lse
 * ([B, H, Lq], may be NULL) are the attention of the shard's queries over the
 * shard's keys only; wanattn_lse_merge combines the shards exactly.  table ==
 * NULL: no rotation (g and the offsets only need to be >= 0).
 * Workspace: wanattn_partial_fwd_workspace_bytes(B, Lk, H, D, table != NULL):
 * the key/value tiles and the 256-byte work counter (no tail split).
 * ------------------------------------------------------------------------- */
size_t wanattn_partial_fwd_workspace_bytes(int B, int Lk, int H, int D, int with_rope);

int wanattn_partial_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int Lq, int Lk, int H, int D,
                        wanattn_grid g, wanattn_rope r, const float* table,
                        int q_offset, int k_offset, float scale,
                        void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Exact merge of R partial results over disjoint key sets (same source):
 *   LSE = ln sum_r exp(LSE_r),  O = sum_r exp(LSE_r - LSE) O_r.
 * o_parts, lse_parts: host arrays of R (1..16) device pointers to [B, L, H, D]
 * bf16 and [B, H, L] fp32 partials; o: [B, L, H, D] bf16 out; lse: [B, H, L]
 * fp32 out or NULL.  Parts with LSE_r = -inf (no keys) get weight 0; if all
 * are -inf, O = 0 and LSE = -inf.  o may alias o_parts[0] (each element is
 * read before it is written, by the same thread).
 * ------------------------------------------------------------------------- */
int wanattn_lse_merge(const void* const* o_parts, const float* const* lse_parts, int R,
                      void* o, float* lse, int B, int L, int H, int D, void* stream);

/* ---------------------------------------------------------------------------
 * Cross-attention forward: video-token queries over text-token keys and values
 * ([lit619] Key takeaways, Backbone: cross-attention to umT5 embeddings;
 * [notes] config table: 512 text tokens).  No RoPE.  Keys j >= k_lens[b] are
 * padding: they are excluded and never read (their contents may be anything,
 * NaN included).  k_lens: device int32 [B], each clamped to [0, Lk]; NULL
 * means every key is valid.  A row with no valid key gets O = 0 and
 * LSE = -inf.  lse may be NULL.
 * Workspace (required, 16-byte aligned): wanattn_cross_fwd_workspace_bytes(B,
 * Lk, H, D) bytes.  It receives the text keys and values rewritten in 64-key
 * tiles of every (b, h): K as [B, H, ceil(Lk/64), 64, D] bf16 and V
 * transposed as [B, H, ceil(Lk/64), D, 64] bf16, keys past k_lens[b] zero,
 * then a 256-byte work counter (taken from by the workgroups when Lk > 512,
 * where 8-wave workgroups run); each part starts on a 256-byte boundary
 * (10.5 MB at Lk = 512, H = 40).  Its contents on return are unspecified.
 * ------------------------------------------------------------------------- */
size_t wanattn_cross_fwd_workspace_bytes(int B, int Lk, int H, int D);

int wanattn_cross_fwd(const void* q, const void* k, const void* v, const int32_t* k_lens,
                      void* o, float* lse, int B, int Lq, int Lk, int H, int D, float scale,
                      void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Cross-attention backward (training back-propagates through the text
 * cross-attention of every block: [lit619] Key takeaways, Backbone; [notes]
 * 3. Training).  The calculus of wanattn_cross_fwd, given its o and lse
 * (lse required) and the output gradient dout:
 *   P_ij = exp(scale <q_i, k_j> - LSE_i) for valid keys j < k_lens[b], else 0;
 *   Delta_i = <dout_i, o_i>;  dV_j = sum_i P_ij dout_i;
 *   dS_ij = P_ij (<dout_i, v_j> - Delta_i);
 *   dq_i = scale sum_j dS_ij k_j;  dk_j = scale sum_i dS_ij q_i.
 * Padded keys (j >= k_lens[b]) get dk = dv = 0 and are never read; rows with
 * no valid key (LSE = -inf) get dq = 0.  dq: [B, Lq, H, D]; dk, dv: [B, Lk,
 * H, D] bf16.  k_lens: device int32 [B] (clamped to [0, Lk]) or NULL (all
 * valid).  The score product runs in fp16 on power-of-two-scaled 64-token
 * tiles, as in the self-attention backward.
 * Workspace (required, 16-byte aligned): wanattn_cross_bwd_workspace_bytes
 * (the self-attention backward's layout over Lq query and Lk key tokens,
 * including the partial sums of a split query range: at the 720p text shape,
 * B = 1, Lq = 75,600, Lk = 512, H = 40, the query range is split 7 ways, and
 * the tail split's partials of the dQ pass).
 * ------------------------------------------------------------------------- */
size_t wanattn_cross_bwd_workspace_bytes(int B, int Lq, int Lk, int H, int D);

int wanattn_cross_bwd(const void* q, const void* k, const void* v, const int32_t* k_lens,
                      const void* o, const float* lse, const void* dout,
                      void* dq, void* dk, void* dv,
                      int B, int Lq, int Lk, int H, int D, float scale,
                      void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Allocation-free variant of wanattn_self_fwd, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, semantics and results as
 * wanattn_self_fwd (the same kernels run), minus the workspace: the K/V tiles
 * and the tail split's partials go to a static device array of the library,
 * 256 MiB per GPU, held from the library's load until the process ends.  The
 * call allocates and frees nothing.  Its first call on a device looks up that
 * device's copy of the array (hipGetSymbolAddress) with the device current.
 * Limit: wanattn_self_fwd_workspace_bytes(B, L, H, D, table != NULL) must not
 * exceed 268435456 (for example B*H*L up to about 500,000 token-heads with
 * RoPE: L = 32,760 with 12 heads, or 75,600 with 5); larger problems return
 * WANATTN_ERR_WORKSPACE before anything is enqueued.  All calls on one GPU
 * share its array: calls that overlap on that GPU (different streams or host
 * threads without ordering between them) race and give undefined results;
 * calls ordered on one stream are safe.  Nothing in the array needs to start
 * at zero (every byte read is written earlier in the same call).
 * ------------------------------------------------------------------------- */
int wanattn_self_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int L, int H, int D, wanattn_grid g, wanattn_rope r,
                             const float* table, float scale, void* stream);

/* ---------------------------------------------------------------------------
 * Measurement aid (not part of the attention method): a loop of back-to-back
 * bf16 MFMAs (v_mfma_f32_32x32x16_bf16, fp32 accumulation) on every SIMD, the
 * rate against which the attention calls' throughput can be stated next to
 * the published dense peak.  Launches `workgroups` workgroups of 4 waves;
 * each wave issues 4 * iters MFMAs of 32*32*16*2 flop on register operands
 * holding varied values, then writes one float per thread to `sink` (device,
 * workgroups * 256 floats, contents meaningless).  Algorithmic work per call:
 * workgroups * 4 * iters * 131072 flop.  Errors: WANATTN_ERR_NULL (sink),
 * _SHAPE (workgroups outside [1, 2^20] or iters < 1), _ALIGN, _HIP.
 * ------------------------------------------------------------------------- */
int wanattn_measure_mfma_peak(float* sink, int workgroups, int iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WANATTN_H */
