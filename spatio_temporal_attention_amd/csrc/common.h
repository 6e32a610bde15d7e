// Device-side building blocks shared by the wanattn kernels (gfx950 / CDNA4).
//
// * bf16 <-> fp32 helpers (fp32 -> bf16 is round-to-nearest-even via v_cvt_pk_bf16_f32)
// * the 3D RoPE rotation of one (even, odd) element pair
// * staging of 64-row x 128-column tiles into LDS in a row-major layout whose
//   16-byte chunks are XOR-swizzled per row, read back as 16-byte row
//   fragments (MFMA operands whose k index runs along the row), and of
//   transposed (T) tiles whose rows feed the products that contract over
//   tokens
// * MFMA 32x32x16 bf16 wrappers and their register layouts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wanattn {

constexpr int HD = 128;               // head dim (the only one supported)
constexpr int TILE_ROWS = 64;         // rows of one staged tile
constexpr int TILE_ELEMS = TILE_ROWS * HD;
// Backward row statistics of one query tile (1 KB): LSE_i * log2(e) and
// -Delta_i of its 64 rows in the accumulators' row order (512 bytes), then the
// tile's exponent e_q (int bits), then zeros.
constexpr int QSTAT_FLOATS = 4 * TILE_ROWS;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// bf16 helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair (a in the low half), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 p = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, p);
}

// Four fp32 -> packed OCP fp8 e4m3 (round to nearest even), byte 0 = a, saturated
// to +-448 so that out-of-range values never become NaN.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  constexpr float M = 448.f;
  a = fminf(fmaxf(a, -M), M);
  b = fminf(fmaxf(b, -M), M);
  c = fminf(fmaxf(c, -M), M);
  d = fminf(fmaxf(d, -M), M);
  const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)w, true);
}

// Two fp32 -> packed fp16 (round to nearest even).
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f32x2 v = {a, b};
  f16x2 h = __builtin_convertvector(v, f16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// The e for which x * 2^-e lies in [2^14, 2^15) (0 for x == 0): scaling a
// row or tile by 2^-e puts its largest magnitude at the top of the fp16
// range, below its maximum 65504, with full fp16 precision below it.
__device__ __forceinline__ int pow2_exponent_15(float x) {
  if (!(x > 0.f)) return 0;
  int ex;
  frexpf(x, &ex);   // x = f * 2^ex, f in [0.5, 1)
  return ex - 15;
}

// ---------------------------------------------------------------------------
// 3D RoPE.  The table holds (cos, sin) float pairs: time block [f][d_f/2],
// then height block [h][d_h/2], then width block [w][d_w/2].
// ---------------------------------------------------------------------------
struct RopeDev {
  const float2* table;  // nullptr: no rotation
  int gh, gw;           // grid rows and columns (token n -> f = n/(gh*gw), h = (n/gw)%gh, w = n%gw)
  int nf, nh, nw;       // pairs per segment: d_f/2, d_h/2, d_w/2
  int off_h, off_w;     // first table entry of the height and width blocks
};

struct TokenPos { int f, h, w; };

__device__ __forceinline__ TokenPos token_pos(const RopeDev& r, int n) {
  const int hw = r.gh * r.gw;
  TokenPos p;
  p.f = n / hw;
  const int rem = n - p.f * hw;
  p.h = rem / r.gw;
  p.w = rem - p.h * r.gw;
  return p;
}

// (cos, sin) of pair k (0 <= k < 64) of a token at position p.
__device__ __forceinline__ float2 rope_cs(const RopeDev& r, const TokenPos& p, int k) {
  int idx;
  if (k < r.nf) idx = p.f * r.nf + k;
  else if (k < r.nf + r.nh) idx = r.off_h + p.h * r.nh + (k - r.nf);
  else idx = r.off_w + p.w * r.nw + (k - r.nf - r.nh);
  return r.table[idx];
}

// Rotate (x0, x1) by the angle whose (cos, sin) is cs; inverse uses minus the angle.
// Written with explicit fmaf so every kernel rounds identically.
__device__ __forceinline__ void rope_rotate(float& x0, float& x1, float2 cs, bool inverse) {
  const float s = inverse ? -cs.y : cs.y;
  const float y0 = fmaf(x0, cs.x, -(x1 * s));
  const float y1 = fmaf(x0, s, x1 * cs.x);
  x0 = y0;
  x1 = y1;
}

// Rotate the 8 bf16 elements of a 16-byte chunk holding head-dim elements
// [8c, 8c+8) (pairs 4c .. 4c+3) of a token at position p; result rounded to bf16.
__device__ __forceinline__ u32x4 rope_chunk(const RopeDev& r, const TokenPos& p, int c, u32x4 x, bool inverse) {
  u32x4 y;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float x0 = bf16_lo(x[t]);
    float x1 = bf16_hi(x[t]);
    rope_rotate(x0, x1, rope_cs(r, p, 4 * c + t), inverse);
    y[t] = pack_bf16(x0, x1);
  }
  return y;
}


// ---------------------------------------------------------------------------
// LDS tiles: 64 rows x 128 bf16, row-major, 256 bytes per row, no padding.
// The 16 chunks (16 bytes each) of row r are stored at chunk c ^ swz(r).
// LDS has 64 banks of 4 bytes, so a row spans all banks once and a chunk's
// bank group is its physical index.  swz(r) = ((r&3) << 2) | ((r>>2)&3):
// 16 consecutive rows read at one logical chunk (16-byte row fragments, 16
// lanes per LDS cycle) land on 16 distinct chunks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz(int r) {
  return ((r & 3) << 2) | ((r >> 2) & 3);
}

// Offset (in bf16 elements) of element (row, col) inside a tile; col % 8 kept.
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * HD + ((((col >> 3) ^ swz(row)) << 3) | (col & 7));
}

// Read-only arrays (not written during the kernel) read through the
// constant address space: loads at uniform indices become scalar loads into
// SGPRs instead of vector loads into VGPRs.
using const_i32 = const __attribute__((address_space(4))) int;
__device__ __forceinline__ const_i32* const_ptr(const int* p) { return (const_i32*)p; }

// Wait for this wave's outstanding global (and LDS-DMA) loads.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0); }

// Workgroup barrier ordering LDS accesses only.  Unlike __syncthreads() it
// does not wait for the wave's outstanding global loads (and so not for LDS
// DMA in flight); callers wait for those explicitly with wait_vmem() before
// the barrier that publishes them.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup barrier for kernels whose LDS is written only by DMA copies: the
// wave's own LDS reads have returned (lgkmcnt 0), copies still in flight are
// not waited for (callers wait for those with wait_vmem() before the barrier
// that publishes them), and the compiler keeps memory accesses on their side
// of it.  (A release/acquire fence would add a wait for every copy in flight.)
__device__ __forceinline__ void dma_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0); vmcnt and expcnt not waited for
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Tiles of 128-byte rows: the fp8 key tile (64 keys x 128 d, 8 KB) and the
// V^T tile (128 d x 64 keys in bf16, 16 KB).  The 8 16-byte chunks of row r
// sit at chunk c ^ swz8(r), swz8(r) = (r >> 1) & 7: the 16 rows a 16-lane
// pass reads at one logical chunk (two rows per 256-byte bank cycle) land on
// 16 distinct bank groups.
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int tile8_off(int row, int chunk) { return row * 128 + ((chunk ^ swz8(row)) << 4); }

// Staging from contiguous 16 KB tiles (all rows present) by NW waves: each
// wave issues 16/NW copies of 1 KB; copy i of wave w fills LDS bytes
// [(16384/NW)*w + 1024*i, +1024), lane l the 16 bytes at 16*l of that block.
// The lane byte offsets into the tile do not depend on the tile, so they
// are computed once.
//   row tile (64 rows x 256 B): rows (64/NW)*w + 4i + l/16, logical chunk
//     (l%16) ^ swz(row) (the layout of tile_off);
//   T tile (128 rows x 128 B): rows (128/NW)*w + 8i + l/8, logical chunk
//     (l%8) ^ swz8(row).
template <int NW>
__device__ __forceinline__ uint32_t rowtile_lane_off(int wave, int i, int lane) {
  const int r = (64 / NW) * wave + 4 * i + (lane >> 4);
  return (uint32_t)(r * 256 + (((lane & 15) ^ swz(r)) << 4));
}
template <int NW>
__device__ __forceinline__ uint32_t ttile_lane_off(int wave, int i, int lane) {
  const int r = (128 / NW) * wave + 8 * i + (lane >> 3);
  return (uint32_t)(r * 128 + (((lane & 7) ^ swz8(r)) << 4));
}
template <int NW>
__device__ __forceinline__ uint8_t* tile_lds_block(void* lds_tile, int wave, int i) {
  return reinterpret_cast<uint8_t*>(lds_tile) + (16384 / NW) * wave + 1024 * i;
}
// Raw buffer resource over `bytes` bytes at `base` (stride 0; dword 3 as for
// gfx9 raw buffers).  Copies through it keep the per-tile step in the scalar
// soffset and the lane offset in a 32-bit voffset (buffer_load ... lds).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// An empty asm statement that reads and rewrites x in place: x is computed
// before this point and nothing that produces it moves below it.
__device__ __forceinline__ void pin_vgprs(bf16x8& x) {
  u32x4 w = __builtin_bit_cast(u32x4, x);
  asm volatile("" : "+v"(w));
  x = __builtin_bit_cast(bf16x8, w);
}

// One 1 KB copy: 64 lanes x 16 bytes from base + soff + voff into lds_block.
__device__ __forceinline__ void buf_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds_block) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_block, 16, voff, soff, 0,
                                           0);
}

// A-side fragment of O^T += V^T P^T from a V^T tile: lane l gets d-row `row`,
// key positions [16*kg + 8*(l/32), +8).  Within each 16-key group the tile
// stores key k at position k with bits 2 and 3 swapped, so these 8 positions
// hold keys {16kg + 4*(l/32) + e, 16kg + 8 + 4*(l/32) + e : e = 0..3}: the k
// order of a 32x32 accumulator block's registers (see mfma32 below).
__device__ __forceinline__ bf16x8 lds_vt_frag(const uint16_t* lds, int row, int kg, int half) {
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint8_t*>(lds) + tile8_off(row, 2 * kg + half));
}


// 16-byte row fragment: elements [8*chunk, 8*chunk+8) of `row`.
__device__ __forceinline__ bf16x8 lds_row_frag(const uint16_t* lds, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(lds + tile_off(row, chunk * 8));
}

// ---------------------------------------------------------------------------
// MFMA 32x32x16 bf16 (fp32 accumulate).  Register layout (lane l, wave64):
//   A[32 x 16]: lane holds A[l%32][8*(l/32) + t], t = 0..7
//   B[16 x 32]: lane holds B[8*(l/32) + t][l%32]
//   C[32 x 32]: lane holds C[8*(j/4) + 4*(l/32) + j%4][l%32], j = 0..15
// A contraction over the 32 rows of an accumulator block can reuse that
// block's registers as the k-side operand of the next MFMA if the k index is
// permuted: accumulator entries j = 8g .. 8g+7 of lane l hold rows
// 16g + 8*(t/4) + 4*(l/32) + t%4 (t = j - 8g), which is k index 8*(l/32) + t
// of a 16-deep step when row and k index differ by swapping bits 2 and 3.
// The T tiles store their tokens in exactly that order (lds_vt_frag).
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// The same product with both operands holding fp16 bit patterns.
__device__ __forceinline__ f32x16 mfma32_f16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}

// Pack accumulator entries 8g .. 8g+7 (after an elementwise map already
// applied) into a bf16x8 k-side operand.
__device__ __forceinline__ bf16x8 pack_acc8(const float* v) {
  u32x4 w;
#pragma unroll
  for (int t = 0; t < 4; ++t) w[t] = pack_bf16(v[2 * t], v[2 * t + 1]);
  return __builtin_bit_cast(bf16x8, w);
}

// Butterfly across the two 32-lane halves of the wave (v_permlane32_swap:
// after swapping a register with itself, the two results hold the lower and
// the upper half's value in every lane).
__device__ __forceinline__ float xor32_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// XCD-aware workgroup order: the hardware deals workgroups round-robin over
// the 8 XCDs (each with its own L2).  Return a logical index such that every
// XCD receives a contiguous range of logical indices, so workgroups that share
// K/V (same batch and head) run on the same XCD.  Kernels order the logical
// index as ((head, batch), tile) with the batch item innermost, so that items
// of unequal work (variable lengths) spread evenly over the XCDs.
__device__ __forceinline__ int xcd_remap(int wg, int total) {
  constexpr int NXCD = 8;
  const int q = total / NXCD;
  const int r = total % NXCD;
  const int xcd = wg % NXCD;
  const int slot = wg / NXCD;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// Work counter.  The XCDs of a chip run at unequal speeds (a few percent
// apart), yet each receives a fixed eighth of a launch's workgroups (workgroup
// x on XCD x % 8), so with one fixed item per workgroup the slowest XCD ends
// the launch.  Instead the workgroups take their items from a counter, in the
// order of the items' index, and the launch holds work_grid(n) workgroups for
// n items: the faster XCDs go on to their spare workgroups and take more
// items, and workgroups that draw a value past the last item leave at once.
// The counter is an int and reaches work_grid(n) - 1: launchers refuse a
// launch whose work_grid exceeds INT_MAX (work_fits).
__host__ __device__ constexpr int64_t work_grid(int64_t n_items) { return n_items + (n_items + 7) / 8; }
__host__ __device__ constexpr bool work_fits(int64_t n_items) { return work_grid(n_items) <= 0x7fffffff; }

// The workgroup's item (the counter's next value): its first thread draws it
// and shares it through LDS.  Every thread of the workgroup calls it, before
// any other barrier.
__device__ __forceinline__ int take_work_item(int* work) {
  __shared__ int drawn;
  if (threadIdx.x == 0) drawn = __hip_atomic_fetch_add(work, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(drawn);
}

// The counter starts at zero: a kernel rather than a memset, so that callers
// may capture the launches in a graph.
namespace {   // one copy per translation unit
__global__ void work_reset_kernel(int* work) { *work = 0; }
}  // namespace

}  // namespace wanattn
