// Shared device helpers for the gfx950 kernels: element types, MFMA
// fragments, layout maps and small wave-level primitives.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vs_attn.h"

namespace vs {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

constexpr int BLK = 64;  // tile edge: 64 query rows x 64 keys
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(_Float16 x) { return (float)x; }

// --- MFMA wrappers (lane layouts verified on gfx950) ------------------------
// 16x16x32 bf16: lane l supplies A[l%16][8*(l/16)+j], B[8*(l/16)+j][l%16]
// (j=0..7) and receives C[4*(l/16)+i][l%16] (i=0..3).
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// The same shape on fp16 operands (identical lane layout).
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
__device__ __forceinline__ f32x4 mfma_f16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                 0, 0);
}
// 16-bit MFMA operands travel in bf16x8 containers; F16 says the bits are
// fp16 (tiles and fragments are only moved, never converted, on the way).
template <bool F16>
__device__ __forceinline__ f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
  if constexpr (F16) return mfma_f16(a, b, c);
  else return mfma_bf16(a, b, c);
}
// 16x16x4 f32: lane l supplies A[l%16][l/16], B[l/16][l%16]; C as above.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16). Within each 16-lane group,
// lane r' points at 4 consecutive b16 elements X[k0 + r'/4][n0 + 4*(r'%4) ..+3]
// of a row-major tile; lane r then receives X[k0 + i][n0 + r], i = 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4*)((__attribute__((address_space(3))) void*)(p)));
}
// Two transpose reads 4 rows apart, joined into one 8-slot MFMA operand
// (whole-vector shuffle: element-wise assembly from the 16-bit lanes was
// observed to be mis-compiled into a broadcast of element 0).
__device__ __forceinline__ bf16x8 lds_read_tr16_x2(const bf16* p, int row_pitch) {
  const bf16x4 lo = lds_read_tr16(p);
  const bf16x4 hi = lds_read_tr16(p + 4 * row_pitch);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ float wave_shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// --- work order across XCDs ---------------------------------------------------
// A work item is (block rank, head within its kv group, kv group); block rank
// 0 is the heaviest (causal work shrinks along the rank). Items are taken in
// clusters of `bpc` consecutive block ranks x the `hpg` heads of ONE kv group,
// and cluster c runs on XCD c % 8 (the dispatcher deals workgroups to the 8
// XCDs in turn). Round r = c / 8 gives all 8 XCDs the same kv group
// (r % G) and 8 neighbouring block groups, so the workgroups resident on an
// XCD at a time work on one kv head's K/V (or one group's Q/dO) and on
// neighbouring blocks whose tiles its L2 serves more than once, while over
// the rounds every XCD gets an even share of every group and of heavy and
// light blocks. The grid is rounded up to whole rounds; workgroups past the
// last block return false and exit at once.
__device__ __forceinline__ bool xcd_group_item(int b, int G, int nblk, int bpc, int hpg, int* blk, int* hh,
                                               int* g) {
  const int csize = bpc * hpg;
  const int x = b & 7, r = (b >> 3) / csize, k = (b >> 3) % csize;
  *g = r % G;
  *blk = ((r / G) * 8 + x) * bpc + k / hpg;
  *hh = k % hpg;
  return *blk < nblk;
}
__host__ inline unsigned xcd_group_grid(int G, int nblk, int bpc, int hpg) {
  const int nbg = (nblk + bpc - 1) / bpc;
  return (unsigned)(G * ((nbg + 7) / 8) * 8 * bpc * hpg);
}
// Query-major kernels (two workgroups per CU, 64 per XCD): clusters of 8
// query blocks x the group's q heads. Key-major kernels (one workgroup per CU,
// 32 per XCD): clusters of 8 key blocks of one kv head (measured against 12,
// 16, 32 and 64: neighbouring key blocks share most of their query tiles, and
// shorter clusters keep more of an XCD's concurrent blocks adjacent).
constexpr int QMAJOR_BPC = 8;
constexpr int KMAJOR_BPC = 8;

// --- layout maps -------------------------------------------------------------
// Global 64-block of local block J of rank `rank` (NB = local blocks per shard).
__device__ __host__ __forceinline__ int64_t global_block(int kind, int P, int NB, int rank, int J) {
  if (kind == VS_CONTIG) return (int64_t)rank * NB + J;
  if (kind == VS_STRIPED) return (int64_t)J * P + rank;
  const int CB = NB >> 1;  // zigzag: two chunks of CB blocks
  return J < CB ? (int64_t)rank * CB + J : (int64_t)(2 * P - 1 - rank) * CB + (J - CB);
}

// Owner rank and local block of global block G; returns the owner.
__device__ __host__ __forceinline__ int owner_of_block(int kind, int P, int NB, int64_t G, int* J) {
  if (kind == VS_CONTIG) { *J = (int)(G % NB); return (int)(G / NB); }
  if (kind == VS_STRIPED) { *J = (int)(G / P); return (int)(G % P); }
  const int CB = NB >> 1;
  const int chunk = (int)(G / CB);
  const int off = (int)(G % CB);
  if (chunk < P) { *J = off; return chunk; }
  *J = CB + off;
  return 2 * P - 1 - chunk;
}

// Number of local blocks J of shard `rank` whose global block is <= G
// (global blocks are increasing in J for every layout).
__device__ __forceinline__ int blocks_upto(int kind, int P, int NB, int rank, int64_t G) {
  int lo = 0, hi = NB;  // first J with global_block > G
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (global_block(kind, P, NB, rank, mid) <= G) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Debug builds (VS_DEBUG_BOUNDS): a value read from a mask that becomes part
// of an address must lie in [lo, hi); one that does not is counted in *dbg
// and replaced by lo, so the kernel still touches only valid memory and
// finishes. Release builds return v unchecked.
__device__ __forceinline__ int dbg_clamp(int v, int lo, int hi, int32_t* dbg) {
#ifdef VS_DEBUG_BOUNDS
  if (v < lo || v >= hi) {
    if (dbg) atomicAdd(dbg, 1);
    return lo;
  }
#endif
  return v;
}

__device__ __forceinline__ int lower_bound_i32(const int32_t* a, int n, int64_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// ---- one-position stripes (VS_STRIPED1) ---------------------------------------
// Local position l of rank r is global position l P + r (P <= 32), so local
// query block I spans global blocks I P .. I P + P - 1: row a of it lies in
// global block I P + qa(a), qa(a) = (a P + r) >> 6, and key b of local block
// J of shard s in J P + kb(b), kb(b) = (b P + s) >> 6. An entry of tile
// (I, J) lies on global block-diagonal o P + qa - kb, o = I - J.

// Bits lo .. lo + len - 1 (len <= 64) of a slash bitmap of W words; bits
// outside the bitmap read as 0.
__device__ __forceinline__ uint64_t sbit_window(const uint32_t* sb, int W, int64_t lo, int len) {
  const int64_t w0 = lo >> 5;                 // floor(lo / 32), also for lo < 0
  const int sh = (int)(lo - w0 * 32);
  auto word = [&](int64_t i) -> uint64_t { return (i >= 0 && i < W) ? (uint64_t)sb[i] : 0ull; };
  const uint64_t lo64 = word(w0) | (word(w0 + 1) << 32);
  uint64_t x = lo64 >> sh;
  if (sh) x |= word(w0 + 2) << (64 - sh);
  return len >= 64 ? x : (x & ((1ull << len) - 1ull));
}
// The selected diagonals a tile at block offset o meets: bit i is diagonal
// o P - P + 1 + i (i < 2P - 1; negative diagonals read 0).
__device__ __forceinline__ uint64_t s1_tile_window(const uint32_t* sb, int W, int P, int o) {
  return sbit_window(sb, W, (int64_t)o * P - P + 1, 2 * P - 1);
}
// Key b of such a tile: bit x of the result says whether rows with qa = x
// lie on a selected diagonal (o P + x - kb(b) = o P - P + 1 + (x + P - 1 - kb)),
// and rows below the returned threshold are above the causal edge (o = 0:
// b P + s <= a P + r).
__device__ __forceinline__ uint32_t s1_key_window(uint64_t tile_win, int P, int s, int b) {
  const int kb = (b * P + s) >> 6;
  return (uint32_t)(tile_win >> (P - 1 - kb));
}
__device__ __forceinline__ int s1_key_threshold(int o, int r, int s, int b) {
  return o == 0 ? b + (s > r ? 1 : 0) : 0;
}
// First row of local query block I (rank r) at or below global column mg:
// rows a >= the result have (64 I + a) P + r >= mg (BLK: none).
__device__ __forceinline__ int s1_causal_row(int64_t mg, int r, int P, int I) {
  const int64_t num = mg - r - (int64_t)BLK * I * P;
  return num <= 0 ? 0 : (int)(num >= (int64_t)BLK * P ? BLK : (num + P - 1) / P);
}
// First local query block of rank r with a row at or below global column mg.
__device__ __forceinline__ int s1_first_qblock(int64_t mg, int r, int P) {
  const int64_t num = mg - r - (int64_t)(BLK - 1) * P;
  return num <= 0 ? 0 : (int)((num + (int64_t)BLK * P - 1) / ((int64_t)BLK * P));
}
// A vertical column (global mg) in query block I: the rows it is active for
// outside the listed tiles are its causal rows (threshold) whose diagonal
// I P + qa - floor(mg / 64) is not selected (bit qa of the window).
__device__ __forceinline__ uint32_t s1_vert_window(const uint32_t* sb, int W, int P, int I, int64_t mg) {
  return ~(uint32_t)sbit_window(sb, W, (int64_t)I * P - (mg >> 6), P);
}

}  // namespace vs

namespace vs {

// --- staged 64 x 128 bf16 tiles -----------------------------------------------
// A tile holds 64 rows of 128 bf16 (256 B = 16 chunks of 16 B), unpadded, with
// the 16-byte chunks of row r permuted by an XOR swizzle of row bits 0, 1 and
// 3. LDS on gfx950 serves a 128-bit read to 16 lanes per cycle (same
// half-wave, same parity of lane bits 2..4) and a 64-bit read to a half-wave,
// over 64 banks of 4 bytes (measured with per-pattern probes under the
// SQ_LDS_BANK_CONFLICT counter). The swizzle keeps both access patterns of
// the attention kernels free of bank conflicts under that service order:
// (a) MFMA-operand reads, 16 lanes reading one chunk from the 16 rows
// {8q + 4t + i} (an earlier swizzle that also used row bit 4 cost every
// such read a second cycle), and (b) the transpose reads, where 16 lanes read
// two chunks from 4 consecutive rows and lane groups read rows 8 apart.
constexpr int TD = 128;                 // head dim of the staged tiles
constexpr int TCH = TD / 8;             // chunks per row
constexpr int TILE_ELEMS = BLK * TD;    // 8192 bf16 = 16 KiB
__device__ __forceinline__ int tile_swz(int r) { return ((r & 3) << 1) | (((r >> 3) & 1) << 3); }
__device__ __forceinline__ int tile_off(int r, int lc) { return r * TD + ((lc ^ tile_swz(r)) << 3); }

// Asynchronous global -> LDS copy of one tile by a 256-thread workgroup
// (gfx950 global_load_lds_dwordx4: lane L of a wave writes 16 B at the
// wave-uniform LDS address + 16 L). Wave w copies the 1 KiB segments
// s = w + 4 c (rows 4 s .. 4 s + 3); lane L carries local row 4 s + L / 16,
// physical chunk L % 16. src_row[c] is the global row for that local row.
__device__ __forceinline__ int dma_local_row(int wave, int c, int lane) { return 4 * (wave + 4 * c) + (lane >> 4); }
__device__ __forceinline__ void dma_tile(bf16* lds_tile, const bf16* gbase, int64_t row_stride, const int* src_row,
                                         int wave, int lane) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int s = wave + 4 * c;
    const int r = 4 * s + (lane >> 4);
    const int lc = (lane & 15) ^ tile_swz(r);
    const bf16* g = gbase + (int64_t)src_row[c] * row_stride + lc * 8;
    __builtin_amdgcn_global_load_lds((const void*)g,
                                     (__attribute__((address_space(3))) void*)(
                                         (__attribute__((address_space(3))) bf16*)(lds_tile + s * 512)),
                                     16, 0, 0);
  }
}
// The same copy with the address split into a wave-uniform part (tile base,
// 64-bit, scalar registers) and a 32-bit per-lane part, so no per-piece
// 64-bit multiply is spent on it. Lane L of wave w carries local rows
// r_c = r0 + 16 c with r0 = 4 w + L / 16 < 16; the swizzle does not use row
// bits 4 and 5, so every piece of a lane has the same column offset.
// `wave` must be wave-uniform (readfirstlane) for the LDS side to stay scalar.
struct DmaLane {
  uint32_t r0;          // local row of the c = 0 piece
  uint32_t col;         // byte offset of the lane's swizzled 16-byte column
};
__device__ __forceinline__ DmaLane dma_lane(int wave, int lane) {
  DmaLane d;
  d.r0 = 4 * wave + (lane >> 4);
  d.col = (((lane & 15) ^ tile_swz((int)d.r0)) << 4);
  return d;
}
__device__ __forceinline__ void dma_copy16(const char* g, bf16* lds) {
  __builtin_amdgcn_global_load_lds((const void*)g,
                                   (__attribute__((address_space(3))) void*)(
                                       (__attribute__((address_space(3))) bf16*)(lds)),
                                   16, 0, 0);
}
// 64 consecutive rows starting at `tile` (wave-uniform), row pitch row_bytes.
__device__ __forceinline__ void dma_tile_rows(bf16* lds_tile, const char* tile, uint32_t row_bytes, const DmaLane& d,
                                              int wave) {
  const uint32_t lo = d.r0 * row_bytes;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    dma_copy16(tile + (size_t)(16 * c) * row_bytes + (lo + d.col), lds_tile + (wave + 4 * c) * 512);
}
// 64 gathered rows of `base` (wave-uniform): this lane's pieces come from rows
// src_row[c]. Offsets are 32-bit and the row product 24-bit: the caller keeps
// rows and row_bytes below 2^24 and rows * row_bytes below 2^32.
__device__ __forceinline__ void dma_tile_gather(bf16* lds_tile, const char* base, const int* src_row,
                                                uint32_t row_bytes, const DmaLane& d, int wave) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
    dma_copy16(base + (__umul24((uint32_t)src_row[c], row_bytes) + d.col), lds_tile + (wave + 4 * c) * 512);
}
// Host check for the 32-bit tile-copy offsets: a bf16 view of `rows` rows
// with row pitch `row_stride` elements keeps rows and the pitch in bytes
// below 2^24 and their product below 2^32.
__host__ inline bool dma_offsets_fit(int64_t rows, int64_t row_stride) {
  const int64_t rb = row_stride * 2;
  return rows < (1 << 24) && rb < (1 << 24) && rows * rb < (int64_t(1) << 32);
}
// Wait for this wave's outstanding memory operations (incl. LDS copies).
__device__ __forceinline__ void wait_all_mem() { __builtin_amdgcn_s_waitcnt(0); }

// Cross-lane exchange between the four 16-lane groups of a wave.
__device__ __forceinline__ float xor16(float v) { return __shfl_xor(v, 16, 64); }
__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, 64); }
// Max / sum over lanes n, n + 16, n + 32, n + 48 (result in all four), with
// the gfx950 row swaps: swapping 16-lane rows (then 32-lane halves) between
// two copies of a value leaves each lane holding its own value and its
// partner's, in one order or the other, so a symmetric op needs no select.
__device__ __forceinline__ float group4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Round 8 fp32 weights to a bf16 pair (hi = bf16(w), lo = bf16(w - hi)).
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
// hi = bf16(w) (round to nearest even), lo = bf16(w - hi), for two values at
// once: one packed convert per pair for each half, and the hi halves widened
// back to fp32 by a shift and a mask.
__device__ __forceinline__ void split_pair(float w0, float w1, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{w0, w1}, bf16x2));
  const float h0 = __builtin_bit_cast(float, hi << 16), h1 = __builtin_bit_cast(float, hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{w0 - h0, w1 - h1}, bf16x2));
}
// split_pair over eight values: element i of (hi, lo) is w0[i] for i < 4 and
// w1[i - 4] otherwise.
__device__ __forceinline__ void split8(const f32x4& w0, const f32x4& w1, bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
  split_pair(w0[0], w0[1], h[0], l[0]);
  split_pair(w0[2], w0[3], h[1], l[1]);
  split_pair(w1[0], w1[1], h[2], l[2]);
  split_pair(w1[2], w1[3], h[3], l[3]);
  hi = __builtin_bit_cast(bf16x8, i32x4{(int)h[0], (int)h[1], (int)h[2], (int)h[3]});
  lo = __builtin_bit_cast(bf16x8, i32x4{(int)l[0], (int)l[1], (int)l[2], (int)l[3]});
}
// Eight fp32 weights (P or dS) as MFMA operands. bf16: the hi + lo pair of
// split8 (two MFMAs per product). fp16: one operand rounded to nearest even
// (11 significant bits; lo is left untouched and not used), or with PAIR an
// fp16 hi + lo pair (hi = fp16(w), lo = fp16(w - hi): 22 significant bits
// down to fp16's 2^-24 spacing), for products that sum very many weights.
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
__device__ __forceinline__ uint32_t f16_pair_bits(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}
template <bool F16, bool PAIR = !F16>
__device__ __forceinline__ void weights8(const f32x4& w0, const f32x4& w1, bf16x8& hi, bf16x8& lo) {
  if constexpr (F16) {
    const uint32_t h0 = f16_pair_bits(w0[0], w0[1]);
    const uint32_t h1 = f16_pair_bits(w0[2], w0[3]);
    const uint32_t h2 = f16_pair_bits(w1[0], w1[1]);
    const uint32_t h3 = f16_pair_bits(w1[2], w1[3]);
    hi = __builtin_bit_cast(bf16x8, i32x4{(int)h0, (int)h1, (int)h2, (int)h3});
    if constexpr (PAIR) {
      const f16x8 hv = __builtin_bit_cast(f16x8, hi);
      const uint32_t l0 = f16_pair_bits(w0[0] - (float)hv[0], w0[1] - (float)hv[1]);
      const uint32_t l1 = f16_pair_bits(w0[2] - (float)hv[2], w0[3] - (float)hv[3]);
      const uint32_t l2 = f16_pair_bits(w1[0] - (float)hv[4], w1[1] - (float)hv[5]);
      const uint32_t l3 = f16_pair_bits(w1[2] - (float)hv[6], w1[3] - (float)hv[7]);
      lo = __builtin_bit_cast(bf16x8, i32x4{(int)l0, (int)l1, (int)l2, (int)l3});
    }
  } else {
    split8(w0, w1, hi, lo);
  }
}

}  // namespace vs

namespace vs {

constexpr int MAX_LDS_W = 512;   // slash-bitmap words kept in LDS (sequences up to 2^20 tokens)

// The tile sequence of one (q head, local query block) against the visible
// shard: its listed slash tiles, then its vertical columns gathered 64 at a
// time. Descriptors are staged through LDS by asynchronous copies (wave 0
// copies the list entry or the 64 column positions of a tile into a 64-int
// slot) and decoded by every wave after a barrier into the four copy rows of
// the lane, the tile mode (0 = full tile, 1 = per-key thresholds apply) and,
// for tid < 64, the threshold of key row tid: query rows with offset below it
// are inactive for that key (causal edge or a column already covered by a
// listed tile).
struct BlockTiles {
  const int32_t* tile_col;
  const int32_t* vl;          // the shard's vertical columns of this head
  const uint32_t* sbits;      // LDS copy of the head's slash bitmap
  int t0, nt, ve, nvc, total;
  int64_t G;                  // global block of the query block
  int kind, P, KB, src;
  int32_t* dbg = nullptr;     // debug builds: bounds-violation counter
  int64_t cap = 0;            // debug builds: capacity of tile_col

  // Tile order: the nvc vertical chunks first, then the listed tiles from the
  // query block's own diagonal outwards (the list holds them far to near).
  // The largest scores of a row usually sit in the sink / outlier columns or
  // next to the diagonal, so the online-softmax reference is set by the first
  // tiles and the O rescale is rarely needed afterwards.
  __device__ __forceinline__ void init(int t0_, int t1_, int ve_) {
    t0 = t0_; nt = t1_ - t0_; ve = ve_;
#ifdef VS_DEBUG_BOUNDS
    t0 = dbg_clamp(t0, 0, (int)cap + 1, dbg);
    nt = dbg_clamp(nt, 0, min(KB, (int)cap - t0) + 1, dbg);
    ve = dbg_clamp(ve, 0, KB * BLK + 1, dbg);
#endif
    nvc = (ve + BLK - 1) / BLK;
    total = nt + nvc;
  }
  __device__ __forceinline__ bool vert(int it) const { return it < nvc; }
  __device__ __forceinline__ void desc_copy(int it, int* slot, int wave, int lane) const {
    if (wave != 0) return;
    const int32_t* s = vert(it) ? vl + min(it * BLK + lane, ve - 1) : tile_col + t0 + (nt - 1 - (it - nvc));
    __builtin_amdgcn_global_load_lds((const void*)s,
                                     (__attribute__((address_space(3))) void*)(
                                         (__attribute__((address_space(3))) int*)(slot)),
                                     4, 0, 0);
  }
  // Listed tile: its first key row (wave-uniform) and whether it is the
  // diagonal tile (mode 1: key k active for rows >= k).
  __device__ __forceinline__ int tile_row(const int* slot, int& mode) const {
    const int e = __builtin_amdgcn_readfirstlane(slot[0]);
    mode = (e & VS_TILE_DIAG) ? 1 : 0;
    return dbg_clamp(e & VS_TILE_MASK, 0, KB, dbg) * BLK;
  }
  // Vertical chunk `it`: the key rows of this lane's copy pieces and, for
  // tid < BLK, the key's row threshold (rows below it are inactive: the causal
  // edge, and columns already covered by a listed tile of this block).
  __device__ __forceinline__ void vert_rows(int it, const int* slot, int* rows, int& thr, int wave, int lane,
                                            int tid) const {
#pragma unroll
    for (int c = 0; c < 4; ++c) rows[c] = dbg_clamp(slot[dma_local_row(wave, c, lane)], 0, KB * BLK, dbg);
    thr = BLK;
    if (tid < BLK && it * BLK + tid < ve) {
      const int m = dbg_clamp(slot[tid], 0, KB * BLK, dbg);
      const int64_t j = G - global_block(kind, P, KB, src, m / BLK);
      if (!((sbits[j >> 5] >> (j & 31)) & 1u)) thr = (j == 0) ? (m % BLK) : 0;
    }
  }
  // The same under one-position stripes: key tid's causal threshold and the
  // window of diagonals (bit qa) on which its rows are not already covered by
  // a listed tile of query block I (rank `rank`); W words of sbits.
  __device__ __forceinline__ void vert_rows_s1(int it, const int* slot, int* rows, int& thr, uint32_t& win, int wave,
                                               int lane, int tid, int I, int rank, int W) const {
#pragma unroll
    for (int c = 0; c < 4; ++c) rows[c] = dbg_clamp(slot[dma_local_row(wave, c, lane)], 0, KB * BLK, dbg);
    thr = BLK;
    win = 0;
    if (tid < BLK && it * BLK + tid < ve) {
      const int64_t mg = (int64_t)dbg_clamp(slot[tid], 0, KB * BLK, dbg) * P + src;
      thr = s1_causal_row(mg, rank, P, I);
      win = s1_vert_window(sbits, W, P, I, mg);
    }
  }
  // The same calls as RingTiles (one visible shard at local row 0; the call
  // site's cursor `c` is not needed).
  __device__ __forceinline__ void gather_rows(int, const int* slot, int* rows, int wave, int lane, int) const {
#pragma unroll
    for (int c = 0; c < 4; ++c) rows[c] = dbg_clamp(slot[dma_local_row(wave, c, lane)], 0, KB * BLK, dbg);
  }
  __device__ __forceinline__ bool vert(int it, int) const { return vert(it); }
  __device__ __forceinline__ int nvert() const { return nvc; }
  __device__ __forceinline__ void vert_rows(int it, const int* slot, int* rows, int& thr, int wave, int lane, int tid,
                                            int) const {
    vert_rows(it, slot, rows, thr, wave, lane, tid);
  }
  __device__ __forceinline__ int64_t row0(int, int) const { return 0; }
};

// ---- several ring steps in one launch ----------------------------------------
// One rank's ring steps walked by one launch with every visible shard
// resident: the tile sequence of a (q head, query block) takes the vertical
// columns of all steps, gathered 64 at a time across the steps' shards,
// then every step's listed tiles; the online-softmax state (or the dQ
// accumulator) carries across the steps, so the output is written once
// instead of being merged step by step.
constexpr int MAX_RING_STEPS = 32;

// Per-step mask arrays and visible shard (kernel argument).
struct RingSteps {
  const int32_t* tile_ptr[MAX_RING_STEPS];
  const int32_t* tile_col[MAX_RING_STEPS];
  const int32_t* vloc[MAX_RING_STEPS];
  const int32_t* vert_end[MAX_RING_STEPS];
  int32_t src[MAX_RING_STEPS];
  int32_t nsteps;
  int64_t cap;   // capacity of every step's tile_col (debug-build checks)
};

// Per-step arrays of the key-major gradient parts (kernel argument): one
// launch covers the key blocks of every step's visible shard.
struct RingStepsKV {
  const int32_t* csc_ptr[MAX_RING_STEPS];
  const int32_t* csc_row[MAX_RING_STEPS];
  const int32_t* vloc[MAX_RING_STEPS];
  const int32_t* vloc_cnt[MAX_RING_STEPS];
  const int32_t* vcum[MAX_RING_STEPS];
  int32_t src[MAX_RING_STEPS];
  int32_t nsteps;
};

// LDS table of one list row across the steps.
struct RingTable {
  int vcum[MAX_RING_STEPS + 1];  // vertical columns of the steps before step s
  int tcum[MAX_RING_STEPS + 1];  // listed tiles of the steps before step s
  int t0[MAX_RING_STEPS], nt[MAX_RING_STEPS];
  int src[MAX_RING_STEPS];       // visible shard of step s
};

__device__ __forceinline__ int rfl(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Tile sequence over the steps, with the calls of BlockTiles. Tile t lies in
// step s with cum[s] <= t < cum[s + 1]; each call site walks its tiles in
// increasing order and keeps its own step cursor (c = 0: descriptor copies,
// 1 and 2: the kernel's two copy sites), so finding the step is a short
// forward scan. Key rows of step s's shard start at row0 = src[s] * KB * 64
// of the tensors that hold every shard in storage order.
// Tile sequence over the steps, with the calls of BlockTiles. Tiles
// 0 .. nv - 1 are vertical chunks: chunk t holds the columns at positions
// 64 t .. 64 t + 63 of the steps' vertical lists laid end to end (step s's
// columns at vcum[s] .. vcum[s + 1] - 1), so a chunk can gather rows of
// several shards and its copy rows are storage rows of the tensors that hold
// every shard (shard src at row src * KB * 64). Tile nv + u is listed tile u
// of the steps' lists laid end to end: step s with tcum[s] <= u < tcum[s + 1],
// its rows from row0 = src[s] * KB * 64. Each call site walks its tiles in
// increasing order and keeps its own step cursor (c = 0: descriptor copies,
// 1 and 2: the kernel's two copy sites), so finding the step of a listed
// tile is a short forward scan.
struct RingTiles {
  const RingSteps* rs;
  RingTable* tb;
  const uint32_t* sbits;      // LDS copy of the head's slash bitmap (the same in every step)
  int64_t vl_off;             // the head's first entry in each step's vloc
  int64_t G;                  // global block of the query block
  int kind, P, KB, total, nv, vt;
  int cur[3];
  int32_t* dbg = nullptr;     // debug builds: bounds-violation counter

  // Wave 0 fills the table of list row u (= h * QB + I); the caller
  // synchronises the workgroup before start().
  __device__ __forceinline__ void fill(int64_t u, int wave, int lane) {
    if (wave != 0) return;
    const int n = rs->nsteps;
    int nt = 0, ve = 0;
    if (lane < n) {
      int a0 = rs->tile_ptr[lane][u], a1 = rs->tile_ptr[lane][u + 1];
      ve = rs->vert_end[lane][u];
#ifdef VS_DEBUG_BOUNDS
      a0 = dbg_clamp(a0, 0, (int)rs->cap + 1, dbg);
      a1 = a0 + dbg_clamp(a1 - a0, 0, min(KB, (int)rs->cap - a0) + 1, dbg);
      ve = dbg_clamp(ve, 0, KB * BLK + 1, dbg);
#endif
      tb->t0[lane] = a0;
      tb->nt[lane] = a1 - a0;
      tb->src[lane] = rs->src[lane];
      nt = a1 - a0;
    }
    int ti = nt, vi = ve;   // inclusive scans over the steps
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(ti, off, 64), z = __shfl_up(vi, off, 64);
      if (lane >= off) {
        ti += y;
        vi += z;
      }
    }
    if (lane < n) {
      tb->tcum[lane + 1] = ti;
      tb->vcum[lane + 1] = vi;
    }
    if (lane == 0) tb->tcum[0] = tb->vcum[0] = 0;
  }
  __device__ __forceinline__ void start() {
    vt = rfl(tb->vcum[rs->nsteps]);
    nv = (vt + BLK - 1) / BLK;
    total = nv + rfl(tb->tcum[rs->nsteps]);
    cur[0] = cur[1] = cur[2] = 0;
  }
  // step of listed tile t (t >= nv)
  __device__ __forceinline__ int step_of(int t, int c) {
    const int u = t - nv;
    int s = cur[c];
    while (s + 1 < rs->nsteps && u >= rfl(tb->tcum[s + 1])) ++s;
    cur[c] = s;
    return s;
  }
  // step holding vertical position pos (< vt): the last s with vcum[s] <= pos
  __device__ __forceinline__ int vstep(int pos) const {
    int lo = 0, hi = rs->nsteps - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tb->vcum[mid] <= pos) lo = mid; else hi = mid - 1;
    }
    return lo;
  }
  __device__ __forceinline__ bool vert(int t, int) const { return t < nv; }
  __device__ __forceinline__ int nvert() const { return nv; }
  __device__ __forceinline__ void desc_copy(int t, int* slot, int wave, int lane) {
    if (t >= nv) step_of(t, 0);
    if (wave != 0) return;
    const int32_t* p;
    if (t < nv) {
      const int pos = min(t * BLK + lane, vt - 1);
      const int s = vstep(pos);
      p = rs->vloc[s] + vl_off + (pos - tb->vcum[s]);
    } else {
      const int s = cur[0];
      const int it = t - nv - rfl(tb->tcum[s]);
      p = rs->tile_col[s] + rfl(tb->t0[s]) + (rfl(tb->nt[s]) - 1 - it);
    }
    __builtin_amdgcn_global_load_lds((const void*)p,
                                     (__attribute__((address_space(3))) void*)(
                                         (__attribute__((address_space(3))) int*)(slot)),
                                     4, 0, 0);
  }
  __device__ __forceinline__ int tile_row(const int* slot, int& mode) const {
    const int e = __builtin_amdgcn_readfirstlane(slot[0]);
    mode = (e & VS_TILE_DIAG) ? 1 : 0;
    return dbg_clamp(e & VS_TILE_MASK, 0, KB, dbg) * BLK;
  }
  // storage row of the column at chunk position r of vertical chunk t
  __device__ __forceinline__ int vrow(int t, const int* slot, int r) const {
    const int s = vstep(min(t * BLK + r, vt - 1));
    return tb->src[s] * KB * BLK + dbg_clamp(slot[r], 0, KB * BLK, dbg);
  }
  // copy rows of this lane's four pieces of vertical chunk t
  __device__ __forceinline__ void gather_rows(int t, const int* slot, int* rows, int wave, int lane, int) const {
#pragma unroll
    for (int k = 0; k < 4; ++k) rows[k] = vrow(t, slot, dma_local_row(wave, k, lane));
  }
  __device__ __forceinline__ void vert_rows(int t, const int* slot, int* rows, int& thr, int wave, int lane, int tid,
                                            int c) {
    gather_rows(t, slot, rows, wave, lane, c);
    thr = BLK;
    if (tid < BLK && t * BLK + tid < vt) {
      const int s = vstep(t * BLK + tid);
      const int m = dbg_clamp(slot[tid], 0, KB * BLK, dbg);
      const int64_t j = G - global_block(kind, P, KB, tb->src[s], m / BLK);
      if (!((sbits[j >> 5] >> (j & 31)) & 1u)) thr = (j == 0) ? (m % BLK) : 0;
    }
  }
  // first storage row of tile t's shard (vertical chunks: rows are storage rows)
  __device__ __forceinline__ int64_t row0(int t, int c) {
    return t < nv ? 0 : (int64_t)rs->src[step_of(t, c)] * KB * BLK;
  }
};

}  // namespace vs

namespace vs {

// Four transpose-read pairs (eight ds_read_b64_tr_b16, each pair 4 rows apart)
// issued back to back with one LDS wait at the end. Issued as one asm block
// so the compiler does not hold them behind outstanding global->LDS copies
// into other stages (it cannot prove the intrinsic form does not alias them);
// the block waits for its own results before returning them.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
}
// (p + 4 rows of a 256-byte-pitch tile = p + 1024 bytes)
__device__ __forceinline__ void lds_read_tr16_x2_4(const bf16* p0, const bf16* p1, const bf16* p2, const bf16* p3,
                                                   bf16x8* out) {
  typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
  i32x2 r0, r1, r2, r3, r4, r5, r6, r7;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:1024\n\t"
      "ds_read_b64_tr_b16 %2, %9\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:1024\n\t"
      "ds_read_b64_tr_b16 %4, %10\n\t"
      "ds_read_b64_tr_b16 %5, %10 offset:1024\n\t"
      "ds_read_b64_tr_b16 %6, %11\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:1024\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
      : "v"(lds_addr(p0)), "v"(lds_addr(p1)), "v"(lds_addr(p2)), "v"(lds_addr(p3))
      : "memory");
  out[0] = __builtin_bit_cast(bf16x8, i32x4{r0[0], r0[1], r1[0], r1[1]});
  out[1] = __builtin_bit_cast(bf16x8, i32x4{r2[0], r2[1], r3[0], r3[1]});
  out[2] = __builtin_bit_cast(bf16x8, i32x4{r4[0], r4[1], r5[0], r5[1]});
  out[3] = __builtin_bit_cast(bf16x8, i32x4{r6[0], r6[1], r7[0], r7[1]});
}

}  // namespace vs
