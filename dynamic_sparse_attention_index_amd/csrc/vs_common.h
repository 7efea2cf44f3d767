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

// --- MFMA wrappers (lane layouts verified on gfx950) ------------------------
// 16x16x32 bf16: lane l supplies A[l%16][8*(l/16)+j], B[8*(l/16)+j][l%16]
// (j=0..7) and receives C[4*(l/16)+i][l%16] (i=0..3).
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

__device__ __forceinline__ int lower_bound_i32(const int32_t* a, int n, int64_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

}  // namespace vs
