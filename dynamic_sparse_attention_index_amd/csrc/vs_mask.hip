// Active-region compaction: from the shared vertical/slash index to the
// per-(head, query block) tile lists, their transpose, the shard's vertical
// columns and exact active-entry counts of one (rank, ring step).
//
// Follows the MTraining review, page 1, section 三.2 item 3: after the index is
// shared, each worker determines the active region of its local attention
// sub-matrix from the indices of the active verticals and slashes. The review
// times a 2.08 ms host step next to the index build (section 五, latency
// breakdown); here the whole conversion is integer work on the GPU.
//
// Four launches: per-head setup (slash bitmap, the shard's vertical columns and
// their per-block prefix counts), list lengths, one exclusive scan, list fill.
#include "vs_common.h"
#include "vs_internal.h"

namespace vs {

struct MaskArgs {
  const int32_t* vert_idx; const int32_t* vert_cnt; int64_t vert_stride;
  const int32_t* slash_idx; const int32_t* slash_cnt; int64_t slash_stride;
  int kind, P, NB, T, W, Hq, rank, src;
  int64_t tile_cap;
  int32_t *tile_ptr, *tile_col, *csc_ptr, *csc_row, *vloc, *vloc_cnt, *vcum, *vert_end;
  uint32_t* slash_bits;
  int64_t* n_active;
  int32_t* status;
};

constexpr int MASK_THREADS = 1024;

// Several ring steps of one rank built by the same four launches (grid.y =
// step): the fields that differ per step (visible shard, output arrays).
constexpr int MAX_MASK_STEPS = 32;
struct MaskRing {
  int32_t src[MAX_MASK_STEPS];
  int32_t *tile_ptr[MAX_MASK_STEPS], *tile_col[MAX_MASK_STEPS], *csc_ptr[MAX_MASK_STEPS], *csc_row[MAX_MASK_STEPS];
  int32_t *vloc[MAX_MASK_STEPS], *vloc_cnt[MAX_MASK_STEPS], *vcum[MAX_MASK_STEPS], *vert_end[MAX_MASK_STEPS];
  uint32_t* slash_bits[MAX_MASK_STEPS];
  int64_t* n_active[MAX_MASK_STEPS];
  int32_t* status[MAX_MASK_STEPS];
};
// The arguments of this workgroup's step (the shared ones from `a`).
__device__ __forceinline__ MaskArgs step_args(const MaskArgs& a, const MaskRing* rg) {
  if (!rg) return a;
  const int s = blockIdx.y;
  MaskArgs b = a;
  b.src = rg->src[s];
  b.tile_ptr = rg->tile_ptr[s]; b.tile_col = rg->tile_col[s]; b.csc_ptr = rg->csc_ptr[s]; b.csc_row = rg->csc_row[s];
  b.vloc = rg->vloc[s]; b.vloc_cnt = rg->vloc_cnt[s]; b.vcum = rg->vcum[s]; b.vert_end = rg->vert_end[s];
  b.slash_bits = rg->slash_bits[s]; b.n_active = rg->n_active[s]; b.status = rg->status[s];
  return b;
}

// Block-wide exclusive scan of one int per thread (1024 threads = 16 waves).
__device__ __forceinline__ int block_exclusive_scan(int x, int* total, int* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < MASK_THREADS / 64; ++w) { int t = sh[w]; sh[w] = run; run += t; }
    sh[MASK_THREADS / 64] = run;
  }
  __syncthreads();
  int res = sh[wave] + incl - x;
  *total = sh[MASK_THREADS / 64];
  __syncthreads();
  return res;
}

// Launch 1: grid = Hq, one workgroup per head.
__device__ __forceinline__ void mask_head_body(const MaskArgs& a) {
  __shared__ int sh[MASK_THREADS / 64 + 1];
  const int h = blockIdx.x;
  const int32_t* S = a.slash_idx + (int64_t)h * a.slash_stride;
  const int ns = a.slash_cnt[h];
  if (h == 0 && threadIdx.x == 0) a.status[0] = VS_OK;
  // slash bitmap
  for (int w = threadIdx.x; w < a.W; w += MASK_THREADS) {
    int lo = lower_bound_i32(S, ns, (int64_t)w * 32);
    int hi = lower_bound_i32(S, ns, (int64_t)w * 32 + 32);
    uint32_t bits = 0;
    for (int e = lo; e < hi; ++e) {
      const int d = S[e] - w * 32;
      if (d >= 0 && d < 32) bits |= 1u << d;
    }
    a.slash_bits[(int64_t)h * a.W + w] = bits;
  }
  // vertical columns of the visible shard, order-preserving compaction
  const int32_t* V = a.vert_idx + (int64_t)h * a.vert_stride;
  const int nv = a.vert_cnt[h];
  int32_t* out = a.vloc + (int64_t)h * a.NB * BLK;
  int base = 0;
  for (int c0 = 0; c0 < nv; c0 += MASK_THREADS) {
    const int e = c0 + threadIdx.x;
    int keep = 0, local = 0;
    if (e < nv) {
      const int64_t m = V[e];
      if (m >= 0 && m < (int64_t)a.T * BLK) {
        int J;
        keep = owner_of_block(a.kind, a.P, a.NB, m / BLK, &J) == a.src;
        local = J * BLK + (int)(m % BLK);
      }
    }
    int tot;
    const int pos = block_exclusive_scan(keep, &tot, sh);
    if (keep && base + pos < a.NB * BLK) out[base + pos] = local;
    base += tot;
  }
  base = min(base, a.NB * BLK);  // only reachable with repeated positions in the input
  if (threadIdx.x == 0) a.vloc_cnt[h] = base;
  __syncthreads();
  // vcum[J] = number of shard verticals in local blocks < J
  for (int J = threadIdx.x; J <= a.NB; J += MASK_THREADS)
    a.vcum[(int64_t)h * (a.NB + 1) + J] = lower_bound_i32(out, base, (int64_t)J * BLK);
}

// Launches 2 and 4 give one wave to each list row: rows [0, Hq*NB) are the
// (h, I) rows of the CSR, rows [Hq*NB, 2*Hq*NB) the (h, J) columns of the CSC;
// the lanes stride over the head's slash list 64 entries at a time.
constexpr int ROW_WAVES = 4;   // waves per workgroup of the row kernels

__device__ __forceinline__ int wave_sum_i32(int x) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Launch 2: list lengths.
__device__ __forceinline__ void mask_count_body(const MaskArgs& a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * ROW_WAVES + (threadIdx.x >> 6);
  const int64_t nrow = (int64_t)a.Hq * a.NB;
  if (t >= 2 * nrow) return;
  const bool csr = t < nrow;
  const int64_t u = csr ? t : t - nrow;
  const int h = (int)(u / a.NB), B = (int)(u % a.NB);
  const int32_t* S = a.slash_idx + (int64_t)h * a.slash_stride;
  const int ns = a.slash_cnt[h];
  int cnt = 0;
  if (csr) {  // key blocks G - j of the visible shard
    const int64_t G = global_block(a.kind, a.P, a.NB, a.rank, B);
    for (int e = lane; e < ns; e += 64) {
      const int j = S[e];
      int J;
      if (j >= 0 && j <= G && owner_of_block(a.kind, a.P, a.NB, G - j, &J) == a.src) ++cnt;
    }
    cnt = wave_sum_i32(cnt);
    if (lane == 0) a.tile_ptr[1 + u] = cnt;
  } else {    // query blocks G' + j of this rank
    const int64_t Gp = global_block(a.kind, a.P, a.NB, a.src, B);
    for (int e = lane; e < ns; e += 64) {
      const int j = S[e];
      int I;
      if (j >= 0 && Gp + j < a.T && owner_of_block(a.kind, a.P, a.NB, Gp + j, &I) == a.rank) ++cnt;
    }
    cnt = wave_sum_i32(cnt);
    if (lane == 0) a.csc_ptr[1 + u] = cnt;
  }
}

// Launch 3: one workgroup; in-place inclusive scan of both length arrays.
// The running total is kept in 64 bits, so a list larger than the int32
// entries can hold is still seen to exceed the capacity (tile_cap < 2^31);
// the stored prefix values are then wrong, but they are overwritten below.
__device__ int64_t scan_inplace(int32_t* p, int64_t n, int* sh) {
  int64_t run = 0;
  if (threadIdx.x == 0) p[0] = 0;
  for (int64_t c0 = 0; c0 < n; c0 += MASK_THREADS) {
    const int64_t e = c0 + threadIdx.x;
    const int x = e < n ? p[1 + e] : 0;   // one row's count: at most T
    int tot;
    const int pos = block_exclusive_scan(x, &tot, sh);
    if (e < n) p[1 + e] = (int32_t)(run + pos + x);
    run += tot;
  }
  return run;
}

// On overflow every list is made empty before any consumer runs: both
// pointer arrays become all zeros and the per-head vertical counts zero
// (vert_end is zeroed by the fill launch), so attention calls queued behind
// this mask on the stream read no list entry and compute nothing for the
// step; only the status word and n_active (exact counts) are meaningful.
__device__ __forceinline__ void mask_scan_body(const MaskArgs& a) {
  __shared__ int sh[MASK_THREADS / 64 + 1];
  const int64_t n = (int64_t)a.Hq * a.NB;
  const int64_t tiles = scan_inplace(a.tile_ptr, n, sh);
  const int64_t cols = scan_inplace(a.csc_ptr, n, sh);
  __syncthreads();
  if (tiles > a.tile_cap || cols > a.tile_cap) {
    for (int64_t e = threadIdx.x; e <= n; e += MASK_THREADS) {
      a.tile_ptr[e] = 0;
      a.csc_ptr[e] = 0;
    }
    for (int h = threadIdx.x; h < a.Hq; h += MASK_THREADS) a.vloc_cnt[h] = 0;
    if (threadIdx.x == 0) a.status[0] = VS_ERR_CAPACITY;
  }
}

// Launch 4: fill the lists; the CSR half also writes vert_end and n_active.
// Order-preserving compaction per 64-entry chunk: a lane's output position is
// the running count plus the matches of the lanes below it (ballot).
__device__ __forceinline__ void mask_fill_body(const MaskArgs& a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * ROW_WAVES + (threadIdx.x >> 6);
  const int64_t nrow = (int64_t)a.Hq * a.NB;
  if (t >= 2 * nrow) return;
  const bool csr = t < nrow;
  const int64_t u = csr ? t : t - nrow;
  const int h = (int)(u / a.NB), B = (int)(u % a.NB);
  const int32_t* S = a.slash_idx + (int64_t)h * a.slash_stride;
  const int ns = a.slash_cnt[h];
  const bool fits = a.status[0] == VS_OK;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (csr) {
    const int64_t G = global_block(a.kind, a.P, a.NB, a.rank, B);
    const int32_t* vc = a.vcum + (int64_t)h * (a.NB + 1);
    int32_t* dst = a.tile_col + a.tile_ptr[u];
    int n = 0;
    int act = 0, covered = 0;   // this lane's share
    // descending j gives ascending key blocks (same predicate as the count)
    for (int c0 = 0; c0 < ns; c0 += 64) {
      const int e = ns - 1 - (c0 + lane);
      int J = 0, j = -1;
      bool ok = false;
      if (e >= 0) {
        j = S[e];
        ok = j >= 0 && j <= G && owner_of_block(a.kind, a.P, a.NB, G - j, &J) == a.src;
      }
      const uint64_t m = __builtin_amdgcn_ballot_w64(ok);
      if (ok) {
        if (fits) dst[n + __builtin_popcountll(m & below)] = J | (j == 0 ? VS_TILE_DIAG : 0);
        if (j == 0) {
          act += BLK * (BLK + 1) / 2;
        } else {
          act += BLK * BLK;
          covered += vc[J + 1] - vc[J];
        }
      }
      n += __builtin_popcountll(m);
    }
    const int J_le = blocks_upto(a.kind, a.P, a.NB, a.src, G);
    const int J_lt = blocks_upto(a.kind, a.P, a.NB, a.src, G - 1);
    // vertical columns in earlier blocks not covered by a listed tile: full
    // columns; in the query block's own global block (when its diagonal is
    // not selected): the causal part of each column
    int vpart = 0;
    if (J_le > J_lt) {  // the shard holds the query block's own global block
      const bool diag_sel = (a.slash_bits[(int64_t)h * a.W] & 1u) != 0;
      if (!diag_sel) {
        const int32_t* vl = a.vloc + (int64_t)h * a.NB * BLK;
        for (int e = vc[J_lt] + lane; e < vc[J_le]; e += 64) vpart += BLK - (vl[e] % BLK);
      }
    }
    act = wave_sum_i32(act);
    covered = wave_sum_i32(covered);
    vpart = wave_sum_i32(vpart);
    if (lane == 0) {
      a.vert_end[u] = fits ? vc[J_le] : 0;
      a.n_active[u] = (int64_t)act + (int64_t)BLK * (vc[J_lt] - covered) + vpart;
    }
  } else {
    if (!fits) return;
    const int64_t Gp = global_block(a.kind, a.P, a.NB, a.src, B);
    int32_t* dst = a.csc_row + a.csc_ptr[u];
    int n = 0;
    for (int c0 = 0; c0 < ns; c0 += 64) {
      const int e = c0 + lane;
      int I = 0, j = -1;
      bool ok = false;
      if (e < ns) {
        j = S[e];
        ok = j >= 0 && Gp + j < a.T && owner_of_block(a.kind, a.P, a.NB, Gp + j, &I) == a.rank;
      }
      const uint64_t m = __builtin_amdgcn_ballot_w64(ok);
      if (ok) dst[n + __builtin_popcountll(m & below)] = I | (j == 0 ? VS_TILE_DIAG : 0);
      n += __builtin_popcountll(m);
    }
  }
}

__global__ void __launch_bounds__(MASK_THREADS) mask_head_kernel(MaskArgs a) { mask_head_body(a); }
__global__ void __launch_bounds__(64 * ROW_WAVES) mask_count_kernel(MaskArgs a) { mask_count_body(a); }
__global__ void __launch_bounds__(MASK_THREADS) mask_scan_kernel(MaskArgs a) { mask_scan_body(a); }
__global__ void __launch_bounds__(64 * ROW_WAVES) mask_fill_kernel(MaskArgs a) { mask_fill_body(a); }
__global__ void __launch_bounds__(MASK_THREADS) mask_head_ring_kernel(MaskArgs a, MaskRing rg) {
  mask_head_body(step_args(a, &rg));
}
__global__ void __launch_bounds__(64 * ROW_WAVES) mask_count_ring_kernel(MaskArgs a, MaskRing rg) {
  mask_count_body(step_args(a, &rg));
}
__global__ void __launch_bounds__(MASK_THREADS) mask_scan_ring_kernel(MaskArgs a, MaskRing rg) {
  mask_scan_body(step_args(a, &rg));
}
__global__ void __launch_bounds__(64 * ROW_WAVES) mask_fill_ring_kernel(MaskArgs a, MaskRing rg) {
  mask_fill_body(step_args(a, &rg));
}

int launch_block_mask(const int32_t* vert_idx, const int32_t* vert_cnt, int64_t vert_stride,
                      const int32_t* slash_idx, const int32_t* slash_cnt, int64_t slash_stride,
                      int rank, int src, vs_mask* m, hipStream_t stream) {
  MaskArgs a;
  a.vert_idx = vert_idx; a.vert_cnt = vert_cnt; a.vert_stride = vert_stride;
  a.slash_idx = slash_idx; a.slash_cnt = slash_cnt; a.slash_stride = slash_stride;
  a.kind = m->lay.kind; a.P = m->lay.P; a.NB = m->QB; a.T = m->T; a.W = m->W; a.Hq = m->Hq;
  a.rank = rank; a.src = src; a.tile_cap = m->tile_cap;
  a.tile_ptr = m->tile_ptr; a.tile_col = m->tile_col; a.csc_ptr = m->csc_ptr; a.csc_row = m->csc_row;
  a.vloc = m->vloc; a.vloc_cnt = m->vloc_cnt; a.vcum = m->vcum; a.vert_end = m->vert_end;
  a.slash_bits = m->slash_bits; a.n_active = m->n_active; a.status = m->status;
  const int64_t nrows = 2 * (int64_t)m->Hq * m->QB;   // one wave per list row
  const int tpb = 64 * ROW_WAVES;
  const unsigned nblk = (unsigned)((nrows + ROW_WAVES - 1) / ROW_WAVES);
  hipLaunchKernelGGL(mask_head_kernel, dim3(m->Hq), dim3(MASK_THREADS), 0, stream, a);
  hipLaunchKernelGGL(mask_count_kernel, dim3(nblk), dim3(tpb), 0, stream, a);
  hipLaunchKernelGGL(mask_scan_kernel, dim3(1), dim3(MASK_THREADS), 0, stream, a);
  hipLaunchKernelGGL(mask_fill_kernel, dim3(nblk), dim3(tpb), 0, stream, a);
  return hipGetLastError() == hipSuccess ? VS_OK : VS_ERR_HIP;
}

// Steps 0 .. nsteps-1 of rank `rank` into ms[0 .. nsteps-1] (every mask
// carved for the same shape and layout), the four launches shared by up to
// MAX_MASK_STEPS steps.
int launch_block_mask_ring(const int32_t* vert_idx, const int32_t* vert_cnt, int64_t vert_stride,
                           const int32_t* slash_idx, const int32_t* slash_cnt, int64_t slash_stride,
                           int rank, vs_mask* ms, int nsteps, hipStream_t stream) {
  const vs_mask* m = &ms[0];
  MaskArgs a;
  a.vert_idx = vert_idx; a.vert_cnt = vert_cnt; a.vert_stride = vert_stride;
  a.slash_idx = slash_idx; a.slash_cnt = slash_cnt; a.slash_stride = slash_stride;
  a.kind = m->lay.kind; a.P = m->lay.P; a.NB = m->QB; a.T = m->T; a.W = m->W; a.Hq = m->Hq;
  a.rank = rank; a.src = -1; a.tile_cap = m->tile_cap;
  const int64_t nrows = 2 * (int64_t)m->Hq * m->QB;
  const int tpb = 64 * ROW_WAVES;
  const unsigned nblk = (unsigned)((nrows + ROW_WAVES - 1) / ROW_WAVES);
  for (int s0 = 0; s0 < nsteps; s0 += MAX_MASK_STEPS) {
    const int ns = nsteps - s0 < MAX_MASK_STEPS ? nsteps - s0 : MAX_MASK_STEPS;
    MaskRing rg{};
    for (int i = 0; i < ns; ++i) {
      vs_mask& x = ms[s0 + i];
      const int src = ((rank - (s0 + i)) % a.P + a.P) % a.P;
      x.rank = rank;
      x.src = src;
      rg.src[i] = src;
      rg.tile_ptr[i] = x.tile_ptr; rg.tile_col[i] = x.tile_col; rg.csc_ptr[i] = x.csc_ptr; rg.csc_row[i] = x.csc_row;
      rg.vloc[i] = x.vloc; rg.vloc_cnt[i] = x.vloc_cnt; rg.vcum[i] = x.vcum; rg.vert_end[i] = x.vert_end;
      rg.slash_bits[i] = x.slash_bits; rg.n_active[i] = x.n_active; rg.status[i] = x.status;
    }
    hipLaunchKernelGGL(mask_head_ring_kernel, dim3(m->Hq, ns), dim3(MASK_THREADS), 0, stream, a, rg);
    hipLaunchKernelGGL(mask_count_ring_kernel, dim3(nblk, ns), dim3(tpb), 0, stream, a, rg);
    hipLaunchKernelGGL(mask_scan_ring_kernel, dim3(1, ns), dim3(MASK_THREADS), 0, stream, a, rg);
    hipLaunchKernelGGL(mask_fill_ring_kernel, dim3(nblk, ns), dim3(tpb), 0, stream, a, rg);
  }
  return hipGetLastError() == hipSuccess ? VS_OK : VS_ERR_HIP;
}

}  // namespace vs
