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
        if (a.kind == VS_STRIPED1) {
          keep = (int)(m % a.P) == a.src;
          local = (int)(m / a.P);
        } else {
          int J;
          keep = owner_of_block(a.kind, a.P, a.NB, m / BLK, &J) == a.src;
          local = J * BLK + (int)(m % BLK);
        }
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

// ---- one-position stripes (VS_STRIPED1) ---------------------------------------
// Local position l of rank r is global position l P + r, so local query block
// I (rank r) spans global blocks I P .. I P + P - 1 and local key block J
// (shard s) global blocks J P .. J P + P - 1 (P <= 32). Row a of the query
// block lies in global block I P + qa(a), qa(a) = (a P + r) >> 6, and key b in
// J P + kb(b), kb(b) = (b P + s) >> 6. An entry of tile (I, J) lies on global
// block-diagonal o P + qa - kb with o = I - J, and every (qa, kb) pair occurs,
// so with o >= 1 the tile meets diagonals o P - P + 1 .. o P + P - 1 (all of
// them causal). With o = 0 it meets 0 .. P - 1 causally (diagonal 0 partly:
// b P + s <= a P + r); negative ones lie above the rows.

// Selected diagonals a stripe-1 tile at block offset o meets, as the mask
// kernels read them (bit i: diagonal o P - P + 1 + i for o >= 1; diagonal i
// for o = 0).
__device__ __forceinline__ uint64_t s1_window(const uint32_t* sb, int W, int P, int o) {
  return o == 0 ? sbit_window(sb, W, 0, P) : sbit_window(sb, W, (int64_t)o * P - P + 1, 2 * P - 1);
}
// A listed tile is full (unflagged) when every diagonal it meets is selected.
__device__ __forceinline__ bool s1_full(uint64_t win, int P, int o) {
  return o > 0 && win == ((2 * P - 1 >= 64) ? ~0ull : ((1ull << (2 * P - 1)) - 1ull));
}
// First row a of the query block with qa(a) >= x (x in 0 .. P): rows with
// qa = x are [first(x), first(x + 1)).
__device__ __forceinline__ int s1_first(int x, int r, int P) {
  return x == 0 ? 0 : min(BLK, (BLK * x - r + P - 1) / P);
}

// Per-workgroup tables of the stripe-1 counts for one (rank r, shard s):
//   fq[x]  first row with qa >= x (x = 0 .. P), fk[y] the same for keys;
//   cd[d + P - 1] = entries with qa - kb = d (d = -(P-1) .. P-1);
//   cd0 = causal entries with qa == kb (b P + s <= a P + r).
struct S1Tables {
  int fq[33], fk[33];
  int cd[63];
  int cd0;
};
__device__ void s1_tables(S1Tables& t, int r, int s, int P) {
  const int tid = threadIdx.x;
  if (tid <= P) {
    t.fq[tid] = s1_first(tid, r, P);
    t.fk[tid] = s1_first(tid, s, P);
  }
  __syncthreads();
  if (tid < 2 * P - 1) {
    const int d = tid - (P - 1);
    int c = 0;
    for (int x = 0; x < P; ++x) {
      const int y = x - d;
      if (y >= 0 && y < P) c += (t.fq[x + 1] - t.fq[x]) * (t.fk[y + 1] - t.fk[y]);
    }
    t.cd[tid] = c;
  }
  if (tid == 0) {
    int c = 0;
    for (int aa = 0; aa < BLK; ++aa) {
      const int x = ((aa * P + r) >> 6);
      const int hi = min(t.fk[x + 1] - 1, aa - (r < s ? 1 : 0));   // b <= a (r >= s) or b < a
      c += max(0, hi - t.fk[x] + 1);
    }
    t.cd0 = c;
  }
  __syncthreads();
}
// Slash-active entries of a listed tile at offset o with window `win`.
__device__ __forceinline__ int s1_tile_count(const S1Tables& t, uint64_t win, int P, int o) {
  int c = 0;
  if (o > 0) {
    while (win) {
      const int i = __builtin_ctzll(win);
      win &= win - 1;
      c += t.cd[i];               // diagonal o P - P + 1 + i: qa - kb = i - (P - 1)
    }
  } else {
    if (win & 1ull) c += t.cd0;
    win &= ~1ull;
    while (win) {
      const int i = __builtin_ctzll(win);
      win &= win - 1;
      c += t.cd[i + P - 1];
    }
  }
  return c;
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
  if (a.kind == VS_STRIPED1) {   // block offsets o = I - J with a selected diagonal in the tile's window
    const uint32_t* sb = a.slash_bits + (int64_t)h * a.W;
    const int n_o = csr ? B + 1 : a.NB - B;   // CSR row I: J = 0 .. I; CSC column J: I = J .. NB - 1
    for (int o = lane; o < n_o; o += 64) cnt += s1_window(sb, a.W, a.P, o) != 0ull;
    cnt = wave_sum_i32(cnt);
    if (lane == 0) (csr ? a.tile_ptr : a.csc_ptr)[1 + u] = cnt;
    return;
  }
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
__device__ void mask_fill_s1(const MaskArgs& a, const S1Tables& tb, bool csr, int64_t u, int h, int B);

__device__ __forceinline__ void mask_fill_body(const MaskArgs& a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * ROW_WAVES + (threadIdx.x >> 6);
  const int64_t nrow = (int64_t)a.Hq * a.NB;
  if (a.kind == VS_STRIPED1) {
    __shared__ S1Tables tb;
    s1_tables(tb, a.rank, a.src, a.P);
    if (t >= 2 * nrow) return;
    const bool csr = t < nrow;
    const int64_t u = csr ? t : t - nrow;
    mask_fill_s1(a, tb, csr, u, (int)(u / a.NB), (int)(u % a.NB));
    return;
  }
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

// Launch 4 under one-position stripes. CSR row (h, I): key blocks J = I - o
// ascending with a selected diagonal in the window, flagged unless the window
// is wholly selected; n_active adds each listed tile's slash entries and, per
// vertical column of the shard, its causal rows on unselected diagonals.
// vert_end: the columns at or before the block's last row,
// l P + s <= (64 I + 63) P + r, i.e. l < 64 I + 64 - [r < s].
// CSC column (h, J): query blocks I = J + o ascending, the same flags.
__device__ void mask_fill_s1(const MaskArgs& a, const S1Tables& tb, bool csr, int64_t u, int h, int B) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const uint32_t* sb = a.slash_bits + (int64_t)h * a.W;
  const bool fits = a.status[0] == VS_OK;
  const int P = a.P;
  if (csr) {
    const int I = B;
    int32_t* dst = a.tile_col + a.tile_ptr[u];
    int n = 0, act = 0;
    for (int c0 = 0; c0 <= I; c0 += 64) {
      const int J = c0 + lane, o = I - J;
      uint64_t win = 0;
      if (J <= I) win = s1_window(sb, a.W, P, o);
      const bool ok = win != 0ull;
      const uint64_t m = __builtin_amdgcn_ballot_w64(ok);
      if (ok) {
        if (fits) dst[n + __builtin_popcountll(m & below)] = J | (s1_full(win, P, o) ? 0 : VS_TILE_DIAG);
        act += s1_tile_count(tb, win, P, o);
      }
      n += __builtin_popcountll(m);
    }
    const int32_t* vl = a.vloc + (int64_t)h * a.NB * BLK;
    const int nv = a.vloc_cnt[h];
    const int ve = lower_bound_i32(vl, nv, (int64_t)BLK * I + BLK - (a.rank < a.src ? 1 : 0));
    int vpart = 0;
    for (int e = lane; e < ve; e += 64) {
      const int64_t mg = (int64_t)vl[e] * P + a.src;          // global column
      // first causal row: (64 I + c) P + r >= mg
      const int64_t num = mg - a.rank - (int64_t)BLK * I * P;
      const int c = num <= 0 ? 0 : (int)min<int64_t>(BLK, (num + P - 1) / P);
      // bit x: diagonal I P + x - floor(mg / 64) selected (negative ones: rows above the column)
      const uint64_t win = sbit_window(sb, a.W, (int64_t)I * P - (mg >> 6), P);
      for (int x = 0; x < P; ++x)
        if (!((win >> x) & 1ull)) vpart += max(0, tb.fq[x + 1] - max(tb.fq[x], c));
    }
    act = wave_sum_i32(act);
    vpart = wave_sum_i32(vpart);
    if (lane == 0) {
      a.vert_end[u] = fits ? ve : 0;
      a.n_active[u] = (int64_t)act + vpart;
    }
  } else {
    if (!fits) return;
    const int J = B;
    int32_t* dst = a.csc_row + a.csc_ptr[u];
    int n = 0;
    for (int c0 = 0; J + c0 < a.NB; c0 += 64) {
      const int o = c0 + lane, I = J + o;
      uint64_t win = 0;
      if (I < a.NB) win = s1_window(sb, a.W, P, o);
      const bool ok = win != 0ull;
      const uint64_t m = __builtin_amdgcn_ballot_w64(ok);
      if (ok) dst[n + __builtin_popcountll(m & below)] = I | (s1_full(win, P, o) ? 0 : VS_TILE_DIAG);
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
