// Backward of the block-sparse vertical-slash attention over one ring step.
//
// The pages describe the sparse forward (MTraining review, page 1, section
// 三.2 item 3) and train with it, so the gradient is the exact gradient of
// softmax attention restricted to the same active set, the index being held
// fixed: with the final row statistics LSE and delta = rowsum(dO * O),
//   P = exp(z - LSE), dV += P^T dO, dS = P * (dO.V - delta),
//   dQ += dS K * scale, dK += dS^T Q * scale.
//
// Three kernels, no atomics except for vertical columns:
//   * dq_kernel     -- query-major like the forward: one workgroup per
//                      (q head, query block) recomputes P and dP over the same
//                      tiles and gathered vertical chunks and owns its dQ rows;
//   * dkdv_kernel   -- key-major over slash tiles: one workgroup per (kv head,
//                      key block) walks the CSC lists of every q head of the
//                      group and owns the key block's dK/dV rows;
//   * dkdv_vert_kernel -- the shard's vertical columns, 64 gathered columns per
//                      work item against a range of query blocks, added to
//                      dK/dV with fp32 atomics (a column can belong to several
//                      q heads of the group).
#include <type_traits>

#include "vs_common.h"
#include "vs_internal.h"

namespace vs {

constexpr int BWD_THREADS = 256;
constexpr int VERT_SEG = 128;          // query blocks per vertical work item (at most)
constexpr int VERT_SEG_MIN = 8;        // ... and at least, when the range is shortened
constexpr int VERT_ITEMS_MIN = 2048;   // shorten the range until there are this many items
constexpr int VERT_GRID = 2048;        // persistent workgroups for vertical columns

struct BwdArgs {
  const void *q, *k, *v, *dout;
  int64_t qsh, qsn, ksh, ksn, vsh, vsn, dsh, dsn;
  const float *lse, *delta;
  const int32_t *tile_ptr, *tile_col, *csc_ptr, *csc_row, *vloc, *vloc_cnt, *vcum, *vert_end;
  const uint32_t* slash_bits;
  float *dq, *dk, *dv;
  int Hq, Hkv, QB, KB, W, kind, P, rank, src;
  float scale, scale_log2;
  int overwrite;   // dq and slash dk/dv written, not added (VS_BWD_OVERWRITE)
  int32_t* dbg;    // debug builds: bounds-violation counter (null otherwise)
  int64_t cap;     // capacity of tile_col / csc_row (debug-build checks)
};

// Zero 64 rows of D = TD floats at `rows` with a workgroup of BWD_THREADS
// (an overwriting part's rows that receive no contribution).
__device__ __forceinline__ void zero_rows64(float* rows, int tid) {
#pragma unroll
  for (int j = 0; j < BLK * TD / 4 / BWD_THREADS; ++j)
    *(f32x4*)(rows + 4 * (tid + j * BWD_THREADS)) = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Row/key permutation inside a 64-wide tile (see the forward kernel): value i
// of subtile t in lane group g is position 32*(t/2) + 8*g + 4*(t%2) + i.
__device__ __forceinline__ int pos_of(int t, int g, int i) { return 32 * (t >> 1) + 8 * g + 4 * (t & 1) + i; }
__device__ __forceinline__ int pos_row(int t, int m) { return 32 * (t >> 1) + 8 * (m >> 2) + 4 * (t & 1) + (m & 3); }

template <typename T, int D>
struct BwdTile {
  static constexpr int KP = D + (sizeof(T) == 2 ? 8 : 4);
  static constexpr int CPR = D * (int)sizeof(T) / 16;
  static constexpr int CPT = BLK * CPR / BWD_THREADS;
  static constexpr int NK = (sizeof(T) == 2) ? D / 32 : D / 4;   // contraction steps over D
  using Frag = typename std::conditional<sizeof(T) == 2, bf16x8, float>::type;
};

// Load a lane's fragment of row `row` (contraction slots of lane group g) from global.
template <typename T, int D>
__device__ __forceinline__ void load_row_frag(const T* row, int g, typename BwdTile<T, D>::Frag* f) {
  constexpr int NK = BwdTile<T, D>::NK;
  if constexpr (sizeof(T) == 2) {
    #pragma unroll
    for (int ks = 0; ks < NK; ++ks) f[ks] = *(const bf16x8*)(row + 32 * ks + 8 * g);
  } else {
    #pragma unroll
    for (int ks = 0; ks < NK; ++ks) f[ks] = row[4 * ks + g];
  }
}

// acc[t] = X_lds[pos_row(t, m)] . frag  (a 16x16 block of (X F^T)^T per subtile)
template <typename T, int D>
__device__ __forceinline__ void rows_dot_frag(const T* X, int n16, int g4,
                                              const typename BwdTile<T, D>::Frag* f, f32x4* acc) {
  constexpr int KP = BwdTile<T, D>::KP, NK = BwdTile<T, D>::NK;
  #pragma unroll
  for (int t = 0; t < 4; ++t) {
    acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const T* xr = X + pos_row(t, n16) * KP;
    if constexpr (sizeof(T) == 2) {
      #pragma unroll
      for (int ks = 0; ks < NK; ++ks) acc[t] = mfma_bf16(*(const bf16x8*)(xr + 32 * ks + 8 * g4), f[ks], acc[t]);
    } else {
      #pragma unroll
      for (int ks = 0; ks < NK; ++ks) acc[t] = mfma_f32(xr[4 * ks + g4], f[ks], acc[t]);
    }
  }
}

// out[dt] += X_lds^T(d, slots) * w  where w[t][i] weights position pos_of(t, g4, i)
// (contraction over the 64 tile positions; X row-major [64][KP]).
// For bf16 inputs the fp32 weights (P or dS) are carried as a pair of bf16
// values w = hi + lo (hi = bf16(w), lo = bf16(w - hi)), two MFMAs sharing the
// X operand: the gradient sums run over up to a whole sequence of rows, and a
// single bf16 rounding of every weight (relative 2^-9) would dominate their
// error; the pair leaves about 2^-17.
template <typename T, int D>
__device__ __forceinline__ void colsT_times(const T* X, int n16, int g4, const f32x4* w, f32x4* out) {
  constexpr int KP = BwdTile<T, D>::KP;
  if constexpr (sizeof(T) == 2) {
    bf16x8 wh[2], wl[2];
    #pragma unroll
    for (int c = 0; c < 2; ++c)
      #pragma unroll
      for (int e = 0; e < 2; ++e)
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = w[2 * c + e][i];
          const bf16 hi = (bf16)x;
          wh[c][4 * e + i] = hi;
          wl[c][4 * e + i] = (bf16)(x - (float)hi);
        }
    #pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      #pragma unroll
      for (int c = 0; c < 2; ++c) {
        const T* base = X + (32 * c + 8 * g4 + (n16 >> 2)) * KP + 16 * dt + 4 * (n16 & 3);
        const bf16x8 xa = lds_read_tr16_x2(base, KP);
        out[dt] = mfma_bf16(xa, wh[c], out[dt]);
        out[dt] = mfma_bf16(xa, wl[c], out[dt]);
      }
  } else {
    #pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      #pragma unroll
      for (int t = 0; t < 4; ++t)
        #pragma unroll
        for (int i = 0; i < 4; ++i) out[dt] = mfma_f32(X[pos_of(t, g4, i) * KP + 16 * dt + n16], w[t][i], out[dt]);
  }
}

// Stage 64 rows (given per thread chunk) of a [*, D] tensor into an LDS tile.
template <typename T, int D>
__device__ __forceinline__ void stage_rows(T* dst, const T* base, int64_t sn, const int* rows, int tid) {
  constexpr int KP = BwdTile<T, D>::KP, CPR = BwdTile<T, D>::CPR, CPT = BwdTile<T, D>::CPT;
  #pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = tid + c * BWD_THREADS;
    const int r = ch / CPR, col = (ch % CPR) * (16 / (int)sizeof(T));
    *(i32x4*)(dst + r * KP + col) = *(const i32x4*)(base + (int64_t)rows[c] * sn + col);
  }
}

// ---------------------------------------------------------------------------
// dQ: query-major. Wave w owns query rows 16w..16w+15 of block I.
template <typename T, int D>
__global__ void __launch_bounds__(BWD_THREADS) dq_kernel(BwdArgs a) {
  using Tl = BwdTile<T, D>;
  constexpr int KP = Tl::KP, CPR = Tl::CPR, CPT = Tl::CPT, NK = Tl::NK;
  __shared__ __attribute__((aligned(16))) T Ks[BLK * KP];
  __shared__ __attribute__((aligned(16))) T Vs[BLK * KP];
  __shared__ int thr_sh[BLK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, n16 = lane & 15;
  int rank_i, hh_i, g_i;
  if (!xcd_group_item(blockIdx.x, a.Hkv, a.QB, QMAJOR_BPC, a.Hq / a.Hkv, &rank_i, &hh_i, &g_i)) return;
  const int I = a.QB - 1 - rank_i;
  const int h = g_i * (a.Hq / a.Hkv) + hh_i;
  const int kvh = h / (a.Hq / a.Hkv);
  const int64_t u = (int64_t)h * a.QB + I;
  const int rowoff = wave * 16 + n16;
  const int64_t grow = (int64_t)I * BLK + rowoff;
  const int t0 = dbg_clamp(a.tile_ptr[u], 0, (int)a.cap + 1, a.dbg);
  const int nt = dbg_clamp(a.tile_ptr[u + 1] - t0, 0, min(a.KB, (int)a.cap - t0) + 1, a.dbg);
  const int ve = dbg_clamp(a.vert_end[u], 0, a.KB * BLK + 1, a.dbg);
  const int total = nt + (ve + BLK - 1) / BLK;
  if (total == 0) return;

  typename Tl::Frag qf[NK], df[NK];
  load_row_frag<T, D>((const T*)a.q + h * a.qsh + grow * a.qsn, g4, qf);
  load_row_frag<T, D>((const T*)a.dout + h * a.dsh + grow * a.dsn, g4, df);
  const float lse2 = a.lse[(int64_t)h * a.QB * BLK + grow] * LOG2E;
  const float dl = a.delta[(int64_t)h * a.QB * BLK + grow];
  const bool row_live = lse2 > -INFINITY;
  const int64_t G = global_block(a.kind, a.P, a.QB, a.rank, I);
  const int32_t* vl = a.vloc + (int64_t)h * a.KB * BLK;
  const uint32_t* sb = a.slash_bits + (int64_t)h * a.W;
  const T* kbase = (const T*)a.k + kvh * a.ksh;
  const T* vbase = (const T*)a.v + kvh * a.vsh;

  f32x4 acc[D / 16];
  #pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int it = 0; it < total; ++it) {
    int rows[CPT];
    int mode;
    if (it < nt) {
      const int e = a.tile_col[t0 + it];
      const int J = dbg_clamp(e & VS_TILE_MASK, 0, a.KB, a.dbg);
      mode = (e & VS_TILE_DIAG) ? 1 : 0;
      #pragma unroll
      for (int c = 0; c < CPT; ++c) rows[c] = J * BLK + (tid + c * BWD_THREADS) / CPR;
      if (tid < BLK) thr_sh[tid] = tid;
    } else {
      const int base = (it - nt) * BLK;
      mode = 1;
      #pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int idx = base + (tid + c * BWD_THREADS) / CPR;
        rows[c] = dbg_clamp(idx < ve ? vl[idx] : vl[base], 0, a.KB * BLK, a.dbg);
      }
      if (tid < BLK) {
        const int idx = base + tid;
        int thr = BLK;
        if (idx < ve) {
          const int m = dbg_clamp(vl[idx], 0, a.KB * BLK, a.dbg);
          const int64_t j = G - global_block(a.kind, a.P, a.KB, a.src, m / BLK);
          if (!((sb[j >> 5] >> (j & 31)) & 1u)) thr = (j == 0) ? (m % BLK) : 0;
        }
        thr_sh[tid] = thr;
      }
    }
    stage_rows<T, D>(Ks, kbase, a.ksn, rows, tid);
    stage_rows<T, D>(Vs, vbase, a.vsn, rows, tid);
    __syncthreads();
    f32x4 s[4], dp[4];
    rows_dot_frag<T, D>(Ks, n16, g4, qf, s);    // S^T: [key][row]
    rows_dot_frag<T, D>(Vs, n16, g4, df, dp);   // dP^T
    #pragma unroll
    for (int t = 0; t < 4; ++t)
      #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool act = row_live && !(mode && thr_sh[pos_of(t, g4, i)] > rowoff);
        const float p = act ? __builtin_amdgcn_exp2f(s[t][i] * a.scale_log2 - lse2) : 0.f;
        s[t][i] = p * (dp[t][i] - dl);          // dS
      }
    colsT_times<T, D>(Ks, n16, g4, s, acc);      // dQ^T += K^T dS^T
    __syncthreads();
  }
  float* out = a.dq + ((int64_t)h * a.QB * BLK + grow) * D;
  #pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    f32x4 r = *(f32x4*)(out + 16 * dt + 4 * g4);
    #pragma unroll
    for (int i = 0; i < 4; ++i) r[i] += acc[dt][i] * a.scale;
    *(f32x4*)(out + 16 * dt + 4 * g4) = r;
  }
}

// ---------------------------------------------------------------------------
// Shared core of the key-major kernels: wave w owns 16 keys (kf/vf fragments);
// the staged query block (Qs, dOs, per-row lse2/delta) is processed against
// them. thr[lane]: rows with row offset < thr are inactive for this lane's key
// (key-side causal / vertical threshold); BLK = inactive everywhere.
template <typename T, int D>
__device__ __forceinline__ void key_block_step(const T* Qs, const T* dOs, const float* lse_sh, const float* dl_sh,
                                               const typename BwdTile<T, D>::Frag* kf,
                                               const typename BwdTile<T, D>::Frag* vf, int thr, int n16, int g4,
                                               float scale_log2, f32x4* acc_dk, f32x4* acc_dv) {
  f32x4 s[4], dp[4];
  rows_dot_frag<T, D>(Qs, n16, g4, kf, s);     // S: [row][key], rows permuted
  rows_dot_frag<T, D>(dOs, n16, g4, vf, dp);   // dP
  f32x4 ds[4];
  #pragma unroll
  for (int t = 0; t < 4; ++t)
    #pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = pos_of(t, g4, i);
      const float l2 = lse_sh[r];
      const bool act = r >= thr && l2 > -INFINITY;
      const float p = act ? __builtin_amdgcn_exp2f(s[t][i] * scale_log2 - l2) : 0.f;
      s[t][i] = p;
      ds[t][i] = p * (dp[t][i] - dl_sh[r]);
    }
  colsT_times<T, D>(dOs, n16, g4, s, acc_dv);   // dV^T += dO^T P
  colsT_times<T, D>(Qs, n16, g4, ds, acc_dk);   // dK^T += Q^T dS
}

template <typename T, int D>
__device__ __forceinline__ void stage_query_block(T* Qs, T* dOs, float* lse_sh, float* dl_sh, const BwdArgs& a,
                                                  int h, int I, int tid) {
  constexpr int CPR = BwdTile<T, D>::CPR, CPT = BwdTile<T, D>::CPT;
  int rows[CPT];
  #pragma unroll
  for (int c = 0; c < CPT; ++c) rows[c] = I * BLK + (tid + c * BWD_THREADS) / CPR;
  stage_rows<T, D>(Qs, (const T*)a.q + h * a.qsh, a.qsn, rows, tid);
  stage_rows<T, D>(dOs, (const T*)a.dout + h * a.dsh, a.dsn, rows, tid);
  if (tid < BLK) {
    const int64_t r = (int64_t)h * a.QB * BLK + (int64_t)I * BLK + tid;
    lse_sh[tid] = a.lse[r] * LOG2E;
    dl_sh[tid] = a.delta[r];
  }
}

// dK/dV over slash tiles: grid = Hkv * KB, item -> (kv head, key block J).
template <typename T, int D>
__global__ void __launch_bounds__(BWD_THREADS) dkdv_kernel(BwdArgs a) {
  using Tl = BwdTile<T, D>;
  constexpr int KP = Tl::KP, NK = Tl::NK;
  __shared__ __attribute__((aligned(16))) T Qs[BLK * KP];
  __shared__ __attribute__((aligned(16))) T dOs[BLK * KP];
  __shared__ float lse_sh[BLK], dl_sh[BLK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, n16 = lane & 15;
  int J, kvh, hh_unused;
  if (!xcd_group_item(blockIdx.x, a.Hkv, a.KB, KMAJOR_BPC, 1, &J, &hh_unused, &kvh)) return;
  const int grp = a.Hq / a.Hkv;
  const int keyoff = wave * 16 + n16;
  const int64_t krow = (int64_t)J * BLK + keyoff;
  typename Tl::Frag kf[NK], vf[NK];
  load_row_frag<T, D>((const T*)a.k + kvh * a.ksh + krow * a.ksn, g4, kf);
  load_row_frag<T, D>((const T*)a.v + kvh * a.vsh + krow * a.vsn, g4, vf);
  f32x4 acc_dk[D / 16], acc_dv[D / 16];
  #pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc_dk[dt] = acc_dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  bool any = false;
  for (int hh = 0; hh < grp; ++hh) {
    const int h = kvh * grp + hh;
    const int64_t cu = (int64_t)h * a.KB + J;
    const int c0 = dbg_clamp(a.csc_ptr[cu], 0, (int)a.cap + 1, a.dbg);
    const int c1 = c0 + dbg_clamp(a.csc_ptr[cu + 1] - c0, 0, min(a.QB, (int)a.cap - c0) + 1, a.dbg);
    for (int e = c0; e < c1; ++e) {
      const int ent = a.csc_row[e];
      const int I = dbg_clamp(ent & VS_TILE_MASK, 0, a.QB, a.dbg);
      stage_query_block<T, D>(Qs, dOs, lse_sh, dl_sh, a, h, I, tid);
      __syncthreads();
      // diagonal tile: key k is active for rows >= k
      const int thr = (ent & VS_TILE_DIAG) ? keyoff : 0;
      key_block_step<T, D>(Qs, dOs, lse_sh, dl_sh, kf, vf, thr, n16, g4, a.scale_log2, acc_dk, acc_dv);
      any = true;
      __syncthreads();
    }
  }
  if (!any) return;
  float* dkr = a.dk + ((int64_t)kvh * a.KB * BLK + krow) * D;
  float* dvr = a.dv + ((int64_t)kvh * a.KB * BLK + krow) * D;
  #pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    f32x4 x = *(f32x4*)(dkr + 16 * dt + 4 * g4);
    f32x4 y = *(f32x4*)(dvr + 16 * dt + 4 * g4);
    #pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] += acc_dk[dt][i] * a.scale;
      y[i] += acc_dv[dt][i];
    }
    *(f32x4*)(dkr + 16 * dt + 4 * g4) = x;
    *(f32x4*)(dvr + 16 * dt + 4 * g4) = y;
  }
}

// dK/dV of vertical columns. Work items (h, chunk of 64 columns, query-block
// segment) are enumerated from the device-side vertical counts; a fixed grid
// strides over them and every workgroup exits after the last item.
template <typename T, int D>
__global__ void __launch_bounds__(BWD_THREADS) dkdv_vert_kernel(BwdArgs a) {
  using Tl = BwdTile<T, D>;
  constexpr int KP = Tl::KP, NK = Tl::NK;
  __shared__ __attribute__((aligned(16))) T Qs[BLK * KP];
  __shared__ __attribute__((aligned(16))) T dOs[BLK * KP];
  __shared__ float lse_sh[BLK], dl_sh[BLK];
  __shared__ int any_sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, n16 = lane & 15;
  const int nseg = (a.QB + VERT_SEG - 1) / VERT_SEG;
  auto vcnt = [&](int h) { return dbg_clamp(a.vloc_cnt[h], 0, a.KB * BLK + 1, a.dbg); };
  int64_t total = 0;
  for (int h = 0; h < a.Hq; ++h) total += (int64_t)((vcnt(h) + BLK - 1) / BLK) * nseg;
  const int grp = a.Hq / a.Hkv;
  for (int64_t w = blockIdx.x; w < total; w += gridDim.x) {
    // decode (h, chunk, seg)
    int64_t r = w;
    int h = 0;
    for (; h < a.Hq; ++h) {
      const int64_t n = (int64_t)((vcnt(h) + BLK - 1) / BLK) * nseg;
      if (r < n) break;
      r -= n;
    }
    // segments rotate with the chunk: the dispatcher deals workgroups to the
    // eight XCDs in turn, and without the rotation one XCD would get every
    // chunk's last (always full) segment
    const int chunk = (int)(r / nseg), seg = (int)((r % nseg + chunk) % nseg);
    const int kvh = h / grp;
    const int cnt = vcnt(h);
    const int32_t* vl = a.vloc + (int64_t)h * a.KB * BLK;
    const uint32_t* sb = a.slash_bits + (int64_t)h * a.W;
    const int slot = chunk * BLK + wave * 16 + n16;
    const bool valid = slot < cnt;
    const int m = dbg_clamp(vl[valid ? slot : chunk * BLK], 0, a.KB * BLK, a.dbg);
    const int64_t gb = global_block(a.kind, a.P, a.KB, a.src, m / BLK);
    typename Tl::Frag kf[NK], vf[NK];
    load_row_frag<T, D>((const T*)a.k + kvh * a.ksh + (int64_t)m * a.ksn, g4, kf);
    load_row_frag<T, D>((const T*)a.v + kvh * a.vsh + (int64_t)m * a.vsn, g4, vf);
    f32x4 acc_dk[D / 16], acc_dv[D / 16];
    #pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc_dk[dt] = acc_dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int I0 = seg * VERT_SEG, I1 = min(a.QB, I0 + VERT_SEG);
    bool touched = false;
    for (int I = I0; I < I1; ++I) {
      const int64_t G = global_block(a.kind, a.P, a.QB, a.rank, I);
      const int64_t j = G - gb;
      int thr = BLK;
      if (valid && j >= 0 && !((sb[j >> 5] >> (j & 31)) & 1u)) thr = (j == 0) ? (m % BLK) : 0;
      if (tid == 0) any_sh = 0;
      __syncthreads();
      if (thr < BLK) any_sh = 1;
      __syncthreads();
      if (!any_sh) continue;
      stage_query_block<T, D>(Qs, dOs, lse_sh, dl_sh, a, h, I, tid);
      __syncthreads();
      key_block_step<T, D>(Qs, dOs, lse_sh, dl_sh, kf, vf, thr, n16, g4, a.scale_log2, acc_dk, acc_dv);
      touched = true;
      __syncthreads();
    }
    if (touched && valid) {
      float* dkr = a.dk + ((int64_t)kvh * a.KB * BLK + m) * D;
      float* dvr = a.dv + ((int64_t)kvh * a.KB * BLK + m) * D;
      #pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
          atomicAdd(dkr + 16 * dt + 4 * g4 + i, acc_dk[dt][i] * a.scale);
          atomicAdd(dvr + 16 * dt + 4 * g4 + i, acc_dv[dt][i]);
        }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16, head dim 128 (the production path). Same tiling as the forward: 64-row
// query blocks and 64-key tiles staged in swizzled LDS tiles by asynchronous
// copies, two stages, one barrier per tile; each wave covers 32 rows x 32 keys.


// dQ, query-major. Wave (rh, kh) = rows 32 rh.. of the block, keys 32 kh.. of
// every tile; the two key halves' partial dQ are added through LDS at the end.
// dS enters the dQ product of a vertical chunk as a hi + lo pair in both
// operand formats (bf16 pair, or fp16 pair on fp16 inputs): dQ_n sums dS k_m
// over every active key of the row, and the vertical columns hold the large
// outlier keys whose terms dominate that sum (a single fp16 dS everywhere
// put dQ at 1.9e-2 of the oracle at 262144 tokens). Listed slash tiles take
// dS as one fp16 operand on the fp16 path.
// RING: the tile sequence runs over several ring steps (RingTiles, `rs`; K/V
// hold every shard in storage order) and dQ accumulates across them.
// S1 (one-position stripes): per-key thresholds and diagonal windows, as in
// the forward.
template <bool F16, bool RING = false, bool S1 = false>
__device__ __forceinline__ void dq_d128(const BwdArgs& a, const RingSteps* rs = nullptr) {
  constexpr int D = TD;
  __shared__ __attribute__((aligned(16))) bf16 K0[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 V0[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 K1[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 V1[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) int thr0_sh[BLK];
  __shared__ __attribute__((aligned(16))) int thr1_sh[BLK];
  __shared__ __attribute__((aligned(16))) uint32_t win_sh[2][S1 ? BLK : 4];
  __shared__ int desc0_sh[BLK], desc1_sh[BLK];
  __shared__ uint32_t sbits[MAX_LDS_W];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, n16 = lane & 15;
  const int rh = wave & 1, kh = wave >> 1;
  int rank_i, hh_i, g_i;
  if (!xcd_group_item(blockIdx.x, a.Hkv, a.QB, QMAJOR_BPC, a.Hq / a.Hkv, &rank_i, &hh_i, &g_i)) return;
  const int I = a.QB - 1 - rank_i;
  const int h = g_i * (a.Hq / a.Hkv) + hh_i;
  const int kvh = h / (a.Hq / a.Hkv);
  const int64_t u = (int64_t)h * a.QB + I;
  const int64_t row_base = (int64_t)I * BLK + 32 * rh;

  typename std::conditional<RING, RingTiles, BlockTiles>::type bt;
  if constexpr (RING) {
    __shared__ RingTable rtab;
    bt.rs = rs; bt.tb = &rtab; bt.sbits = sbits; bt.vl_off = (int64_t)h * a.KB * BLK;
    bt.G = global_block(a.kind, a.P, a.QB, a.rank, I);
    bt.kind = a.kind; bt.P = a.P; bt.KB = a.KB; bt.dbg = a.dbg;
    bt.fill(u, wave, lane);
    __syncthreads();
    bt.start();
  } else {
    bt.tile_col = a.tile_col; bt.vl = a.vloc + (int64_t)h * a.KB * BLK; bt.sbits = sbits;
    bt.G = global_block(a.kind, a.P, a.QB, a.rank, I);
    bt.kind = a.kind; bt.P = a.P; bt.KB = a.KB; bt.src = a.src; bt.dbg = a.dbg; bt.cap = a.cap;
    bt.init(a.tile_ptr[u], a.tile_ptr[u + 1], a.vert_end[u]);
  }
  const int total = bt.total;
  if (total == 0) {
    if (a.overwrite) zero_rows64(a.dq + ((int64_t)h * a.QB * BLK + (int64_t)I * BLK) * TD, tid);
    return;
  }
  const uint32_t* sbg = a.slash_bits + (int64_t)h * a.W;
  for (int w = tid; w < a.W; w += BWD_THREADS) sbits[w] = sbg[w];

  const char* kbase = (const char*)((const bf16*)a.k + kvh * a.ksh);
  const char* vbase = (const char*)((const bf16*)a.v + kvh * a.vsh);
  const uint32_t krb = (uint32_t)a.ksn * 2, vrb = (uint32_t)a.vsn * 2;   // row pitch in bytes
  const DmaLane dlane = dma_lane(wave, lane);
  // start the copy of tile t into (Kn, Vn); its row thresholds go to thn
  // (S1: its diagonal windows to wn)
  auto issue = [&](int t, const int* slot, bf16* Kn, bf16* Vn, int* thn, uint32_t* wn) -> int {
    int thr = tid, mode = 1;
    uint32_t win = ~0u;
    const int64_t sr0 = bt.row0(t, 1);   // the tile's shard
    const char* kb = kbase + sr0 * krb;
    const char* vb = vbase + sr0 * vrb;
    if (!bt.vert(t, 1)) {
      const int r0 = bt.tile_row(slot, mode);
      if constexpr (S1) {
        if (tid < BLK) {
          const int o = I - r0 / BLK;
          win = s1_key_window(s1_tile_window(sbits, a.W, a.P, o), a.P, a.src, tid);
          thr = s1_key_threshold(o, a.rank, a.src, tid);
        }
      }
      dma_tile_rows(Kn, kb + (int64_t)r0 * krb, krb, dlane, wave);
      dma_tile_rows(Vn, vb + (int64_t)r0 * vrb, vrb, dlane, wave);
    } else {
      int rows[4];
      if constexpr (S1) bt.vert_rows_s1(t, slot, rows, thr, win, wave, lane, tid, I, a.rank, a.W);
      else bt.vert_rows(t, slot, rows, thr, wave, lane, tid, 1);
      dma_tile_gather(Kn, kb, rows, krb, dlane, wave);
      dma_tile_gather(Vn, vb, rows, vrb, dlane, wave);
    }
    if (tid < BLK) {
      thn[tid] = thr;
      if constexpr (S1) wn[tid] = win;
    }
    return mode;
  };
  bf16x8 qf[2][4], df[2][4];
  float lse2[2], dl[2];
#pragma unroll
  for (int rs = 0; rs < 2; ++rs) {
    const int64_t grow = row_base + 16 * rs + n16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qf[rs][ks] = *(const bf16x8*)((const bf16*)a.q + h * a.qsh + grow * a.qsn + 32 * ks + 8 * g4);
      df[rs][ks] = *(const bf16x8*)((const bf16*)a.dout + h * a.dsh + grow * a.dsn + 32 * ks + 8 * g4);
    }
    // an empty row (LSE = -inf) gets +inf, so exp2(S * scale - LSE) is 0
    // for it without a per-element select
    const float lr = a.lse[(int64_t)h * a.QB * BLK + grow];
    lse2[rs] = lr == -INFINITY ? INFINITY : lr * LOG2E;
    dl[rs] = a.delta[(int64_t)h * a.QB * BLK + grow];
  }
  f32x4 acc[2][8];
#pragma unroll
  for (int rs = 0; rs < 2; ++rs)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[rs][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sl2 = a.scale_log2;
  int mode_c = 0;
  int qa_l[2] = {0, 0};   // S1: global-block offset qa of this lane's two rows
  if constexpr (S1) {
#pragma unroll
    for (int rs = 0; rs < 2; ++rs) qa_l[rs] = ((32 * rh + 16 * rs + n16) * a.P + a.rank) >> 6;
  }

  // VCH: the tile is a vertical chunk (dS as a hi + lo pair in the dQ product)
  auto step = [&]<bool VCH>(int it, const bf16* Ks, const bf16* Vs, const int* thc, const uint32_t* wc, bf16* Kn,
                            bf16* Vn, int* thn, uint32_t* wn, int* dn_next, const int* dn_cur) {
    wait_all_mem();
    __syncthreads();
    const int mode = mode_c;
    if (it + 1 < total) {
      mode_c = issue(it + 1, dn_cur, Kn, Vn, thn, wn);
      if (it + 2 < total) bt.desc_copy(it + 2, dn_next, wave, lane);
    }
    // S^T and dP^T for keys 32 kh + 8 g + 4 t + i, rows 16 rs + n of the wave
    f32x4 s[2][2], dp[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int kr = 32 * kh + 8 * (n16 >> 2) + 4 * t + (n16 & 3);
#pragma unroll
      for (int rs = 0; rs < 2; ++rs) s[rs][t] = dp[rs][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 kf = *(const bf16x8*)(Ks + tile_off(kr, 4 * ks + g4));
        const bf16x8 vf = *(const bf16x8*)(Vs + tile_off(kr, 4 * ks + g4));
#pragma unroll
        for (int rs = 0; rs < 2; ++rs) {
          s[rs][t] = mma16<F16>(kf, qf[rs][ks], s[rs][t]);
          dp[rs][t] = mma16<F16>(vf, df[rs][ks], dp[rs][t]);
        }
      }
    }
    if (mode) {   // wave-uniform: diagonal tile or vertical chunk
      // row thresholds of this lane's 8 keys (two 16-byte reads)
      const i32x4 th0 = *(const i32x4*)(thc + 32 * kh + 8 * g4);
      const i32x4 th1 = *(const i32x4*)(thc + 32 * kh + 8 * g4 + 4);
      i32x4 w0 = i32x4{-1, -1, -1, -1}, w1 = w0;
      if constexpr (S1) {
        w0 = *(const i32x4*)(wc + 32 * kh + 8 * g4);
        w1 = *(const i32x4*)(wc + 32 * kh + 8 * g4 + 4);
      }
#pragma unroll
      for (int rs = 0; rs < 2; ++rs)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            bool off = (t == 0 ? th0[i] : th1[i]) > 32 * rh + 16 * rs + n16;
            if constexpr (S1) off = off || !(((uint32_t)(t == 0 ? w0[i] : w1[i]) >> qa_l[rs]) & 1u);
            if (off) s[rs][t][i] = -INFINITY;
          }
    }
#pragma unroll
    for (int rs = 0; rs < 2; ++rs)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rs][t][i], sl2, -lse2[rs]));
          s[rs][t][i] = p * (dp[rs][t][i] - dl[rs]);
        }
    // dQ^T += K^T dS^T over this wave's 32 keys (PR: dS as a hi + lo pair);
    // the transposed K operand of block dt + 1 is read after the first MFMA
    // of block dt (two register sets: a third spills registers here)
    auto dq_product = [&]<bool PR>() {
      bf16x8 dsh[2], dsl[2];
#pragma unroll
      for (int rs = 0; rs < 2; ++rs) weights8<F16, PR>(s[rs][0], s[rs][1], dsh[rs], dsl[rs]);
      const int vr = 32 * kh + 8 * g4 + (n16 >> 2);
      bf16x8 ka[2];
      auto rdk = [&](int dt, int b) {
        const int lc = 2 * dt + ((n16 & 3) >> 1);
        ka[b] = lds_read_tr16_x2(Ks + tile_off(vr, lc) + 4 * (n16 & 1), D);
      };
      rdk(0, 0);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        if (dt + 1 < 8) rdk(dt + 1, (dt + 1) & 1);
        const int b = dt & 1;
#pragma unroll
        for (int rs = 0; rs < 2; ++rs) {
          acc[rs][dt] = mma16<F16>(ka[b], dsh[rs], acc[rs][dt]);
          if constexpr (PR) acc[rs][dt] = mma16<F16>(ka[b], dsl[rs], acc[rs][dt]);
        }
      }
      constexpr int MPB = PR ? 4 : 2;   // MFMAs per column block
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (dt + 1 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, MPB - 1, 0);
      }
    };
    dq_product.template operator()<VCH || !F16>();
  };

  bt.desc_copy(0, desc0_sh, wave, lane);
  if (total > 1) bt.desc_copy(1, desc1_sh, wave, lane);
  wait_all_mem();
  __syncthreads();
  mode_c = issue(0, desc0_sh, K0, V0, thr0_sh, win_sh[0]);
  // With fp16 operands the vertical chunks, which lead the sequence (in the
  // resident ring those of every step), take the pair and the listed tiles
  // one operand; one-position stripes keep the pair on every tile, as does
  // the bf16 operand format.
  // Stages are fixed per call site (tile parity) so the compiler can tell the
  // stage being read from the one being filled and keeps its copy wait at
  // the step's barrier.
  auto even = [&]<bool PR>(int it) {
    step.template operator()<PR>(it, K0, V0, thr0_sh, win_sh[0], K1, V1, thr1_sh, win_sh[1], desc0_sh, desc1_sh);
  };
  auto odd = [&]<bool PR>(int it) {
    step.template operator()<PR>(it, K1, V1, thr1_sh, win_sh[1], K0, V0, thr0_sh, win_sh[0], desc1_sh, desc0_sh);
  };
  auto walk = [&]<bool PR>(int it0, int it1) {
    int it = it0;
    if ((it & 1) && it < it1) odd.template operator()<PR>(it++);
    for (; it < it1; it += 2) {
      even.template operator()<PR>(it);
      if (it + 1 < it1) odd.template operator()<PR>(it + 1);
    }
  };
  if constexpr (F16 && !S1) {
    walk.template operator()<true>(0, bt.nvert());
    walk.template operator()<false>(bt.nvert(), total);
  } else {   // pairs throughout (bf16 operands, one-position stripes)
    for (int it = 0; it < total; it += 2) {
      even.template operator()<true>(it);
      if (it + 1 < total) odd.template operator()<true>(it + 1);
    }
  }
  __syncthreads();
  float* xo = (float*)(rh == 0 ? K0 : V0);   // [2 rs][8 dt][64 lanes] f32x4 per row half
  if (kh == 1) {
#pragma unroll
    for (int rs = 0; rs < 2; ++rs)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) *(f32x4*)(xo + ((rs * 8 + dt) * 64 + lane) * 4) = acc[rs][dt];
  }
  __syncthreads();
  if (kh == 1) return;
#pragma unroll
  for (int rs = 0; rs < 2; ++rs) {
    float* out = a.dq + ((int64_t)h * a.QB * BLK + row_base + 16 * rs + n16) * D;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const f32x4 o1 = *(const f32x4*)(xo + ((rs * 8 + dt) * 64 + lane) * 4);
      f32x4 r = a.overwrite ? f32x4{0.f, 0.f, 0.f, 0.f} : *(f32x4*)(out + 16 * dt + 4 * g4);
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] += (acc[rs][dt][i] + o1[i]) * a.scale;
      *(f32x4*)(out + 16 * dt + 4 * g4) = r;
    }
  }
}
__global__ void __launch_bounds__(BWD_THREADS, 2) dq_bf16_d128_kernel(BwdArgs a) { dq_d128<false>(a); }
__global__ void __launch_bounds__(BWD_THREADS, 2) dq_f16_d128_kernel(BwdArgs a) { dq_d128<true>(a); }
__global__ void __launch_bounds__(BWD_THREADS, 2) dq_s1_bf16_d128_kernel(BwdArgs a) {
  dq_d128<false, false, true>(a);
}
__global__ void __launch_bounds__(BWD_THREADS, 2) dq_s1_f16_d128_kernel(BwdArgs a) { dq_d128<true, false, true>(a); }
__global__ void __launch_bounds__(BWD_THREADS, 2) dq_ring_bf16_d128_kernel(BwdArgs a, RingSteps rs) {
  dq_d128<false, true>(a, &rs);
}
__global__ void __launch_bounds__(BWD_THREADS, 2) dq_ring_f16_d128_kernel(BwdArgs a, RingSteps rs) {
  dq_d128<true, true>(a, &rs);
}


// The two halves of kv_block, for the software-pipelined dK/dV kernel:
// kv_sdp computes S and dP of a staged tile (MFMA only); kv_grad turns them
// into P and dS (hi + lo pairs) and adds dV^T += dO^T P, dK^T += Q^T dS.
__device__ __forceinline__ void kv_frag(const bf16* Qs, const bf16* Os, int rh, int g4, int n16, bf16x8 (*qa)[4],
                                        bf16x8 (*oa)[4]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int qr = 32 * rh + 8 * (n16 >> 2) + 4 * t + (n16 & 3);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qa[t][ks] = *(const bf16x8*)(Qs + tile_off(qr, 4 * ks + g4));
      oa[t][ks] = *(const bf16x8*)(Os + tile_off(qr, 4 * ks + g4));
    }
  }
}
template <bool F16>
__device__ __forceinline__ void kv_sdp(const bf16x8 (*qa)[4], const bf16x8 (*oa)[4], const bf16x8 (*kf)[4],
                                       const bf16x8 (*vf)[4], f32x4 (*s)[2], f32x4 (*dp)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s[kt][t] = dp[kt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        s[kt][t] = mma16<F16>(qa[t][ks], kf[kt][ks], s[kt][t]);
        dp[kt][t] = mma16<F16>(oa[t][ks], vf[kt][ks], dp[kt][t]);
      }
  }
}
// The staged row LSE in log2 units, +inf for an empty row (so exp2(S * scale
// - LSE) is 0 there without a per-element select); one wave converts a
// staged tile's 64 values in place.
__device__ __forceinline__ void lse_to_log2(float* lsh, int lane) {
  const float v = lsh[lane];
  lsh[lane] = v == -INFINITY ? INFINITY : v * LOG2E;
}
// per-row lse and delta of the wave's rows 32 rh + 8 g + 4 t + i; LOG2 says
// whether the staged LSE was already converted by lse_to_log2
template <bool LOG2>
__device__ __forceinline__ void kv_rowstats(const float* lsh, const float* dsh_, int rh, int g4, f32x4* l2,
                                            f32x4* dd) {
  const int r0 = 32 * rh + 8 * g4;
  l2[0] = *(const f32x4*)(lsh + r0);
  l2[1] = *(const f32x4*)(lsh + r0 + 4);
  if constexpr (!LOG2) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) l2[t][i] = l2[t][i] == -INFINITY ? INFINITY : l2[t][i] * LOG2E;
  }
  dd[0] = *(const f32x4*)(dsh_ + r0);
  dd[1] = *(const f32x4*)(dsh_ + r0 + 4);
}
// l2: row LSE in log2 units, +inf for an empty row (kv_rowstats); on a
// masked tile key kt of this lane is active for rows >= thr[kt]. S1: and only
// for the rows 4 t + i of this lane whose global-block offset qa[4 t + i] is
// a set bit of win[kt]. MASK = 0 / 1: the tile is known unmasked / masked at
// compile time (no branch in the caller's scheduling region); MASK = 2: the
// wave-uniform `diag` decides.
template <bool F16, bool PAIR = !F16, bool S1 = false, int MASK = 2>
__device__ __forceinline__ void kv_pds(f32x4 (*s)[2], const f32x4 (*dp)[2], const f32x4* l2, const f32x4* dd,
                                       int diag, const int* thr, int rh, int g4, float sl2, bf16x8* ph,
                                       bf16x8* pl, bf16x8* dh, bf16x8* dl, const uint32_t* win = nullptr,
                                       const int* qa = nullptr) {
  const int r0 = 32 * rh + 8 * g4;
  if (MASK == 1 || (MASK == 2 && diag)) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bool off = r0 + 4 * t + i < thr[kt];
          if constexpr (S1) off = off || !((win[kt] >> qa[4 * t + i]) & 1u);
          if (off) s[kt][t][i] = -INFINITY;
        }
  }
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    f32x4 ds[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][t][i], sl2, -l2[t][i]));
        s[kt][t][i] = pr;
        ds[t][i] = pr * (dp[kt][t][i] - dd[t][i]);
      }
    weights8<F16, PAIR>(s[kt][0], s[kt][1], ph[kt], pl[kt]);
    weights8<F16, PAIR>(ds[0], ds[1], dh[kt], dl[kt]);
  }
}
template <bool F16, bool PAIR = !F16>
__device__ __forceinline__ void kv_grad(const bf16* Qs, const bf16* Os, const bf16x8* ph, const bf16x8* pl,
                                        const bf16x8* dh, const bf16x8* dl, int rh, int g4, int n16,
                                        f32x4 (*acc_dk)[8], f32x4 (*acc_dv)[8]) {
  constexpr int D = TD;
  const int rr = 32 * rh + 8 * g4 + (n16 >> 2);
  // The transposed operands of column block dt + 2 are read while the MFMAs
  // of block dt run (three register sets, order pinned below); with one set
  // every block would wait out a full LDS round trip.
  bf16x8 oT[3], qT[3];
  auto rd = [&](int dt, int b) {
    const int lc = 2 * dt + ((n16 & 3) >> 1);
    oT[b] = lds_read_tr16_x2(Os + tile_off(rr, lc) + 4 * (n16 & 1), D);
    qT[b] = lds_read_tr16_x2(Qs + tile_off(rr, lc) + 4 * (n16 & 1), D);
  };
  rd(0, 0);
  rd(1, 1);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    if (dt + 2 < 8) rd(dt + 2, (dt + 2) % 3);
    const int b = dt % 3;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      acc_dv[kt][dt] = mma16<F16>(oT[b], ph[kt], acc_dv[kt][dt]);
      if constexpr (PAIR) acc_dv[kt][dt] = mma16<F16>(oT[b], pl[kt], acc_dv[kt][dt]);
      acc_dk[kt][dt] = mma16<F16>(qT[b], dh[kt], acc_dk[kt][dt]);
      if constexpr (PAIR) acc_dk[kt][dt] = mma16<F16>(qT[b], dl[kt], acc_dk[kt][dt]);
    }
  }
  constexpr int MPB = PAIR ? 8 : 4;   // MFMAs per column block
  // reads of block dt + 2 go out after the first MFMA of block dt
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (dt + 2 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, MPB - 1, 0);
  }
}

// One staged query block against the wave's keys, without pipelining (the
// vertical-column kernel): thr[kt] = rows of the block with offset below it
// are inactive for key kt of this lane (BLK: the whole block); the LSE is
// staged in natural-log units.
template <bool F16, bool PAIR = !F16>
__device__ __forceinline__ void kv_block(const bf16* Qs, const bf16* Os, const float* lsh, const float* dsh_,
                                         const bf16x8 (*kf)[4], const bf16x8 (*vf)[4], const int* thr,
                                         int rh, int g4, int n16, float sl2, f32x4 (*acc_dk)[8],
                                         f32x4 (*acc_dv)[8]) {
  bf16x8 qa[2][4], oa[2][4];
  kv_frag(Qs, Os, rh, g4, n16, qa, oa);
  f32x4 s[2][2], dp[2][2];
  kv_sdp<F16>(qa, oa, kf, vf, s, dp);
  f32x4 l2[2], dd[2];
  kv_rowstats<false>(lsh, dsh_, rh, g4, l2, dd);
  // thresholds apply under a wave-uniform branch: most blocks have none
  const int masked = __builtin_amdgcn_ballot_w64(thr[0] != 0 || thr[1] != 0) != 0ull ? 1 : 0;
  bf16x8 ph[2], pl[2], dh[2], dl[2];
  kv_pds<F16, PAIR>(s, dp, l2, dd, masked, thr, rh, g4, sl2, ph, pl, dh, dl);
  kv_grad<F16, PAIR>(Qs, Os, ph, pl, dh, dl, rh, g4, n16, acc_dk, acc_dv);
}

// Copy the Q and dO rows of query block I of head h and its lse/delta.
__device__ __forceinline__ void stage_qblock(bf16* Qn, bf16* On, float* ln, const BwdArgs& a, int h, int I, int wave,
                                             int lane, const DmaLane& dl) {
  const int64_t r0 = (int64_t)I * BLK;
  const uint32_t qrb = (uint32_t)a.qsn * 2, orb = (uint32_t)a.dsn * 2;
  dma_tile_rows(Qn, (const char*)((const bf16*)a.q + h * a.qsh + r0 * a.qsn), qrb, dl, wave);
  dma_tile_rows(On, (const char*)((const bf16*)a.dout + h * a.dsh + r0 * a.dsn), orb, dl, wave);
  if (wave < 2) {
    const float* src = (wave == 0 ? a.lse : a.delta) + (int64_t)h * a.QB * BLK + (int64_t)I * BLK + lane;
    __builtin_amdgcn_global_load_lds((const void*)src,
                                     (__attribute__((address_space(3))) void*)(
                                         (__attribute__((address_space(3))) float*)(ln + wave * BLK)),
                                     4, 0, 0);
  }
}

// Combine the two row halves' dK/dV partials (rh = 1 -> rh = 0 through LDS)
// and add them to dk/dv (plain stores when `atomic` is 0, fp32 atomics
// otherwise; with `overwrite` the plain stores replace the old values).
// keys[kt]: output row of this lane's key kt (-1 = none).
__device__ __forceinline__ void kv_finish(float* xbuf_dk, float* xbuf_dv, f32x4 (*acc_dk)[8], f32x4 (*acc_dv)[8],
                                          float* dk, float* dv, const int64_t* keys, int kh, int rh, int lane, int g4,
                                          float scale, bool atomic, bool overwrite) {
  constexpr int D = TD;
  float* xk = xbuf_dk + kh * (2 * 8 * 64 * 4);
  float* xv = xbuf_dv + kh * (2 * 8 * 64 * 4);
  __syncthreads();
  if (rh == 1) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        *(f32x4*)(xk + ((kt * 8 + dt) * 64 + lane) * 4) = acc_dk[kt][dt];
        *(f32x4*)(xv + ((kt * 8 + dt) * 64 + lane) * 4) = acc_dv[kt][dt];
      }
  }
  __syncthreads();
  if (rh == 1) return;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    if (keys[kt] < 0) continue;
    float* kr = dk + keys[kt] * D;
    float* vr = dv + keys[kt] * D;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const f32x4 k1 = *(const f32x4*)(xk + ((kt * 8 + dt) * 64 + lane) * 4);
      const f32x4 v1 = *(const f32x4*)(xv + ((kt * 8 + dt) * 64 + lane) * 4);
      if (atomic) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          atomicAdd(kr + 16 * dt + 4 * g4 + i, (acc_dk[kt][dt][i] + k1[i]) * scale);
          atomicAdd(vr + 16 * dt + 4 * g4 + i, acc_dv[kt][dt][i] + v1[i]);
        }
      } else {
        f32x4 x = overwrite ? f32x4{0.f, 0.f, 0.f, 0.f} : *(f32x4*)(kr + 16 * dt + 4 * g4);
        f32x4 y = overwrite ? f32x4{0.f, 0.f, 0.f, 0.f} : *(f32x4*)(vr + 16 * dt + 4 * g4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] += (acc_dk[kt][dt][i] + k1[i]) * scale;
          y[i] += acc_dv[kt][dt][i] + v1[i];
        }
        *(f32x4*)(kr + 16 * dt + 4 * g4) = x;
        *(f32x4*)(vr + 16 * dt + 4 * g4) = y;
      }
    }
  }
}

// dK/dV over slash tiles: one workgroup per (kv head, key block J); walks the
// CSC lists of every q head of the group and owns the key block's dK/dV rows.
// Software pipeline over the (q head, query block) tiles of the walk: step i
// computes S and dP of tile i + 1 on the matrix cores while the vector ALU
// turns S and dP of tile i into P and dS, then adds tile i's dV and dK. Three
// (Q, dO) stages: tile i (gradient products), tile i + 1 (S, dP), tile i + 2
// (being copied). One workgroup per CU (the accumulators and K/V fragments
// take more than half the registers), so LDS has room for the third stage.
//
// RING: one launch covers several ring steps: workgroup b belongs to step
// b / (gridDim.x / nsteps) (a whole number of XCD rounds per step), reads
// that step's CSC lists and writes the dK/dV rows of its visible shard in
// tensors that hold every shard in storage order (as K/V do).
//
// S1 (one-position stripes): keys of a flagged tile carry a causal threshold
// and a window of diagonals (as in the forward), built per tile from the
// tile's q head's slash bitmap.
template <bool F16, bool RING = false, bool S1 = false>
__device__ __forceinline__ void dkdv_d128(const BwdArgs& a0, const RingStepsKV* rk = nullptr) {
  BwdArgs a = a0;
  int b = blockIdx.x;
  int64_t srow0 = 0, kv_hrows = (int64_t)a0.KB * BLK;   // shard's first row; rows per kv head
  if constexpr (RING) {
    const int per = gridDim.x / rk->nsteps;
    const int st = b / per;
    b -= st * per;
    a.csc_ptr = rk->csc_ptr[st]; a.csc_row = rk->csc_row[st]; a.vloc = rk->vloc[st]; a.vcum = rk->vcum[st];
    a.src = rk->src[st];
    srow0 = (int64_t)a.src * a.KB * BLK;
    kv_hrows = (int64_t)a.P * a.KB * BLK;
  }
  __shared__ __attribute__((aligned(16))) bf16 QO0[2 * TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 QO1[2 * TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 QO2[2 * TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) float L0[2 * BLK];
  __shared__ __attribute__((aligned(16))) float L1[2 * BLK];
  __shared__ __attribute__((aligned(16))) float L2[2 * BLK];
  __shared__ int desc_sh[3][BLK];   // CSC entry of tile t in slot t % 3 (the copy fills all 64 words)
  __shared__ int head_sh[3];        // q head (within the group) of tile t in slot t % 3
  auto QOst = [&]<int p>() -> bf16* {
    if constexpr (p == 0) return QO0;
    else if constexpr (p == 1) return QO1;
    else return QO2;
  };
  auto Lst = [&]<int p>() -> float* {
    if constexpr (p == 0) return L0;
    else if constexpr (p == 1) return L1;
    else return L2;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const DmaLane dlane = dma_lane(wave, lane);
  const int g4 = lane >> 4, n16 = lane & 15;
  const int kh = wave >> 1, rh = wave & 1;
  int J, kvh, hh_unused;
  if (!xcd_group_item(b, a.Hkv, a.KB, KMAJOR_BPC, 1, &J, &hh_unused, &kvh)) return;
  const int grp = a.Hq / a.Hkv;
  // The walk is the concatenation of the group's q heads' CSC lists for this
  // key block. Per-head ranges sit in lanes 0 .. grp-1 and are read back with
  // readlane by a wave-uniform head index (an SGPR array indexed at run time
  // compiles into compare/select chains).
  int cst_l = 0, cnt_l = 0;
  if (lane < grp) {
    const int64_t cu = (int64_t)(kvh * grp + lane) * a.KB + J;
    cst_l = dbg_clamp(a.csc_ptr[cu], 0, (int)a.cap + 1, a.dbg);
    cnt_l = dbg_clamp(a.csc_ptr[cu + 1] - cst_l, 0, min(a.QB, (int)a.cap - cst_l) + 1, a.dbg);
  }
  int total = 0;
  for (int hh = 0; hh < grp; ++hh) total += __builtin_amdgcn_readlane(cnt_l, hh);
  // Vertical columns are left to the vertical-column kernel over every query
  // block (with hi + lo weights there), so this kernel drops them from its
  // tiles: lane hh < grp holds the 64-bit set of key block J's columns that
  // are verticals of the group's q head hh.
  uint32_t vm_lo_l = 0, vm_hi_l = 0;
  if (lane < grp) {
    const int64_t hq = kvh * grp + lane;
    const int32_t* vc = a.vcum + hq * (a.KB + 1);
    const int32_t* vl = a.vloc + hq * a.KB * BLK;
    const int e0 = dbg_clamp(vc[J], 0, a.KB * BLK + 1, a.dbg);
    const int e1 = e0 + dbg_clamp(vc[J + 1] - e0, 0, a.KB * BLK - e0 + 1, a.dbg);
    for (int e = e0; e < e1; ++e) {
      const int b = vl[e] & (BLK - 1);
      if (b < 32) vm_lo_l |= 1u << b;
      else vm_hi_l |= 1u << (b - 32);
    }
  }
  if (total == 0) {
    if (a.overwrite) {
      const int64_t r0 = ((int64_t)kvh * kv_hrows + srow0 + (int64_t)J * BLK) * TD;
      zero_rows64(a.dk + r0, tid);
      zero_rows64(a.dv + r0, tid);
    }
    return;
  }
  // per-head row-0 offsets (bytes) of Q and dO, and of the head's lse / delta rows
  const int64_t q_off_l = lane < grp ? (int64_t)(kvh * grp + lane) * a.qsh * 2 : 0;
  const int64_t o_off_l = lane < grp ? (int64_t)(kvh * grp + lane) * a.dsh * 2 : 0;
  auto rl64 = [&](int64_t v, int hh) -> int64_t {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)(uint64_t)v, hh);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)v >> 32), hh);
    return (int64_t)(((uint64_t)hi << 32) | lo);
  };
  // cursor (head, position) of the next descriptor copy; copies are issued
  // for walk positions 0, 1, 2, ... in order
  int cur_h = 0, cur_p = 0;
  auto cur_skip = [&]() {
    while (cur_h < grp && cur_p >= __builtin_amdgcn_readlane(cnt_l, cur_h)) {
      ++cur_h;
      cur_p = 0;
    }
  };
  cur_skip();
  auto desc_copy = [&](int it) {
    if (wave == 0) {
      const int e = __builtin_amdgcn_readlane(cst_l, cur_h) + cur_p;
      __builtin_amdgcn_global_load_lds((const void*)(a.csc_row + e),
                                       (__attribute__((address_space(3))) void*)(
                                           (__attribute__((address_space(3))) int*)(desc_sh[it % 3])),
                                       4, 0, 0);
      if (lane == 0) head_sh[it % 3] = cur_h;   // the walk position's q head
    }
    ++cur_p;
    cur_skip();
  };
  // start the copy of tile t into stage p; returns its diagonal flag (bit 0),
  // its q head within the group (bits 1..3) and, S1, its query block (bits 4..)
  auto issue = [&]<int p>(int t) -> int {
    const int e = __builtin_amdgcn_readfirstlane(desc_sh[t % 3][0]);
    const int hh = __builtin_amdgcn_readfirstlane(head_sh[t % 3]);
    const int I = dbg_clamp(e & VS_TILE_MASK, 0, a.QB, a.dbg);
    bf16* qo = QOst.template operator()<p>();
    float* ls = Lst.template operator()<p>();
    const int64_t r0 = (int64_t)I * BLK;
    const uint32_t qrb = (uint32_t)a.qsn * 2, orb = (uint32_t)a.dsn * 2;
    dma_tile_rows(qo, (const char*)a.q + rl64(q_off_l, hh) + r0 * qrb, qrb, dlane, wave);
    dma_tile_rows(qo + TILE_ELEMS, (const char*)a.dout + rl64(o_off_l, hh) + r0 * orb, orb, dlane, wave);
    if (wave < 2) {
      const float* src = (wave == 0 ? a.lse : a.delta) + (int64_t)(kvh * grp + hh) * a.QB * BLK + r0 + lane;
      __builtin_amdgcn_global_load_lds((const void*)src,
                                       (__attribute__((address_space(3))) void*)(
                                           (__attribute__((address_space(3))) float*)(ls + wave * BLK)),
                                       4, 0, 0);
    }
    return ((e & VS_TILE_DIAG) ? 1 : 0) | (hh << 1) | (S1 ? (I << 4) : 0);
  };
  int qa_r[8] = {};   // S1: global-block offset qa of this lane's eight rows
  if constexpr (S1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) qa_r[j] = ((32 * rh + 8 * g4 + j) * a.P + a.rank) >> 6;
  }

  bf16x8 kf[2][4], vf[2][4];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int64_t krow = srow0 + (int64_t)J * BLK + 32 * kh + 16 * kt + n16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      kf[kt][ks] = *(const bf16x8*)((const bf16*)a.k + kvh * a.ksh + krow * a.ksn + 32 * ks + 8 * g4);
      vf[kt][ks] = *(const bf16x8*)((const bf16*)a.v + kvh * a.vsh + krow * a.vsn + 32 * ks + 8 * g4);
    }
  }
  f32x4 acc_dk[2][8], acc_dv[2][8];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc_dk[kt][dt] = acc_dv[kt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sl2 = a.scale_log2;
  f32x4 s_c[2][2], dp_c[2][2];
  int diag_c = 0, diag_n1 = 0;

  // step i (stage p = i % 3): S/dP of tile i in (s_c, dp_c); tile i + 1 is
  // in stage p + 1, tile i + 2's descriptor in slot (i + 2) % 3.
  auto step = [&]<int p>(int i) {
    constexpr int p1 = (p + 1) % 3, p2 = (p + 2) % 3;
    wait_all_mem();
    __syncthreads();   // tile i + 1 and descriptor i + 2 have landed; step i - 1 is done everywhere
    const int diag_i = diag_c;
    int diag_n2 = 0;
    if (i + 2 < total) diag_n2 = issue.template operator()<p2>(i + 2);
    if (i + 3 < total) desc_copy(i + 3);
    // S, dP of tile i + 1 (the last step computes them from a stale stage and
    // drops them): fragments and this tile's row statistics are read first, so
    // the region below holds only MFMAs and vector ops, interleaved one MFMA
    // per six vector ops
    const bf16* Qn = QOst.template operator()<p1>();
    bf16x8 qa[2][4], oa[2][4];
    kv_frag(Qn, Qn + TILE_ELEMS, rh, g4, n16, qa, oa);
    // tile i + 1's LSE has landed: wave 0 converts it for step i + 1
    if (wave == 0) lse_to_log2(Lst.template operator()<p1>(), lane);
    f32x4 l2[2], dd[2];
    const float* Lc = Lst.template operator()<p>();
    kv_rowstats<true>(Lc, Lc + BLK, rh, g4, l2, dd);
    // key kt of this lane is active for rows >= thr[kt]: its index on the
    // diagonal tile, 0 elsewhere, and never (BLK) for a vertical of the head
    const int hh_i = S1 ? (diag_i >> 1) & 7 : diag_i >> 1;
    const uint32_t vlo = __builtin_amdgcn_readlane(vm_lo_l, hh_i), vhi = __builtin_amdgcn_readlane(vm_hi_l, hh_i);
    int thr[2];
    uint32_t win[2] = {~0u, ~0u};
    if constexpr (S1) {
      const int o = (diag_i >> 4) - J;
      const uint64_t tw = s1_tile_window(a.slash_bits + (int64_t)(kvh * grp + hh_i) * a.W, a.W, a.P, o);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int key = 32 * kh + 16 * kt + n16;
        const bool vert = ((kh ? vhi : vlo) >> (16 * kt + n16)) & 1u;
        win[kt] = s1_key_window(tw, a.P, a.src, key);
        thr[kt] = vert ? BLK : s1_key_threshold(o, a.rank, a.src, key);
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int key = 32 * kh + 16 * kt + n16;
        const bool vert = ((kh ? vhi : vlo) >> (16 * kt + n16)) & 1u;
        thr[kt] = vert ? BLK : ((diag_i & 1) ? key : 0);
      }
    }
    const int masked = ((diag_i & 1) || vlo || vhi) ? 1 : 0;
    __builtin_amdgcn_sched_barrier(0);
    f32x4 s_n[2][2], dp_n[2][2];
    bf16x8 ph[2], pl[2], dh[2], dl[2];
    // the MFMAs of S, dP (tile i + 1) and the vector ops of P, dS (tile i)
    // form one branch-free region per case (a branch inside it would split
    // the interleave and leave the MFMAs and the exponentials back to back)
    auto sdp_pds = [&]<int MASK>() {
      kv_sdp<F16>(qa, oa, kf, vf, s_n, dp_n);
      kv_pds<F16, !F16, S1, MASK>(s_c, dp_c, l2, dd, 0, thr, rh, g4, sl2, ph, pl, dh, dl, win, qa_r);
      constexpr int VPM = F16 ? 4 : 6;   // vector ops per MFMA (fp16 weights need one convert per pair)
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    if (masked) sdp_pds.template operator()<1>();
    else sdp_pds.template operator()<0>();
    const bf16* Qc = QOst.template operator()<p>();
    kv_grad<F16>(Qc, Qc + TILE_ELEMS, ph, pl, dh, dl, rh, g4, n16, acc_dk, acc_dv);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        s_c[kt][t] = s_n[kt][t];
        dp_c[kt][t] = dp_n[kt][t];
      }
    diag_c = diag_n1;
    diag_n1 = diag_n2;
  };

#pragma unroll
  for (int t = 0; t < 3; ++t)
    if (t < total) desc_copy(t);
  wait_all_mem();
  __syncthreads();
  diag_c = issue.template operator()<0>(0);
  if (total > 1) diag_n1 = issue.template operator()<1>(1);
  wait_all_mem();
  __syncthreads();
  if (wave == 0) lse_to_log2(L0, lane);   // tile 0's LSE, seen after step 0's barrier
  {
    bf16x8 qa[2][4], oa[2][4];
    kv_frag(QO0, QO0 + TILE_ELEMS, rh, g4, n16, qa, oa);
    kv_sdp<F16>(qa, oa, kf, vf, s_c, dp_c);
  }
  for (int i0 = 0; i0 < total; i0 += 3) {
    step.template operator()<0>(i0);
    if (i0 + 1 < total) step.template operator()<1>(i0 + 1);
    if (i0 + 2 < total) step.template operator()<2>(i0 + 2);
  }
  int64_t keys[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
    keys[kt] = (int64_t)kvh * kv_hrows + srow0 + (int64_t)J * BLK + 32 * kh + 16 * kt + n16;
  wait_all_mem();
  kv_finish((float*)QO0, (float*)QO1, acc_dk, acc_dv, a.dk, a.dv, keys, kh, rh, lane, g4, a.scale, false,
            a.overwrite != 0);
}
__global__ void __launch_bounds__(BWD_THREADS, 1) dkdv_bf16_d128_kernel(BwdArgs a) { dkdv_d128<false>(a); }
__global__ void __launch_bounds__(BWD_THREADS, 1) dkdv_f16_d128_kernel(BwdArgs a) { dkdv_d128<true>(a); }
__global__ void __launch_bounds__(BWD_THREADS, 1) dkdv_s1_bf16_d128_kernel(BwdArgs a) {
  dkdv_d128<false, false, true>(a);
}
__global__ void __launch_bounds__(BWD_THREADS, 1) dkdv_s1_f16_d128_kernel(BwdArgs a) {
  dkdv_d128<true, false, true>(a);
}
__global__ void __launch_bounds__(BWD_THREADS, 1) dkdv_ring_bf16_d128_kernel(BwdArgs a, RingStepsKV rk) {
  dkdv_d128<false, true>(a, &rk);
}
__global__ void __launch_bounds__(BWD_THREADS, 1) dkdv_ring_f16_d128_kernel(BwdArgs a, RingStepsKV rk) {
  dkdv_d128<true, true>(a, &rk);
}

// dK/dV of vertical columns: work items (head, 64-column chunk of the shard's
// verticals, range of VERT_SEG query blocks) enumerated from the device-side
// counts; a fixed grid strides over them. Query blocks before the chunk's
// first column are skipped; within the range every block is processed with
// per-key thresholds (causal edge, columns covered by a listed tile).
// Results are added with fp32 atomics (a column can be a vertical of several
// q heads of the group). A vertical column sums P and dS over up to every row
// of the sequence and of the group's q heads, so the weights always enter as
// hi + lo pairs (fp16 pairs on fp16 operands): one rounding of each weight
// to fp16 leaves an error that grows with the square root of that count and
// reached 0.1 in dV on the outlier columns of the 131072-token layer.
//
// RING: the work items of several ring steps in one launch (each step's
// verticals in its visible shard, written to tensors holding every shard).
// S1 (one-position stripes): the causal rows of a column follow from its
// global position l P + src.
template <bool F16, bool RING = false, bool S1 = false>
__device__ __forceinline__ void dkdv_vert_d128(const BwdArgs& a, const RingStepsKV* rk = nullptr) {
  __shared__ __attribute__((aligned(16))) bf16 QO0[2 * TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 QO1[2 * TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) float L0[2 * BLK];
  __shared__ __attribute__((aligned(16))) float L1[2 * BLK];
  bf16* Q0 = QO0;
  bf16* O0 = QO0 + TILE_ELEMS;
  bf16* Q1 = QO1;
  bf16* O1 = QO1 + TILE_ELEMS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const DmaLane dlane = dma_lane(wave, lane);
  const int g4 = lane >> 4, n16 = lane & 15;
  const int kh = wave >> 1, rh = wave & 1;
  // Query-block range per item: VERT_SEG blocks, halved (down to
  // VERT_SEG_MIN) while there are fewer than VERT_ITEMS_MIN items, so a ring
  // step with few vertical columns still spreads over the whole GPU instead
  // of walking long ranges in a few workgroups. Every workgroup derives the
  // same partition from the device-side counts.
  // per step: its chunks of 64 verticals over all heads (steps in LDS)
  __shared__ int step_chunks[RING ? MAX_RING_STEPS : 1];
  const int nst = RING ? rk->nsteps : 1;
  auto vcnt_of = [&](int st) -> const int32_t* {
    if constexpr (RING) return rk->vloc_cnt[st];
    else return a.vloc_cnt;
  };
  if (tid < nst) {
    int c = 0;
    for (int h = 0; h < a.Hq; ++h) c += (dbg_clamp(vcnt_of(tid)[h], 0, a.KB * BLK + 1, a.dbg) + BLK - 1) / BLK;
    step_chunks[tid] = c;
  }
  __syncthreads();
  int64_t nchunks = 0;
  for (int st = 0; st < nst; ++st) nchunks += step_chunks[st];
  int seg_len = VERT_SEG;
  while (seg_len > VERT_SEG_MIN && nchunks * ((a.QB + seg_len - 1) / seg_len) < VERT_ITEMS_MIN) seg_len >>= 1;
  const int nseg = (a.QB + seg_len - 1) / seg_len;
  const int64_t nwork = nchunks * nseg;
  const int grp = a.Hq / a.Hkv;
  const float sl2 = a.scale_log2;
  const int64_t kv_hrows = (int64_t)(RING ? a.P : 1) * a.KB * BLK;   // rows per kv head of k, v, dk, dv
  for (int64_t w = blockIdx.x; w < nwork; w += gridDim.x) {
    int64_t r = w;
    int st = 0;
    for (; st + 1 < nst; ++st) {
      const int64_t n = (int64_t)step_chunks[st] * nseg;
      if (r < n) break;
      r -= n;
    }
    const int32_t* vloc_cnt = vcnt_of(st);
    const int32_t* vloc = a.vloc;
    int src = a.src;
    if constexpr (RING) {
      vloc = rk->vloc[st];
      src = rk->src[st];
    }
    const int64_t srow0 = RING ? (int64_t)src * a.KB * BLK : 0;
    auto vcnt = [&](int hq) { return dbg_clamp(vloc_cnt[hq], 0, a.KB * BLK + 1, a.dbg); };
    int h = 0;
    for (; h < a.Hq; ++h) {
      const int64_t n = (int64_t)((vcnt(h) + BLK - 1) / BLK) * nseg;
      if (r < n) break;
      r -= n;
    }
    // segments rotate with the chunk: the dispatcher deals workgroups to the
    // eight XCDs in turn, and without the rotation one XCD would get every
    // chunk's last (always full) segment
    const int chunk = (int)(r / nseg), seg = (int)((r % nseg + chunk) % nseg);
    const int kvh = h / grp;
    const int cnt = vcnt(h);
    const int32_t* vl = vloc + (int64_t)h * a.KB * BLK;
    int I_first;   // the first query block with a row at or below the chunk's first column
    if constexpr (S1) {
      I_first = s1_first_qblock((int64_t)dbg_clamp(vl[chunk * BLK], 0, a.KB * BLK, a.dbg) * a.P + src, a.rank, a.P);
    } else {
      const int64_t gb_min = global_block(a.kind, a.P, a.KB, src, dbg_clamp(vl[chunk * BLK], 0, a.KB * BLK, a.dbg) / BLK);
      I_first = blocks_upto(a.kind, a.P, a.QB, a.rank, gb_min - 1);
    }
    const int I_lo = max(seg * seg_len, I_first);
    const int I_hi = min(a.QB, (seg + 1) * seg_len);
    const int total = I_hi - I_lo;
    if (total <= 0) continue;
    __syncthreads();  // the previous item's exchange has been read
    int m[2];
    int64_t gbk[2];
    bool valid[2];
    bf16x8 kf[2][4], vf[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int slot = chunk * BLK + 32 * kh + 16 * kt + n16;
      valid[kt] = slot < cnt;
      m[kt] = dbg_clamp(vl[valid[kt] ? slot : chunk * BLK], 0, a.KB * BLK, a.dbg);
      gbk[kt] = S1 ? (int64_t)m[kt] * a.P + src : global_block(a.kind, a.P, a.KB, src, m[kt] / BLK);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        kf[kt][ks] = *(const bf16x8*)((const bf16*)a.k + kvh * a.ksh + (srow0 + m[kt]) * a.ksn + 32 * ks + 8 * g4);
        vf[kt][ks] = *(const bf16x8*)((const bf16*)a.v + kvh * a.vsh + (srow0 + m[kt]) * a.vsn + 32 * ks + 8 * g4);
      }
    }
    f32x4 acc_dk[2][8], acc_dv[2][8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc_dk[kt][dt] = acc_dv[kt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto step = [&](int it, const bf16* Qs, const bf16* Os, const float* Ls, bf16* Qn, bf16* On, float* Ln) {
      wait_all_mem();
      __syncthreads();
      if (it + 1 < total) stage_qblock(Qn, On, Ln, a, h, I_lo + it + 1, wave, lane, dlane);
      int thr[2];
      if constexpr (S1) {   // gbk: the column's global position
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) thr[kt] = valid[kt] ? s1_causal_row(gbk[kt], a.rank, a.P, I_lo + it) : BLK;
      } else {
        const int64_t G = global_block(a.kind, a.P, a.QB, a.rank, I_lo + it);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          // every causal row of the column, inside listed tiles too (the slash
          // kernel leaves vertical columns out of its tiles)
          const int64_t j = G - gbk[kt];
          thr[kt] = BLK;
          if (valid[kt] && j >= 0) thr[kt] = (j == 0) ? (m[kt] % BLK) : 0;
        }
      }
      kv_block<F16, true>(Qs, Os, Ls, Ls + BLK, kf, vf, thr, rh, g4, n16, sl2, acc_dk, acc_dv);
    };
    stage_qblock(Q0, O0, L0, a, h, I_lo, wave, lane, dlane);
    for (int it = 0; it < total; it += 2) {
      step(it, Q0, O0, L0, Q1, O1, L1);
      if (it + 1 < total) step(it + 1, Q1, O1, L1, Q0, O0, L0);
    }
    int64_t keys[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) keys[kt] = valid[kt] ? (int64_t)kvh * kv_hrows + srow0 + m[kt] : -1;
    kv_finish((float*)QO0, (float*)QO1, acc_dk, acc_dv, a.dk, a.dv, keys, kh, rh, lane, g4, a.scale, true, false);
  }
}
__global__ void __launch_bounds__(BWD_THREADS, 1) dkdv_vert_bf16_d128_kernel(BwdArgs a) { dkdv_vert_d128<false>(a); }
__global__ void __launch_bounds__(BWD_THREADS, 1) dkdv_vert_f16_d128_kernel(BwdArgs a) { dkdv_vert_d128<true>(a); }
__global__ void __launch_bounds__(BWD_THREADS, 1) dkdv_vert_s1_bf16_d128_kernel(BwdArgs a) {
  dkdv_vert_d128<false, false, true>(a);
}
__global__ void __launch_bounds__(BWD_THREADS, 1) dkdv_vert_s1_f16_d128_kernel(BwdArgs a) {
  dkdv_vert_d128<true, false, true>(a);
}
__global__ void __launch_bounds__(BWD_THREADS, 1) dkdv_vert_ring_bf16_d128_kernel(BwdArgs a, RingStepsKV rk) {
  dkdv_vert_d128<false, true>(a, &rk);
}
__global__ void __launch_bounds__(BWD_THREADS, 1) dkdv_vert_ring_f16_d128_kernel(BwdArgs a, RingStepsKV rk) {
  dkdv_vert_d128<true, true>(a, &rk);
}

// ---------------------------------------------------------------------------
// delta[row] = dO[row] . O[row]; D/4 threads per row.
template <typename T>
__global__ void bwd_prep_kernel(const float* o, const T* dout, int64_t dsh, int64_t dsn, int64_t Nq, int64_t rows,
                                int D, float* delta) {
  const int per = D / 4;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t r = t / per;
  const int c = (int)(t % per) * 4;
  float x = 0.f;
  if (r < rows) {
    const int64_t h = r / Nq, n = r % Nq;
    const f32x4 ov = *(const f32x4*)(o + r * D + c);
    const T* dr = dout + h * dsh + n * dsn + c;
    #pragma unroll
    for (int i = 0; i < 4; ++i) x += ov[i] * to_f32(dr[i]);
  }
    for (int off = per / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  if (r < rows && c == 0) delta[r] = x;
}

int launch_bwd_prep(const float* o, int dtype, TView dout, int Hq, int64_t Nq, int D, float* delta,
                    hipStream_t stream) {
  const int64_t rows = (int64_t)Hq * Nq;
  const int64_t n = rows * (D / 4);
  const int tpb = 256;
  const dim3 grid((unsigned)((n + tpb - 1) / tpb));
  if (dtype == VS_F16)
    hipLaunchKernelGGL(bwd_prep_kernel<_Float16>, grid, dim3(tpb), 0, stream, o, (const _Float16*)dout.ptr, dout.sh,
                       dout.sn, Nq, rows, D, delta);
  else if (dtype == VS_BF16)
    hipLaunchKernelGGL(bwd_prep_kernel<bf16>, grid, dim3(tpb), 0, stream, o, (const bf16*)dout.ptr, dout.sh, dout.sn,
                       Nq, rows, D, delta);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<float>, grid, dim3(tpb), 0, stream, o, (const float*)dout.ptr, dout.sh,
                       dout.sn, Nq, rows, D, delta);
  return hipGetLastError() == hipSuccess ? VS_OK : VS_ERR_HIP;
}

// delta[row] = dO[row] . O[row] from bf16 dO, writing the fp16 copy of dO
// on the way (one read of dO instead of one for the copy and one for delta).
// A value with a biased bf16 exponent >= 127 + 16 (|x| >= 65536, inf, NaN)
// sets *status = VS_ERR_RANGE.
__global__ void bwd_prep_f16_kernel(const float* o, const uint16_t* dout, uint16_t* dout16, int64_t rows, int D,
                                    float* delta, int32_t* status) {
  const int per = D / 4;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t r = t / per;
  const int c = (int)(t % per) * 4;
  float x = 0.f;
  bool bad = false;
  if (r < rows) {
    const f32x4 ov = *(const f32x4*)(o + r * D + c);
    typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
    const u32x2 w = *(const u32x2*)(dout + r * D + c);
    u32x2 h;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t e0 = (w[j] >> 7) & 0xffu, e1 = (w[j] >> 23) & 0xffu;
      bad |= (e0 >= 143u) | (e1 >= 143u);
      const float f0 = __builtin_bit_cast(float, w[j] << 16), f1 = __builtin_bit_cast(float, w[j] & 0xffff0000u);
      x += ov[2 * j] * f0;       // same accumulation order as bwd_prep_kernel
      x += ov[2 * j + 1] * f1;
      h[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{f0, f1}, f16x2));
    }
    *(u32x2*)(dout16 + r * D + c) = h;
  }
  for (int off = per / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  if (r < rows && c == 0) delta[r] = x;
  if (bad) *status = VS_ERR_RANGE;
}

int launch_bwd_prep_f16(const float* o, const void* dout, void* dout16, int Hq, int64_t Nq, int D, float* delta,
                        int32_t* status, hipStream_t stream) {
  const int64_t rows = (int64_t)Hq * Nq;
  const int64_t n = rows * (D / 4);
  const int tpb = 256;
  hipLaunchKernelGGL(bwd_prep_f16_kernel, dim3((unsigned)((n + tpb - 1) / tpb)), dim3(tpb), 0, stream, o,
                     (const uint16_t*)dout, (uint16_t*)dout16, rows, D, delta, status);
  return hipGetLastError() == hipSuccess ? VS_OK : VS_ERR_HIP;
}

// n floats (a multiple of 4) set to zero
__global__ void zero_f32_kernel(float* p, int64_t n) {
  for (int64_t i = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x); i < n; i += 4 * (int64_t)gridDim.x * blockDim.x)
    *(f32x4*)(p + i) = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <typename T, int D>
static void launch_bwd_typed(const BwdArgs& a, int parts, hipStream_t stream) {
  if (parts & VS_BWD_OVERWRITE) {   // these kernels add: clear their outputs first
    const int64_t nq = (int64_t)a.Hq * a.QB * BLK * D, nk = (int64_t)a.Hkv * a.KB * BLK * D;
    if (parts & VS_BWD_DQ) hipLaunchKernelGGL(zero_f32_kernel, dim3(1024), dim3(256), 0, stream, a.dq, nq);
    if (parts & VS_BWD_DKDV) {
      hipLaunchKernelGGL(zero_f32_kernel, dim3(1024), dim3(256), 0, stream, a.dk, nk);
      hipLaunchKernelGGL(zero_f32_kernel, dim3(1024), dim3(256), 0, stream, a.dv, nk);
    }
  }
  if (parts & VS_BWD_DQ)
    hipLaunchKernelGGL((dq_kernel<T, D>), dim3(xcd_group_grid(a.Hkv, a.QB, QMAJOR_BPC, a.Hq / a.Hkv)), dim3(BWD_THREADS), 0, stream, a);
  if (parts & VS_BWD_DKDV)
    hipLaunchKernelGGL((dkdv_kernel<T, D>), dim3(xcd_group_grid(a.Hkv, a.KB, KMAJOR_BPC, 1)), dim3(BWD_THREADS), 0, stream, a);
  if (parts & VS_BWD_DKDV_VERT)
    hipLaunchKernelGGL((dkdv_vert_kernel<T, D>), dim3(VERT_GRID), dim3(BWD_THREADS), 0, stream, a);
}

int launch_attn_bwd(int dtype, int D, TView q, TView k, TView v, TView dout, const float* lse,
                    const float* delta, const vs_mask* m, float scale, float* dq, float* dk, float* dv,
                    int parts, hipStream_t stream) {
  BwdArgs a;
  a.q = q.ptr; a.k = k.ptr; a.v = v.ptr; a.dout = dout.ptr;
  a.qsh = q.sh; a.qsn = q.sn; a.ksh = k.sh; a.ksn = k.sn; a.vsh = v.sh; a.vsn = v.sn;
  a.dsh = dout.sh; a.dsn = dout.sn;
  a.lse = lse; a.delta = delta;
  a.tile_ptr = m->tile_ptr; a.tile_col = m->tile_col; a.csc_ptr = m->csc_ptr; a.csc_row = m->csc_row;
  a.vloc = m->vloc; a.vloc_cnt = m->vloc_cnt; a.vcum = m->vcum; a.vert_end = m->vert_end;
  a.slash_bits = m->slash_bits;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.Hq = m->Hq; a.Hkv = m->Hkv; a.QB = m->QB; a.KB = m->KB; a.W = m->W; a.kind = m->lay.kind;
  a.P = m->lay.P; a.rank = m->rank; a.src = m->src;
  a.scale = scale; a.scale_log2 = scale * LOG2E;
  a.dbg = debug_word(); a.cap = m->tile_cap;
  a.overwrite = 0;
  if ((dtype == VS_BF16 || dtype == VS_F16) && D == 128) {
    const bool f16 = dtype == VS_F16;
    a.overwrite = (parts & VS_BWD_OVERWRITE) ? 1 : 0;
    if (m->W > MAX_LDS_W) return VS_ERR_UNSUPPORTED;
    const int64_t krows = (int64_t)m->KB * BLK, qrows = (int64_t)m->QB * BLK;
    if (!dma_offsets_fit(krows, k.sn) || !dma_offsets_fit(krows, v.sn) || !dma_offsets_fit(qrows, q.sn) ||
        !dma_offsets_fit(qrows, dout.sn))
      return VS_ERR_UNSUPPORTED;
    if (a.Hq / a.Hkv > 8) return VS_ERR_UNSUPPORTED;
    const dim3 qgrid(xcd_group_grid(a.Hkv, a.QB, QMAJOR_BPC, a.Hq / a.Hkv)), kgrid(xcd_group_grid(a.Hkv, a.KB, KMAJOR_BPC, 1));
    const bool s1 = m->lay.kind == VS_STRIPED1;
    if (parts & VS_BWD_DQ)
      hipLaunchKernelGGL(s1 ? (f16 ? dq_s1_f16_d128_kernel : dq_s1_bf16_d128_kernel)
                            : (f16 ? dq_f16_d128_kernel : dq_bf16_d128_kernel),
                         qgrid, dim3(BWD_THREADS), 0, stream, a);
    if (parts & VS_BWD_DKDV)
      hipLaunchKernelGGL(s1 ? (f16 ? dkdv_s1_f16_d128_kernel : dkdv_s1_bf16_d128_kernel)
                            : (f16 ? dkdv_f16_d128_kernel : dkdv_bf16_d128_kernel),
                         kgrid, dim3(BWD_THREADS), 0, stream, a);
    if (parts & VS_BWD_DKDV_VERT)
      hipLaunchKernelGGL(s1 ? (f16 ? dkdv_vert_s1_f16_d128_kernel : dkdv_vert_s1_bf16_d128_kernel)
                            : (f16 ? dkdv_vert_f16_d128_kernel : dkdv_vert_bf16_d128_kernel),
                         dim3(VERT_GRID), dim3(BWD_THREADS), 0, stream, a);
  }
  else if (m->lay.kind == VS_STRIPED1) return VS_ERR_UNSUPPORTED;   // one-position stripes: D = 128 only
  else if (dtype == VS_BF16 && D == 64) launch_bwd_typed<bf16, 64>(a, parts, stream);
  else if (dtype == VS_F32 && D == 64) launch_bwd_typed<float, 64>(a, parts, stream);
  else return VS_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? VS_OK : VS_ERR_HIP;
}

// Several ring steps of one rank per launch (groups of up to MAX_RING_STEPS):
// k, v, dk, dv hold every shard in storage order (shard r at rows
// r * KB * 64). dQ accumulates over the steps of a group; with
// VS_BWD_OVERWRITE the first group writes dq (later groups add to it) and
// every group writes its visible shards' dk/dv rows (the vertical part then
// adds to them).
int launch_attn_bwd_ring(int dtype, TView q, TView k, TView v, TView dout, const float* lse, const float* delta,
                         const vs_mask* ms, int nsteps, float scale, float* dq, float* dk, float* dv, int parts,
                         hipStream_t stream) {
  const vs_mask* m = &ms[0];
  if (dtype != VS_BF16 && dtype != VS_F16) return VS_ERR_UNSUPPORTED;
  if (m->W > MAX_LDS_W || m->Hq / m->Hkv > 8) return VS_ERR_UNSUPPORTED;
  // 32-bit copy offsets: over every shard for K/V (the dQ kernel's vertical
  // chunks gather storage rows), over the rank's rows for Q/dO
  const int64_t krows = (int64_t)m->lay.P * m->KB * BLK, qrows = (int64_t)m->QB * BLK;
  if (!dma_offsets_fit(krows, k.sn) || !dma_offsets_fit(krows, v.sn) || !dma_offsets_fit(qrows, q.sn) ||
      !dma_offsets_fit(qrows, dout.sn))
    return VS_ERR_UNSUPPORTED;
  BwdArgs a;
  a.q = q.ptr; a.k = k.ptr; a.v = v.ptr; a.dout = dout.ptr;
  a.qsh = q.sh; a.qsn = q.sn; a.ksh = k.sh; a.ksn = k.sn; a.vsh = v.sh; a.vsn = v.sn;
  a.dsh = dout.sh; a.dsn = dout.sn;
  a.lse = lse; a.delta = delta;
  a.tile_ptr = nullptr; a.tile_col = nullptr; a.csc_ptr = nullptr; a.csc_row = nullptr;
  a.vloc = nullptr; a.vloc_cnt = nullptr; a.vcum = nullptr; a.vert_end = nullptr;
  a.slash_bits = m->slash_bits;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.Hq = m->Hq; a.Hkv = m->Hkv; a.QB = m->QB; a.KB = m->KB; a.W = m->W; a.kind = m->lay.kind;
  a.P = m->lay.P; a.rank = m->rank; a.src = -1;
  a.scale = scale; a.scale_log2 = scale * LOG2E;
  a.dbg = debug_word(); a.cap = m->tile_cap;
  const bool f16 = dtype == VS_F16;
  const unsigned qgrid = xcd_group_grid(a.Hkv, a.QB, QMAJOR_BPC, a.Hq / a.Hkv);
  const unsigned kgrid = xcd_group_grid(a.Hkv, a.KB, KMAJOR_BPC, 1);
  for (int s0 = 0; s0 < nsteps; s0 += MAX_RING_STEPS) {
    const int ns = nsteps - s0 < MAX_RING_STEPS ? nsteps - s0 : MAX_RING_STEPS;
    RingSteps rs{};
    RingStepsKV rk{};
    rs.nsteps = rk.nsteps = ns;
    rs.cap = m->tile_cap;
    for (int s = 0; s < ns; ++s) {
      const vs_mask& x = ms[s0 + s];
      rs.tile_ptr[s] = x.tile_ptr; rs.tile_col[s] = x.tile_col; rs.vloc[s] = x.vloc; rs.vert_end[s] = x.vert_end;
      rs.src[s] = x.src;
      rk.csc_ptr[s] = x.csc_ptr; rk.csc_row[s] = x.csc_row; rk.vloc[s] = x.vloc; rk.vloc_cnt[s] = x.vloc_cnt;
      rk.vcum[s] = x.vcum; rk.src[s] = x.src;
    }
    // dq: the first group may overwrite, later groups add; dk/dv: every
    // group's shards are its own (a rank sees each shard at one step), so
    // the overwrite holds for every group
    a.overwrite = (s0 == 0 && (parts & VS_BWD_OVERWRITE)) ? 1 : 0;
    if (parts & VS_BWD_DQ)
      hipLaunchKernelGGL(f16 ? dq_ring_f16_d128_kernel : dq_ring_bf16_d128_kernel, dim3(qgrid), dim3(BWD_THREADS), 0,
                         stream, a, rs);
    a.overwrite = (parts & VS_BWD_OVERWRITE) ? 1 : 0;
    if (parts & VS_BWD_DKDV)
      hipLaunchKernelGGL(f16 ? dkdv_ring_f16_d128_kernel : dkdv_ring_bf16_d128_kernel, dim3(kgrid * ns),
                         dim3(BWD_THREADS), 0, stream, a, rk);
    if (parts & VS_BWD_DKDV_VERT)
      hipLaunchKernelGGL(f16 ? dkdv_vert_ring_f16_d128_kernel : dkdv_vert_ring_bf16_d128_kernel, dim3(VERT_GRID),
                         dim3(BWD_THREADS), 0, stream, a, rk);
  }
  return hipGetLastError() == hipSuccess ? VS_OK : VS_ERR_HIP;
}

}  // namespace vs
