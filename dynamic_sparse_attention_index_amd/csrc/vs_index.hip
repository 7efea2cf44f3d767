// Online sparse-index approximation on the GPU.
//
// MTraining review, page 1, section 三.2 item 1: the last queries are scored
// against the keys, cumulative attention statistics are formed along the
// vertical (column) and slash (diagonal) directions, and the minimum number of
// verticals and slashes that recall the target attention mass is estimated;
// item 2: verticals at token level, slashes aggregated over 64x64 blocks.
// The budget is the "online top-p" of section 五.
//
// Passes:
//   1. rowstat  -- per kv head and key range, the (max, sum exp) of every scored
//                  row of every q head of the group (one K read, MFMA, exp);
//   2. combine  -- the row log-sum-exp;
//   3. colsum   -- recompute the logits, P = exp(z - LSE), column sums per q
//                  head = vertical mass v(m); block sums of v = slash mass s(j)
//                  (the scored rows lie in the last 64-block, so diagonal j
//                  collects exactly key block T-1-j);
//   4. select   -- per head, exact top-p by radix select on the fp32 bit
//                  patterns with fixed-point mass histograms, then ascending
//                  compaction.
#include <algorithm>
#include <type_traits>

#include "vs_common.h"
#include "vs_internal.h"

namespace vs {

// Key-range splits per pass: about IDX_WAVE_TARGET waves over all q heads
// (one wave per q head and split), i.e. two waves per SIMD on 256 CUs
// whatever the group size (one wave per SIMD leaves the exponentials and the
// scoring MFMAs of a wave to run back to back).
constexpr int IDX_WAVE_TARGET = 2048;
__host__ inline int64_t idx_nsplit(int Hq, int64_t ntiles) {
  return std::min<int64_t>(ntiles, std::max<int64_t>(1, IDX_WAVE_TARGET / Hq));
}

struct IndexArgs {
  const void* q; const void* k;
  int64_t qsh, qsn, ksh, ksn;
  int Hq, Hkv, last_q, kind, P, NB, T, nsplit, tiles_per;
  // tiles walked by passes 1 and 3: all T (k holds every shard, storage
  // order) or, for one rank's share, the NB tiles of rank `rank_fixed`
  // (k holds that shard only); rank_fixed < 0 for the first case
  int ntiles, rank_fixed;
  int64_t n_global;
  float scale_log2;
  float* part;       // [Hq, 64, nsplit, 2]
  float* lse2;       // [Hq, 64] (log2 domain)
  float* vert; float* slash;
  // combine pass: partial (max, sum) pair s of row t at
  // cmb_in[(t * cmb_tstride + s * cmb_sstride) * 2], s < cmb_n; writes lse2,
  // or (max, sum) of the row to cmb_stats when that is set
  const float* cmb_in; int cmb_n; int64_t cmb_tstride, cmb_sstride;
  float* cmb_stats;
};

template <typename T, int D>
struct IdxTile {
  static constexpr int KP = D + (sizeof(T) == 2 ? 8 : 4);
  static constexpr int CPR = D * (int)sizeof(T) / 16;
  static constexpr int NK = (sizeof(T) == 2) ? D / 32 : D / 4;
  using Frag = typename std::conditional<sizeof(T) == 2, bf16x8, float>::type;
};

// One wave holds the 64 scored rows of its q head as A operands (4 subtiles of
// 16 rows) and multiplies them with the staged 64-key tile: acc[rs][kt] lane
// (g, n) = S[row 16 rs + 4 g + i][key 16 kt + n].
template <typename T, int D>
__device__ __forceinline__ void score_tile(const T* Ks, const typename IdxTile<T, D>::Frag (*qa)[IdxTile<T, D>::NK],
                                           int n16, int g4, f32x4 (*acc)[4]) {
  constexpr int KP = IdxTile<T, D>::KP, NK = IdxTile<T, D>::NK;
  #pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const T* kr = Ks + (16 * kt + n16) * KP;
    typename IdxTile<T, D>::Frag kb[NK];
    if constexpr (sizeof(T) == 2) {
      #pragma unroll
      for (int ks = 0; ks < NK; ++ks) kb[ks] = *(const bf16x8*)(kr + 32 * ks + 8 * g4);
    } else {
      #pragma unroll
      for (int ks = 0; ks < NK; ++ks) kb[ks] = kr[4 * ks + g4];
    }
    #pragma unroll
    for (int rs = 0; rs < 4; ++rs) {
      acc[rs][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      #pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        if constexpr (sizeof(T) == 2) acc[rs][kt] = mfma_bf16(qa[rs][ks], kb[ks], acc[rs][kt]);
        else acc[rs][kt] = mfma_f32(qa[rs][ks], kb[ks], acc[rs][kt]);
      }
    }
  }
}

template <typename T, int D>
__device__ __forceinline__ void load_q_rows(const IndexArgs& a, int h, int n16, int g4,
                                            typename IdxTile<T, D>::Frag (*qa)[IdxTile<T, D>::NK]) {
  constexpr int NK = IdxTile<T, D>::NK;
  #pragma unroll
  for (int rs = 0; rs < 4; ++rs) {
    const int r = 16 * rs + n16;
    const T* qr = (const T*)a.q + h * a.qsh + (int64_t)r * a.qsn;
    #pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      if constexpr (sizeof(T) == 2) {
        qa[rs][ks] = r < a.last_q ? *(const bf16x8*)(qr + 32 * ks + 8 * g4) : bf16x8{};
      } else {
        qa[rs][ks] = r < a.last_q ? qr[4 * ks + g4] : 0.f;
      }
    }
  }
}

// Stage key tile `tau` (storage order) of kv head `kvh` into LDS; returns its global block.
template <typename T, int D>
__device__ __forceinline__ int64_t stage_key_tile(T* Ks, const IndexArgs& a, int kvh, int tau, int tid, int nthr) {
  constexpr int KP = IdxTile<T, D>::KP, CPR = IdxTile<T, D>::CPR;
  const T* kb = (const T*)a.k + kvh * a.ksh + (int64_t)tau * BLK * a.ksn;
  for (int ch = tid; ch < BLK * CPR; ch += nthr) {
    const int r = ch / CPR, col = (ch % CPR) * (16 / (int)sizeof(T));
    *(i32x4*)(Ks + r * KP + col) = *(const i32x4*)(kb + (int64_t)r * a.ksn + col);
  }
  if (a.rank_fixed >= 0) return global_block(a.kind, a.P, a.NB, a.rank_fixed, tau);
  return global_block(a.kind, a.P, a.NB, tau / a.NB, tau % a.NB);
}

// The same copy split in two, for workgroups of at least BLK * CPR / KPF_N
// threads: key_tile_load issues the global loads of tile `tau` into
// registers (they stay in flight while the current tile is scored), and
// key_tile_store writes them to LDS.
constexpr int KPF_N = 4;
template <typename T, int D>
__device__ __forceinline__ void key_tile_load(i32x4* r, const IndexArgs& a, int kvh, int tau, int tid, int nthr) {
  constexpr int CPR = IdxTile<T, D>::CPR;
  const T* kb = (const T*)a.k + kvh * a.ksh + (int64_t)tau * BLK * a.ksn;
#pragma unroll
  for (int j = 0; j < KPF_N; ++j) {
    const int ch = tid + j * nthr;
    if (ch < BLK * CPR) {
      const int row = ch / CPR, col = (ch % CPR) * (16 / (int)sizeof(T));
      r[j] = *(const i32x4*)(kb + (int64_t)row * a.ksn + col);
    }
  }
}
template <typename T, int D>
__device__ __forceinline__ void key_tile_store(T* Ks, const i32x4* r, int tid, int nthr) {
  constexpr int KP = IdxTile<T, D>::KP, CPR = IdxTile<T, D>::CPR;
#pragma unroll
  for (int j = 0; j < KPF_N; ++j) {
    const int ch = tid + j * nthr;
    if (ch < BLK * CPR) *(i32x4*)(Ks + (ch / CPR) * KP + (ch % CPR) * (16 / (int)sizeof(T))) = r[j];
  }
}
__device__ __forceinline__ int64_t key_tile_block(const IndexArgs& a, int tau) {
  if (a.rank_fixed >= 0) return global_block(a.kind, a.P, a.NB, a.rank_fixed, tau);
  return global_block(a.kind, a.P, a.NB, tau / a.NB, tau % a.NB);
}

// Pass 1: grid (nsplit, Hkv), 64 * group threads (one wave per q head).
template <typename T, int D>
__global__ void __launch_bounds__(512) index_rowstat_kernel(IndexArgs a) {
  using Tl = IdxTile<T, D>;
  __shared__ __attribute__((aligned(16))) T Ks[BLK * Tl::KP];
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, n16 = lane & 15;
  const int kvh = blockIdx.y, grp = a.Hq / a.Hkv, h = kvh * grp + wave;
  typename Tl::Frag qa[4][Tl::NK];
  load_q_rows<T, D>(a, h, n16, g4, qa);
  const int row0 = BLK - a.last_q;          // row offset of scored row 0 in the last block
  float m[4][4], l[4][4];
  #pragma unroll
  for (int rs = 0; rs < 4; ++rs)
    #pragma unroll
    for (int i = 0; i < 4; ++i) { m[rs][i] = -INFINITY; l[rs][i] = 0.f; }
  const int tau0 = blockIdx.x * a.tiles_per;
  const int tau1 = min(a.ntiles, tau0 + a.tiles_per);
  // with enough threads, the next tile's loads are issued before this tile
  // is scored (wave-uniform choice)
  const bool pf = nthr * KPF_N >= BLK * Tl::CPR;
  i32x4 kreg[KPF_N];
  if (pf && tau0 < tau1) key_tile_load<T, D>(kreg, a, kvh, tau0, tid, nthr);
  for (int tau = tau0; tau < tau1; ++tau) {
    int64_t G;
    if (pf) {
      key_tile_store<T, D>(Ks, kreg, tid, nthr);
      G = key_tile_block(a, tau);
    } else {
      G = stage_key_tile<T, D>(Ks, a, kvh, tau, tid, nthr);
    }
    __syncthreads();
    if (pf && tau + 1 < tau1) key_tile_load<T, D>(kreg, a, kvh, tau + 1, tid, nthr);
    f32x4 acc[4][4];
    score_tile<T, D>(Ks, qa, n16, g4, acc);
    const bool last = G == a.T - 1;
    if (!last && a.last_q == BLK) {
      // no masked entry in this tile (wave-uniform): the running maximum is
      // taken on the raw scores (scale > 0 keeps their order) and every
      // exponential is one fused multiply-add away from its score
      #pragma unroll
      for (int rs = 0; rs < 4; ++rs)
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float tmax = fmaxf(fmaxf(acc[rs][0][i], acc[rs][1][i]), fmaxf(acc[rs][2][i], acc[rs][3][i])) *
                             a.scale_log2;
          if (tmax > m[rs][i]) {
            l[rs][i] *= __builtin_amdgcn_exp2f(m[rs][i] - tmax);
            m[rs][i] = tmax;
          }
          #pragma unroll
          for (int kt = 0; kt < 4; ++kt)
            l[rs][i] += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[rs][kt][i], a.scale_log2, -m[rs][i]));
        }
      __syncthreads();
      continue;
    }
    #pragma unroll
    for (int rs = 0; rs < 4; ++rs)
      #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rs + 4 * g4 + i;
        float x[4], tmax = -INFINITY;
        #pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          float z = acc[rs][kt][i] * a.scale_log2;
          if (r >= a.last_q || (last && 16 * kt + n16 > row0 + r)) z = -INFINITY;
          x[kt] = z;
          tmax = fmaxf(tmax, z);
        }
        if (tmax > m[rs][i]) {
          l[rs][i] *= __builtin_amdgcn_exp2f(m[rs][i] - tmax);
          m[rs][i] = tmax;
        }
        if (m[rs][i] > -INFINITY)
          #pragma unroll
          for (int kt = 0; kt < 4; ++kt) l[rs][i] += __builtin_amdgcn_exp2f(x[kt] - m[rs][i]);
      }
    __syncthreads();
  }
  // combine the 16 key lanes of each row
  #pragma unroll
  for (int rs = 0; rs < 4; ++rs)
    #pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mm = m[rs][i], ll = l[rs][i];
      #pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const float mo = __shfl_xor(mm, off, 64), lo = __shfl_xor(ll, off, 64);
        const float mn = fmaxf(mm, mo);
        const float base = mn == -INFINITY ? 0.f : mn;
        ll = ll * __builtin_amdgcn_exp2f(mm - base) + lo * __builtin_amdgcn_exp2f(mo - base);
        mm = mn;
      }
      if (n16 == 0) {
        const int r = 16 * rs + 4 * g4 + i;
        float* p = a.part + (((int64_t)h * BLK + r) * a.nsplit + blockIdx.x) * 2;
        p[0] = mm;
        p[1] = ll;
      }
    }
}

// Pass 2: one wave per (q head, row); lanes stride over the partial pairs
// (key-range splits, or ranks).
constexpr int COMB_THREADS = 256;
__global__ void __launch_bounds__(COMB_THREADS) index_combine_kernel(IndexArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (COMB_THREADS / 64) + (threadIdx.x >> 6);
  if (t >= a.Hq * BLK) return;
  const float* p = a.cmb_in + (int64_t)t * a.cmb_tstride * 2;
  const int64_t ss = a.cmb_sstride * 2;
  float mm = -INFINITY;
  for (int s = lane; s < a.cmb_n; s += 64) mm = fmaxf(mm, p[s * ss]);
  #pragma unroll
  for (int off = 32; off > 0; off >>= 1) mm = fmaxf(mm, __shfl_xor(mm, off, 64));
  float ll = 0.f;
  if (mm > -INFINITY)
    for (int s = lane; s < a.cmb_n; s += 64) ll += p[s * ss + 1] * __builtin_amdgcn_exp2f(p[s * ss] - mm);
  #pragma unroll
  for (int off = 32; off > 0; off >>= 1) ll += __shfl_xor(ll, off, 64);
  if (lane == 0) {
    if (a.cmb_stats) {
      a.cmb_stats[2 * t] = mm;
      a.cmb_stats[2 * t + 1] = ll;
    } else {
      a.lse2[t] = ll > 0.f ? mm + log2f(ll) : -INFINITY;
    }
  }
}

// Pass 3: grid (nsplit, Hkv); vertical mass per key and slash mass per block.
template <typename T, int D>
__global__ void __launch_bounds__(512) index_colsum_kernel(IndexArgs a) {
  using Tl = IdxTile<T, D>;
  __shared__ __attribute__((aligned(16))) T Ks[BLK * Tl::KP];
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, n16 = lane & 15;
  const int kvh = blockIdx.y, grp = a.Hq / a.Hkv, h = kvh * grp + wave;
  typename Tl::Frag qa[4][Tl::NK];
  load_q_rows<T, D>(a, h, n16, g4, qa);
  float lse[4][4];
  #pragma unroll
  for (int rs = 0; rs < 4; ++rs)
    #pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rs + 4 * g4 + i;
      lse[rs][i] = r < a.last_q ? a.lse2[h * BLK + r] : -INFINITY;
    }
  const int row0 = BLK - a.last_q;
  const float inv_rows = 1.f / (float)a.last_q;
  const int tau0 = blockIdx.x * a.tiles_per;
  const int tau1 = min(a.ntiles, tau0 + a.tiles_per);
  // with enough threads, the next tile's loads are issued before this tile
  // is scored (wave-uniform choice)
  const bool pf = nthr * KPF_N >= BLK * Tl::CPR;
  i32x4 kreg[KPF_N];
  if (pf && tau0 < tau1) key_tile_load<T, D>(kreg, a, kvh, tau0, tid, nthr);
  for (int tau = tau0; tau < tau1; ++tau) {
    int64_t G;
    if (pf) {
      key_tile_store<T, D>(Ks, kreg, tid, nthr);
      G = key_tile_block(a, tau);
    } else {
      G = stage_key_tile<T, D>(Ks, a, kvh, tau, tid, nthr);
    }
    __syncthreads();
    if (pf && tau + 1 < tau1) key_tile_load<T, D>(kreg, a, kvh, tau + 1, tid, nthr);
    f32x4 acc[4][4];
    score_tile<T, D>(Ks, qa, n16, g4, acc);
    const bool last = G == a.T - 1;
    // no masked entry in this tile (wave-uniform): every scored row is live
    // (its LSE is finite) and no key lies beyond it
    const bool plain = !last && a.last_q == BLK;
    float col[4];
    #pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      float c = 0.f;
      if (plain) {
        #pragma unroll
        for (int rs = 0; rs < 4; ++rs)
          #pragma unroll
          for (int i = 0; i < 4; ++i)
            c += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[rs][kt][i], a.scale_log2, -lse[rs][i]));
      } else {
        #pragma unroll
        for (int rs = 0; rs < 4; ++rs)
          #pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * rs + 4 * g4 + i;
            const bool act = lse[rs][i] > -INFINITY && !(last && 16 * kt + n16 > row0 + r);
            if (act) c += __builtin_amdgcn_exp2f(acc[rs][kt][i] * a.scale_log2 - lse[rs][i]);
          }
      }
      c += __shfl_xor(c, 16, 64);
      c += __shfl_xor(c, 32, 64);
      col[kt] = c * inv_rows;
    }
    if (g4 == 0)
      #pragma unroll
      for (int kt = 0; kt < 4; ++kt) a.vert[(int64_t)h * a.n_global + G * BLK + 16 * kt + n16] = col[kt];
    float bs = col[0] + col[1] + col[2] + col[3];
    #pragma unroll
    for (int off = 1; off < 16; off <<= 1) bs += __shfl_xor(bs, off, 64);
    if (lane == 0) a.slash[(int64_t)h * a.T + (a.T - 1 - G)] = bs;
    __syncthreads();
  }
}

// ---- exact budget selection -------------------------------------------------
// Radix select on the fp32 bit patterns of one (head, direction)'s scores
// (non-negative: bit order = value order), each digit weighted by its
// fixed-point mass (top-p) or by one (fixed count), spread over many
// workgroups: a pass is one launch of per-chunk histograms (LDS, then merged
// into a global histogram with 64-bit atomics) and one launch that scans the
// global histogram and fixes the digit. Digits: bits 31-20, 19-8, 7-0. Then a
// count launch and a write launch compact the kept indices in ascending
// order. The joint budget runs one selection per head over both directions:
// they share the histogram and state of direction 0, and in the pooled order
// the vertical ties come before the slash ties.
constexpr int SEL_CHUNK = 4096;              // scores per workgroup
constexpr int SEL_WG = 256;                  // threads of the chunk kernels
constexpr int SEL_PER = SEL_CHUNK / SEL_WG;  // scores per thread
constexpr int SEL_BINS = 4096;               // 12-bit digits
constexpr int SCAN_THREADS = 1024;           // one thread per 4 bins

struct SelState {
  unsigned long long rem;     // mass still to collect at or below the fixed prefix
  unsigned long long k_tie;   // after the last pass: ties at the cutoff to keep
  uint32_t prefix;            // fixed high bits of the cutoff pattern
  int mode;                   // 0: selecting, 1: keep every index, 2: keep none
  int pad[2];
};

enum { BUDGET_TOP_P = 0, BUDGET_TOP_K = 1, BUDGET_JOINT = 2 };

struct SelectArgs {
  const float* vert; const float* slash;
  int32_t *vert_idx, *vert_cnt, *slash_idx, *slash_cnt;
  int64_t n_vert; int n_slash;
  float top_p;
  int budget;                 // BUDGET_*
  int k_vert, k_slash;        // counts of the fixed-count budget
  unsigned long long* hist;   // [Hq][2][SEL_BINS]
  SelState* state;            // [Hq][2]
  int* counts;                // [Hq][2][max_chunks][2]: (above the cutoff, at it)
  int max_chunks;
};

// round_half_even(x * 2^40) for a non-negative fp32 x <= 2^23, in integers:
// x = m * 2^(E - 150) with the 24-bit significand m (E = 1 for subnormals),
// so x * 2^40 = m * 2^(E - 110): a left shift, or a right shift rounded half
// to even. Equal to rint((double)x * 2^40) for every such x (checked
// exhaustively on the host); no fp64 arithmetic or f64 -> u64 conversion.
__device__ __forceinline__ uint64_t fixed_mass(float x) {
  const uint32_t b = __float_as_uint(x);
  const uint32_t e = b >> 23, f = b & 0x7FFFFFu;
  const uint64_t m = e ? (uint64_t)(f | 0x800000u) : (uint64_t)f;
  const int sh = (e ? (int)e : 1) - 110;
  if (sh >= 0) return m << sh;
  const int r = -sh;
  if (r >= 64) return 0;
  const uint64_t q = m >> r, rem = m & ((1ull << r) - 1), half = 1ull << (r - 1);
  return q + ((rem > half || (rem == half && (q & 1))) ? 1u : 0u);
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
  #pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
  #pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// the scores of (h, dir), their count and outputs
struct SelView {
  const float* x; int32_t* out; int32_t* cnt; int n;
};
__device__ __forceinline__ SelView sel_view(const SelectArgs& a, int h, int dir) {
  SelView v;
  if (dir == 0) {
    v.x = a.vert + h * a.n_vert; v.out = a.vert_idx + h * a.n_vert; v.cnt = a.vert_cnt + h; v.n = (int)a.n_vert;
  } else {
    v.x = a.slash + (int64_t)h * a.n_slash; v.out = a.slash_idx + (int64_t)h * a.n_slash; v.cnt = a.slash_cnt + h;
    v.n = a.n_slash;
  }
  return v;
}

// the histogram / state slot a (head, direction) selects with
__device__ __forceinline__ int sel_slot(const SelectArgs& a, int h, int dir) {
  return a.budget == BUDGET_JOINT ? 2 * h : 2 * h + dir;
}

__device__ __forceinline__ void sel_digit_bits(int pass, int& shift, int& width) {
  shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
  width = pass == 2 ? 8 : 12;
}

// grid (Hq, 2): clear the global histogram, set the mode
__global__ void __launch_bounds__(SEL_WG) sel_init_kernel(SelectArgs a) {
  const int hd = blockIdx.x * 2 + blockIdx.y;
  unsigned long long* gh = a.hist + (int64_t)hd * SEL_BINS;
  for (int b = threadIdx.x; b < SEL_BINS; b += SEL_WG) gh[b] = 0;
  if (threadIdx.x == 0) {
    SelState s{};
    if (a.budget == BUDGET_TOP_K) {
      const int64_t n = blockIdx.y ? a.n_slash : a.n_vert;
      const int k = blockIdx.y ? a.k_slash : a.k_vert;
      s.mode = k >= n ? 1 : (k > 0 ? 0 : 2);
      s.rem = k > 0 ? (unsigned long long)k : 0ull;
    } else {
      s.mode = a.top_p >= 1.f ? 1 : (a.top_p > 0.f ? 0 : 2);
    }
    a.state[hd] = s;
  }
}

// grid (max_chunks, Hq, 2): histogram of one chunk's scores that carry the
// fixed prefix, by the pass's digit, merged into the global histogram
__global__ void __launch_bounds__(SEL_WG) sel_hist_kernel(SelectArgs a, int pass) {
  __shared__ unsigned long long lh[SEL_BINS];
  const int h = blockIdx.y, dir = blockIdx.z, hd = sel_slot(a, h, dir);
  const SelView v = sel_view(a, h, dir);
  const int c0 = blockIdx.x * SEL_CHUNK;
  if (c0 >= v.n) return;
  const SelState st = a.state[hd];
  if (st.mode != 0) return;
  const bool by_count = a.budget == BUDGET_TOP_K;
  int shift, width;
  sel_digit_bits(pass, shift, width);
  const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + width));
  const uint32_t dmask = (1u << width) - 1u;
  const int tid = threadIdx.x;
  for (int b = tid; b < SEL_BINS; b += SEL_WG) lh[b] = 0;
  uint32_t bits[SEL_PER];
  #pragma unroll
  for (int k = 0; k < SEL_PER; ++k) {
    const int i = c0 + tid + k * SEL_WG;
    bits[k] = i < v.n ? __float_as_uint(v.x[i]) : 0xFFFFFFFFu;
  }
  __syncthreads();
  #pragma unroll
  for (int k = 0; k < SEL_PER; ++k) {
    const int i = c0 + tid + k * SEL_WG;
    if (i < v.n && (bits[k] & hi_mask) == st.prefix)
      atomicAdd(&lh[(bits[k] >> shift) & dmask],
                by_count ? 1ull : (unsigned long long)fixed_mass(__uint_as_float(bits[k])));
  }
  __syncthreads();
  unsigned long long* gh = a.hist + (int64_t)hd * SEL_BINS;
  for (int b = tid; b < SEL_BINS; b += SEL_WG)
    if (lh[b]) atomicAdd(&gh[b], lh[b]);
}

// grid (Hq, 2): scan the global histogram for the pass's digit. With the
// suffix mass S(b) = sum of bins b' >= b, the digit is the largest b >= 1
// with S(b) >= rem (0 if none) and the mass above it leaves the budget. The
// histogram is cleared for the next pass (and the next call).
__global__ void __launch_bounds__(SCAN_THREADS) sel_scan_kernel(SelectArgs a, int pass) {
  __shared__ unsigned long long wsum[SCAN_THREADS / 64];
  __shared__ int wcnt[SCAN_THREADS / 64];
  __shared__ unsigned long long wab[SCAN_THREADS / 64];
  if (a.budget == BUDGET_JOINT && blockIdx.y) return;
  const int hd = blockIdx.x * 2 + blockIdx.y;
  const SelState st = a.state[hd];
  if (st.mode != 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NW = SCAN_THREADS / 64;
  int shift, width;
  sel_digit_bits(pass, shift, width);
  const int nbins = 1 << width;
  unsigned long long* gh = a.hist + (int64_t)hd * SEL_BINS;
  // thread t holds bins 4t .. 4t + 3
  unsigned long long v[4];
  #pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = 4 * tid + j;
    v[j] = b < nbins ? gh[b] : 0ull;
  }
  #pragma unroll
  for (int j = 0; j < 4; ++j) gh[4 * tid + j] = 0;
  const unsigned long long loc = v[0] + v[1] + v[2] + v[3];
  // suffix sums over threads: within the wave, then across waves
  unsigned long long suf = loc;
  #pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long t = __shfl_down(suf, off, 64);
    if (lane + off < 64) suf += t;
  }
  if (lane == 0) wsum[wave] = suf;
  __syncthreads();
  unsigned long long above_waves = 0, total = 0;
  #pragma unroll
  for (int w = 0; w < NW; ++w) {
    total += wsum[w];
    if (w > wave) above_waves += wsum[w];
  }
  unsigned long long rem = st.rem;   // the fixed-count budget sets it at init
  if (pass == 0 && a.budget != BUDGET_TOP_K) {
    const unsigned long long pq = (unsigned long long)__builtin_rint((double)a.top_p * 4294967296.0);
    const unsigned __int128 prod = (unsigned __int128)pq * total;
    rem = (unsigned long long)((prod + 0xFFFFFFFFull) >> 32);   // ceil(pq * total / 2^32)
    if (rem == 0) {
      if (tid == 0) a.state[hd].mode = 2;
      return;
    }
  }
  unsigned long long s = above_waves + suf - loc;   // mass of the bins above this thread's
  int c = 0;
  #pragma unroll
  for (int j = 3; j >= 0; --j) {
    s += v[j];   // S(4 t + j)
    c += (4 * tid + j >= 1 && s >= rem) ? 1 : 0;
  }
  c = wave_sum_i32(c);
  if (lane == 0) wcnt[wave] = c;
  __syncthreads();
  int bstar = 0;
  #pragma unroll
  for (int w = 0; w < NW; ++w) bstar += wcnt[w];
  unsigned long long ab = 0;
  #pragma unroll
  for (int j = 0; j < 4; ++j) ab += (4 * tid + j > bstar) ? v[j] : 0ull;
  ab = wave_sum_u64(ab);
  if (lane == 0) wab[wave] = ab;
  __syncthreads();
  if (tid == 0) {
    unsigned long long above = 0;
    for (int w = 0; w < NW; ++w) above += wab[w];
    SelState ns = st;
    ns.rem = rem - above;
    ns.prefix = st.prefix | ((uint32_t)bstar << shift);
    if (pass == 2) {
      if (a.budget == BUDGET_TOP_K) {
        ns.k_tie = ns.rem;
      } else {
        const unsigned long long qstar = fixed_mass(__uint_as_float(ns.prefix));
        ns.k_tie = qstar ? (ns.rem + qstar - 1) / qstar : 0;
      }
    }
    a.state[hd] = ns;
  }
}

// grid (max_chunks, Hq, 2): per chunk, the scores above the cutoff and at it
__global__ void __launch_bounds__(SEL_WG) sel_count_kernel(SelectArgs a) {
  __shared__ int red[2][SEL_WG / 64];
  const int h = blockIdx.y, dir = blockIdx.z, hd = h * 2 + dir;
  const SelView v = sel_view(a, h, dir);
  const int c0 = blockIdx.x * SEL_CHUNK;
  if (c0 >= v.n) return;
  const SelState st = a.state[sel_slot(a, h, dir)];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int n_gt = 0, n_tie = 0;
  if (st.mode == 0) {
    #pragma unroll
    for (int k = 0; k < SEL_PER; ++k) {
      const int i = c0 + tid + k * SEL_WG;
      if (i < v.n) {
        const uint32_t b = __float_as_uint(v.x[i]);
        n_gt += b > st.prefix ? 1 : 0;
        n_tie += b == st.prefix ? 1 : 0;
      }
    }
  }
  n_gt = wave_sum_i32(n_gt);
  n_tie = wave_sum_i32(n_tie);
  if (lane == 0) { red[0][wave] = n_gt; red[1][wave] = n_tie; }
  __syncthreads();
  if (tid == 0) {
    int g = 0, t = 0;
    for (int w = 0; w < SEL_WG / 64; ++w) { g += red[0][w]; t += red[1][w]; }
    int* cc = a.counts + ((int64_t)hd * a.max_chunks + blockIdx.x) * 2;
    cc[0] = g;
    cc[1] = t;
  }
}

// grid (max_chunks, Hq, 2): write the chunk's kept indices in ascending order:
// scores above the cutoff, and the ties at it up to k_tie in index order.
// Each wave owns a contiguous quarter of the chunk; ballots give positions.
__global__ void __launch_bounds__(SEL_WG) sel_write_kernel(SelectArgs a) {
  constexpr int NW = SEL_WG / 64, QUART = SEL_CHUNK / NW;
  __shared__ int wgt[NW], wtie[NW];
  const int h = blockIdx.y, dir = blockIdx.z, hd = h * 2 + dir;
  const SelView v = sel_view(a, h, dir);
  const int chunk = blockIdx.x, c0 = chunk * SEL_CHUNK;
  if (c0 >= v.n) return;
  const SelState st = a.state[sel_slot(a, h, dir)];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nchunks = (v.n + SEL_CHUNK - 1) / SEL_CHUNK;
  if (st.mode == 1) {
    for (int i = c0 + tid; i < min(v.n, c0 + SEL_CHUNK); i += SEL_WG) v.out[i] = i;
    if (chunk == 0 && tid == 0) *v.cnt = v.n;
    return;
  }
  if (st.mode == 2) {
    if (chunk == 0 && tid == 0) *v.cnt = 0;
    return;
  }
  // above-cutoff and tie counts of the chunks before this one, and of all
  const int* cc = a.counts + (int64_t)hd * a.max_chunks * 2;
  int g_before = 0, t_before = 0, g_all = 0, t_all = 0;
  for (int c = lane; c < nchunks; c += 64) {
    const int g = cc[2 * c], t = cc[2 * c + 1];
    g_all += g; t_all += t;
    if (c < chunk) { g_before += g; t_before += t; }
  }
  g_before = wave_sum_i32(g_before); t_before = wave_sum_i32(t_before);
  g_all = wave_sum_i32(g_all); t_all = wave_sum_i32(t_all);
  // joint budget, slashes: the vertical ties come first in the pooled order
  int t_off = 0;
  if (a.budget == BUDGET_JOINT && dir == 1) {
    const int* cv = a.counts + (int64_t)(h * 2) * a.max_chunks * 2;
    const int nch_v = (int)((a.n_vert + SEL_CHUNK - 1) / SEL_CHUNK);
    for (int c = lane; c < nch_v; c += 64) t_off += cv[2 * c + 1];
    t_off = wave_sum_i32(t_off);
  }
  const unsigned long long k_tie = st.k_tie;
  const unsigned long long kept_off = min((unsigned long long)t_off, k_tie);   // ties the verticals took
  const uint32_t xstar = st.prefix;
  if (chunk == 0 && tid == 0)
    *v.cnt = g_all + (int)(min((unsigned long long)(t_off + t_all), k_tie) - kept_off);
  // this wave's quarter: counts, then the waves before it
  const int w0 = min(v.n, c0 + wave * QUART), w1 = min(v.n, w0 + QUART);
  int n_gt = 0, n_tie = 0;
  for (int i = w0 + lane; i < w1; i += 64) {
    const uint32_t b = __float_as_uint(v.x[i]);
    n_gt += b > xstar ? 1 : 0;
    n_tie += b == xstar ? 1 : 0;
  }
  n_gt = wave_sum_i32(n_gt);
  n_tie = wave_sum_i32(n_tie);
  if (lane == 0) { wgt[wave] = n_gt; wtie[wave] = n_tie; }
  __syncthreads();
  unsigned long long ties_seen = (unsigned long long)(t_off + t_before);   // in the pooled order
  int gt_before = g_before;
  for (int w = 0; w < wave; ++w) { gt_before += wgt[w]; ties_seen += (unsigned long long)wtie[w]; }
  // kept before this wave: every above-cutoff score, and this direction's
  // share of the first k_tie ties
  int base = gt_before + (int)(min(ties_seen, k_tie) - kept_off);
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int cs = w0; cs < w1; cs += 64) {
    const int i = cs + lane;
    const bool ok = i < w1;
    const uint32_t b = ok ? __float_as_uint(v.x[i]) : 0u;
    const bool is_tie = ok && b == xstar;
    const unsigned long long tmask = __ballot(is_tie);
    const unsigned long long tie_rank = ties_seen + __popcll(tmask & below);
    const bool keep = ok && (b > xstar || (is_tie && tie_rank < k_tie));
    const unsigned long long kmask = __ballot(keep);
    if (keep) v.out[base + __popcll(kmask & below)] = i;
    base += __popcll(kmask);
    ties_seen += __popcll(tmask);
  }
}

size_t select_workspace_bytes(int Hq, int64_t n_global) {
  const int64_t chunks = (n_global + SEL_CHUNK - 1) / SEL_CHUNK;
  return (size_t)Hq * 2 * (SEL_BINS * sizeof(unsigned long long) + sizeof(SelState) + chunks * 2 * sizeof(int)) + 256;
}

// the passes' partials and row LSE, then (256-byte aligned) the selection's
static size_t index_pass_bytes(int Hq, int Hkv, int64_t n_global) {
  const int64_t T = n_global / BLK;
  const int64_t nsplit = idx_nsplit(Hq, T);
  return ((size_t)(Hq * BLK * nsplit * 2 + Hq * BLK) * sizeof(float) + 255) & ~(size_t)255;
}

size_t index_workspace_bytes(int Hq, int Hkv, int64_t n_global, int D, int last_q) {
  (void)D; (void)last_q;
  return index_pass_bytes(Hq, Hkv, n_global) + select_workspace_bytes(Hq, n_global);
}

// Shared set-up: the tiles walked (all T, or the NB tiles of rank_fixed) and
// their split over workgroups; the workspace holds the split partials and
// the row LSE.
static IndexArgs index_args(TView q_last, int Hq, int last_q, TView k, int Hkv, const vs_layout& lay, float scale,
                            int rank_fixed, void* ws) {
  IndexArgs a{};
  a.q = q_last.ptr; a.k = k.ptr;
  a.qsh = q_last.sh; a.qsn = q_last.sn; a.ksh = k.sh; a.ksn = k.sn;
  a.Hq = Hq; a.Hkv = Hkv; a.last_q = last_q; a.kind = lay.kind; a.P = lay.P;
  a.n_global = lay.n_global;
  a.T = (int)(lay.n_global / BLK);
  a.NB = a.T / lay.P;
  a.rank_fixed = rank_fixed;
  a.ntiles = rank_fixed >= 0 ? a.NB : a.T;
  a.nsplit = (int)idx_nsplit(Hq, a.ntiles);
  a.tiles_per = (a.ntiles + a.nsplit - 1) / a.nsplit;
  a.nsplit = (a.ntiles + a.tiles_per - 1) / a.tiles_per;
  a.scale_log2 = scale * LOG2E;
  a.part = (float*)ws;
  a.lse2 = a.part + (int64_t)Hq * BLK * a.nsplit * 2;
  return a;
}

static bool launch_rowstat(int dtype, int D, const IndexArgs& a, hipStream_t stream) {
  const dim3 grid(a.nsplit, a.Hkv), block(64 * (a.Hq / a.Hkv));
  if (dtype == VS_BF16 && D == 128) hipLaunchKernelGGL((index_rowstat_kernel<bf16, 128>), grid, block, 0, stream, a);
  else if (dtype == VS_BF16 && D == 64) hipLaunchKernelGGL((index_rowstat_kernel<bf16, 64>), grid, block, 0, stream, a);
  else if (dtype == VS_F32 && D == 64) hipLaunchKernelGGL((index_rowstat_kernel<float, 64>), grid, block, 0, stream, a);
  else return false;
  return true;
}

static bool launch_colsum(int dtype, int D, const IndexArgs& a, hipStream_t stream) {
  const dim3 grid(a.nsplit, a.Hkv), block(64 * (a.Hq / a.Hkv));
  if (dtype == VS_BF16 && D == 128) hipLaunchKernelGGL((index_colsum_kernel<bf16, 128>), grid, block, 0, stream, a);
  else if (dtype == VS_BF16 && D == 64) hipLaunchKernelGGL((index_colsum_kernel<bf16, 64>), grid, block, 0, stream, a);
  else if (dtype == VS_F32 && D == 64) hipLaunchKernelGGL((index_colsum_kernel<float, 64>), grid, block, 0, stream, a);
  else return false;
  return true;
}

static void launch_combine(IndexArgs a, const float* in, int n, int64_t tstride, int64_t sstride, float* stats,
                           hipStream_t stream) {
  a.cmb_in = in; a.cmb_n = n; a.cmb_tstride = tstride; a.cmb_sstride = sstride; a.cmb_stats = stats;
  hipLaunchKernelGGL(index_combine_kernel, dim3((a.Hq * BLK + COMB_THREADS / 64 - 1) / (COMB_THREADS / 64)),
                     dim3(COMB_THREADS), 0, stream, a);
}

int launch_index_select(const float* vert_score, const float* slash_score, int Hq, int64_t n_global, int budget,
                        float top_p, int k_vert, int k_slash, int32_t* vert_idx, int32_t* vert_cnt,
                        int32_t* slash_idx, int32_t* slash_cnt, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (ws_bytes < select_workspace_bytes(Hq, n_global)) return VS_ERR_WORKSPACE;
  SelectArgs s;
  s.vert = vert_score; s.slash = slash_score; s.vert_idx = vert_idx; s.vert_cnt = vert_cnt;
  s.slash_idx = slash_idx; s.slash_cnt = slash_cnt; s.n_vert = n_global; s.n_slash = (int)(n_global / BLK);
  s.top_p = top_p;
  s.budget = budget; s.k_vert = k_vert; s.k_slash = k_slash;
  s.max_chunks = (int)((n_global + SEL_CHUNK - 1) / SEL_CHUNK);
  char* w = (char*)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
  s.hist = (unsigned long long*)w;
  w += (size_t)Hq * 2 * SEL_BINS * sizeof(unsigned long long);
  s.state = (SelState*)w;
  w += (size_t)Hq * 2 * sizeof(SelState);
  s.counts = (int*)w;
  const dim3 heads(Hq, 2), chunks(s.max_chunks, Hq, 2);
  hipLaunchKernelGGL(sel_init_kernel, heads, dim3(SEL_WG), 0, stream, s);
  for (int pass = 0; pass < 3; ++pass) {
    hipLaunchKernelGGL(sel_hist_kernel, chunks, dim3(SEL_WG), 0, stream, s, pass);
    hipLaunchKernelGGL(sel_scan_kernel, heads, dim3(SCAN_THREADS), 0, stream, s, pass);
  }
  hipLaunchKernelGGL(sel_count_kernel, chunks, dim3(SEL_WG), 0, stream, s);
  hipLaunchKernelGGL(sel_write_kernel, chunks, dim3(SEL_WG), 0, stream, s);
  return hipGetLastError() == hipSuccess ? VS_OK : VS_ERR_HIP;
}

int launch_index_build(int dtype, int D, TView q_last, int Hq, int last_q, TView k, int Hkv,
                       const vs_layout& lay, float scale, float top_p, float* vert_score,
                       float* slash_score, int32_t* vert_idx, int32_t* vert_cnt, int32_t* slash_idx,
                       int32_t* slash_cnt, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (ws_bytes < index_workspace_bytes(Hq, Hkv, lay.n_global, D, last_q)) return VS_ERR_WORKSPACE;
  IndexArgs a = index_args(q_last, Hq, last_q, k, Hkv, lay, scale, -1, ws);
  a.vert = vert_score; a.slash = slash_score;
  if (!launch_rowstat(dtype, D, a, stream)) return VS_ERR_UNSUPPORTED;
  launch_combine(a, a.part, a.nsplit, a.nsplit, 1, nullptr, stream);
  launch_colsum(dtype, D, a, stream);
  const size_t off = index_pass_bytes(Hq, Hkv, lay.n_global);
  return launch_index_select(vert_score, slash_score, Hq, lay.n_global, BUDGET_TOP_P, top_p, 0, 0, vert_idx, vert_cnt,
                             slash_idx, slash_cnt, (char*)ws + off, ws_bytes - off, stream);
}

int launch_index_rank_stats(int dtype, int D, TView q_last, int Hq, int last_q, TView k_local, int Hkv,
                            const vs_layout& lay, int rank, float scale, float* stats, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  if (ws_bytes < index_workspace_bytes(Hq, Hkv, lay.n_global, D, last_q)) return VS_ERR_WORKSPACE;
  IndexArgs a = index_args(q_last, Hq, last_q, k_local, Hkv, lay, scale, rank, ws);
  if (!launch_rowstat(dtype, D, a, stream)) return VS_ERR_UNSUPPORTED;
  launch_combine(a, a.part, a.nsplit, a.nsplit, 1, stats, stream);
  return hipGetLastError() == hipSuccess ? VS_OK : VS_ERR_HIP;
}

int launch_index_rank_mass(int dtype, int D, TView q_last, int Hq, int last_q, TView k_local, int Hkv,
                           const vs_layout& lay, int rank, float scale, const float* all_stats, float* vert_score,
                           float* slash_score, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (ws_bytes < index_workspace_bytes(Hq, Hkv, lay.n_global, D, last_q)) return VS_ERR_WORKSPACE;
  IndexArgs a = index_args(q_last, Hq, last_q, k_local, Hkv, lay, scale, rank, ws);
  a.vert = vert_score; a.slash = slash_score;
  // the gathered stats are [P][Hq * 64][2]: row t of rank s at (s * Hq * 64 + t) * 2
  launch_combine(a, all_stats, lay.P, 1, (int64_t)Hq * BLK, nullptr, stream);
  if (!launch_colsum(dtype, D, a, stream)) return VS_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? VS_OK : VS_ERR_HIP;
}

}  // namespace vs
