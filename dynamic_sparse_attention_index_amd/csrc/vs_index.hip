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

constexpr int IDX_SPLIT_TARGET = 1024;   // workgroups per pass (over all kv heads)

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
  for (int tau = tau0; tau < tau1; ++tau) {
    const int64_t G = stage_key_tile<T, D>(Ks, a, kvh, tau, tid, nthr);
    __syncthreads();
    f32x4 acc[4][4];
    score_tile<T, D>(Ks, qa, n16, g4, acc);
    const bool last = G == a.T - 1;
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
  for (int tau = tau0; tau < tau1; ++tau) {
    const int64_t G = stage_key_tile<T, D>(Ks, a, kvh, tau, tid, nthr);
    __syncthreads();
    f32x4 acc[4][4];
    score_tile<T, D>(Ks, qa, n16, g4, acc);
    const bool last = G == a.T - 1;
    float col[4];
    #pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      float c = 0.f;
      #pragma unroll
      for (int rs = 0; rs < 4; ++rs)
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rs + 4 * g4 + i;
          const bool act = lse[rs][i] > -INFINITY && !(last && 16 * kt + n16 > row0 + r);
          if (act) c += __builtin_amdgcn_exp2f(acc[rs][kt][i] * a.scale_log2 - lse[rs][i]);
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

// ---- exact top-p selection ---------------------------------------------------
constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int SEL_UNROLL = 8;   // loads in flight per thread in each sweep

struct SelectArgs {
  const float* vert; const float* slash;
  int32_t *vert_idx, *vert_cnt, *slash_idx, *slash_cnt;
  int64_t n_vert; int n_slash;
  float top_p;
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

// One wave over a 256-digit mass histogram h (lane l holds digits 4l..4l+3).
// With the suffix mass S(b) = sum of h[b'] for b' >= b, returns the digit
// b* = the largest b >= 1 with S(b) >= rem (0 when there is none) and stores
// S(b* + 1), the mass of the digits above it, in *above. The histogram total
// goes to *total.
__device__ __forceinline__ int sel_digit(const unsigned long long* h, unsigned long long rem, int lane,
                                         unsigned long long* above, unsigned long long* total) {
  unsigned long long v[4];
  #pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = h[4 * lane + j];
  const unsigned long long loc = v[0] + v[1] + v[2] + v[3];
  unsigned long long suf = loc;   // inclusive suffix over lanes
  #pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long t = __shfl_down(suf, off, 64);
    if (lane + off < 64) suf += t;
  }
  *total = __shfl(suf, 0, 64);
  unsigned long long s = suf - loc;
  int cnt = 0;
  #pragma unroll
  for (int j = 3; j >= 0; --j) {
    s += v[j];   // S(4 lane + j)
    cnt += (4 * lane + j >= 1 && s >= rem) ? 1 : 0;
  }
  const int b = wave_sum_i32(cnt);
  unsigned long long ab = 0;
  #pragma unroll
  for (int j = 0; j < 4; ++j) ab += (4 * lane + j > b) ? v[j] : 0ull;
  *above = wave_sum_u64(ab);
  return b;
}

// grid (Hq, 2): y = 0 vertical scores, y = 1 slash scores.
__global__ void __launch_bounds__(SEL_THREADS) topp_select_kernel(SelectArgs a) {
  __shared__ unsigned long long hist[SEL_WAVES][256];
  __shared__ unsigned long long sel_rem;
  __shared__ uint32_t sel_prefix;
  __shared__ int sel_empty;
  const int h = blockIdx.x;
  const bool is_vert = blockIdx.y == 0;
  const int n = is_vert ? (int)a.n_vert : a.n_slash;
  const float* x = is_vert ? a.vert + h * a.n_vert : a.slash + (int64_t)h * a.n_slash;
  int32_t* out = is_vert ? a.vert_idx + h * a.n_vert : a.slash_idx + (int64_t)h * a.n_slash;
  int32_t* cnt = is_vert ? a.vert_cnt + h : a.slash_cnt + h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  if (a.top_p >= 1.f) {
    for (int i = tid; i < n; i += SEL_THREADS) out[i] = i;
    if (tid == 0) *cnt = n;
    return;
  }
  if (!(a.top_p > 0.f)) {
    if (tid == 0) *cnt = 0;
    return;
  }
  // Radix select on the fp32 bit pattern (non-negative: bit order = value
  // order), 8 bits a pass, each digit weighted by its fixed-point mass. The
  // first pass sees every score, so its histogram total is the whole mass
  // and sets the target ceil(p * total).
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    const uint32_t prefix = pass == 0 ? 0u : sel_prefix;
    unsigned long long* hw = hist[wave];
    #pragma unroll
    for (int j = 0; j < 4; ++j) hw[lane + 64 * j] = 0;
    for (int c0 = 0; c0 < n; c0 += SEL_THREADS * SEL_UNROLL) {
      uint32_t bits[SEL_UNROLL];
      #pragma unroll
      for (int k = 0; k < SEL_UNROLL; ++k) {
        const int i = c0 + tid + k * SEL_THREADS;
        bits[k] = i < n ? __float_as_uint(x[i]) : 0u;
      }
      #pragma unroll
      for (int k = 0; k < SEL_UNROLL; ++k) {
        const int i = c0 + tid + k * SEL_THREADS;
        if (i < n && (bits[k] & hi_mask) == prefix)
          atomicAdd(&hw[(bits[k] >> shift) & 255u], fixed_mass(__uint_as_float(bits[k])));
      }
    }
    __syncthreads();
    if (tid < 256) {
      unsigned long long t = 0;
      #pragma unroll
      for (int w = 0; w < SEL_WAVES; ++w) t += hist[w][tid];
      hist[0][tid] = t;
    }
    __syncthreads();
    if (wave == 0) {
      unsigned long long rem = pass == 0 ? 0ull : sel_rem, above, total;
      if (pass == 0) {
        // the target needs the total first: a second wave-wide sum
        unsigned long long loc = 0;
        #pragma unroll
        for (int j = 0; j < 4; ++j) loc += hist[0][4 * lane + j];
        const unsigned long long tot = wave_sum_u64(loc);
        const unsigned long long pq = (unsigned long long)__builtin_rint((double)a.top_p * 4294967296.0);
        const unsigned __int128 prod = (unsigned __int128)pq * tot;
        rem = (unsigned long long)((prod + 0xFFFFFFFFull) >> 32);   // ceil(pq * tot / 2^32)
      }
      const int b = sel_digit(hist[0], rem, lane, &above, &total);
      if (lane == 0) {
        sel_empty = rem == 0;
        sel_rem = rem - above;
        sel_prefix = prefix | ((uint32_t)b << shift);
      }
    }
    __syncthreads();
    if (sel_empty) {
      if (tid == 0) *cnt = 0;
      return;
    }
  }
  const uint32_t xstar = sel_prefix;
  const unsigned long long qstar = fixed_mass(__uint_as_float(xstar));
  const unsigned long long k_tie = qstar ? (sel_rem + qstar - 1) / qstar : 0;
  // ascending compaction: x > x*, or x == x* among the first k_tie ties (in
  // index order). Each wave owns a contiguous index range; pass A counts its
  // keeps and ties, one barrier, then pass B writes positions from ballots.
  __shared__ int wave_gt[SEL_WAVES], wave_tie[SEL_WAVES];
  const int per = (n + SEL_WAVES - 1) / SEL_WAVES;
  const int w0 = min(n, wave * per), w1 = min(n, w0 + per);
  int n_gt = 0, n_tie = 0;
  for (int c0 = w0; c0 < w1; c0 += 64 * SEL_UNROLL) {
    uint32_t bits[SEL_UNROLL];
    #pragma unroll
    for (int k = 0; k < SEL_UNROLL; ++k) {
      const int i = c0 + lane + 64 * k;
      bits[k] = i < w1 ? __float_as_uint(x[i]) : 0u;
    }
    #pragma unroll
    for (int k = 0; k < SEL_UNROLL; ++k) {
      const bool ok = c0 + lane + 64 * k < w1;
      n_gt += (ok && bits[k] > xstar) ? 1 : 0;
      n_tie += (ok && bits[k] == xstar) ? 1 : 0;
    }
  }
  n_gt = wave_sum_i32(n_gt);
  n_tie = wave_sum_i32(n_tie);
  if (lane == 0) {
    wave_gt[wave] = n_gt;
    wave_tie[wave] = n_tie;
  }
  __syncthreads();
  // this wave's output base, and the ties before its range
  unsigned long long ties_before = 0, run_ties = 0;
  int base = 0, total_kept = 0;
  for (int w = 0; w < SEL_WAVES; ++w) {
    const unsigned long long room = k_tie > run_ties ? k_tie - run_ties : 0;
    const int kept_w = wave_gt[w] + (int)min((unsigned long long)wave_tie[w], room);
    if (w < wave) base += kept_w;
    if (w == wave) ties_before = run_ties;
    total_kept += kept_w;
    run_ties += (unsigned long long)wave_tie[w];
  }
  unsigned long long ties_seen = ties_before;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = w0; c0 < w1; c0 += 64 * SEL_UNROLL) {
    uint32_t bits[SEL_UNROLL];
    #pragma unroll
    for (int k = 0; k < SEL_UNROLL; ++k) {
      const int i = c0 + lane + 64 * k;
      bits[k] = i < w1 ? __float_as_uint(x[i]) : 0u;
    }
    #pragma unroll
    for (int k = 0; k < SEL_UNROLL; ++k) {
      const int i = c0 + lane + 64 * k;
      const bool ok = i < w1;
      const bool is_tie = ok && bits[k] == xstar;
      const unsigned long long tmask = __ballot(is_tie);
      const unsigned long long tie_rank = ties_seen + __popcll(tmask & below);
      const bool keep = ok && (bits[k] > xstar || (is_tie && tie_rank < k_tie));
      const unsigned long long kmask = __ballot(keep);
      if (keep) out[base + __popcll(kmask & below)] = i;
      base += __popcll(kmask);
      ties_seen += __popcll(tmask);
    }
  }
  if (tid == 0) *cnt = total_kept;
}

size_t index_workspace_bytes(int Hq, int Hkv, int64_t n_global, int D, int last_q) {
  (void)D; (void)last_q;
  const int64_t T = n_global / BLK;
  const int64_t nsplit = std::min<int64_t>(T, std::max<int64_t>(1, IDX_SPLIT_TARGET / Hkv));
  return (size_t)(Hq * BLK * nsplit * 2 + Hq * BLK) * sizeof(float) + 256;
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
  a.nsplit = (int)std::min<int64_t>(a.ntiles, std::max<int64_t>(1, IDX_SPLIT_TARGET / Hkv));
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

int launch_index_select(const float* vert_score, const float* slash_score, int Hq, int64_t n_global, float top_p,
                        int32_t* vert_idx, int32_t* vert_cnt, int32_t* slash_idx, int32_t* slash_cnt,
                        hipStream_t stream) {
  SelectArgs s;
  s.vert = vert_score; s.slash = slash_score; s.vert_idx = vert_idx; s.vert_cnt = vert_cnt;
  s.slash_idx = slash_idx; s.slash_cnt = slash_cnt; s.n_vert = n_global; s.n_slash = (int)(n_global / BLK);
  s.top_p = top_p;
  hipLaunchKernelGGL(topp_select_kernel, dim3(Hq, 2), dim3(SEL_THREADS), 0, stream, s);
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
  return launch_index_select(vert_score, slash_score, Hq, lay.n_global, top_p, vert_idx, vert_cnt, slash_idx,
                             slash_cnt, stream);
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
