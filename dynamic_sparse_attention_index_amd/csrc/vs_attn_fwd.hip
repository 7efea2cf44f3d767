// Block-sparse attention forward over the active region of one ring step,
// and the log-sum-exp merge of partial results.
//
// Computes, for every query row, softmax attention restricted to the active
// entries of the vertical-slash set (MTraining review, page 1, section 三.2
// item 3: only the active entries of the local sub-matrix are computed; item 2:
// slashes at 64x64 block granularity, verticals at token granularity). The
// incremental-softmax merge follows the Ring Attention overview page, section
// 2.1.
//
// One workgroup = one (q head, 64-row query block); four waves of 16 rows.
// Work per block: the listed slash tiles (dense 64x64 on MFMA, causal predicate
// only on the block's own diagonal tile), then the shard's vertical columns
// gathered 64 at a time into a dense tile (columns already inside a listed tile
// or beyond the causal edge are masked). S^T = K Q^T keeps one query row per
// lane, so the online-softmax state is per lane and O^T = V^T P^T consumes P
// straight from registers; V^T fragments come from the row-major V tile via
// the gfx950 LDS transpose read.
#include <type_traits>
#include <utility>

#include "vs_common.h"
#include "vs_internal.h"

namespace vs {

constexpr int FWD_THREADS = 256;  // 4 waves

struct FwdArgs {
  const void* q; const void* k; const void* v;
  int64_t qsh, qsn, ksh, ksn, vsh, vsn;
  const int32_t* tile_ptr; const int32_t* tile_col;
  const int32_t* vloc; const int32_t* vert_end; const uint32_t* slash_bits;
  float* o; float* lse;
  int32_t* status;   // head-pair kernel: written VS_ERR_ARG if a pair's active sets differ
  int Hq, Hkv, QB, KB, W, kind, P, rank, src, accumulate;
  float scale_log2;
  int32_t* dbg;      // debug builds: bounds-violation counter (null otherwise)
  int64_t cap;       // capacity of tile_col (debug-build checks)
};

// Physical key (0..63) held by S^T output value i of 16-key subtile t in lane
// group g: subtile t covers keys 32*(t/2) + 8*g + 4*(t%2) + i, so each lane
// group later supplies 8 consecutive keys to the P.V contraction.
__device__ __forceinline__ int key_of(int t, int g, int i) { return 32 * (t >> 1) + 8 * g + 4 * (t & 1) + i; }
// Key row read by lane row m (0..15) of subtile t for the A operand of S^T.
__device__ __forceinline__ int key_row(int t, int m) { return 32 * (t >> 1) + 8 * (m >> 2) + 4 * (t & 1) + (m & 3); }

template <typename T, int D>
struct FwdTile {
  static constexpr int KP = D + (sizeof(T) == 2 ? 8 : 4);       // LDS row pitch (elements)
  static constexpr int CPR = D * (int)sizeof(T) / 16;            // 16-byte chunks per row
  static constexpr int CPT = BLK * CPR / FWD_THREADS;            // chunks per thread
  static_assert(CPT >= 1 && BLK * CPR % FWD_THREADS == 0, "tile split");
};

template <typename T, int D>
__global__ void __launch_bounds__(FWD_THREADS) attn_fwd_kernel(FwdArgs a) {
  using Tl = FwdTile<T, D>;
  constexpr int KP = Tl::KP, CPR = Tl::CPR, CPT = Tl::CPT;
  __shared__ __attribute__((aligned(16))) T Ks[BLK * KP];
  __shared__ __attribute__((aligned(16))) T Vs[BLK * KP];
  __shared__ int thr_sh[BLK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, n16 = lane & 15;
  // work item: heavy (late) query blocks first, clustered per XCD and kv group
  int rank_i, hh_i, g_i;
  if (!xcd_group_item(blockIdx.x, a.Hkv, a.QB, QMAJOR_BPC, a.Hq / a.Hkv, &rank_i, &hh_i, &g_i)) return;
  const int I = a.QB - 1 - rank_i;
  const int h = g_i * (a.Hq / a.Hkv) + hh_i;
  const int kvh = h / (a.Hq / a.Hkv);
  const int64_t u = (int64_t)h * a.QB + I;
  const int rowoff = wave * 16 + n16;  // this lane's query row within the block
  const int64_t grow = (int64_t)I * BLK + rowoff;

  const T* qrow = (const T*)a.q + h * a.qsh + grow * a.qsn;
  const T* kbase = (const T*)a.k + kvh * a.ksh;
  const T* vbase = (const T*)a.v + kvh * a.vsh;

  // Q fragment (B operand of S^T): this lane's row, contraction slots of group g4
  constexpr int NQ = (sizeof(T) == 2) ? D / 32 : D / 4;
  typedef typename std::conditional<sizeof(T) == 2, bf16x8, float>::type QFrag;
  QFrag qf[NQ];
  if constexpr (sizeof(T) == 2) {
    #pragma unroll
    for (int ks = 0; ks < NQ; ++ks) qf[ks] = *(const bf16x8*)(qrow + 32 * ks + 8 * g4);
  } else {
    #pragma unroll
    for (int ks = 0; ks < NQ; ++ks) qf[ks] = qrow[4 * ks + g4];
  }

  const int t0 = dbg_clamp(a.tile_ptr[u], 0, (int)a.cap + 1, a.dbg);
  const int nt = dbg_clamp(a.tile_ptr[u + 1] - t0, 0, min(a.KB, (int)a.cap - t0) + 1, a.dbg);
  const int ve = dbg_clamp(a.vert_end[u], 0, a.KB * BLK + 1, a.dbg);
  const int total = nt + (ve + BLK - 1) / BLK;
  const int64_t G = global_block(a.kind, a.P, a.QB, a.rank, I);
  const int32_t* vl = a.vloc + (int64_t)h * a.KB * BLK;
  const uint32_t* sb = a.slash_bits + (int64_t)h * a.W;

  f32x4 acc[D / 16];
  #pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // staging registers for the next tile
  i32x4 kreg[CPT], vreg[CPT];
  int mode_next = 0, thr_next = 0;

  auto fetch = [&](int it) {
    int src_rows[CPT];
    if (it < nt) {
      const int e = a.tile_col[t0 + it];
      const int J = dbg_clamp(e & VS_TILE_MASK, 0, a.KB, a.dbg);
      mode_next = (e & VS_TILE_DIAG) ? 1 : 0;
      #pragma unroll
      for (int c = 0; c < CPT; ++c) src_rows[c] = J * BLK + (tid + c * FWD_THREADS) / CPR;
      thr_next = tid < BLK ? tid : 0;  // causal threshold inside the diagonal tile
    } else {
      const int base = (it - nt) * BLK;
      mode_next = 1;
      #pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int slot = (tid + c * FWD_THREADS) / CPR;
        const int idx = base + slot;
        src_rows[c] = dbg_clamp(idx < ve ? vl[idx] : vl[base], 0, a.KB * BLK, a.dbg);
      }
      if (tid < BLK) {
        const int idx = base + tid;
        int thr = BLK;  // never active
        if (idx < ve) {
          const int m = dbg_clamp(vl[idx], 0, a.KB * BLK, a.dbg);
          const int64_t gb = global_block(a.kind, a.P, a.KB, a.src, m / BLK);
          const int64_t j = G - gb;
          const bool covered = (sb[j >> 5] >> (j & 31)) & 1u;
          if (!covered) thr = (j == 0) ? (m % BLK) : 0;
        }
        thr_next = thr;
      }
    }
    #pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int col = ((tid + c * FWD_THREADS) % CPR) * (16 / (int)sizeof(T));
      kreg[c] = *(const i32x4*)(kbase + src_rows[c] * a.ksn + col);
      vreg[c] = *(const i32x4*)(vbase + src_rows[c] * a.vsn + col);
    }
  };

  if (total > 0) fetch(0);
  for (int it = 0; it < total; ++it) {
    #pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + c * FWD_THREADS;
      const int r = ch / CPR, col = (ch % CPR) * (16 / (int)sizeof(T));
      *(i32x4*)(Ks + r * KP + col) = kreg[c];
      *(i32x4*)(Vs + r * KP + col) = vreg[c];
    }
    if (tid < BLK) thr_sh[tid] = thr_next;
    const int mode = mode_next;
    __syncthreads();
    if (it + 1 < total) fetch(it + 1);

    // ---- S^T = K Q^T for this wave's 16 rows x 64 keys
    f32x4 s[4];
    #pragma unroll
    for (int t = 0; t < 4; ++t) {
      s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      const T* krow = Ks + key_row(t, n16) * KP;
      if constexpr (sizeof(T) == 2) {
        #pragma unroll
        for (int ks = 0; ks < NQ; ++ks)
          s[t] = mfma_bf16(*(const bf16x8*)(krow + 32 * ks + 8 * g4), qf[ks], s[t]);
      } else {
        #pragma unroll
        for (int ks = 0; ks < NQ; ++ks) s[t] = mfma_f32(krow[4 * ks + g4], qf[ks], s[t]);
      }
    }
    // ---- scale, mask, online softmax (log2 domain)
    float mx = -INFINITY;
    #pragma unroll
    for (int t = 0; t < 4; ++t)
      #pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = s[t][i] * a.scale_log2;
        if (mode && thr_sh[key_of(t, g4, i)] > rowoff) x = -INFINITY;
        s[t][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, wave_shfl_xor(mx, 16));
    mx = fmaxf(mx, wave_shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.f;
    #pragma unroll
    for (int t = 0; t < 4; ++t)
      #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[t][i] - m_use);
        s[t][i] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    #pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      #pragma unroll
      for (int i = 0; i < 4; ++i) acc[dt][i] *= alpha;

    // ---- O^T += V^T P^T
    if constexpr (sizeof(T) == 2) {
      bf16x8 pf[2];
      #pragma unroll
      for (int c = 0; c < 2; ++c)
        #pragma unroll
        for (int e = 0; e < 2; ++e)
          #pragma unroll
          for (int i = 0; i < 4; ++i) pf[c][4 * e + i] = (bf16)s[2 * c + e][i];
      #pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        #pragma unroll
        for (int c = 0; c < 2; ++c) {
          const T* base = Vs + (32 * c + 8 * g4 + (n16 >> 2)) * KP + 16 * dt + 4 * (n16 & 3);
          acc[dt] = mfma_bf16(lds_read_tr16_x2(base, KP), pf[c], acc[dt]);
        }
    } else {
      #pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        #pragma unroll
        for (int t = 0; t < 4; ++t)
          #pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[dt] = mfma_f32(Vs[key_of(t, g4, i) * KP + 16 * dt + n16], s[t][i], acc[dt]);
    }
    __syncthreads();
  }

  // ---- epilogue: normalise, write or merge
  float l_tot = l_run + wave_shfl_xor(l_run, 16);
  l_tot = l_tot + wave_shfl_xor(l_tot, 32);
  const bool nonempty = l_tot > 0.f;
  const float inv = nonempty ? 1.f / l_tot : 0.f;
  const float lse_new = nonempty ? (m_run + log2f(l_tot)) * LN2 : -INFINITY;
  float* orow = a.o + ((int64_t)h * a.QB * BLK + grow) * D;
  float* lrow = a.lse + (int64_t)h * a.QB * BLK + grow;
  if (!a.accumulate) {
    #pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      f32x4 r;
      #pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = acc[dt][i] * inv;
      *(f32x4*)(orow + 16 * dt + 4 * g4) = r;
    }
    if (g4 == 0) *lrow = lse_new;
  } else {
    const float lse_old = *lrow;
    const float mxl = fmaxf(lse_old, lse_new);
    const float base = (mxl == -INFINITY) ? 0.f : mxl;
    const float wa = expf(lse_old - base), wb = expf(lse_new - base);
    const float tot = wa + wb;
    const float ca = tot > 0.f ? wa / tot : 0.f;
    const float cb = tot > 0.f ? wb / tot * inv : 0.f;
    #pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      f32x4 old = *(f32x4*)(orow + 16 * dt + 4 * g4);
      f32x4 r;
      #pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = ca * old[i] + cb * acc[dt][i];
      *(f32x4*)(orow + 16 * dt + 4 * g4) = r;
    }
    // every lane of the row has read lse_old before the wave writes it
    if (g4 == 0) *lrow = tot > 0.f ? base + logf(tot) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// bf16, head dim 128 (the production path). Each wave owns 32 query rows and
// one half (32 keys) of every 64-key tile, so a K/V fragment read from LDS
// feeds two MFMAs and a wave reads only its half of the tile; the two key
// halves keep separate online-softmax states, merged through LDS at the end
// (the same log-sum-exp merge as across ring steps).
//
// Software pipeline: step i computes S for tile i + 1 (an MFMA chain that
// does not depend on the softmax) together with the softmax and P.V of tile
// i, so the matrix cores and the vector ALU work at the same time. K tiles
// are therefore staged one tile ahead of V tiles: during step i LDS holds
// K[i+1] (being read), V[i] (being read), and receives K[i+2] and V[i+1]
// through asynchronous global->LDS copies, in two K and two V stages (64 KiB,
// two workgroups per CU). Descriptors (list entries or gathered vertical
// rows) arrive one step before the K copy that needs them; what the V copy
// needs (the same descriptor, read again) stays in LDS in between.
//
// F16: the inputs are fp16 (exact copies of bf16 data, see vs_convert_f16)
// and P is one fp16 operand, so P.V takes one MFMA instead of the hi + lo pair.
//
// HP = 2 (grouped-query packing): two q heads of one kv group share the
// workgroup (eight waves, four per head) and every K/V tile copy, which the
// first head's waves issue. Valid when the two heads have the same active
// set (an index selected per kv head); each workgroup checks that its pair's
// lists agree and otherwise writes VS_ERR_ARG to a.status and returns.
//
// RING: the tile sequence runs over several ring steps (RingTiles, `rs`):
// K/V hold every shard in storage order and each tile's copy starts at its
// step's shard; the online-softmax state carries across the steps.
//
// S1 (one-position stripes): a flagged tile's keys carry a causal threshold
// and a window of diagonals, entry (a, b) active when a >= thr[b] and bit
// qa(a) of win[b] is set; vertical chunks keep each column's causal rows on
// unselected diagonals (the rest lies in listed tiles).
template <bool F16, int HP, bool RING = false, bool S1 = false>
__device__ __forceinline__ void attn_fwd_d128(const FwdArgs& a, const RingSteps* rs = nullptr) {
  constexpr int D = TD;
  __shared__ __attribute__((aligned(16))) bf16 K0[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 K1[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 V0[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 V1[TILE_ELEMS];
  __shared__ float xs[HP * 2 * 2 * 64 * 2];
  // descriptor and row thresholds of tile t live in slot t % 3 from the
  // descriptor copy (step t - 3) to the softmax (step t)
  __shared__ int thr_sh[3][BLK];
  __shared__ uint32_t win_sh[S1 ? 3 : 1][BLK];
  __shared__ int desc_sh[3][BLK];
  __shared__ uint32_t sbits[MAX_LDS_W];
  // stages are chosen at compile time (the loop is unrolled by two) so the
  // compiler can tell the stages being read from the ones being filled
  auto Kst = [&]<int p>() -> bf16* {
    if constexpr (p == 0) return K0;
    else return K1;
  };
  auto Vst = [&]<int p>() -> bf16* {
    if constexpr (p == 0) return V0;
    else return V1;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave8 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hs = wave8 >> 2;                 // head slot in the workgroup (0 unless HP = 2)
  const int wave = wave8 & 3;                // wave among its head's four
  const int g4 = lane >> 4, n16 = lane & 15;
  const int rh = wave & 1, kh = wave >> 1;   // row half, key half
  int rank_i, hh_i, g_i;
  if (!xcd_group_item(blockIdx.x, a.Hkv, a.QB, QMAJOR_BPC, a.Hq / a.Hkv / HP, &rank_i, &hh_i, &g_i)) return;
  const int I = a.QB - 1 - rank_i;
  const int h0 = g_i * (a.Hq / a.Hkv) + HP * hh_i;   // the workgroup's first head: its lists drive the walk
  const int h = h0 + hs;
  const int kvh = g_i;
  const int64_t u = (int64_t)h0 * a.QB + I;
  const int64_t row_base = (int64_t)I * BLK + 32 * rh;   // this wave's first query row
  if constexpr (HP == 2) {
    const int64_t u1 = u + a.QB;
    const int t0 = dbg_clamp(a.tile_ptr[u], 0, (int)a.cap + 1, a.dbg);
    const int nt0 = dbg_clamp(a.tile_ptr[u + 1] - t0, 0, min(a.KB, (int)a.cap - t0) + 1, a.dbg);
    const int ve0 = dbg_clamp(a.vert_end[u], 0, a.KB * BLK + 1, a.dbg);
    const int t1 = dbg_clamp(a.tile_ptr[u1], 0, (int)a.cap + 1, a.dbg);
    const int nt1 = dbg_clamp(a.tile_ptr[u1 + 1] - t1, 0, min(a.KB, (int)a.cap - t1) + 1, a.dbg);
    const int ve1 = dbg_clamp(a.vert_end[u1], 0, a.KB * BLK + 1, a.dbg);
    int mism = (nt0 != nt1 || ve0 != ve1) ? 1 : 0;
    if (!mism) {
      for (int i = tid; i < nt0; i += HP * FWD_THREADS) mism |= a.tile_col[t0 + i] != a.tile_col[t1 + i];
      const int32_t* v0 = a.vloc + (int64_t)h0 * a.KB * BLK;
      for (int i = tid; i < ve0; i += HP * FWD_THREADS) mism |= v0[i] != v0[(int64_t)a.KB * BLK + i];
    }
    if (__syncthreads_or(mism)) {
      if (tid == 0) *a.status = VS_ERR_ARG;
      return;
    }
  }

  const bf16* qb = (const bf16*)a.q + h * a.qsh;
  const char* kbase = (const char*)((const bf16*)a.k + kvh * a.ksh);
  const char* vbase = (const char*)((const bf16*)a.v + kvh * a.vsh);
  const uint32_t krb = (uint32_t)a.ksn * 2, vrb = (uint32_t)a.vsn * 2;   // row pitch in bytes
  const DmaLane dl = dma_lane(wave, lane);

  typename std::conditional<RING, RingTiles, BlockTiles>::type bt;
  if constexpr (RING) {
    __shared__ RingTable rtab;
    bt.rs = rs; bt.tb = &rtab; bt.sbits = sbits; bt.vl_off = (int64_t)h0 * a.KB * BLK;
    bt.G = global_block(a.kind, a.P, a.QB, a.rank, I);
    bt.kind = a.kind; bt.P = a.P; bt.KB = a.KB; bt.dbg = a.dbg;
    bt.fill(u, wave8, lane);
    __syncthreads();
    bt.start();
  } else {
    bt.tile_col = a.tile_col; bt.vl = a.vloc + (int64_t)h0 * a.KB * BLK; bt.sbits = sbits;
    bt.G = global_block(a.kind, a.P, a.QB, a.rank, I);
    bt.kind = a.kind; bt.P = a.P; bt.KB = a.KB; bt.src = a.src; bt.dbg = a.dbg; bt.cap = a.cap;
    bt.init(a.tile_ptr[u], a.tile_ptr[u + 1], a.vert_end[u]);
  }
  const int total = bt.total;
  const uint32_t* sbg = a.slash_bits + (int64_t)h0 * a.W;
  for (int w = tid; w < a.W; w += HP * FWD_THREADS) sbits[w] = sbg[w];

  bf16x8 qf[2][4];
#pragma unroll
  for (int rs = 0; rs < 2; ++rs)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[rs][ks] = *(const bf16x8*)(qb + (row_base + 16 * rs + n16) * a.qsn + 32 * ks + 8 * g4);

  f32x4 acc[2][8];
#pragma unroll
  for (int rs = 0; rs < 2; ++rs)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[rs][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  const float sl2 = a.scale_log2;

  int mode_pend = 0;   // mode of the tile whose V copy was started last
  int qa_l[2] = {0, 0};   // S1: global-block offset qa of this lane's two rows
  if constexpr (S1) {
#pragma unroll
    for (int rs = 0; rs < 2; ++rs) qa_l[rs] = ((32 * rh + 16 * rs + n16) * a.P + a.rank) >> 6;
  }

  // start the K copy of tile t into K stage p and record its row thresholds
  auto issue_k = [&]<int p>(int t) {
    bf16* ks = Kst.template operator()<p>();
    const int* slot = desc_sh[t % 3];
    int thr = tid;
    uint32_t win = ~0u;
    const char* kb = kbase + bt.row0(t, 1) * krb;   // the tile's shard
    if (!bt.vert(t, 1)) {
      int mode;
      const int r0 = bt.tile_row(slot, mode);
      if constexpr (S1) {
        if (tid < BLK) {
          const int o = I - r0 / BLK;
          win = s1_key_window(s1_tile_window(sbits, a.W, a.P, o), a.P, a.src, tid);
          thr = s1_key_threshold(o, a.rank, a.src, tid);
        }
      }
      if (hs == 0) dma_tile_rows(ks, kb + (int64_t)r0 * krb, krb, dl, wave);
    } else {
      int rows[4];
      if constexpr (S1) bt.vert_rows_s1(t, slot, rows, thr, win, wave, lane, tid, I, a.rank, a.W);
      else bt.vert_rows(t, slot, rows, thr, wave, lane, tid, 1);
      if (hs == 0) dma_tile_gather(ks, kb, rows, krb, dl, wave);
    }
    if (tid < BLK) {
      thr_sh[t % 3][tid] = thr;
      if constexpr (S1) win_sh[t % 3][tid] = win;
    }
  };
  // start the V copy of tile t into V stage p (descriptor read again)
  auto issue_v = [&]<int p>(int t) {
    bf16* vs_ = Vst.template operator()<p>();
    const int* slot = desc_sh[t % 3];
    const char* vb = vbase + bt.row0(t, 2) * vrb;   // the tile's shard
    if (!bt.vert(t, 2)) {
      const int r0 = bt.tile_row(slot, mode_pend);
      if (hs == 0) dma_tile_rows(vs_, vb + (int64_t)r0 * vrb, vrb, dl, wave);
    } else {
      if (hs == 0) {
        int rows[4];
        bt.gather_rows(t, slot, rows, wave, lane, 2);
        dma_tile_gather(vs_, vb, rows, vrb, dl, wave);
      }
      mode_pend = 1;
    }
  };
  // S^T for 32 keys (this wave's half) x 32 rows from K stage p: s[rs][t]
  // lane (g, n) = S[row 16 rs + n][key 32 kh + 8 g + 4 t + i]
  auto qk = [&]<int p>(f32x4 (&s)[2][2]) {
    const bf16* Ks = Kst.template operator()<p>();
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int kr = 32 * kh + 8 * (n16 >> 2) + 4 * t + (n16 & 3);
#pragma unroll
      for (int rs = 0; rs < 2; ++rs) s[rs][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 kf = *(const bf16x8*)(Ks + tile_off(kr, 4 * ks + g4));
#pragma unroll
        for (int rs = 0; rs < 2; ++rs) s[rs][t] = mma16<F16>(kf, qf[rs][ks], s[rs][t]);
      }
    }
  };
  // online softmax of S (thresholds in slot p when mode is set) and
  // O^T += V^T P^T from V stage p
  // S of the next tile (from K stage pk) is computed inside the branch-free
  // exponential section so its MFMAs interleave with the vector work.
  auto softmax_pv = [&]<int p, int pk>(f32x4 (&s)[2][2], int mode, const int* thr, const uint32_t* win,
                                        f32x4 (&s_next)[2][2]) {
    if (mode) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 32 * kh + 8 * g4 + 4 * t + i;
          const int th = thr[key];
          uint32_t wk = ~0u;
          if constexpr (S1) wk = win[key];
#pragma unroll
          for (int rs = 0; rs < 2; ++rs) {
            bool off = th > 32 * rh + 16 * rs + n16;
            if constexpr (S1) off = off || !((wk >> qa_l[rs]) & 1u);
            if (off) s[rs][t][i] = -INFINITY;
          }
        }
    }
    // P as a hi + lo bf16 pair (two MFMAs per product), or one fp16 operand
    // (F16; 8x finer rounding than bf16): with bf16 P alone the
    // O error (a few 1e-3) passes into delta = rowsum(dO * O) and from there,
    // scaled by large outlier keys, into dQ beyond the 2e-2 bound
    bf16x8 pf[2], pl[2];
    bool rescale = false;
    float alpha[2], m_use[2];
#pragma unroll
    for (int rs = 0; rs < 2; ++rs) {
      float mx = fmaxf(fmaxf(fmaxf(s[rs][0][0], s[rs][0][1]), fmaxf(s[rs][0][2], s[rs][0][3])),
                       fmaxf(fmaxf(s[rs][1][0], s[rs][1][1]), fmaxf(s[rs][1][2], s[rs][1][3])));
      mx = group4_max(mx);
      // Exact running max: the largest probability of the row is then exactly
      // 1 in bf16, which keeps the dominant term of O free of rounding (a
      // stale reference doubles the O error on peaked rows).
      const float mt = mx * sl2;
      const bool up = mt > m_run[rs];
      const float m_new = up ? mt : m_run[rs];
      m_use[rs] = (m_new == -INFINITY) ? 0.f : m_new;
      alpha[rs] = up ? __builtin_amdgcn_exp2f(m_run[rs] - m_use[rs]) : 1.f;
      rescale |= up;
      m_run[rs] = m_new;
    }
    if (__builtin_amdgcn_ballot_w64(rescale)) {
#pragma unroll
      for (int rs = 0; rs < 2; ++rs)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[rs][dt][i] *= alpha[rs];
    }
#pragma unroll
    for (int rs = 0; rs < 2; ++rs) {
      float psum = 0.f;
      f32x4 pr[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[t][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rs][t][i], sl2, -m_use[rs]));
          psum += pr[t][i];
        }
      weights8<F16>(pr[0], pr[1], pf[rs], pl[rs]);
      l_run[rs] = l_run[rs] * alpha[rs] + psum;
    }
    qk.template operator()<pk>(s_next);
    // 8 K-fragment reads, then one MFMA of the next S per three vector ops
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // O^T += V^T P^T by 16-column blocks dt of V; the transposed V operand of
    // block dt + 2 is read after the first MFMA of block dt (three register
    // sets, order pinned below), so a read has three MFMAs (fp16; seven with
    // bf16 pairs) to land and only blocks 0 and 1 wait out an LDS round trip
    const bf16* Vs = Vst.template operator()<p>();
    const int vr = 32 * kh + 8 * g4 + (n16 >> 2);
    const int vb = (n16 & 3) >> 1, vo = 4 * (n16 & 1);
    bf16x8 va[3];
    auto rdv = [&](int dt, int b) { va[b] = lds_read_tr16_x2(Vs + tile_off(vr, 2 * dt + vb) + vo, D); };
    rdv(0, 0);
    rdv(1, 1);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      if (dt + 2 < 8) rdv(dt + 2, (dt + 2) % 3);
#pragma unroll
      for (int rs = 0; rs < 2; ++rs) {
        acc[rs][dt] = mma16<F16>(va[dt % 3], pf[rs], acc[rs][dt]);
        if constexpr (!F16) acc[rs][dt] = mma16<F16>(va[dt % 3], pl[rs], acc[rs][dt]);
      }
    }
    constexpr int MPB = F16 ? 2 : 4;   // MFMAs per column block
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (dt + 2 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, MPB - 1, 0);
    }
  };

  f32x4 s_cur[2][2];
  // step i (stage parity p = i % 2): S of tile i is in s_cur, K[i+1] in K
  // stage 1-p, V[i] in V stage p, descriptor i+2 in slot (i+2) % 3.
  auto step = [&]<int p>(int i) {
    constexpr int q = 1 - p;
    wait_all_mem();
    __syncthreads();   // copies issued in step i-1 have landed; step i-1 is done everywhere
    const int mode_i = mode_pend;
    if (i + 1 < total) issue_v.template operator()<q>(i + 1);
    if (i + 2 < total) issue_k.template operator()<p>(i + 2);
    if (i + 3 < total) bt.desc_copy(i + 3, desc_sh[i % 3], wave8, lane);
    // (the last step computes a next S from a stale stage and drops it)
    f32x4 s_next[2][2];
    softmax_pv.template operator()<p, q>(s_cur, mode_i, thr_sh[i % 3], win_sh[S1 ? i % 3 : 0], s_next);
#pragma unroll
    for (int rs = 0; rs < 2; ++rs)
#pragma unroll
      for (int t = 0; t < 2; ++t) s_cur[rs][t] = s_next[rs][t];
  };

  if (total > 0) {
#pragma unroll
    for (int t = 0; t < 3; ++t)
      if (t < total) bt.desc_copy(t, desc_sh[t], wave8, lane);
    wait_all_mem();
    __syncthreads();
    issue_k.template operator()<0>(0);
    issue_v.template operator()<0>(0);
    if (total > 1) issue_k.template operator()<1>(1);
    wait_all_mem();
    __syncthreads();
    qk.template operator()<0>(s_cur);
  }
  for (int i0 = 0; i0 < total; i0 += 2) {
    step.template operator()<0>(i0);
    if (i0 + 1 < total) step.template operator()<1>(i0 + 1);
  }

  // ---- merge the two key halves (kh = 1 hands its state to kh = 0 via LDS)
#pragma unroll
  for (int rs = 0; rs < 2; ++rs) l_run[rs] = group4_sum(l_run[rs]);
  __syncthreads();  // every wave is past its last read of the stages
  // [2 rs][8 dt][64 lanes] f32x4 = 16 KiB per row half: K stage 0 / V stage 0
  float* xo = (float*)(hs == 0 ? (rh == 0 ? K0 : V0) : (rh == 0 ? K1 : V1));
  if (kh == 1) {
#pragma unroll
    for (int rs = 0; rs < 2; ++rs) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) *(f32x4*)(xo + ((rs * 8 + dt) * 64 + lane) * 4) = acc[rs][dt];
      xs[(((hs * 2 + rh) * 2 + rs) * 64 + lane) * 2 + 0] = m_run[rs];
      xs[(((hs * 2 + rh) * 2 + rs) * 64 + lane) * 2 + 1] = l_run[rs];
    }
  }
  __syncthreads();
  if (kh == 1) return;
#pragma unroll
  for (int rs = 0; rs < 2; ++rs) {
    const float m1 = xs[(((hs * 2 + rh) * 2 + rs) * 64 + lane) * 2 + 0];
    const float l1 = xs[(((hs * 2 + rh) * 2 + rs) * 64 + lane) * 2 + 1];
    const float m0 = m_run[rs];
    const float mm = fmaxf(m0, m1);
    const float mb = (mm == -INFINITY) ? 0.f : mm;
    const float w0 = __builtin_amdgcn_exp2f(m0 - mb), w1 = __builtin_amdgcn_exp2f(m1 - mb);
    const float l_tot = l_run[rs] * w0 + l1 * w1;
    const bool nonempty = l_tot > 0.f;
    const float inv = nonempty ? 1.f / l_tot : 0.f;
    const float lse_new = nonempty ? (mm + log2f(l_tot)) * LN2 : -INFINITY;
    const int64_t grow = row_base + 16 * rs + n16;
    float* orow = a.o + ((int64_t)h * a.QB * BLK + grow) * D;
    float* lrow = a.lse + (int64_t)h * a.QB * BLK + grow;
    // O and LSE are written once and not read again by this kernel: stream
    // them past the caches (non-temporal) so they do not evict K/V tiles
    float ca = 0.f, cb = inv;
    if (a.accumulate) {
      const float lse_old = *lrow;
      const float mxl = fmaxf(lse_old, lse_new);
      const float base = (mxl == -INFINITY) ? 0.f : mxl;
      const float wa = expf(lse_old - base), wb = expf(lse_new - base);
      const float tot = wa + wb;
      ca = tot > 0.f ? wa / tot : 0.f;
      cb = tot > 0.f ? wb / tot * inv : 0.f;
      if (g4 == 0) *lrow = tot > 0.f ? base + logf(tot) : -INFINITY;
    } else if (g4 == 0) {
      *lrow = lse_new;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const f32x4 o1 = *(const f32x4*)(xo + ((rs * 8 + dt) * 64 + lane) * 4);
      f32x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = (acc[rs][dt][i] * w0 + o1[i] * w1) * cb;
      if (a.accumulate) {
        const f32x4 old = *(const f32x4*)(orow + 16 * dt + 4 * g4);
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] += ca * old[i];
      }
      __builtin_nontemporal_store(r, (f32x4*)(orow + 16 * dt + 4 * g4));
    }
  }
}
__global__ void __launch_bounds__(FWD_THREADS, 2) attn_fwd_bf16_d128_kernel(FwdArgs a) {
  attn_fwd_d128<false, 1>(a);
}
__global__ void __launch_bounds__(FWD_THREADS, 2) attn_fwd_f16_d128_kernel(FwdArgs a) { attn_fwd_d128<true, 1>(a); }
__global__ void __launch_bounds__(FWD_THREADS, 2) attn_fwd_ring_bf16_d128_kernel(FwdArgs a, RingSteps rs) {
  attn_fwd_d128<false, 1, true>(a, &rs);
}
__global__ void __launch_bounds__(FWD_THREADS, 2) attn_fwd_ring_f16_d128_kernel(FwdArgs a, RingSteps rs) {
  attn_fwd_d128<true, 1, true>(a, &rs);
}
__global__ void __launch_bounds__(FWD_THREADS, 2) attn_fwd_s1_bf16_d128_kernel(FwdArgs a) {
  attn_fwd_d128<false, 1, false, true>(a);
}
__global__ void __launch_bounds__(FWD_THREADS, 2) attn_fwd_s1_f16_d128_kernel(FwdArgs a) {
  attn_fwd_d128<true, 1, false, true>(a);
}
__global__ void __launch_bounds__(2 * FWD_THREADS, 1) attn_fwd_pair_bf16_d128_kernel(FwdArgs a) {
  attn_fwd_d128<false, 2>(a);
}
__global__ void __launch_bounds__(2 * FWD_THREADS, 1) attn_fwd_pair_f16_d128_kernel(FwdArgs a) {
  attn_fwd_d128<true, 2>(a);
}

int launch_attn_fwd(int dtype, int D, TView q, TView k, TView v, const vs_mask* m, float scale,
                    float* o, float* lse, int accumulate, hipStream_t stream) {
  FwdArgs a;
  a.q = q.ptr; a.k = k.ptr; a.v = v.ptr;
  a.qsh = q.sh; a.qsn = q.sn; a.ksh = k.sh; a.ksn = k.sn; a.vsh = v.sh; a.vsn = v.sn;
  a.tile_ptr = m->tile_ptr; a.tile_col = m->tile_col; a.vloc = m->vloc; a.vert_end = m->vert_end;
  a.slash_bits = m->slash_bits; a.o = o; a.lse = lse; a.status = nullptr;
  a.Hq = m->Hq; a.Hkv = m->Hkv; a.QB = m->QB; a.KB = m->KB; a.W = m->W; a.kind = m->lay.kind;
  a.P = m->lay.P; a.rank = m->rank; a.src = m->src; a.accumulate = accumulate;
  a.scale_log2 = scale * LOG2E;
  a.dbg = debug_word(); a.cap = m->tile_cap;
  const dim3 grid(xcd_group_grid(m->Hkv, m->QB, QMAJOR_BPC, m->Hq / m->Hkv)), block(FWD_THREADS);
  if ((dtype == VS_BF16 || dtype == VS_F16) && D == 128) {
    if (m->W > MAX_LDS_W) return VS_ERR_UNSUPPORTED;
    const int64_t krows = (int64_t)m->KB * BLK;
    if (!dma_offsets_fit(krows, k.sn) || !dma_offsets_fit(krows, v.sn)) return VS_ERR_UNSUPPORTED;
    const bool s1 = m->lay.kind == VS_STRIPED1;
    if (dtype == VS_F16) {
      if (s1) hipLaunchKernelGGL(attn_fwd_s1_f16_d128_kernel, grid, block, 0, stream, a);
      else hipLaunchKernelGGL(attn_fwd_f16_d128_kernel, grid, block, 0, stream, a);
    } else {
      if (s1) hipLaunchKernelGGL(attn_fwd_s1_bf16_d128_kernel, grid, block, 0, stream, a);
      else hipLaunchKernelGGL(attn_fwd_bf16_d128_kernel, grid, block, 0, stream, a);
    }
  }
  else if (m->lay.kind == VS_STRIPED1) return VS_ERR_UNSUPPORTED;   // one-position stripes: D = 128 only
  else if (dtype == VS_BF16 && D == 64) hipLaunchKernelGGL((attn_fwd_kernel<bf16, 64>), grid, block, 0, stream, a);
  else if (dtype == VS_F32 && D == 64) hipLaunchKernelGGL((attn_fwd_kernel<float, 64>), grid, block, 0, stream, a);
  else return VS_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? VS_OK : VS_ERR_HIP;
}

// Two q heads per workgroup sharing the K/V tile copies (requires equal active
// sets within each head pair; checked per workgroup, reported in *status).
int launch_attn_fwd_packed(int dtype, TView q, TView k, TView v, const vs_mask* m, float scale, float* o,
                           float* lse, int accumulate, int32_t* status, hipStream_t stream) {
  FwdArgs a;
  a.q = q.ptr; a.k = k.ptr; a.v = v.ptr;
  a.qsh = q.sh; a.qsn = q.sn; a.ksh = k.sh; a.ksn = k.sn; a.vsh = v.sh; a.vsn = v.sn;
  a.tile_ptr = m->tile_ptr; a.tile_col = m->tile_col; a.vloc = m->vloc; a.vert_end = m->vert_end;
  a.slash_bits = m->slash_bits; a.o = o; a.lse = lse; a.status = status;
  a.Hq = m->Hq; a.Hkv = m->Hkv; a.QB = m->QB; a.KB = m->KB; a.W = m->W; a.kind = m->lay.kind;
  a.P = m->lay.P; a.rank = m->rank; a.src = m->src; a.accumulate = accumulate;
  a.scale_log2 = scale * LOG2E;
  a.dbg = debug_word(); a.cap = m->tile_cap;
  if (m->W > MAX_LDS_W) return VS_ERR_UNSUPPORTED;
  const int64_t krows = (int64_t)m->KB * BLK;
  if (!dma_offsets_fit(krows, k.sn) || !dma_offsets_fit(krows, v.sn)) return VS_ERR_UNSUPPORTED;
  const dim3 grid(xcd_group_grid(m->Hkv, m->QB, QMAJOR_BPC, m->Hq / m->Hkv / 2)), block(2 * FWD_THREADS);
  if (dtype == VS_F16) hipLaunchKernelGGL(attn_fwd_pair_f16_d128_kernel, grid, block, 0, stream, a);
  else hipLaunchKernelGGL(attn_fwd_pair_bf16_d128_kernel, grid, block, 0, stream, a);
  return hipGetLastError() == hipSuccess ? VS_OK : VS_ERR_HIP;
}

// Several ring steps of one rank in one launch per group of up to
// MAX_RING_STEPS steps: k, v hold every shard in storage order (shard r at
// rows r * KB * 64); the first group honours `accumulate`, later groups merge
// into its result.
int launch_attn_fwd_ring(int dtype, TView q, TView k, TView v, const vs_mask* ms, int nsteps, float scale, float* o,
                         float* lse, int accumulate, hipStream_t stream) {
  const vs_mask* m = &ms[0];
  FwdArgs a;
  a.q = q.ptr; a.k = k.ptr; a.v = v.ptr;
  a.qsh = q.sh; a.qsn = q.sn; a.ksh = k.sh; a.ksn = k.sn; a.vsh = v.sh; a.vsn = v.sn;
  a.tile_ptr = nullptr; a.tile_col = nullptr; a.vloc = nullptr; a.vert_end = nullptr;
  a.slash_bits = m->slash_bits; a.o = o; a.lse = lse; a.status = nullptr;
  a.Hq = m->Hq; a.Hkv = m->Hkv; a.QB = m->QB; a.KB = m->KB; a.W = m->W; a.kind = m->lay.kind;
  a.P = m->lay.P; a.rank = m->rank; a.src = -1;
  a.scale_log2 = scale * LOG2E;
  a.dbg = debug_word(); a.cap = m->tile_cap;
  if (m->W > MAX_LDS_W) return VS_ERR_UNSUPPORTED;
  // 32-bit copy offsets over every shard (vertical chunks gather storage rows)
  const int64_t krows = (int64_t)m->lay.P * m->KB * BLK;
  if (!dma_offsets_fit(krows, k.sn) || !dma_offsets_fit(krows, v.sn)) return VS_ERR_UNSUPPORTED;
  const dim3 grid(xcd_group_grid(m->Hkv, m->QB, QMAJOR_BPC, m->Hq / m->Hkv)), block(FWD_THREADS);
  for (int s0 = 0; s0 < nsteps; s0 += MAX_RING_STEPS) {
    RingSteps rs{};
    rs.nsteps = nsteps - s0 < MAX_RING_STEPS ? nsteps - s0 : MAX_RING_STEPS;
    rs.cap = m->tile_cap;
    for (int s = 0; s < rs.nsteps; ++s) {
      const vs_mask& ms_s = ms[s0 + s];
      rs.tile_ptr[s] = ms_s.tile_ptr; rs.tile_col[s] = ms_s.tile_col; rs.vloc[s] = ms_s.vloc;
      rs.vert_end[s] = ms_s.vert_end; rs.src[s] = ms_s.src;
    }
    a.accumulate = s0 == 0 ? accumulate : 1;
    if (dtype == VS_F16) hipLaunchKernelGGL(attn_fwd_ring_f16_d128_kernel, grid, block, 0, stream, a, rs);
    else if (dtype == VS_BF16) hipLaunchKernelGGL(attn_fwd_ring_bf16_d128_kernel, grid, block, 0, stream, a, rs);
    else return VS_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? VS_OK : VS_ERR_HIP;
}

// ---- log-sum-exp merge ------------------------------------------------------
// One thread per (row, 4 consecutive features).
__global__ void merge_kernel(float* o_acc, float* lse_acc, const float* o_step, const float* lse_step,
                             int64_t rows, int D) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per = D / 4;
  if (t >= rows * per) return;
  const int64_t r = t / per;
  const int c = (int)(t % per) * 4;
  const float la = lse_acc[r], lb = lse_step[r];
  const float mx = fmaxf(la, lb);
  const float base = (mx == -INFINITY) ? 0.f : mx;
  const float wa = expf(la - base), wb = expf(lb - base);
  const float tot = wa + wb;
  const float ca = tot > 0.f ? wa / tot : 0.f, cb = tot > 0.f ? wb / tot : 0.f;
  f32x4 x = *(const f32x4*)(o_acc + r * D + c);
  const f32x4 y = *(const f32x4*)(o_step + r * D + c);
  #pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = ca * x[i] + cb * y[i];
  *(f32x4*)(o_acc + r * D + c) = x;
  // the row's LSE is written by the thread of its first feature group after
  // the other groups of the same row have read it: rows never straddle a
  // wave boundary (D/4 divides 64), and a wave's loads complete before its stores
  if (c == 0) lse_acc[r] = tot > 0.f ? base + logf(tot) : -INFINITY;
}

int launch_merge(float* o_acc, float* lse_acc, const float* o_step, const float* lse_step,
                 int Hq, int64_t Nq, int D, hipStream_t stream) {
  const int64_t rows = (int64_t)Hq * Nq;
  const int64_t n = rows * (D / 4);
  const int tpb = 256;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((n + tpb - 1) / tpb)), dim3(tpb), 0, stream,
                     o_acc, lse_acc, o_step, lse_step, rows, D);
  return hipGetLastError() == hipSuccess ? VS_OK : VS_ERR_HIP;
}

}  // namespace vs
