/*
 * vs_attn.h -- C ABI of the vertical-slash (VS) dynamic sparse attention path
 * for AMD Instinct MI355X (gfx950).
 *
 * The path is the per-rank hot path of MTraining (review page "MTraining:
 * 分布式动态稀疏注意力高效超长上下文训练", xllm-io paper-review):
 *   1. vs_index_build  -- online sparse-index approximation (section 三.2 item 1
 *                         and 2): score the last queries against every key, take
 *                         the attention mass of token-level vertical columns and
 *                         of 64x64 block-level slash diagonals, and keep the
 *                         fewest of each that reach the top-p budget;
 *   2. vs_block_mask   -- each worker derives the active region of its local
 *                         attention sub-matrix from the shared index (section
 *                         三.2 item 3);
 *   3. vs_attn_fwd     -- block-sparse flash attention over only the active
 *                         entries of one ring step (same item);
 *   4. vs_merge_lse    -- incremental-softmax merge of partial results across
 *                         ring steps (Ring Attention overview page,
 *                         intelliparadigm, section 2.1);
 *   5. vs_attn_bwd_prep / vs_attn_bwd -- gradient of the same sparse attention.
 *
 * Conventions shared by every call:
 *   - All data pointers are DEVICE pointers unless stated otherwise. The
 *     library never allocates, frees or retains device memory: every buffer,
 *     including scratch, is owned by the caller.
 *   - Every compute call is asynchronous on `stream` (a hipStream_t; NULL is
 *     the default stream). Host-side validation errors are returned
 *     synchronously; a kernel launch failure returns VS_ERR_HIP. Conditions
 *     found on the device (list capacity overflow) are written to a device
 *     status word that the caller reads after synchronising the stream.
 *   - A token position is "global" when it indexes the whole sequence and
 *     "local" when it indexes one rank's shard in storage order.
 *   - Every `scale` argument must be finite and positive, else VS_ERR_ARG.
 *   - Attention uses natural-log LSE, logits q.k * scale (scale = 1/sqrt(D)),
 *     query head h reads kv head h / (Hq / Hkv). Empty rows give O = 0 and
 *     LSE = -inf and contribute no gradient.
 *   - The active set of query head h with vertical set V_h (global positions)
 *     and slash set S_h (block-diagonal ids, block = 64 tokens) is
 *       M_h[n, m] = [m <= n] and ([m in V_h] or [n/64 - m/64 in S_h]).
 * Supported: D in {64, 128}; dtype f32 or bf16 (q, k, v, dout alike); every
 * local length a multiple of 64; Hq a multiple of Hkv; last_q in [1, 64].
 * The attention calls (vs_attn_fwd, vs_attn_bwd_prep, vs_attn_bwd*) also take
 * fp16 at D = 128: exact copies of bf16 data made by vs_convert_f16, on
 * which the attention weights P and dS enter their products as single fp16
 * operands (11 significant bits) instead of hi + lo bf16 pairs.
 */
#ifndef VS_ATTN_H
#define VS_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VS_OK = 0,
  VS_ERR_ARG = -1,          /* null pointer, inconsistent shape or bad value   */
  VS_ERR_UNSUPPORTED = -2,  /* valid but not implemented (head dim, alignment) */
  VS_ERR_WORKSPACE = -3,    /* workspace or mask buffer too small              */
  VS_ERR_CAPACITY = -4,     /* device-side list capacity exceeded (status word) */
  VS_ERR_HIP = -5,          /* a HIP runtime call or kernel launch failed      */
  VS_ERR_RANGE = -6         /* a value outside the target type (status word)   */
} vs_status;

typedef enum { VS_F32 = 0, VS_BF16 = 1, VS_F16 = 2 } vs_dtype;

/* How global positions are dealt to the P ranks of the context-parallel ring
 * (review page 1, section 三.3):
 *   VS_CONTIG  -- rank r holds [r*N/P, (r+1)*N/P);
 *   VS_STRIPED -- 64-token stripes round-robin: rank r holds global blocks
 *                 G with G mod P == r (the balanced layout);
 *   VS_ZIGZAG  -- 2P equal chunks, rank r holds chunks r and 2P-1-r;
 *   VS_STRIPED1 -- single positions dealt round-robin: rank r holds the
 *                 positions n with n mod P == r (the fine-grained stripes of
 *                 the Ring Attention overview, section 3.1); P <= 32. A
 *                 local 64-row tile then spans P global blocks, so listed
 *                 tiles are mostly partial (VS_TILE_DIAG marks them) and the
 *                 attention kernels evaluate the active set entry by entry in
 *                 them. The index calls refuse this kind for P > 1
 *                 (VS_ERR_UNSUPPORTED): build the index on the keys in global
 *                 order (VS_CONTIG, P = 1); the lists are global positions
 *                 and diagonals, the same under every layout.
 * A shard is stored in ascending global order. P = 1 is the plain sequence. */
typedef enum { VS_CONTIG = 0, VS_STRIPED = 1, VS_ZIGZAG = 2, VS_STRIPED1 = 3 } vs_layout_kind;

typedef struct {
  int32_t kind;      /* vs_layout_kind */
  int32_t P;         /* ranks, >= 1 */
  int64_t n_global;  /* whole sequence length, a multiple of 64*P (128*P for zigzag) */
} vs_layout;

/* A [H, N, D] tensor view; D is contiguous, strides are in elements. */
typedef struct {
  const void* ptr;
  int32_t dtype;     /* vs_dtype */
  int32_t H;
  int64_t N;
  int32_t D;
  int64_t stride_h;
  int64_t stride_n;
} vs_tensor;

/* Flag bit on tile_col / csc_row entries: not every entry of the tile is
 * active, so a predicate applies inside it. Under the 64-token layouts that
 * is exactly the query block's own global block (the causal cut); under
 * VS_STRIPED1 any tile not wholly covered by selected diagonals. */
#define VS_TILE_DIAG 0x40000000
#define VS_TILE_MASK 0x3FFFFFFF

/* Host-side descriptor of the active region of one (rank, ring step), with
 * device arrays carved from one caller-owned device buffer by vs_mask_init.
 * QB = local query blocks, KB = local key blocks (= QB), T = global blocks.
 *   tile_ptr[Hq*QB+1], tile_col[tile_cap]: per (head h, query block I) the
 *       ascending local key blocks J of the visible shard whose 64x64 tile
 *       holds a slash-active entry (CSR), ORed with VS_TILE_DIAG;
 *   csc_ptr[Hq*KB+1], csc_row[tile_cap]: the same pairs per (h, J), listing
 *       ascending I (CSC), ORed with VS_TILE_DIAG;
 *   vloc[Hq*KB*64] (head h at h*KB*64), vloc_cnt[Hq]: ascending local
 *       positions of the visible shard's vertical columns;
 *   vcum[Hq*(KB+1)]: vertical columns of the shard before local block J;
 *   vert_end[Hq*QB]: the first vert_end entries of vloc have an active entry
 *       in query block I (those in a listed tile are covered by it and are
 *       skipped by the kernels);
 *   slash_bits[Hq*W], W = ceil(T/32): bit j set iff j in S_h;
 *   n_active[Hq*QB]: active entries of query block I in this shard (exact);
 *   status[1]: VS_OK or VS_ERR_CAPACITY after vs_block_mask. */
typedef struct {
  int32_t Hq, Hkv, QB, KB, T, W;
  vs_layout lay;
  int64_t tile_cap;
  int32_t rank, src;          /* set by vs_block_mask */
  int32_t* tile_ptr;
  int32_t* tile_col;
  int32_t* csc_ptr;
  int32_t* csc_row;
  int32_t* vloc;
  int32_t* vloc_cnt;
  int32_t* vcum;
  int32_t* vert_end;
  uint32_t* slash_bits;
  int64_t* n_active;
  int32_t* status;
} vs_mask;

/* Human-readable name of a status code (static string). */
const char* vs_status_string(int status);

/* ---- 1. sparse index -------------------------------------------------- */

/* Workspace bytes vs_index_build needs (device memory). */
size_t vs_index_workspace_size(int Hq, int Hkv, int64_t n_global, int D, int last_q);

/* Online sparse-index approximation (review page 1, section 三.2 items 1-2).
 *   q_last: [Hq, last_q, D], the queries at global rows n_global-last_q ..
 *           n_global-1;
 *   k:      [Hkv, n_global, D], every key, shards concatenated in rank order
 *           under `lay` (for P = 1: global order);
 *   scale:  logit scale (1/sqrt(D));
 *   top_p:  target mass; >= 1 keeps every element, <= 0 keeps none.
 * Outputs (device, caller-owned):
 *   vert_score[Hq, n_global]  fp32: v_h(m) = (1/last_q) sum over the scored
 *       rows n >= m of softmax_n(m), indexed by global position;
 *   slash_score[Hq, n_global/64] fp32: s_h(j) = mass on block-diagonal j;
 *   vert_idx[Hq, n_global], vert_cnt[Hq]: per head the selected global
 *       positions, ascending (row stride n_global);
 *   slash_idx[Hq, n_global/64], slash_cnt[Hq]: selected diagonals, ascending.
 * Selection: per head and separately for v and s, the fewest elements in
 * descending score order (ties: lower index first) whose fixed-point mass
 * sum_i round(x_i * 2^40) reaches ceil(round(p * 2^32) * total / 2^32). */
int vs_index_build(vs_tensor q_last, vs_tensor k, vs_layout lay, float scale, float top_p,
                   float* vert_score, float* slash_score,
                   int32_t* vert_idx, int32_t* vert_cnt,
                   int32_t* slash_idx, int32_t* slash_cnt,
                   void* ws, size_t ws_bytes, void* stream);

/* vs_index_build for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments without the workspace, whose role a scratch array
 * inside the library takes: VS_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU, held
 * from the first call on that GPU until the process ends. The call itself
 * allocates nothing. Calls whose vs_index_workspace_size exceeds the scratch
 * return VS_ERR_WORKSPACE before any device work (it holds Hq = 128 q heads
 * at 2^20 tokens). Every call on one GPU uses that GPU's one scratch array:
 * calls that overlap on a GPU (concurrent streams or host threads) race and
 * must be serialised by the caller; consecutive calls on one stream are
 * safe (nothing in the scratch needs to start at zero: every pass writes
 * what it reads). VS_ERR_HIP if the device's scratch address cannot be
 * looked up. Results equal vs_index_build's bit for bit. */
#define VS_NOALLOC_SCRATCH_BYTES (16 << 20)
int vs_index_build_noalloc(vs_tensor q_last, vs_tensor k, vs_layout lay, float scale, float top_p,
                           float* vert_score, float* slash_score, int32_t* vert_idx, int32_t* vert_cnt,
                           int32_t* slash_idx, int32_t* slash_cnt, void* stream);

/* The same index built the distributed way (review page 1, section 三.2
 * item 1: the scored queries are broadcast and every rank scores them
 * against the keys it holds). Per rank r, with exchanges between the calls:
 *   1. vs_index_rank_stats: the rank's partial row statistics;
 *   2. all-gather of the P slots into all_stats[P][Hq][64][2];
 *   3. vs_index_rank_mass: merged row LSE, then the rank's entries of the
 *      vertical and slash scores;
 *   4. all-gather of the score entries (ranks write disjoint entries);
 *   5. vs_index_select on the gathered scores (the same on every rank).
 * On one GPU the ranks run one after another and the exchange buffers are
 * shared. The scores equal vs_index_build's up to fp32 rounding of the
 * merge (the summation order differs), and the selection follows from them
 * by the same rule.
 *
 * vs_index_rank_stats:
 *   q_last:  [Hq, last_q, D], as for vs_index_build;
 *   k_local: [Hkv, n_global / P, D], rank `rank`'s keys in storage order
 *            under `lay`;
 *   stats:   [Hq, 64, 2] fp32 (device, caller-owned; rows >= last_q are
 *            unused): per scored row, the largest logit over the rank's
 *            causal keys in log2 units (logit * log2 e) and the sum of
 *            2^(logit * log2 e - largest); (-inf, 0) when the rank holds no
 *            causal key of the row;
 *   ws:      vs_index_workspace_size(Hq, Hkv, n_global, D, last_q) bytes.
 * Errors: as vs_index_build; VS_ERR_ARG for rank outside [0, P). */
int vs_index_rank_stats(vs_tensor q_last, vs_tensor k_local, vs_layout lay, int rank, float scale,
                        float* stats, void* ws, size_t ws_bytes, void* stream);

/* vs_index_rank_mass:
 *   all_stats: [P, Hq, 64, 2] fp32, every rank's stats slot (read-only);
 *   vert_score [Hq, n_global], slash_score [Hq, n_global / 64]: written only
 *     at the global positions of the rank's keys and at the diagonals of its
 *     key blocks (block-diagonal T-1-G for key block G), other entries are
 *     left as they are;
 *   other arguments and errors as vs_index_rank_stats. */
int vs_index_rank_mass(vs_tensor q_last, vs_tensor k_local, vs_layout lay, int rank, float scale,
                       const float* all_stats, float* vert_score, float* slash_score,
                       void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes vs_index_select needs (device memory; 0 for Hq <= 0 or
 * n_global <= 0). */
size_t vs_index_select_workspace_size(int Hq, int64_t n_global);

/* vs_index_select: the top-p selection of vs_index_build on given scores
 * (vert_score [Hq, n_global], slash_score [Hq, n_global / 64], non-negative
 * fp32); outputs as for vs_index_build; ws: caller-owned scratch of
 * vs_index_select_workspace_size bytes (contents need no initialisation).
 * VS_ERR_ARG for null pointers, Hq <= 0 or a NaN top_p; VS_ERR_UNSUPPORTED if
 * n_global is not a multiple of 64; VS_ERR_WORKSPACE if ws_bytes is too
 * small. */
int vs_index_select(const float* vert_score, const float* slash_score, int Hq, int64_t n_global, float top_p,
                    int32_t* vert_idx, int32_t* vert_cnt, int32_t* slash_idx, int32_t* slash_cnt,
                    void* ws, size_t ws_bytes, void* stream);

/* Per-kv-head variant of the selection (grouped-query attention; the review
 * fixes one index per attention head, page 1, section 三.2 item 1, and this
 * variant takes the head to be the kv head): for every kv group g of R =
 * Hq / Hkv consecutive q heads, v_g = (1/R) sum_{h in g} v_h and likewise
 * s_g (fp32, heads added in ascending order, then scaled by 1/R); the top-p
 * rule of vs_index_select is applied once per group; every q head of the
 * group receives the group's lists. Outputs as vs_index_select ([Hq, ...]).
 * All q heads of a group then share one active set, which is what
 * vs_attn_fwd_packed requires. ws: vs_index_select_group_workspace_size
 * bytes. Errors as vs_index_select, plus VS_ERR_ARG if Hkv <= 0 or
 * Hq % Hkv != 0. */
size_t vs_index_select_group_workspace_size(int Hq, int Hkv, int64_t n_global);
int vs_index_select_group(const float* vert_score, const float* slash_score, int Hq, int Hkv, int64_t n_global,
                          float top_p, int32_t* vert_idx, int32_t* vert_cnt, int32_t* slash_idx,
                          int32_t* slash_cnt, void* ws, size_t ws_bytes, void* stream);

/* Budget kinds of vs_index_select_budget. */
#define VS_BUDGET_TOP_P 0        /* separate top-p on v and on s (vs_index_select) */
#define VS_BUDGET_TOP_K 1        /* a fixed count per head */
#define VS_BUDGET_JOINT_TOP_P 2  /* one top-p over the pooled v and s candidates */

/* vs_index_select_budget: vs_index_select with a choice of budget rule, on
 * the same scores, outputs, workspace and errors (VS_ERR_ARG also for an
 * unknown `budget`).
 *   VS_BUDGET_TOP_P: as vs_index_select; k_vert, k_slash unused.
 *   VS_BUDGET_TOP_K: a fixed count, the form of the budget behind the review's
 *     hand-fixed 95% sparsity (page 1, section 八 item 4): per head the
 *     min(k_vert, n_global) largest vertical scores and the
 *     min(k_slash, n_global / 64) largest slash scores, ties to the lower
 *     index; a count <= 0 keeps none of that direction. top_p unused.
 *   VS_BUDGET_JOINT_TOP_P: the fewest verticals plus slashes of section 三.2
 *     item 1 read as one count: per head the n_global verticals followed by
 *     the n_global / 64 slashes form one candidate list, and the fewest in
 *     descending score order (ties: verticals first, then the lower index)
 *     whose fixed-point mass reaches ceil(round(p * 2^32) * total / 2^32) of
 *     the pooled total are kept (p >= 1: all, p <= 0: none). k_vert, k_slash
 *     unused.
 * Each output list is ascending, with its count in vert_cnt / slash_cnt. */
int vs_index_select_budget(const float* vert_score, const float* slash_score, int Hq, int64_t n_global, int budget,
                           float top_p, int k_vert, int k_slash, int32_t* vert_idx, int32_t* vert_cnt,
                           int32_t* slash_idx, int32_t* slash_cnt, void* ws, size_t ws_bytes, void* stream);

/* ---- 2. active region ------------------------------------------------- */

/* Device bytes of one mask buffer able to hold `tile_cap` (h, I, J) tiles. */
size_t vs_mask_bytes(int Hq, int Hkv, vs_layout lay, int64_t tile_cap);

/* Carve a caller-owned device buffer into the arrays of `m` (host call, no
 * device work). Returns VS_ERR_WORKSPACE if `bytes` is too small. */
int vs_mask_init(vs_mask* m, void* buf, size_t bytes, int Hq, int Hkv, vs_layout lay, int64_t tile_cap);

/* Derive the active region of rank `rank` at ring step `step` (visible KV
 * shard src = (rank - step) mod P) from the shared index (review page 1,
 * section 三.2 item 3). vert_idx/slash_idx rows have strides vert_stride /
 * slash_stride (elements) and hold vert_cnt[h] / slash_cnt[h] ascending
 * entries. Fills every array of `m`. If the tile lists need more than
 * m->tile_cap entries, the device writes VS_ERR_CAPACITY to m->status and
 * leaves every list empty (tile_ptr and csc_ptr all zero, vloc_cnt and
 * vert_end zero; n_active still holds the exact counts), so attention calls
 * queued behind it on the stream read no list entry and compute nothing for
 * the step (vs_attn_fwd then writes O = 0, LSE = -inf, or leaves an
 * accumulating merge unchanged). The caller reads the status word after
 * synchronising. */
int vs_block_mask(const int32_t* vert_idx, const int32_t* vert_cnt, int64_t vert_stride,
                  const int32_t* slash_idx, const int32_t* slash_cnt, int64_t slash_stride,
                  int rank, int step, vs_mask* m, void* stream);

/* The active regions of steps 0 .. nsteps-1 of rank `rank` (1 <= nsteps <=
 * P), written to masks[0 .. nsteps-1] (host array of descriptors carved by
 * vs_mask_init for the same shape, layout and tile_cap), each exactly as
 * vs_block_mask(..., rank, step, &masks[step], ...) writes it, by the same
 * four launches for up to 32 steps at a time (the masks a rank's resident
 * ring consumes). Errors as vs_block_mask, plus VS_ERR_ARG for masks of
 * different shapes; overflow is reported in each mask's own status word. */
int vs_block_mask_ring(const int32_t* vert_idx, const int32_t* vert_cnt, int64_t vert_stride,
                       const int32_t* slash_idx, const int32_t* slash_cnt, int64_t slash_stride,
                       int rank, vs_mask* masks, int nsteps, void* stream);

/* ---- 3./4. forward and merge ----------------------------------------- */

/* Sparse attention of the rank's queries against one visible KV shard,
 * computing only the tiles and vertical columns listed in `m`.
 *   q: [Hq, QB*64, D] (rank's shard), k, v: [Hkv, KB*64, D] (shard m->src);
 *   o: [Hq, QB*64, D] fp32 contiguous, lse: [Hq, QB*64] fp32.
 * accumulate = 0: o, lse receive this step's normalised output and LSE.
 * accumulate = 1: (o, lse) hold a running merge (start: o = 0, lse = -inf)
 *   and this step's result is merged into them in place (same formula as
 *   vs_merge_lse), without writing the step's own output. */
int vs_attn_fwd(vs_tensor q, vs_tensor k, vs_tensor v, const vs_mask* m, float scale,
                float* o, float* lse, int accumulate, void* stream);

/* vs_attn_fwd with two q heads per workgroup: q heads 2i and 2i + 1 of
 * every kv group share the workgroup and every K/V tile copy (half the tile
 * traffic of vs_attn_fwd). Same arguments, outputs and results as
 * vs_attn_fwd, for masks whose two heads of each such pair have identical
 * active sets (built from vs_index_select_group lists). Each workgroup
 * compares its pair's tile list and vertical columns and, if they differ,
 * writes VS_ERR_ARG to the device word *status (set to VS_OK by the caller)
 * and leaves its rows of o / lse unwritten. Supported: bf16 or fp16 operands,
 * D = 128, Hq / Hkv even (else VS_ERR_UNSUPPORTED). */
int vs_attn_fwd_packed(vs_tensor q, vs_tensor k, vs_tensor v, const vs_mask* m, float scale,
                       float* o, float* lse, int accumulate, int32_t* status, void* stream);

/* In-place log-sum-exp merge (Ring Attention overview, section 2.1):
 *   L = log(e^La + e^Lb), O = e^(La-L) Oa + e^(Lb-L) Ob, (0, -inf) = identity.
 * o_acc/o_step: [Hq, Nq, D] fp32 contiguous; lse_acc/lse_step: [Hq, Nq]. */
int vs_merge_lse(float* o_acc, float* lse_acc, const float* o_step, const float* lse_step,
                 int Hq, int64_t Nq, int D, void* stream);

/* ---- 16-bit operand format -------------------------------------------- */

/* dst[i] = fp16(src[i]) for n contiguous bf16 values (src, dst 16-byte
 * aligned device buffers of n * 2 bytes, n a multiple of 8, not overlapping).
 * Not a step of the pages' method: it changes only the bit format the
 * attention kernels read. bf16 keeps 8 significant bits, fp16 11, so the
 * conversion is exact for 2^-17 <= |x| < 65536 and for 0; smaller magnitudes
 * are rounded to fp16's 2^-24 spacing (absolute error <= 2^-25). A value
 * with |x| >= 65536 (including inf) or a NaN is a range error: the kernel
 * writes VS_ERR_RANGE to the device word *status (which the caller sets to
 * VS_OK beforehand and reads after synchronising) and dst is then
 * unspecified. Inputs of larger range are pre-scaled by the caller by a power
 * of two (exact), with the scale folded into `scale` or the outputs.
 * Errors: VS_ERR_ARG for null pointers or n < 0; VS_ERR_UNSUPPORTED for
 * misaligned buffers or n % 8 != 0. */
int vs_convert_f16(const void* src, void* dst, int64_t n, int32_t* status, void* stream);

/* ---- 5. backward ------------------------------------------------------ */

/* delta[h, n] = sum_d dout[h, n, d] * o[h, n, d] (the row term of the
 * softmax gradient), from the FINAL output o [Hq, Nq, D] fp32 contiguous. */
int vs_attn_bwd_prep(const float* o, vs_tensor dout, float* delta, void* stream);

/* vs_attn_bwd_prep for bf16 dO that also writes its fp16 copy (the operand
 * of the fp16 backward kernels), reading dO once: dout [Hq, Nq, D] bf16
 * contiguous (read), dout_f16 [Hq, Nq, D] fp16 contiguous (written, as
 * vs_convert_f16 would), delta as vs_attn_bwd_prep (bit for bit the same as
 * vs_attn_bwd_prep on either copy). Range errors as vs_convert_f16, in the
 * device word *status. VS_ERR_ARG for null pointers or Hq, Nq <= 0;
 * VS_ERR_UNSUPPORTED for D not in {64, 128} or misaligned buffers. */
int vs_attn_bwd_prep_f16(const float* o, const void* dout, void* dout_f16, int Hq, int64_t Nq, int D,
                         float* delta, int32_t* status, void* stream);

/* Gradient contribution of the active entries of `m` (one ring step), using
 * the final lse [Hq, Nq] and delta [Hq, Nq] of the rank's rows:
 *   P = exp(q.k*scale - lse), dV += P^T dO, dS = P (dO.v - delta),
 *   dQ += dS K scale, dK += dS^T Q scale, summed over the q heads of a kv head.
 * dq [Hq, Nq, D], dk/dv [Hkv, Nk, D]: fp32 contiguous, accumulated (+=); the
 * caller zeroes them before the first step. dk/dv contributions of vertical
 * columns are added with fp32 atomics, so their low bits may vary run to run. */
int vs_attn_bwd(vs_tensor q, vs_tensor k, vs_tensor v, vs_tensor dout,
                const float* lse, const float* delta, const vs_mask* m, float scale,
                float* dq, float* dk, float* dv, void* stream);

/* The same gradient in separately launchable parts (each one kernel), for
 * callers that schedule them on different streams or time them apart:
 *   VS_BWD_DQ    -- dq of the rank's rows (query-major over the tile lists);
 *   VS_BWD_DKDV  -- dk/dv of the keys inside listed slash tiles (key-major
 *                   over the CSC lists; plain read-modify-write);
 *   VS_BWD_DKDV_VERT -- dk/dv of the vertical columns (fp32 atomics).
 * At D = 128 (bf16 and fp16 operands) a head's vertical columns belong to
 * VS_BWD_DKDV_VERT over every causal row, also inside that head's listed
 * tiles, which VS_BWD_DKDV then leaves out: a vertical column sums its
 * weights over up to the whole sequence, and that part forms the products
 * with hi + lo weight pairs. (D = 64 and fp32 keep such entries in the tile
 * part.) The sum of the two parts is the same gradient either way.
 * `parts` is an OR of these; VS_BWD_ALL is vs_attn_bwd. Parts that write the
 * same array (the two dk/dv parts) must not run concurrently.
 * With VS_BWD_OVERWRITE also set, the VS_BWD_DQ and VS_BWD_DKDV parts write
 * their arrays instead of adding to them (every row of dq and every key row
 * of dk/dv gets a value, zero where the step has no active entry), so the
 * caller need not zero them for the first ring step; VS_BWD_DKDV_VERT always
 * adds and must then run after VS_BWD_DKDV. */
#define VS_BWD_DQ 1
#define VS_BWD_DKDV 2
#define VS_BWD_DKDV_VERT 4
#define VS_BWD_ALL 7
#define VS_BWD_OVERWRITE 8
int vs_attn_bwd_parts(vs_tensor q, vs_tensor k, vs_tensor v, vs_tensor dout,
                      const float* lse, const float* delta, const vs_mask* m, float scale,
                      float* dq, float* dk, float* dv, int parts, void* stream);

/* ---- a rank's whole ring in one launch --------------------------------- */

/* The ring steps of one rank run as one launch (per group of up to 32 steps)
 * instead of one call per step, with every visible shard resident: the
 * incremental softmax of the Ring Attention overview (section 2.1) is carried
 * inside the kernel across the steps, so O and LSE are written once, and the
 * backward accumulates dQ across the steps and covers the key blocks of
 * every step's shard in one grid.
 *   q:       [Hq, QB*64, D], the rank's queries;
 *   k_all, v_all: [Hkv, P*KB*64, D], every rank's shard in storage order
 *            (shard r at rows r*KB*64 .. (r+1)*KB*64 - 1);
 *   masks:   host array of `nsteps` descriptors (1 <= nsteps <= P), each
 *            filled by vs_block_mask for the same rank and layout at one step
 *            (masks[i].src is the shard it reads); no shard twice;
 *   o, lse:  as vs_attn_fwd; accumulate = 0 writes the result of all the
 *            steps, 1 merges it into (o, lse).
 * Results equal the step-by-step calls (vs_attn_fwd with accumulate = 1 per
 * step) up to fp32 rounding order. Supported: bf16 or fp16 operands at D =
 * 128 (else VS_ERR_UNSUPPORTED); VS_ERR_ARG for inconsistent masks, a shard
 * seen twice or nsteps outside [1, P]. */
int vs_attn_fwd_ring(vs_tensor q, vs_tensor k_all, vs_tensor v_all, const vs_mask* masks, int nsteps, float scale,
                     float* o, float* lse, int accumulate, void* stream);

/* The gradient of the same steps (review page 1, section 三.2 item 3, with
 * the final lse and delta of the rank's rows): dq [Hq, QB*64, D], dk_all,
 * dv_all [Hkv, P*KB*64, D] (shard r's key rows at r*KB*64, as k_all), fp32.
 * `parts` as vs_attn_bwd_parts. Without VS_BWD_OVERWRITE every output adds;
 * with it dq is written (then added to by steps beyond the first 32) and the
 * dk/dv rows of every visible shard are written before the vertical part
 * adds to them (rows of shards no step sees are left alone). */
int vs_attn_bwd_ring(vs_tensor q, vs_tensor k_all, vs_tensor v_all, vs_tensor dout, const float* lse,
                     const float* delta, const vs_mask* masks, int nsteps, float scale, float* dq, float* dk_all,
                     float* dv_all, int parts, void* stream);

/* ---- bounds-checked debug build --------------------------------------------
 * The library also builds as libvsattn_debug.so (macro VS_DEBUG_BOUNDS): there
 * every value an attention kernel reads from a mask and turns into an address
 * (list ranges, tile and query-block numbers, vertical column positions) is
 * checked against the range its use allows; a value outside it is counted in
 * a per-GPU word and replaced by an in-range one, so a corrupted mask gives a
 * count instead of an out-of-bounds access. The release build has no checks.
 *
 * vs_debug_bounds_enabled: 1 in the debug build, 0 in the release build.
 * vs_debug_bounds_count: after the work queued on `stream` so far, *count
 *   (host) receives the number of violations counted on the current GPU since
 *   the last reset (release build: always 0, no device work); reset = 1 clears
 *   the word. Synchronises `stream`. VS_ERR_ARG on a null count. */
int vs_debug_bounds_enabled(void);
int vs_debug_bounds_count(int32_t* count, int reset, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* VS_ATTN_H */
