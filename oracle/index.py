"""Online sparse-index approximation (oracle side).

MTraining review, page 1, section 三.2 "分布式稀疏索引近似", items 1-2:
  * the last ``last_q`` queries are scored against the keys;
  * each rank forms cumulative attention statistics along the vertical
    (token-level column) and slash (diagonal) directions;
  * the smallest number of verticals and slashes that recall the target
    attention mass is kept (the "online top-p budget" of section 五);
  * slash statistics are aggregated at the 64x64 block level to match the
    block matmul tiling, verticals stay token level.

Readings (the pages leave these open):
  * rows are the global positions [N - last_q, N); logits are q.k * scale over
    every causal key (m <= n); A = row softmax;
  * v(m) = (1/last_q) sum_n A[n, m]; s(j) = (1/last_q) sum of A over entries
    with floor(n/64) - floor(m/64) = j; both sum to 1;
  * top-p is applied separately to v and s, per query head;
  * the fewest elements are taken in descending score order, ties to the lower
    index, with exact fixed-point sums (q_i = round(x_i * 2^40),
    target = ceil(round(p * 2^32) * sum q / 2^32));
  * p >= 1 keeps everything, p <= 0 keeps nothing.

Two other budgets on the same scores: a fixed count per head (select_top_k)
and one top-p over the pooled vertical and slash candidates
(select_joint_top_p). select_group_top_p selects once per kv head, on the
mean scores of its q heads (group_scores).
"""
import numpy as np

BLOCK = 64


def row_stats(q_last: np.ndarray, k: np.ndarray, scale: float, n_global: int):
    """Logits and log-sum-exp of the scored rows.

    q_last: [Hq, L, D] rows at global positions n_global-L .. n_global-1.
    k:      [Hkv, N, D] keys in global order.
    Returns a list (per q head) of masked logits z [L, N] (-inf where m > n) and
    lse [Hq, L].
    """
    Hq, L, _ = q_last.shape
    Hkv, N, _ = k.shape
    assert N == n_global
    rows = np.arange(N - L, N)
    cols = np.arange(N)
    causal = cols[None, :] <= rows[:, None]
    zs, lse = [], np.empty((Hq, L))
    for h in range(Hq):
        g = h * Hkv // Hq
        z = (q_last[h].astype(np.float64) @ k[g].astype(np.float64).T) * scale
        z = np.where(causal, z, -np.inf)
        zmax = z.max(axis=1, keepdims=True)
        lse[h] = (zmax + np.log(np.exp(z - zmax).sum(axis=1, keepdims=True)))[:, 0]
        zs.append(z)
    return zs, lse


def scores(q_last: np.ndarray, k: np.ndarray, scale: float, n_global: int):
    """Vertical and slash attention mass, rounded to fp32 (the reported scores).

    Returns (v [Hq, N] float32, s [Hq, N/64] float32, lse [Hq, L] float64).
    """
    Hq, L, _ = q_last.shape
    N = n_global
    T = N // BLOCK
    zs, lse = row_stats(q_last, k, scale, n_global)
    rows = np.arange(N - L, N)
    cols = np.arange(N)
    diag = rows[:, None] // BLOCK - cols[None, :] // BLOCK
    causal = cols[None, :] <= rows[:, None]
    v = np.empty((Hq, N))
    s = np.empty((Hq, T))
    for h in range(Hq):
        a = np.exp(zs[h] - lse[h][:, None])            # exactly 0 where z = -inf
        v[h] = a.sum(axis=0) / L
        s[h] = np.bincount(diag[causal], weights=a[causal], minlength=T)[:T] / L
    return v.astype(np.float32), s.astype(np.float32), lse


def select_top_p(x: np.ndarray, p: float) -> np.ndarray:
    """Fewest indices whose score mass reaches the fraction p (ascending output).

    x: non-negative float32 scores. p is taken as float32.
    """
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[0]
    p32 = np.float32(p)
    if p32 >= 1:
        return np.arange(n, dtype=np.int64)
    if p32 <= 0:
        return np.zeros(0, dtype=np.int64)
    assert (x >= 0).all()
    q = np.rint(x.astype(np.float64) * 2.0 ** 40).astype(np.int64)   # exact: x is fp32
    total = int(q.sum())
    pq = int(np.rint(np.float64(p32) * 2.0 ** 32))
    tgt = -((-pq * total) // 2 ** 32)                                # ceil, exact integers
    if tgt <= 0:
        return np.zeros(0, dtype=np.int64)
    order = np.lexsort((np.arange(n), -x.astype(np.float64)))      # x desc, index asc
    cum = np.cumsum(q[order])
    k = int(np.searchsorted(cum, tgt, side="left")) + 1
    return np.sort(order[:k])


def select_top_k(x: np.ndarray, k: int) -> np.ndarray:
    """Fixed-count budget: the min(k, n) largest scores, ties to the lower
    index (ascending output); k <= 0 keeps nothing.

    The review (page 1, section 八, item 4) reports that its experiments fix
    the sparsity at 95% by hand instead of adapting it; a fixed count of
    verticals and slashes per head is the plain form of such a budget, the
    caller choosing the counts that give the sparsity it wants.
    """
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[0]
    k = max(0, min(int(k), n))
    order = np.lexsort((np.arange(n), -x.astype(np.float64)))      # x desc, index asc
    return np.sort(order[:k])


def select_joint_top_p(v: np.ndarray, s: np.ndarray, p: float):
    """Joint budget: one top-p over the pooled vertical and slash scores.

    Page 1, section 三.2 item 1 asks for the fewest verticals and slashes that
    recall the target mass; read jointly, the count that is minimised is the
    number of verticals plus slashes. The candidates of one head are its n
    verticals followed by its T slashes; the fewest of them in descending
    score order (ties: verticals before slashes, then the lower index) whose
    fixed-point mass reaches p of the pooled total are kept, with the same
    integer rule as select_top_p. Each attention entry is counted once in its
    column and once in its diagonal; the overlap of a chosen column and a
    chosen diagonal is not deducted (the pages give no rule for it).
    Returns (vertical indices, slash indices), each ascending.
    """
    v = np.asarray(v, dtype=np.float32)
    s = np.asarray(s, dtype=np.float32)
    n = v.shape[0]
    kept = select_top_p(np.concatenate([v, s]), p)
    return kept[kept < n], kept[kept >= n] - n


def group_scores(x: np.ndarray, Hkv: int) -> np.ndarray:
    """Per-kv-head scores for grouped-query attention: the mean over the
    R = Hq / Hkv consecutive q heads that share kv head g (fp64).

    The review fixes one sparse index per attention head (page 1, section
    三.2 item 1); this variant takes the head to be the kv head, so every q
    head of a group attends the same positions."""
    x = np.asarray(x, dtype=np.float64)
    Hq = x.shape[0]
    assert Hq % Hkv == 0
    return x.reshape(Hkv, Hq // Hkv, -1).mean(axis=1)


def select_group_top_p(v: np.ndarray, s: np.ndarray, Hkv: int, p: float):
    """Top-p (select_top_p) on the per-kv-head scores, the lists handed to
    every q head of the group: returns (vert, slash), one list per q head.
    v, s: [Hq, N] and [Hq, T] scores; the group scores are rounded to fp32
    before the selection (the selection rule takes fp32 scores)."""
    Hq = v.shape[0]
    R = Hq // Hkv
    gv = group_scores(v, Hkv).astype(np.float32)
    gs = group_scores(s, Hkv).astype(np.float32)
    vg = [select_top_p(gv[g], p) for g in range(Hkv)]
    sg = [select_top_p(gs[g], p) for g in range(Hkv)]
    return [vg[h // R] for h in range(Hq)], [sg[h // R] for h in range(Hq)]


def build_index(q_last, k, scale, n_global, top_p):
    """The whole index step: scores, then separate top-p on v and on s per head.

    Returns dict with v, s (float32), lse, and per-head index arrays
    vert[h] (global token positions) and slash[h] (block-diagonal ids).
    """
    v, s, lse = scores(q_last, k, scale, n_global)
    vert = [select_top_p(v[h], top_p) for h in range(v.shape[0])]
    slash = [select_top_p(s[h], top_p) for h in range(s.shape[0])]
    return {"v": v, "s": s, "lse": lse, "vert": vert, "slash": slash}


def rank_row_stats(q_last, k_shard, pos, scale, n_global):
    """One rank's partial row statistics over the keys it holds.

    The distributed index of the same section (三.2, item 1): the scored
    queries are broadcast, every rank scores them against its local keys only
    and keeps, per scored row, the running maximum and the sum of exponentials
    relative to it (the two numbers an exchange needs to rebuild the row's
    log-sum-exp).

    k_shard: [Hkv, n_local, D] the rank's keys, at global positions ``pos``.
    Returns (m [Hq, L], l [Hq, L]): m = max logit over the rank's causal keys
    (-inf if none), l = sum exp(z - m) (0 if none).
    """
    Hq, L, _ = q_last.shape
    Hkv = k_shard.shape[0]
    rows = np.arange(n_global - L, n_global)
    causal = pos[None, :] <= rows[:, None]
    m = np.full((Hq, L), -np.inf)
    l = np.zeros((Hq, L))
    for h in range(Hq):
        g = h * Hkv // Hq
        z = (q_last[h].astype(np.float64) @ k_shard[g].astype(np.float64).T) * scale
        z = np.where(causal, z, -np.inf)
        mh = z.max(axis=1) if z.shape[1] else np.full(L, -np.inf)
        ok = mh > -np.inf
        m[h] = mh
        l[h, ok] = np.exp(z[ok] - mh[ok, None]).sum(axis=1)
    return m, l


def merge_row_stats(parts):
    """Row log-sum-exp from every rank's (m, l): M = max m, LSE = M + log sum
    l_r exp(m_r - M); -inf for a row no rank saw."""
    ms = np.stack([p[0] for p in parts])
    ls = np.stack([p[1] for p in parts])
    M = ms.max(axis=0)
    ok = M > -np.inf
    lse = np.full(M.shape, -np.inf)
    w = np.where(ms > -np.inf, np.exp(ms - np.where(ok, M, 0.0)[None]), 0.0)
    lse[ok] = M[ok] + np.log((ls * w).sum(axis=0)[ok])
    return lse


def rank_mass(q_last, k_shard, pos, scale, n_global, lse):
    """One rank's share of the vertical and slash mass: v(m) for its keys and
    the slash mass of the 64-blocks it holds (with the scored rows in the last
    block, block-diagonal j collects exactly key block T-1-j). Returns
    (v_local [Hq, n_local], s_part [Hq, T]) in fp64; s_part is zero outside
    the rank's blocks."""
    Hq, L, _ = q_last.shape
    Hkv = k_shard.shape[0]
    T = n_global // BLOCK
    rows = np.arange(n_global - L, n_global)
    causal = pos[None, :] <= rows[:, None]
    diag = rows[:, None] // BLOCK - pos[None, :] // BLOCK
    v = np.zeros((Hq, pos.shape[0]))
    s = np.zeros((Hq, T))
    for h in range(Hq):
        g = h * Hkv // Hq
        z = (q_last[h].astype(np.float64) @ k_shard[g].astype(np.float64).T) * scale
        ok = np.isfinite(lse[h])[:, None] & causal
        a = np.where(ok, np.exp(np.where(ok, z - lse[h][:, None], 0.0)), 0.0)
        v[h] = a.sum(axis=0) / L
        s[h] = np.bincount(diag[ok], weights=a[ok], minlength=T)[:T] / L
    return v, s


def build_index_distributed(q_last, k, scale, n_global, top_p, kind, P):
    """The index built the distributed way: per-rank partial statistics, an
    all-gather of (m, l), the merged row LSE, per-rank mass, then an
    all-gather of v and a sum of the slash parts, and the same top-p on the
    gathered scores. k is [Hkv, N, D] in global order; each rank is handed
    the keys at its shard positions."""
    from .layout import shard_positions
    shards = [shard_positions(kind, n_global, P, r) for r in range(P)]
    parts = [rank_row_stats(q_last, k[:, pos], pos, scale, n_global) for pos in shards]
    lse = merge_row_stats(parts)
    Hq = q_last.shape[0]
    v = np.zeros((Hq, n_global))
    s = np.zeros((Hq, n_global // BLOCK))
    for pos in shards:
        v_r, s_r = rank_mass(q_last, k[:, pos], pos, scale, n_global, lse)
        v[:, pos] = v_r
        s += s_r
    v, s = v.astype(np.float32), s.astype(np.float32)
    vert = [select_top_p(v[h], top_p) for h in range(Hq)]
    slash = [select_top_p(s[h], top_p) for h in range(Hq)]
    return {"v": v, "s": s, "lse": lse, "vert": vert, "slash": slash}
