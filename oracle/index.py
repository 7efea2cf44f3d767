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


def build_index(q_last, k, scale, n_global, top_p):
    """The whole index step: scores, then separate top-p on v and on s per head.

    Returns dict with v, s (float32), lse, and per-head index arrays
    vert[h] (global token positions) and slash[h] (block-diagonal ids).
    """
    v, s, lse = scores(q_last, k, scale, n_global)
    vert = [select_top_p(v[h], top_p) for h in range(v.shape[0])]
    slash = [select_top_p(s[h], top_p) for h in range(s.shape[0])]
    return {"v": v, "s": s, "lse": lse, "vert": vert, "slash": slash}
