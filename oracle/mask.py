"""The active set and its per-block description (oracle side).

MTraining review, page 1: section 三.1 (vertical-slash pattern: slash = a band
of constant n - m, vertical = a key column most queries attend to) and section
三.2 item 3 (after the index is shared, each worker finds the active region of
its local attention sub-matrix from the active verticals and slashes and
computes only those entries), with the granularity of item 2 (token-level
verticals, 64x64 block-level slashes).

Reading: for query head h with vertical set V_h (global token positions) and
slash set S_h (block-diagonal ids),
    M_h[n, m] = [m <= n] and ([m in V_h] or [floor(n/64) - floor(m/64) in S_h]).
M is defined on global positions, so every layout describes the same set.

The per-(rank, step) description mirrors what the attention kernels consume:
  tiles[h][I]  -- ascending local key blocks J of the visible shard whose 64x64
                  block holds at least one slash-active entry of local query
                  block I, each flagged when not all of its 4096 entries are
                  slash-active (so the slash predicate applies inside it;
                  vertical columns are accounted separately, below). Under
                  64-token layouts a local tile is a global tile and the
                  flagged tile is exactly the query block's own diagonal tile;
                  under the one-position stripes of "striped1" a tile spans P
                  global blocks on each side and most listed tiles are
                  partial;
  vloc[h]      -- ascending local positions of the shard's vertical columns;
  vert_end[h][I] -- how many leading vloc entries have an active entry in
                  query block I (they always form a prefix of vloc);
  n_active[h][I] -- number of active entries of query block I in this shard.
Everything is derived from M by definition, block by block.
"""
import numpy as np

from .layout import shard_positions, ring_source

BLOCK = 64


def active(rows_g: np.ndarray, cols_g: np.ndarray, vert_h: np.ndarray, slash_h: np.ndarray):
    """Return (M, M_slash, M_vert) boolean [len(rows), len(cols)] for global positions."""
    causal = cols_g[None, :] <= rows_g[:, None]
    diag = rows_g[:, None] // BLOCK - cols_g[None, :] // BLOCK
    m_slash = causal & np.isin(diag, slash_h)
    m_vert = causal & np.isin(cols_g, vert_h)[None, :]
    return m_slash | m_vert, m_slash, m_vert


def block_description(rows_g, cols_g, vert_h, slash_h):
    """Tile list, vertical prefix length and active count for one query block."""
    M, m_slash, m_vert = active(rows_g, cols_g, vert_h, slash_h)
    kb = cols_g.shape[0] // BLOCK
    qgb = rows_g[0] // BLOCK
    tiles, diag = [], []
    for J in range(kb):
        if m_slash[:, J * BLOCK:(J + 1) * BLOCK].any():
            tiles.append(J)
            diag.append(not bool(m_slash[:, J * BLOCK:(J + 1) * BLOCK].all()))
    is_vert_col = np.isin(cols_g, vert_h)
    vloc = np.nonzero(is_vert_col)[0]
    used = m_vert.any(axis=0)[vloc]
    vert_end = int(used.sum())
    assert used[:vert_end].all() and not used[vert_end:].any(), "vertical columns must form a prefix"
    return {"tiles": np.array(tiles, dtype=np.int64), "diag": np.array(diag, dtype=bool),
            "vert_end": vert_end, "n_active": int(M.sum())}


def step_description(kind, n_global, P, rank, step, vert, slash, heads=None, blocks=None):
    """Description of rank ``rank`` at ring step ``step`` for all (or some) heads/blocks."""
    rows_all = shard_positions(kind, n_global, P, rank)
    cols = shard_positions(kind, n_global, P, ring_source(rank, step, P))
    qb = rows_all.shape[0] // BLOCK
    heads = range(len(vert)) if heads is None else heads
    blocks = range(qb) if blocks is None else blocks
    out = {"QB": qb, "KB": cols.shape[0] // BLOCK, "vloc": {}, "blocks": {}}
    for h in heads:
        out["vloc"][h] = np.nonzero(np.isin(cols, vert[h]))[0]
        for I in blocks:
            out["blocks"][(h, I)] = block_description(rows_all[I * BLOCK:(I + 1) * BLOCK], cols,
                                                      vert[h], slash[h])
    return out


def csc_from_description(desc, h):
    """Per local key block J: ascending (I, diag) pairs whose tile list holds J."""
    cols = {J: [] for J in range(desc["KB"])}
    for I in range(desc["QB"]):
        b = desc["blocks"][(h, I)]
        for J, dg in zip(b["tiles"], b["diag"]):
            cols[int(J)].append((I, bool(dg)))
    return cols


def active_count(n_global, vert_h, slash_h):
    """Number of active entries of one head over the causal N x N square.

    Counted per key column: a column m is active for row n >= m iff m is a
    vertical or the block-diagonal of (n, m) is selected.
    """
    T = n_global // BLOCK
    sel = np.zeros(T, dtype=bool)
    sel[np.asarray(slash_h, dtype=np.int64)] = True
    # slash part: whole selected block-diagonals (diagonal 0 keeps its causal half)
    js = np.nonzero(sel)[0]
    total = int(sum((T - j) * (BLOCK * BLOCK if j > 0 else BLOCK * (BLOCK + 1) // 2) for j in js))
    # vertical columns outside selected block-diagonals
    cnt_sel_upto = np.concatenate([[0], np.cumsum(sel[1:])])     # selected j in [1, x]
    m = np.asarray(vert_h, dtype=np.int64)
    b = m // BLOCK
    own = np.where(sel[0], 0, BLOCK - m % BLOCK)                 # rows of its own block, n >= m
    later = (T - 1 - b) - cnt_sel_upto[T - 1 - b]                # later blocks whose diagonal is off
    total += int(own.sum() + BLOCK * later.sum())
    return total


def sparsity(n_global, vert, slash):
    """1 - active / total over the causal square, per head (page 1, section 四)."""
    tot = n_global * (n_global + 1) // 2
    return np.array([1.0 - active_count(n_global, vert[h], slash[h]) / tot for h in range(len(vert))])
