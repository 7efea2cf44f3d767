"""Whole-group oracle for the full-size GPU tests.

Every row of the q heads of one kv group and every key of that kv group,
computed from the definitions in ``oracle/`` (fp64 numpy), so a full-size
check is not limited to sampled rows or a tail window of keys:

  * O, LSE and dQ of every row: ``oracle.attention.forward_rows`` and
    ``backward_rows`` on each 64-row query block against the block's whole
    active key set (``oracle.mask.active`` on a superset of candidate keys);
  * dK and dV of every key: the per-block key gradients summed over all rows
    and over the group's q heads;
  * for chosen key columns (the planted outlier keys and the most-attended
    vertical columns) the column sums once more in column order, from the
    rows' final LSE and delta, together with the componentwise sums
    sum |terms| that bound the error of rounding the attention weights P and
    dS before their products (a Higham-style dot-product bound: rounding each
    weight to a format with unit roundoff u moves the sum by at most
    u * sum |terms|).

The blocks are dealt round-robin to worker processes forked from the test
process (no program is executed in them); they run only the numpy code
below, never touch the GPU, and leave through os._exit, so no runtime
teardown runs in them. Inputs and the GPU's results are handed over in
module state set before the fork (shared copy-on-write, read only). This
module is test infrastructure.
"""
import multiprocessing as mp
import os

import numpy as np

from oracle import attention as oa
from oracle import mask as om


def candidate_cols(rows, vert_h, slash_h):
    """A superset of the keys the rows can attend (their verticals and the key
    blocks on their selected block diagonals, up to the last row); the oracle's
    active() is then evaluated on these columns only (exact: every other
    column is inactive by definition)."""
    qb = np.unique(rows // 64)
    kb = np.unique((qb[:, None] - np.asarray(slash_h, dtype=np.int64)[None, :]).ravel())
    kb = kb[kb >= 0]
    cols = np.concatenate([np.asarray(vert_h, dtype=np.int64), (kb[:, None] * 64 + np.arange(64)[None, :]).ravel()])
    cols = np.unique(cols)
    return cols[cols <= rows.max()]


_W = {}


def _init(counter):
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass
    _W["counter"] = counter


def _work(task):
    """Blocks I = w, w + W, ... of every q head of the group."""
    w, W = task
    R, N, scale, comps = _W["R"], _W["N"], _W["scale"], _W["comps"]
    T = N // 64
    D = _W["q"].shape[2]
    k, v = np.asarray(_W["k"], dtype=np.float64), np.asarray(_W["v"], dtype=np.float64)
    dk = np.zeros((N, D))
    dv = np.zeros((N, D))
    lse_all = np.full((R, N), np.nan)
    delta_all = np.full((R, N), np.nan)
    err = {c: {"o": 0.0, "lse": 0.0, "dq": 0.0} for c in comps}
    for a in range(R):
        vert, slash = _W["vert"][a], _W["slash"][a]
        for I in range(w, T, W):
            rows = np.arange(64 * I, 64 * I + 64)
            cand = candidate_cols(rows, vert, slash)
            M, _, _ = om.active(rows, cand, vert, slash)
            keep = M.any(axis=0)
            used, M = cand[keep], M[:, keep]
            q = np.asarray(_W["q"][a, rows], dtype=np.float64)
            do = np.asarray(_W["do"][a, rows], dtype=np.float64)
            o, lse = oa.forward_rows(q, k[used], v[used], M, scale)
            dq, dkb, dvb = oa.backward_rows(q, k[used], v[used], M, scale, do)
            dk[used] += dkb
            dv[used] += dvb
            lse_all[a, rows] = lse
            delta_all[a, rows] = (do * o).sum(axis=1)
            fin = np.isfinite(lse)
            for c in comps:
                e = err[c]
                e["o"] = max(e["o"], float(np.abs(_W["o_" + c][a, rows] - o).max()))
                e["dq"] = max(e["dq"], float(np.abs(_W["dq_" + c][a, rows] - dq).max()))
                if fin.any():
                    e["lse"] = max(e["lse"], float(np.abs(_W["lse_" + c][a, rows][fin] - lse[fin]).max()))
        with _W["counter"].get_lock():
            _W["counter"].value += len(range(w, T, W))
    return err, lse_all, delta_all, dk, dv


def column_sums(q, k, v, do, vert, slash, lse, delta, cols, scale):
    """dK, dV of key columns `cols` summed over every active row of every q
    head of the group, in column order, from the rows' final LSE and delta:
    P = exp(z - LSE) on active entries, dS = P (dO.v - delta),
    dK_m = scale sum_n dS_nm q_n, dV_m = sum_n P_nm dO_n. Also returns the
    componentwise sums of |terms| of the P and dS products."""
    R, N, D = q.shape
    rows = np.arange(N)
    kc, vc = k[cols].astype(np.float64), v[cols].astype(np.float64)
    dk = np.zeros((len(cols), D))
    dv = np.zeros((len(cols), D))
    abs_k = np.zeros((len(cols), D))
    abs_v = np.zeros((len(cols), D))
    for a in range(R):
        M, _, _ = om.active(rows, cols, vert[a], slash[a])
        qa, doa = q[a].astype(np.float64), do[a].astype(np.float64)
        fin = np.isfinite(lse[a])
        act = M & fin[:, None]
        z = (qa @ kc.T) * scale
        p = np.where(act, np.exp(z - np.where(fin, lse[a], 0.0)[:, None]), 0.0)
        dp = doa @ vc.T
        ds = np.where(act, p * (dp - np.where(fin, delta[a], 0.0)[:, None]), 0.0)
        dk += (ds.T @ qa) * scale
        dv += p.T @ doa
        abs_k += (np.abs(ds).T @ np.abs(qa)) * scale
        abs_v += p.T @ np.abs(doa)
    return dk, dv, abs_k, abs_v


def whole_group(t, g, Hq, Hkv, vert, slash, scale, gpu, workers=None, log=print):
    """Oracle of kv group g over the whole sequence, compared with the GPU.

    t: inputs (float32 arrays holding the dtype-exact values, global order);
    gpu: {comp: {"o", "lse", "dq": arrays of the group's q heads [R, N(, D)],
                 "dk", "dv": the group's [N, D]}}.
    Returns (per-comp max errors of o / lse / dq / dk / dv over the whole
    group, lse [R, N], delta [R, N], oracle dk [N, D], dv [N, D])."""
    R = Hq // Hkv
    hs = list(range(g * R, (g + 1) * R))
    N = t["q"].shape[1]
    comps = sorted(gpu)
    if workers is None:
        workers = max(1, min(12, len(os.sched_getaffinity(0))))
    _W.clear()
    _W.update({"q": t["q"][hs], "do": t["do"][hs], "k": t["k"][g], "v": t["v"][g], "R": R, "N": N,
               "scale": scale, "comps": comps,
               "vert": [np.asarray(vert[h]) for h in hs], "slash": [np.asarray(slash[h]) for h in hs]})
    for c in comps:
        for name in ("o", "lse", "dq"):
            _W[f"{name}_{c}"] = gpu[c][name]
    ctx = mp.get_context("fork")
    err = {c: {"o": 0.0, "lse": 0.0, "dq": 0.0} for c in comps}
    lse = np.full((R, N), np.nan)
    delta = np.full((R, N), np.nan)
    dk = np.zeros((N, t["k"].shape[2]))
    dv = np.zeros_like(dk)
    counter = ctx.Value("q", 0)
    total_blocks = R * (N // 64)
    try:
        with ctx.Pool(workers, initializer=_init, initargs=(counter,)) as pool:
            pending = pool.map_async(_work, [(w, workers) for w in range(workers)])
            reported = 0
            while not pending.ready():
                pending.wait(15)
                done = counter.value
                if done >= reported + total_blocks // 10:
                    log(f"  whole-group oracle: {done} of {total_blocks} query blocks done")
                    reported = done
            for e, l_, d_, dk_, dv_ in pending.get():
                for c in comps:
                    for key in err[c]:
                        err[c][key] = max(err[c][key], e[c][key])
                sel = ~np.isnan(l_)
                lse[sel] = l_[sel]
                delta[sel] = d_[sel]
                dk += dk_
                dv += dv_
    finally:
        _W.clear()
    assert not np.isnan(lse).any()
    for c in comps:
        err[c]["dk"] = float(np.abs(gpu[c]["dk"] - dk).max())
        err[c]["dv"] = float(np.abs(gpu[c]["dv"] - dv).max())
    return err, lse, delta, dk, dv
