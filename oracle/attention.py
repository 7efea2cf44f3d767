"""Masked softmax attention, its log-sum-exp merge and its gradient (oracle side).

Given the index, the sparse attention of the MTraining review (page 1, section
三.2 item 3: compute only the active entries) is exact softmax attention over
the active set M. This module writes that definition out in fp64:
    LSE_n = log sum_{m: M[n,m]} exp(z_nm),  z = q_n . k_m * scale,
    O_n   = sum_{m: M[n,m]} exp(z_nm - LSE_n) v_m,
with O_n = 0, LSE_n = -inf for a row without active keys.

The merge of partial results across ring steps is the incremental softmax of
the Ring Attention overview (page 4, section 2.1):
    L = log(exp(L_a) + exp(L_b)),  O = exp(L_a - L) O_a + exp(L_b - L) O_b,
with (0, -inf) as identity.

The backward is the textbook gradient of masked softmax attention (the pages do
not spell it out): P = exp(z - LSE) on active entries, dV = P^T dO,
dP = dO V^T, dS = P * (dP - rowsum(P * dP)), dQ = dS K * scale,
dK = dS^T Q * scale. Query heads sharing a kv head add their dK, dV.
"""
import numpy as np


def _masked_lse(z, M):
    zm = np.where(M, z, -np.inf)
    mx = zm.max(axis=1, initial=-np.inf)
    safe = np.where(np.isfinite(mx), mx, 0.0)
    ssum = np.exp(zm - safe[:, None]).sum(axis=1)
    with np.errstate(divide="ignore"):
        return np.where(ssum > 0, safe + np.log(ssum), -np.inf)


def forward_rows(q, k, v, M, scale):
    """q [R, D], k/v [C, D], M [R, C] bool -> (O [R, D], LSE [R])."""
    z = (q.astype(np.float64) @ k.astype(np.float64).T) * scale
    lse = _masked_lse(z, M)
    fin = np.isfinite(lse)
    p = np.where(M & fin[:, None], np.exp(z - np.where(fin, lse, 0.0)[:, None]), 0.0)
    return p @ v.astype(np.float64), lse


def merge(o_a, lse_a, o_b, lse_b):
    """Combine two partial (O, LSE) results of disjoint key sets."""
    mx = np.maximum(lse_a, lse_b)
    safe = np.where(np.isfinite(mx), mx, 0.0)
    wa = np.exp(lse_a - safe)
    wb = np.exp(lse_b - safe)
    tot = wa + wb
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(tot > 0, safe + np.log(tot), -np.inf)
        ca = np.where(tot > 0, wa / tot, 0.0)
        cb = np.where(tot > 0, wb / tot, 0.0)
    return ca[..., None] * o_a + cb[..., None] * o_b, lse


def backward_rows(q, k, v, M, scale, do, lse=None, drow=None):
    """Gradient contributions of the active entries M of rows q against keys k/v.

    lse, drow: the rows' final log-sum-exp and rowsum(P * dP); when omitted they
    are computed from this M (i.e. M is the row's whole active set). Passing the
    final values lets a caller split the keys (ring steps) and add the parts.
    Returns (dQ [R, D], dK [C, D], dV [C, D]).
    """
    q = q.astype(np.float64)
    k = k.astype(np.float64)
    v = v.astype(np.float64)
    do = do.astype(np.float64)
    z = (q @ k.T) * scale
    if lse is None:
        lse = _masked_lse(z, M)
    fin = np.isfinite(lse)
    act = M & fin[:, None]
    p = np.where(act, np.exp(z - np.where(fin, lse, 0.0)[:, None]), 0.0)
    dp = do @ v.T
    if drow is None:
        drow = (p * dp).sum(axis=1)
    ds = np.where(act, p * (dp - drow[:, None]), 0.0)
    return (ds @ k) * scale, (ds.T @ q) * scale, p.T @ do
