"""Full-size workloads on the GPU, in the launch configuration the benchmark
times, checked on sampled outputs against the fp64 oracle.

Both sides use the oracle's index (computed here from the synthetic inputs),
so the attention comparison does not depend on ties at the top-p budget edge;
the GPU index itself is compared with the oracle's separately (same rule as
the small index tests). Checked per workload:
  * O, LSE and dQ of seeded query blocks (first, last, random) against the
    oracle's attention over each row's whole active key set;
  * dK and dV of the last key blocks: keys there are attended only by rows
    at or after them, so the oracle gets their exact gradients from those
    few rows (slash tiles and vertical columns both contribute).
The ring case runs one rank's full ring (every step) at P = 32.
"""
import math
import sys
import time

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import index as oi
from oracle import layout as ol
from oracle import mask as om
from synth import config_by_name, generate

pytestmark = pytest.mark.gpu

TOL = 2e-2   # bf16 inputs, fp32 outputs (absolute)


def _log(msg):
    """Progress lines go to the process's own stderr, past pytest's output
    capture, so a long full-size case keeps reporting its steps."""
    sys.__stderr__.write(f"[fullsize {time.strftime('%H:%M:%S')}] {msg}\n")
    sys.__stderr__.flush()


def _oracle_index(t, cfg):
    N = cfg.N
    ref = oi.build_index(t["q"][:, N - cfg.last_q:], t["k"], cfg.scale, N, cfg.top_p)
    return ref


def _candidate_cols(rows, vert_h, slash_h):
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


def _rows_check(t, cfg, vert, slash, rows_of, got, heads, blocks):
    """O / LSE / dQ of query blocks `blocks` (rows_of(I) -> global rows) of `heads`.
    `got` is one result dict, or a dict of them by name (the oracle rows are
    then computed once and every result is checked against them)."""
    if "o" not in got:
        return _rows_check_many(t, cfg, vert, slash, rows_of, got, heads, blocks)
    return _rows_check_many(t, cfg, vert, slash, rows_of, {"": got}, heads, blocks)[""]


def _rows_check_many(t, cfg, vert, slash, rows_of, gots, heads, blocks):
    Hq, Hkv = cfg.Hq, cfg.Hkv
    worsts = {name: {"o": 0.0, "lse": 0.0, "dq": 0.0} for name in gots}
    for h in heads:
        g = h * Hkv // Hq
        for I in blocks:
            rows = rows_of(I)
            cand = _candidate_cols(rows, vert[h], slash[h])
            M, _, _ = om.active(rows, cand, vert[h], slash[h])
            used = cand[M.any(axis=0)]
            M = M[:, M.any(axis=0)]
            q, do = t["q"][h, rows], t["do"][h, rows]
            k, v = t["k"][g, used], t["v"][g, used]
            o, lse = oa.forward_rows(q, k, v, M, cfg.scale)
            dq, _, _ = oa.backward_rows(q, k, v, M, cfg.scale, do)
            fin = np.isfinite(lse)
            sl = slice(64 * I, 64 * I + 64)
            for name, got in gots.items():
                worst = worsts[name]
                worst["o"] = max(worst["o"], float(np.abs(got["o"][h, sl] - o).max()))
                worst["lse"] = max(worst["lse"],
                                   float(np.abs(got["lse"][h, sl][fin] - lse[fin]).max()) if fin.any() else 0.0)
                worst["dq"] = max(worst["dq"], float(np.abs(got["dq"][h, sl] - dq).max()))
    return worsts


def _tail_active(cfg, vert, slash, row_lo, rows_filter=None):
    """Active (row, key) pairs with row and key at or after row_lo (rows
    filtered; the layouts keep 64-row blocks whole): per row block I, its
    slash tiles inside the window (2080 entries on the diagonal, 4096 off it)
    plus the entries of its verticals in the window that no such tile covers."""
    N = cfg.N
    J0, QB = row_lo // 64, N // 64
    Ib = np.arange(J0, QB)
    if rows_filter is not None:
        Ib = Ib[rows_filter(Ib * 64)]
    total = 0
    for h in range(cfg.Hq):
        sh = np.sort(np.asarray(slash[h]))
        vm = np.sort(np.asarray(vert[h]))
        vm = vm[vm >= row_lo]
        for I in Ib:
            ss = sh[sh <= I - J0]
            total += 4096 * int((ss > 0).sum()) + 2080 * int((ss == 0).sum())
            m = vm[vm < 64 * (I + 1)]
            if len(m):
                covered = np.isin(I - m // 64, ss)
                total += int(np.minimum(64, 64 * (I + 1) - m)[~covered].sum())
    return total


def _tail_start(cfg, vert, slash, first_blocks, rows_filter=None, need=4096, max_blocks=512, end_row=None):
    """Start of the tail window: `first_blocks` key blocks before end_row (the
    sequence end, or a ring rank's last row), doubled until the window holds
    at least `need` active entries (so the dK/dV check is not vacuous when the
    last blocks are attended by nobody)."""
    end_row = cfg.N if end_row is None else end_row
    nb = first_blocks
    while True:
        row_lo = max(0, end_row - 64 * nb)
        cnt = _tail_active(cfg, vert, slash, row_lo, rows_filter)
        if cnt >= need or nb >= max_blocks:
            return row_lo, cnt
        nb *= 2


def _tail_kv_check(t, cfg, vert, slash, row_lo, dk_of, dv_of, rows_filter=None, kv_heads=None):
    """dK / dV of keys at global positions >= row_lo: exact contributions of the
    rows at or after row_lo (optionally only those passing rows_filter).
    dk_of / dv_of may be lists (several results checked against one oracle
    computation); the errors are then lists too. kv_heads: check only these
    kv heads (the q heads of their groups), else all."""
    Hq, Hkv, N = cfg.Hq, cfg.Hkv, cfg.N
    rows = np.arange(row_lo, N)
    if rows_filter is not None:
        rows = rows[rows_filter(rows)]
    keys = np.arange(row_lo, N)
    ref_dk = np.zeros((Hkv, len(keys), cfg.D))
    ref_dv = np.zeros((Hkv, len(keys), cfg.D))
    kv_sel = list(range(Hkv)) if kv_heads is None else sorted(kv_heads)
    for h in range(Hq):
        g = h * Hkv // Hq
        if len(rows) == 0 or g not in kv_sel:
            continue
        if h % 4 == 0:
            _log(f"  oracle dK/dV: q head {h} of {Hq}")
        cand = _candidate_cols(rows, vert[h], slash[h])
        M, _, _ = om.active(rows, cand, vert[h], slash[h])
        used = cand[M.any(axis=0)]
        _, dk, dv = oa.backward_rows(t["q"][h, rows], t["k"][g, used], t["v"][g, used], M[:, M.any(axis=0)],
                                     cfg.scale, t["do"][h, rows])
        sel = used >= row_lo
        ref_dk[g, used[sel] - row_lo] += dk[sel]
        ref_dv[g, used[sel] - row_lo] += dv[sel]
    ks = np.asarray(kv_sel)
    if isinstance(dk_of, (list, tuple)):
        return ([float(np.abs(f(keys)[ks] - ref_dk[ks]).max()) for f in dk_of],
                [float(np.abs(f(keys)[ks] - ref_dv[ks]).max()) for f in dv_of])
    return (float(np.abs(dk_of(keys)[ks] - ref_dk[ks]).max()), float(np.abs(dv_of(keys)[ks] - ref_dv[ks]).max()))


def _contig_case(name, comps=("bf16",)):
    """comps: operand formats of the attention kernels checked on the same
    index and oracle rows: "bf16" (the inputs as given, hi + lo weights) and
    "f16" (exact fp16 copies made by vs_convert_f16, single fp16 weights)."""
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    cfg = config_by_name(name)
    N, Hq, Hkv, D = cfg.N, cfg.Hq, cfg.Hkv, cfg.D
    T = N // 64
    _log(f"{name}: generating N={N} Hq={Hq} Hkv={Hkv}")
    t = generate(cfg)
    _log(f"{name}: oracle index")
    ref = _oracle_index(t, cfg)
    dev = "cuda"
    q, k, v, do = (H.to_dev(t[x], cfg.dtype) for x in ("q", "k", "v", "do"))
    lay = vs.layout("contig", 1, N)
    _log(f"{name}: GPU index vs oracle index")
    H.check_index(H.gpu_index(q[:, N - cfg.last_q:], k, lay, cfg.scale, cfg.top_p), ref, cfg.top_p)
    vert, slash = ref["vert"], ref["slash"]
    m = H.gpu_mask(H.upload_lists(vert, slash, N), Hq, Hkv, lay, 0, 0, H.tile_cap_for(slash, Hq, T))
    assert int(m.arrays()["status"].item()) == 0
    gots, dks, dvs = {}, [], []
    for comp in comps:
        _log(f"{name}: GPU mask + forward + backward (oracle index), {comp} operands")
        ops = [H.as_f16(x) for x in (q, k, v, do)] if comp == "f16" else [q, k, v, do]
        o = torch.empty(Hq, N, D, device=dev)
        lse = torch.empty(Hq, N, device=dev)
        delta = torch.empty(Hq, N, device=dev)
        dq = torch.zeros(Hq, N, D, device=dev)
        dk = torch.zeros(Hkv, N, D, device=dev)
        dv = torch.zeros(Hkv, N, D, device=dev)
        vs.vs_attn_fwd(ops[0], ops[1], ops[2], m, cfg.scale, o, lse)
        vs.vs_attn_bwd_prep(o, ops[3], delta)
        vs.vs_attn_bwd(*ops, lse, delta, m, cfg.scale, dq, dk, dv)
        torch.cuda.synchronize()
        del ops
        gots[comp] = {"o": o.cpu().numpy(), "lse": lse.cpu().numpy(), "dq": dq.cpu().numpy()}
        dk_h, dv_h = dk.cpu().numpy(), dv.cpu().numpy()
        dks.append(lambda keys, a=dk_h: a[:, keys])
        dvs.append(lambda keys, a=dv_h: a[:, keys])
        del o, lse, delta, dq, dk, dv
    rng = np.random.default_rng(cfg.seed + 77)
    heads = sorted(set([0, Hq - 1] + rng.choice(Hq, 2, replace=False).tolist()))
    blocks = sorted(set([0, T - 1, T // 2] + rng.choice(T, 3, replace=False).tolist()))
    _log(f"{name}: oracle rows heads={heads} blocks={blocks}")
    ws = _rows_check(t, cfg, vert, slash, lambda I: np.arange(64 * I, 64 * I + 64), gots, heads, blocks)
    row_lo, n_tail = _tail_start(cfg, vert, slash, 3)
    _log(f"{name}: oracle dK/dV of the last {(N - row_lo) // 64} key blocks ({n_tail} active entries over "
         f"all heads)")
    assert n_tail > 0
    kv_heads = None if Hkv <= 2 else [0, Hkv - 1]     # the first and last kv groups of a wide layer
    eks, evs = _tail_kv_check(t, cfg, vert, slash, row_lo, dks, dvs, kv_heads=kv_heads)
    for comp, ek, ev in zip(comps, eks, evs):
        w = ws[comp]
        _log(f"{name} [{comp}]: max errors O {w['o']:.3e} LSE {w['lse']:.3e} dQ {w['dq']:.3e} "
             f"dK {ek:.3e} dV {ev:.3e}")
    for comp, ek, ev in zip(comps, eks, evs):
        w = ws[comp]
        assert max(w["o"], w["lse"], w["dq"], ek, ev) <= TOL, (comp, w, ek, ev)


@pytest.mark.timeout(600)
def test_fullsize_qwen128k_step():
    """The benchmarked step: 16/2 heads, 131072 tokens, d 128, bf16 inputs,
    fwd + bwd, with bf16 and with fp16 operands."""
    _contig_case("qwen128k", comps=("bf16", "f16"))


@pytest.mark.timeout(900)
def test_fullsize_llama256k_step():
    """32/8 heads, 262144 tokens with Yarn x32 positions, fwd + bwd."""
    _contig_case("llama256k", comps=("bf16", "f16"))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("kind,rank", [("striped", 7), ("zigzag", 20)])
def test_fullsize_qwen512k_ring_rank(kind, rank):
    """One rank of a 524288-token sequence at P = 32: the whole ring (32 steps,
    accumulated forward, per-step backward into each source shard's dK/dV)."""
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    cfg = config_by_name("qwen512k_cp32")
    N, Hq, Hkv, D, P = cfg.N, cfg.Hq, cfg.Hkv, cfg.D, cfg.P
    T = N // 64
    QB = T // P
    _log(f"512k {kind} rank {rank}: generating")
    t = generate(cfg)
    _log("512k: oracle index")
    ref = _oracle_index(t, cfg)
    lay = vs.layout(kind, P, N)
    _log("512k: GPU index (whole sequence, storage order) vs oracle")
    k_store = H.storage_order(t["k"], kind, P)
    H.check_index(H.gpu_index(H.to_dev(t["q"][:, N - cfg.last_q:], cfg.dtype), H.to_dev(k_store, cfg.dtype), lay,
                              cfg.scale, cfg.top_p), ref, cfg.top_p)
    del k_store
    vert, slash = ref["vert"], ref["slash"]
    lists = H.upload_lists(vert, slash, N)
    cap = H.tile_cap_for(slash, Hq, QB)
    dev = "cuda"
    rows_r = ol.shard_positions(kind, N, P, rank)
    rng = np.random.default_rng(cfg.seed + 11 * rank)
    heads = sorted(set([0, Hq - 1] + rng.choice(Hq, 1).tolist()))
    blocks = sorted(set([0, QB - 1] + rng.choice(QB, 3, replace=False).tolist()))
    comps = ("bf16", "f16")
    gots, dk_hs, dv_hs = {}, {}, {}
    for comp in comps:
        conv = H.as_f16 if comp == "f16" else (lambda x: x)
        q = conv(H.to_dev(t["q"][:, rows_r], cfg.dtype))
        do = conv(H.to_dev(t["do"][:, rows_r], cfg.dtype))
        o = torch.zeros(Hq, QB * 64, D, device=dev)
        lse = torch.full((Hq, QB * 64), -math.inf, device=dev)
        _log(f"512k [{comp}]: forward over 32 ring steps")
        kv = {}
        for step in range(P):
            src = ol.ring_source(rank, step, P)
            cols = ol.shard_positions(kind, N, P, src)
            kv[src] = (conv(H.to_dev(t["k"][:, cols], cfg.dtype)), conv(H.to_dev(t["v"][:, cols], cfg.dtype)))
            m = H.gpu_mask(lists, Hq, Hkv, lay, rank, step, cap)
            assert int(m.arrays()["status"].item()) == 0
            vs.vs_attn_fwd(q, kv[src][0], kv[src][1], m, cfg.scale, o, lse, accumulate=1)
        delta = torch.empty(Hq, QB * 64, device=dev)
        vs.vs_attn_bwd_prep(o, do, delta)
        dq = torch.zeros(Hq, QB * 64, D, device=dev)
        dk = {s: torch.zeros(Hkv, QB * 64, D, device=dev) for s in range(P)}
        dv = {s: torch.zeros(Hkv, QB * 64, D, device=dev) for s in range(P)}
        _log(f"512k [{comp}]: backward over 32 ring steps")
        for step in range(P):
            src = ol.ring_source(rank, step, P)
            m = H.gpu_mask(lists, Hq, Hkv, lay, rank, step, cap)
            vs.vs_attn_bwd(q, kv[src][0], kv[src][1], do, lse, delta, m, cfg.scale, dq, dk[src], dv[src])
        torch.cuda.synchronize()
        gots[comp] = {"o": o.cpu().numpy(), "lse": lse.cpu().numpy(), "dq": dq.cpu().numpy()}
        dk_hs[comp] = {s: dk[s].cpu().numpy() for s in range(P)}
        dv_hs[comp] = {s: dv[s].cpu().numpy() for s in range(P)}
        del q, do, o, lse, delta, dq, dk, dv, kv
    _log(f"512k: oracle rows heads={heads} local blocks={blocks}")
    ws = _rows_check(t, cfg, vert, slash, lambda I: rows_r[64 * I:64 * I + 64], gots, heads, blocks)
    # dK/dV of the key blocks from 64 (or more) blocks before this rank's last
    # row to the end, from this rank's rows only (keys past its last row get
    # nothing from it)
    owner = np.empty(N, dtype=np.int64)
    local = np.empty(N, dtype=np.int64)
    for s in range(P):
        c = ol.shard_positions(kind, N, P, s)
        owner[c] = s
        local[c] = np.arange(len(c))
    def gather(store, keys):
        out = np.empty((Hkv, len(keys), D), dtype=np.float32)
        for s in np.unique(owner[keys]):
            sel = owner[keys] == s
            out[:, sel] = store[s][:, local[keys[sel]]]
        return out
    mine = np.zeros(N, dtype=bool)
    mine[rows_r] = True
    # (striped: the rank holds every P-th block, so start 2P blocks back)
    row_lo, n_tail = _tail_start(cfg, vert, slash, 2 * P if kind == "striped" else 3,
                                 rows_filter=lambda rows: mine[rows], max_blocks=1024,
                                 end_row=int(rows_r.max()) + 1)
    _log(f"512k: oracle dK/dV of the last {(N - row_lo) // 64} key blocks, this rank's rows ({n_tail} active)")
    assert n_tail > 0
    eks, evs = _tail_kv_check(t, cfg, vert, slash, row_lo,
                              [lambda keys, c=c: gather(dk_hs[c], keys) for c in comps],
                              [lambda keys, c=c: gather(dv_hs[c], keys) for c in comps],
                              rows_filter=lambda rows: mine[rows])
    for comp, ek, ev in zip(comps, eks, evs):
        w = ws[comp]
        _log(f"512k {kind} rank {rank} [{comp}]: max errors O {w['o']:.3e} LSE {w['lse']:.3e} dQ {w['dq']:.3e} "
             f"dK {ek:.3e} dV {ev:.3e}")
    for comp, ek, ev in zip(comps, eks, evs):
        w = ws[comp]
        assert max(w["o"], w["lse"], w["dq"], ek, ev) <= TOL, (comp, w, ek, ev)
