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
    few rows (slash tiles and vertical columns both contribute);
  * for one whole kv group (the contiguous workloads): O, LSE and dQ of every
    row of its q heads and dK, dV of every key, from the oracle run block by
    block in worker processes, and the planted outlier keys plus the
    most-attended vertical columns once more in column order with the
    componentwise bound of rounding P and dS beside the error.
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
from tests import fullsize_group as fg

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


_candidate_cols = fg.candidate_cols


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


_CACHE = {}


def _inputs_and_scores(name):
    """The workload's inputs and the oracle's index scores (which do not
    depend on the budget), kept for the next case of the same workload."""
    if name not in _CACHE:
        _CACHE.clear()
        cfg = config_by_name(name)
        _log(f"{name}: generating N={cfg.N} Hq={cfg.Hq} Hkv={cfg.Hkv}")
        t = generate(cfg)
        _log(f"{name}: oracle index scores")
        _CACHE[name] = (t, _oracle_index(t, cfg))
    return _CACHE[name]


def _contig_case(name, comps=("bf16",), top_p=None, whole_group=True, mask_heads=None):
    """comps: operand formats of the attention kernels checked on the same
    index and oracle rows: "bf16" (the inputs as given, hi + lo weights) and
    "f16" (exact fp16 copies made by vs_convert_f16, single fp16 weights).
    top_p: another budget than the workload's (the oracle selection is
    re-run on the same scores). mask_heads: also compare the GPU's tile
    lists, vertical columns and counts of sampled query blocks of these heads
    bit for bit with the oracle's description. whole_group: run the
    whole-group check."""
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    cfg = config_by_name(name) if top_p is None else config_by_name(name, top_p=top_p)
    N, Hq, Hkv, D = cfg.N, cfg.Hq, cfg.Hkv, cfg.D
    T = N // 64
    t, scores = _inputs_and_scores(name)
    ref = dict(scores)
    if top_p is not None:
        ref["vert"] = [oi.select_top_p(ref["v"][h], top_p) for h in range(Hq)]
        ref["slash"] = [oi.select_top_p(ref["s"][h], top_p) for h in range(Hq)]
    _log(f"{name}: p = {cfg.top_p}, oracle sparsity {float(om.sparsity(N, ref['vert'], ref['slash']).mean()):.4f}")
    dev = "cuda"
    q, k, v, do = (H.to_dev(t[x], cfg.dtype) for x in ("q", "k", "v", "do"))
    lay = vs.layout("contig", 1, N)
    _log(f"{name}: GPU index vs oracle index")
    H.check_index(H.gpu_index(q[:, N - cfg.last_q:], k, lay, cfg.scale, cfg.top_p), ref, cfg.top_p)
    vert, slash = ref["vert"], ref["slash"]
    m = H.gpu_mask(H.upload_lists(vert, slash, N), Hq, Hkv, lay, 0, 0, H.tile_cap_for(slash, Hq, T))
    assert int(m.arrays()["status"].item()) == 0
    if mask_heads is not None:
        rng = np.random.default_rng(cfg.seed + 5)
        mblocks = sorted(set([0, T - 1] + rng.choice(T, 4, replace=False).tolist()))
        _log(f"{name}: GPU mask vs oracle description, heads {mask_heads}, blocks {mblocks}")
        a = H.mask_to_numpy(m)
        desc = om.step_description("contig", N, 1, 0, 0, vert, slash, heads=mask_heads, blocks=mblocks)
        for h in mask_heads:
            assert np.array_equal(a["vloc"][h * T * 64:h * T * 64 + a["vloc_cnt"][h]], desc["vloc"][h])
            for I in mblocks:
                b = desc["blocks"][(h, I)]
                u = h * T + I
                got = a["tile_col"][a["tile_ptr"][u]:a["tile_ptr"][u + 1]]
                assert got.tolist() == [J | (0x40000000 if d else 0) for J, d in zip(b["tiles"], b["diag"])]
                assert a["vert_end"][u] == b["vert_end"] and a["n_active"][u] == b["n_active"]
        assert int(a["n_active"].sum()) == sum(om.active_count(N, vert[h], slash[h]) for h in range(Hq))
    gots, dks, dvs, group = {}, [], [], {}
    R = Hq // Hkv
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
        hs = slice(GROUP * R, (GROUP + 1) * R)
        group[comp] = {"o": gots[comp]["o"][hs], "lse": gots[comp]["lse"][hs], "dq": gots[comp]["dq"][hs],
                       "dk": dk_h[GROUP], "dv": dv_h[GROUP]}
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
    if whole_group:
        _whole_group_check(name, t, cfg, ref, group)


GROUP = 0   # the kv group checked whole


def _whole_group_check(name, t, cfg, ref, group):
    """Every row of kv group GROUP's q heads and every key of the group, then
    the outlier and most-attended vertical columns with their bounds."""
    Hq, Hkv, N = cfg.Hq, cfg.Hkv, cfg.N
    R = Hq // Hkv
    hs = list(range(GROUP * R, (GROUP + 1) * R))
    vert, slash = ref["vert"], ref["slash"]
    _log(f"{name}: whole-group oracle, kv group {GROUP} ({R} q heads x {N} rows, every key)")
    err, lse, delta, dk_ref, dv_ref = fg.whole_group(t, GROUP, Hq, Hkv, vert, slash, cfg.scale, group, log=_log)
    for comp, e in err.items():
        _log(f"{name} [{comp}] whole group: max errors O {e['o']:.3e} LSE {e['lse']:.3e} dQ {e['dq']:.3e} "
             f"dK {e['dk']:.3e} dV {e['dv']:.3e}")
    # the planted outlier keys and the group's 16 most-attended vertical columns
    top = np.argsort(-ref["v"][hs].astype(np.float64).sum(axis=0), kind="stable")[:16]
    cols = np.unique(np.concatenate([t["outliers"], top])).astype(np.int64)
    q, do = t["q"][hs], t["do"][hs]
    ck, cv, abs_k, abs_v = fg.column_sums(q, t["k"][GROUP], t["v"][GROUP], do, [vert[h] for h in hs],
                                          [slash[h] for h in hs], lse, delta, cols, cfg.scale)
    # the two oracle summation orders (row blocks vs columns) agree
    assert np.abs(ck - dk_ref[cols]).max() <= 1e-9 * max(1.0, np.abs(ck).max())
    assert np.abs(cv - dv_ref[cols]).max() <= 1e-9 * max(1.0, np.abs(cv).max())
    for comp, e in err.items():
        for what, got, ref_c, bnd in (("dK", group[comp]["dk"][cols], ck, abs_k),
                                      ("dV", group[comp]["dv"][cols], cv, abs_v)):
            d = np.abs(got - ref_c)
            i = np.unravel_index(np.argmax(d), d.shape)
            b8 = 2.0 ** -8 * bnd
            ratio = float((d / np.maximum(b8, 1e-30)).max())
            _log(f"{name} [{comp}] {what} on {len(cols)} outlier/vertical columns: max err {d.max():.3e} "
                 f"(column {cols[i[0]]}, bound 2^-8 sum|terms| there {b8[i]:.3e}); "
                 f"max err / 2^-8 sum|terms| = {ratio:.3e}; largest sum|terms| {bnd.max():.3e}")
            e[f"{what.lower()}_cols"] = float(d.max())
    for comp, e in err.items():
        assert max(e["o"], e["lse"], e["dq"], e["dk"], e["dv"]) <= TOL, (comp, e)


@pytest.mark.timeout(900)
def test_fullsize_qwen32k_step():
    """The 32768-token workload (16/2 heads, d 128, bf16 inputs) at its full
    size: GPU index vs the oracle's, masks of sampled blocks bit for bit, then
    the forward (and the backward beside it) on the oracle's index, sampled
    rows and the whole kv group, with bf16 and with fp16 operands."""
    _contig_case("qwen32k", comps=("bf16", "f16"), mask_heads=[0, 15])


@pytest.mark.timeout(1500)
def test_fullsize_qwen128k_step():
    """The benchmarked step: 16/2 heads, 131072 tokens, d 128, bf16 inputs,
    fwd + bwd, with bf16 and with fp16 operands."""
    _contig_case("qwen128k", comps=("bf16", "f16"))


@pytest.mark.timeout(1800)
def test_fullsize_llama256k_step():
    """32/8 heads, 262144 tokens with Yarn x32 positions, fwd + bwd."""
    _contig_case("llama256k", comps=("bf16", "f16"))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("p", [0.8, 0.99])
def test_fullsize_llama256k_budget_sweep(p):
    """The same layer at the other budgets of the sweep (fp16 operands, the
    benchmarked path): index, sampled mask blocks bit for bit, O / LSE / dQ of
    sampled rows and the tail dK / dV."""
    _contig_case("llama256k", comps=("f16",), top_p=p, whole_group=False, mask_heads=[0, 31])


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
    _CACHE.clear()
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
    # the resident calls, as the ring report times them: every shard in
    # storage order, the masks of all steps from one call, one forward and
    # one backward call over the whole ring (fp16 operands)
    _log("512k [f16 resident]: masks, forward and backward over the ring in one call each")
    store = np.concatenate([ol.shard_positions(kind, N, P, s) for s in range(P)])
    k_all = H.as_f16(H.to_dev(t["k"][:, store], cfg.dtype))
    v_all = H.as_f16(H.to_dev(t["v"][:, store], cfg.dtype))
    q = H.as_f16(H.to_dev(t["q"][:, rows_r], cfg.dtype))
    do = H.as_f16(H.to_dev(t["do"][:, rows_r], cfg.dtype))
    masks = [vs.Mask(Hq, Hkv, lay, cap) for _ in range(P)]
    vs.vs_block_mask_ring(*lists, rank, masks)
    o = torch.full((Hq, QB * 64, D), float("nan"), device=dev)
    lse = torch.full((Hq, QB * 64), float("nan"), device=dev)
    vs.vs_attn_fwd_ring(q, k_all, v_all, masks, cfg.scale, o, lse, accumulate=0)
    delta = torch.empty(Hq, QB * 64, device=dev)
    vs.vs_attn_bwd_prep(o, do, delta)
    dq = torch.full((Hq, QB * 64, D), float("nan"), device=dev)
    dk_all = torch.full((Hkv, N, D), float("nan"), device=dev)
    dv_all = torch.full((Hkv, N, D), float("nan"), device=dev)
    vs.vs_attn_bwd_ring(q, k_all, v_all, do, lse, delta, masks, cfg.scale, dq, dk_all, dv_all,
                        vs.VS_BWD_ALL | vs.VS_BWD_OVERWRITE)
    torch.cuda.synchronize()
    for m in masks:
        assert int(m.arrays()["status"].item()) == 0
    gots["f16 resident"] = {"o": o.cpu().numpy(), "lse": lse.cpu().numpy(), "dq": dq.cpu().numpy()}
    dk_hs["f16 resident"] = {s: dk_all[:, s * QB * 64:(s + 1) * QB * 64].cpu().numpy() for s in range(P)}
    dv_hs["f16 resident"] = {s: dv_all[:, s * QB * 64:(s + 1) * QB * 64].cpu().numpy() for s in range(P)}
    del k_all, v_all, q, do, o, lse, delta, dq, dk_all, dv_all, masks
    comps = comps + ("f16 resident",)
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
