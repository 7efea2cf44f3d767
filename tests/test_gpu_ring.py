"""One rank's ring steps in one launch (vs_attn_fwd_ring / vs_attn_bwd_ring)
against the fp64 oracle and against the same steps run one call per step."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import layout as ol
from oracle import mask as om
from synth import config_by_name, generate

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _index(rng, N, Hq, nv, ns):
    T = N // 64
    vert = [np.sort(rng.choice(N, nv, replace=False)) for _ in range(Hq)]
    slash = [np.sort(np.unique(np.concatenate([np.arange(3), rng.choice(T, ns, replace=False)])))
             for _ in range(Hq)]
    return vert, slash


def _ring_case(kind, P, comp, N, Hq=4, Hkv=2, seed=0):
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    rng = np.random.default_rng(seed)
    cfg = config_by_name("qwen32k", N=N, Hq=Hq, Hkv=Hkv, n_out=6, c=2.0)
    vert, slash = _index(rng, N, Hq, 70, 6)
    t = generate(cfg)
    D = cfg.D
    lay = vs.layout(kind, P, N)
    QB = N // 64 // P
    NL = QB * 64
    lists = H.upload_lists(vert, slash, N)
    cap = H.tile_cap_for(slash, Hq, QB)
    # oracle: full outputs and gradients over the global active set
    pos = np.arange(N)
    ref_o, ref_l = np.zeros((Hq, N, D)), np.zeros((Hq, N))
    ref_dq, ref_dk, ref_dv = np.zeros((Hq, N, D)), np.zeros((Hkv, N, D)), np.zeros((Hkv, N, D))
    for h in range(Hq):
        g = h * Hkv // Hq
        M, _, _ = om.active(pos, pos, vert[h], slash[h])
        ref_o[h], ref_l[h] = oa.forward_rows(t["q"][h], t["k"][g], t["v"][g], M, cfg.scale)
        dq, dk, dv = oa.backward_rows(t["q"][h], t["k"][g], t["v"][g], M, cfg.scale, t["do"][h])
        ref_dq[h] += dq
        ref_dk[g] += dk
        ref_dv[g] += dv
    # every shard resident in storage order
    store = np.concatenate([ol.shard_positions(kind, N, P, r) for r in range(P)])
    k_all = H.to_dev_comp(t["k"][:, store], comp)
    v_all = H.to_dev_comp(t["v"][:, store], comp)
    dk_ring = torch.full((Hkv, N, D), float("nan"), device="cuda")
    dv_ring = torch.full((Hkv, N, D), float("nan"), device="cuda")
    dk_step = {r: torch.zeros(Hkv, NL, D, device="cuda") for r in range(P)}   # per shard (contiguous)
    dv_step = {r: torch.zeros(Hkv, NL, D, device="cuda") for r in range(P)}
    worst = {"o": 0.0, "lse": 0.0, "dq": 0.0, "dk": 0.0, "dv": 0.0, "o_vs_steps": 0.0, "dq_vs_steps": 0.0}
    for rank in range(P):
        rows = ol.shard_positions(kind, N, P, rank)
        q = H.to_dev_comp(t["q"][:, rows], comp)
        do = H.to_dev_comp(t["do"][:, rows], comp)
        masks = [vs.Mask(Hq, Hkv, lay, cap) for _ in range(P)]
        vs.vs_block_mask_ring(*lists, rank, masks)
        torch.cuda.synchronize()
        for m in masks:
            assert int(m.arrays()["status"].item()) == 0
        # ring: one launch per group of steps
        o = torch.full((Hq, NL, D), float("nan"), device="cuda")
        lse = torch.full((Hq, NL), float("nan"), device="cuda")
        vs.vs_attn_fwd_ring(q, k_all, v_all, masks, cfg.scale, o, lse, accumulate=0)
        delta = torch.empty(Hq, NL, device="cuda")
        vs.vs_attn_bwd_prep(o, do, delta)
        dq = torch.full((Hq, NL, D), float("nan"), device="cuda")
        # the ring's shards in this rank's step order: every shard once, so
        # the overwrite writes each shard's dk/dv rows; accumulate over ranks
        dk_r = torch.full((Hkv, N, D), float("nan"), device="cuda")
        dv_r = torch.full((Hkv, N, D), float("nan"), device="cuda")
        vs.vs_attn_bwd_ring(q, k_all, v_all, do, lse, delta, masks, cfg.scale, dq, dk_r, dv_r,
                            vs.VS_BWD_ALL | vs.VS_BWD_OVERWRITE)
        # the same steps one call per step
        o_s = torch.zeros(Hq, NL, D, device="cuda")
        l_s = torch.full((Hq, NL), -math.inf, device="cuda")
        dq_s = torch.zeros(Hq, NL, D, device="cuda")
        for step, m in enumerate(masks):
            src = ol.ring_source(rank, step, P)
            sl = slice(src * NL, (src + 1) * NL)
            vs.vs_attn_fwd(q, k_all[:, sl], v_all[:, sl], m, cfg.scale, o_s, l_s, accumulate=1)
        delta_s = torch.empty(Hq, NL, device="cuda")
        vs.vs_attn_bwd_prep(o_s, do, delta_s)
        for step, m in enumerate(masks):
            src = ol.ring_source(rank, step, P)
            sl = slice(src * NL, (src + 1) * NL)
            vs.vs_attn_bwd(q, k_all[:, sl], v_all[:, sl], do, l_s, delta_s, m, cfg.scale, dq_s, dk_step[src],
                           dv_step[src])
        torch.cuda.synchronize()
        assert not torch.isnan(dk_r).any() and not torch.isnan(dq).any() and not torch.isnan(o).any()
        if rank == 0:
            dk_ring.copy_(dk_r)
            dv_ring.copy_(dv_r)
        else:
            dk_ring += dk_r
            dv_ring += dv_r
        go, gl, gdq = o.cpu().numpy(), lse.cpu().numpy(), dq.cpu().numpy()
        fin = np.isfinite(ref_l[:, rows])
        worst["o"] = max(worst["o"], float(np.abs(go - ref_o[:, rows]).max()))
        worst["lse"] = max(worst["lse"], float(np.abs(gl[fin] - ref_l[:, rows][fin]).max()))
        assert (gl[~fin] == -np.inf).all() and (go[~fin] == 0).all()
        worst["dq"] = max(worst["dq"], float(np.abs(gdq - ref_dq[:, rows]).max()))
        worst["o_vs_steps"] = max(worst["o_vs_steps"], float((o - o_s).abs().max()))
        worst["dq_vs_steps"] = max(worst["dq_vs_steps"], float((dq - dq_s).abs().max()))
    torch.cuda.synchronize()
    # dk/dv rows of shard r are at storage rows r * NL ..; global order via `store`
    inv = np.empty(N, dtype=np.int64)
    inv[store] = np.arange(N)
    gdk, gdv = dk_ring.cpu().numpy()[:, inv], dv_ring.cpu().numpy()[:, inv]
    worst["dk"] = float(np.abs(gdk - ref_dk).max())
    worst["dv"] = float(np.abs(gdv - ref_dv).max())
    dk_s = torch.cat([dk_step[r] for r in range(P)], dim=1)     # storage order
    dv_s = torch.cat([dv_step[r] for r in range(P)], dim=1)
    worst["dk_vs_steps"] = float((dk_ring - dk_s).abs().max())
    worst["dv_vs_steps"] = float((dv_ring - dv_s).abs().max())
    print(f"ring {kind} P={P} {comp}: {worst}")
    assert max(worst[x] for x in ("o", "lse", "dq", "dk", "dv")) <= TOL, worst
    # one launch and one call per step compute the same sums in another
    # order: the online-softmax reference of a row, and so the rounding of
    # its weights to the operand format, differs; the two may differ by up to
    # their own distance to the oracle (a step left out or counted twice
    # would move them by O(1))
    own = max(worst[x] for x in ("o", "dq", "dk", "dv"))
    assert max(worst[x] for x in ("o_vs_steps", "dq_vs_steps", "dk_vs_steps", "dv_vs_steps")) <= 2 * own + 1e-6, \
        worst


@pytest.mark.parametrize("kind,P,comp", [("striped", 4, "f16"), ("zigzag", 2, "f16"), ("striped", 4, "bf16"),
                                         ("contig", 4, "f16")])
def test_ring_launch(kind, P, comp):
    _ring_case(kind, P, comp, N=64 * 32)


def test_ring_launch_more_steps_than_one_group():
    """40 steps: the launcher splits them into groups of at most 32, the
    later group merging into (forward) or adding to (backward) the first."""
    _ring_case("striped", 40, "f16", N=64 * 80, Hq=2, Hkv=1, seed=5)


@pytest.mark.parametrize("kind,P", [("striped", 4), ("zigzag", 2), ("contig", 4), ("striped", 40),
                                    ("striped1", 4), ("striped1", 32)])
def test_block_mask_ring_equals_per_step(kind, P):
    """vs_block_mask_ring writes every step's active region exactly as one
    vs_block_mask call per step does (every array, bit for bit, over the
    filled lengths), also past one group of 32 steps."""
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    rng = np.random.default_rng(P)
    N, Hq, Hkv = 64 * 2 * P * (2 if P > 8 else 8), 4, 2
    vert, slash = _index(rng, N, Hq, 50, 5)
    lay = vs.layout(kind, P, N)
    QB = N // 64 // P
    lists = H.upload_lists(vert, slash, N)
    cap = H.tile_cap_for(slash, Hq, QB)
    for rank in sorted({0, P - 1, P // 2}):
        masks = [vs.Mask(Hq, Hkv, lay, cap) for _ in range(P)]
        vs.vs_block_mask_ring(*lists, rank, masks)
        torch.cuda.synchronize()
        for step in range(P):
            ref = H.gpu_mask(lists, Hq, Hkv, lay, rank, step, cap)
            a, b = H.mask_to_numpy(masks[step]), H.mask_to_numpy(ref)
            assert masks[step].desc.src == ref.desc.src == ol.ring_source(rank, step, P)
            for name in ("tile_ptr", "csc_ptr", "vloc_cnt", "vcum", "vert_end", "slash_bits", "n_active", "status"):
                assert np.array_equal(a[name], b[name]), (rank, step, name)
            n = int(b["tile_ptr"][-1])
            assert np.array_equal(a["tile_col"][:n], b["tile_col"][:n]) and \
                np.array_equal(a["csc_row"][:n], b["csc_row"][:n]), (rank, step)
            for h in range(Hq):
                c = int(b["vloc_cnt"][h])
                assert np.array_equal(a["vloc"][h * QB * 64:h * QB * 64 + c], b["vloc"][h * QB * 64:h * QB * 64 + c])
