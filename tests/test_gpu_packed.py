"""Per-kv-head index and the head-pair forward (two q heads of a kv group per
workgroup, sharing the K/V tile copies), against the oracle and against the
one-head-per-workgroup forward."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import index as oi
from oracle import layout as ol
from synth import config_by_name, generate

pytestmark = pytest.mark.gpu


def _group_lists(vs, H, cfg, q, k, lay):
    """GPU scores of the per-q-head index, then the per-kv-head selection on
    the GPU; the lists must equal the oracle's rule on the GPU's scores."""
    N, Hq, Hkv = cfg.N, cfg.Hq, cfg.Hkv
    T = N // 64
    idx = H.gpu_index(q[:, N - cfg.last_q:], k, lay, cfg.scale, cfg.top_p)
    vidx = torch.full((Hq, N), -7, dtype=torch.int32, device="cuda")
    sidx = torch.full((Hq, T), -7, dtype=torch.int32, device="cuda")
    vcnt = torch.empty(Hq, dtype=torch.int32, device="cuda")
    scnt = torch.empty(Hq, dtype=torch.int32, device="cuda")
    ws = torch.empty(vs.index_select_group_workspace_size(Hq, Hkv, N), dtype=torch.uint8, device="cuda")
    vs.vs_index_select_group(idx["v"], idx["s"], Hq, Hkv, N, cfg.top_p, vidx, vcnt, sidx, scnt, ws)
    torch.cuda.synchronize()
    got = {"vidx": vidx, "vcnt": vcnt, "sidx": sidx, "scnt": scnt}
    vert, slash = H.lists_from_gpu(got)
    # the group scores are the fp32 mean of the q heads' fp32 scores (heads in
    # ascending order): the oracle's rule on those exact values
    gv = idx["v"].cpu().numpy().reshape(Hkv, Hq // Hkv, N)
    gs = idx["s"].cpu().numpy().reshape(Hkv, Hq // Hkv, T)
    R = Hq // Hkv
    for g in range(Hkv):
        acc_v, acc_s = np.zeros(N, np.float32), np.zeros(T, np.float32)
        for r in range(R):
            acc_v = (acc_v + gv[g, r]).astype(np.float32)
            acc_s = (acc_s + gs[g, r]).astype(np.float32)
        ev = oi.select_top_p((acc_v * np.float32(1.0 / R)).astype(np.float32), cfg.top_p)
        es = oi.select_top_p((acc_s * np.float32(1.0 / R)).astype(np.float32), cfg.top_p)
        for h in range(g * R, (g + 1) * R):
            assert np.array_equal(vert[h], ev), h
            assert np.array_equal(slash[h], es), h
    # and the oracle's whole group selection on the GPU scores agrees to the
    # index bar (fp64 mean vs fp32 mean may only move entries at the cutoff)
    ov, os_ = oi.select_group_top_p(idx["v"].cpu().numpy(), idx["s"].cpu().numpy(), Hkv, cfg.top_p)
    for h in range(Hq):
        for a_, b_, x in ((vert[h], ov[h], oi.group_scores(idx["v"].cpu().numpy(), Hkv)[h // R]),
                          (slash[h], os_[h], oi.group_scores(idx["s"].cpu().numpy(), Hkv)[h // R])):
            diff = np.setxor1d(a_, b_)
            if len(diff):
                assert (np.abs(x[diff] - x[b_].min()) <= 1e-5).all()
    return vert, slash, (vidx, vcnt, sidx, scnt), idx


@pytest.mark.parametrize("comp", ["f16", "bf16"])
def test_group_index_and_packed_forward(comp):
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    cfg = config_by_name("qwen32k", N=64 * 40, Hq=8, Hkv=2, n_out=5, c=3.0)
    t = generate(cfg, tensors=("q", "k", "v"))
    N, Hq, Hkv, D = cfg.N, cfg.Hq, cfg.Hkv, cfg.D
    T = N // 64
    lay = vs.layout("contig", 1, N)
    qb, kb = H.to_dev(t["q"], "bf16"), H.to_dev(t["k"], "bf16")
    vert, slash, lists, idx = _group_lists(vs, H, cfg, qb, kb, lay)
    q, k, v = (H.to_dev_comp(t[x], comp) for x in ("q", "k", "v"))
    m = H.gpu_mask(lists, Hq, Hkv, lay, 0, 0, H.tile_cap_for(slash, Hq, T))
    o1, l1 = torch.empty(Hq, N, D, device="cuda"), torch.empty(Hq, N, device="cuda")
    o2, l2 = torch.full((Hq, N, D), float("nan"), device="cuda"), torch.full((Hq, N), float("nan"), device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    vs.vs_attn_fwd(q, k, v, m, cfg.scale, o1, l1)
    vs.vs_attn_fwd_packed(q, k, v, m, cfg.scale, o2, l2, status)
    torch.cuda.synchronize()
    assert int(status.item()) == vs.VS_OK
    # same tiles in the same order per head: bit-identical results
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    pos = np.arange(N)
    err = 0.0
    from oracle import mask as om
    for h in (0, 3, 6):
        M, _, _ = om.active(pos, pos, vert[h], slash[h])
        o_ref, l_ref = oa.forward_rows(t["q"][h], t["k"][h * Hkv // Hq], t["v"][h * Hkv // Hq], M, cfg.scale)
        err = max(err, float(np.abs(o2[h].cpu().numpy() - o_ref).max()))
        fin = np.isfinite(l_ref)
        err = max(err, float(np.abs(l2[h].cpu().numpy()[fin] - l_ref[fin]).max()))
    print(f"packed fwd {comp}: max err vs oracle {err:.3e}")
    assert err <= 2e-2
    # per-q-head lists (pairs differ): every workgroup refuses, reported in status
    idx_lists = H.upload_lists(*H.lists_from_gpu(idx), N)
    m2 = H.gpu_mask(idx_lists, Hq, Hkv, lay, 0, 0, H.tile_cap_for(H.lists_from_gpu(idx)[1], Hq, T))
    status.zero_()
    vs.vs_attn_fwd_packed(q, k, v, m2, cfg.scale, o2, l2, status)
    torch.cuda.synchronize()
    assert int(status.item()) == vs.VS_ERR_ARG


def test_packed_forward_ring_accumulate():
    """Striped P = 4, rank 1, every ring step merged in place: the packed and
    the per-head forward agree bit for bit after the whole ring."""
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    cfg = config_by_name("qwen32k", N=64 * 32, Hq=4, Hkv=1, n_out=4, c=2.0)
    t = generate(cfg, tensors=("q", "k", "v"))
    N, Hq, Hkv, D, P, rank = cfg.N, cfg.Hq, cfg.Hkv, cfg.D, 4, 1
    lay = vs.layout("striped", P, N)
    QB = N // 64 // P
    rng = np.random.default_rng(9)
    vg = np.sort(rng.choice(N, 80, replace=False))
    sg = np.sort(np.unique(np.concatenate([np.arange(3), rng.choice(N // 64, 5, replace=False)])))
    vert, slash = [vg] * Hq, [sg] * Hq
    lists = H.upload_lists(vert, slash, N)
    cap = H.tile_cap_for(slash, Hq, QB)
    q = H.to_dev_comp(H.shard(t["q"], "striped", P, rank), "f16")
    outs = []
    for packed in (False, True):
        o = torch.zeros(Hq, QB * 64, D, device="cuda")
        lse = torch.full((Hq, QB * 64), -math.inf, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        for step in range(P):
            src = ol.ring_source(rank, step, P)
            k = H.to_dev_comp(H.shard(t["k"], "striped", P, src), "f16")
            v = H.to_dev_comp(H.shard(t["v"], "striped", P, src), "f16")
            m = H.gpu_mask(lists, Hq, Hkv, lay, rank, step, cap)
            if packed:
                vs.vs_attn_fwd_packed(q, k, v, m, cfg.scale, o, lse, status, accumulate=1)
            else:
                vs.vs_attn_fwd(q, k, v, m, cfg.scale, o, lse, accumulate=1)
        torch.cuda.synchronize()
        assert int(status.item()) == vs.VS_OK
        outs.append((o, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_group_select_one_head_per_group_is_per_head_select():
    """With one q head per kv head the per-kv-head selection is the per-head
    selection, bit for bit (the group mean of one head is that head)."""
    import dynamic_sparse_attention_index_amd as vs
    rng = np.random.default_rng(31)
    Hq, N = 3, 64 * 48
    T = N // 64
    v = torch.tensor(rng.exponential(1.0, (Hq, N)) ** 3, dtype=torch.float32, device="cuda")
    s = torch.tensor(rng.exponential(1.0, (Hq, T)) ** 3, dtype=torch.float32, device="cuda")
    outs = []
    for group in (False, True):
        vi = torch.full((Hq, N), -1, dtype=torch.int32, device="cuda")
        si = torch.full((Hq, T), -1, dtype=torch.int32, device="cuda")
        vc, sc = (torch.empty(Hq, dtype=torch.int32, device="cuda") for _ in range(2))
        if group:
            ws = torch.empty(vs.index_select_group_workspace_size(Hq, Hq, N), dtype=torch.uint8, device="cuda")
            vs.vs_index_select_group(v, s, Hq, Hq, N, 0.9, vi, vc, si, sc, ws)
        else:
            ws = torch.empty(vs.index_select_workspace_size(Hq, N), dtype=torch.uint8, device="cuda")
            vs.vs_index_select(v, s, Hq, N, 0.9, vi, vc, si, sc, ws)
        torch.cuda.synchronize()
        outs.append((vc.cpu(), sc.cpu(), vi.cpu(), si.cpu()))
    (vc0, sc0, vi0, si0), (vc1, sc1, vi1, si1) = outs
    assert torch.equal(vc0, vc1) and torch.equal(sc0, sc1)
    for h in range(Hq):
        assert torch.equal(vi0[h, :vc0[h]], vi1[h, :vc1[h]]) and torch.equal(si0[h, :sc0[h]], si1[h, :sc1[h]])
        assert np.array_equal(vi1[h, :vc1[h]].numpy(), oi.select_top_p(v[h].cpu().numpy(), 0.9))


def test_packed_forward_single_pair():
    """Two q heads sharing one kv head (one pair per group), bf16 operands."""
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    cfg = config_by_name("qwen32k", N=64 * 12, Hq=2, Hkv=1, n_out=3, c=2.0)
    t = generate(cfg, tensors=("q", "k", "v"))
    N, Hq, D = cfg.N, cfg.Hq, cfg.D
    rng = np.random.default_rng(5)
    vg = np.sort(rng.choice(N, 40, replace=False))
    sg = np.array([0, 1, 5], dtype=np.int64)
    lists = H.upload_lists([vg] * Hq, [sg] * Hq, N)
    lay = vs.layout("contig", 1, N)
    m = H.gpu_mask(lists, Hq, 1, lay, 0, 0, H.tile_cap_for([sg] * Hq, Hq, N // 64))
    q, k, v = (H.to_dev(t[x], "bf16") for x in ("q", "k", "v"))
    o1, l1 = torch.empty(Hq, N, D, device="cuda"), torch.empty(Hq, N, device="cuda")
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    vs.vs_attn_fwd(q, k, v, m, cfg.scale, o1, l1)
    vs.vs_attn_fwd_packed(q, k, v, m, cfg.scale, o2, l2, st)
    torch.cuda.synchronize()
    assert int(st.item()) == vs.VS_OK
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
