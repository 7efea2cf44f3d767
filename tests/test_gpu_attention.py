"""GPU sparse forward / merge / backward vs the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import layout as ol
from oracle import mask as om
from synth import config_by_name, generate

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4, "f16": 2e-2}


def _cfg(dtype, **kw):
    """Config whose inputs are `dtype` values; "f16" (fp16 operands) runs on
    bf16 inputs converted exactly by the library."""
    return config_by_name("qwen32k", dtype="bf16" if dtype == "f16" else dtype, **kw)


def _index(rng, N, Hq, nv, ns, band=3):
    T = N // 64
    vert = [np.sort(rng.choice(N, nv, replace=False)) for _ in range(Hq)]
    slash = [np.sort(np.unique(np.concatenate([np.arange(band), rng.choice(T, ns, replace=False)])))
             for _ in range(Hq)]
    return vert, slash


def _fwd_case(cfg, vert, slash, kind="contig", P=1, accumulate_steps=False, comp=None):
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    comp = comp or cfg.dtype
    t = generate(cfg, tensors=("q", "k", "v"))
    N, Hq, Hkv, D = cfg.N, cfg.Hq, cfg.Hkv, cfg.D
    lay = vs.layout(kind, P, N)
    QB = N // 64 // P
    lists = H.upload_lists(vert, slash, N)
    cap = H.tile_cap_for(slash, Hq, QB)
    worst = 0.0
    for rank in range(P):
        q = H.to_dev_comp(H.shard(t["q"], kind, P, rank), comp)
        o_acc = torch.zeros(Hq, QB * 64, D, device="cuda")
        l_acc = torch.full((Hq, QB * 64), -math.inf, device="cuda")
        ref_o = np.zeros((Hq, QB * 64, D))
        ref_l = np.full((Hq, QB * 64), -np.inf)
        for step in range(P):
            src = ol.ring_source(rank, step, P)
            k = H.to_dev_comp(H.shard(t["k"], kind, P, src), comp)
            v = H.to_dev_comp(H.shard(t["v"], kind, P, src), comp)
            m = H.gpu_mask(lists, Hq, Hkv, lay, rank, step, cap)
            if accumulate_steps:
                vs.vs_attn_fwd(q, k, v, m, cfg.scale, o_acc, l_acc, accumulate=1)
            else:
                o = torch.empty(Hq, QB * 64, D, device="cuda")
                lse = torch.empty(Hq, QB * 64, device="cuda")
                vs.vs_attn_fwd(q, k, v, m, cfg.scale, o, lse)
                vs.vs_merge_lse(o_acc, l_acc, o, lse)
            ref = H.oracle_step_forward(t["q"], t["k"], t["v"], vert, slash, kind, P, rank, step, cfg.scale)
            for (h, I), (o_r, l_r) in ref.items():
                sl = slice(64 * I, 64 * I + 64)
                ref_o[h, sl], ref_l[h, sl] = oa.merge(ref_o[h, sl], ref_l[h, sl], o_r, l_r)
        torch.cuda.synchronize()
        go, gl = o_acc.cpu().numpy(), l_acc.cpu().numpy()
        err = np.abs(go - ref_o).max()
        fin = np.isfinite(ref_l)
        assert (gl[~fin] == -np.inf).all() and (go[~fin] == 0).all()
        lerr = np.abs(gl[fin] - ref_l[fin]).max() if fin.any() else 0.0
        worst = max(worst, err, lerr)
        print(f"fwd {comp} D={cfg.D} {kind} P={P} rank={rank}: max|dO|={err:.3e} max|dLSE|={lerr:.3e}")
        assert err <= TOL[comp] and lerr <= TOL[comp], (rank, err, lerr)
    return worst


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 128), ("bf16", 64), ("f32", 64)])
def test_fwd_random_index_contig(dtype, D):
    rng = np.random.default_rng(1)
    cfg = _cfg(dtype, N=64 * 24, Hq=4, Hkv=2, D=D, n_out=5, c=2.0)
    vert, slash = _index(rng, cfg.N, cfg.Hq, 150, 5)
    slash[1] = slash[1][slash[1] != 0]        # a head without the diagonal block: causal verticals + empty rows
    vert[2] = np.zeros(0, dtype=np.int64)     # a head without verticals
    _fwd_case(cfg, vert, slash, comp=dtype)


@pytest.mark.parametrize("kind,P,comp", [("striped", 4, "bf16"), ("zigzag", 2, "bf16"), ("contig", 2, "bf16"),
                                         ("striped", 4, "f16")])
def test_fwd_ring_merge(kind, P, comp):
    rng = np.random.default_rng(2)
    cfg = config_by_name("qwen32k", N=64 * 32, Hq=4, Hkv=1, n_out=4, c=2.0)
    vert, slash = _index(rng, cfg.N, cfg.Hq, 100, 6)
    _fwd_case(cfg, vert, slash, kind, P, accumulate_steps=False, comp=comp)
    _fwd_case(cfg, vert, slash, kind, P, accumulate_steps=True, comp=comp)


def _stripe1_index(rng, N, Hq, P):
    """Random lists plus the cases one-position stripes single out: a head
    whose diagonals 1 .. 3P + 1 are all selected (whole windows: full tiles)
    and diagonal 0 is not, and a head without verticals."""
    vert, slash = _index(rng, N, Hq, 100, 6)
    run = min(N // 64, 3 * P + 2)
    slash[1] = np.union1d(slash[1][slash[1] != 0], np.arange(1, run)).astype(np.int64)
    vert[2] = np.zeros(0, dtype=np.int64)
    return vert, slash


@pytest.mark.parametrize("P,comp", [(2, "bf16"), (2, "f16"), (3, "f16"), (4, "bf16"), (8, "f16"), (32, "f16")])
def test_fwd_stripe1(P, comp):
    """One-position stripes: every (rank, step) of the ring, merged per rank,
    against the oracle (per-entry predicate in partial tiles, vertical
    columns outside the listed tiles' selected diagonals)."""
    rng = np.random.default_rng(20 + P)
    cfg = config_by_name("qwen32k", N=64 * P * (2 if P > 8 else 32 // P * 2), Hq=4, Hkv=2, n_out=4, c=2.0)
    vert, slash = _stripe1_index(rng, cfg.N, cfg.Hq, P)
    _fwd_case(cfg, vert, slash, "striped1", P, accumulate_steps=P % 2 == 0, comp=comp)


def test_fwd_full_budget_is_dense_causal_sdpa():
    """All verticals and slashes selected -> dense causal attention (torch SDPA on the GPU, fp32)."""
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    cfg = config_by_name("qwen32k", N=64 * 20, Hq=2, Hkv=1, n_out=3, c=1.0)
    t = generate(cfg, tensors=("q", "k", "v"))
    N, Hq, D = cfg.N, cfg.Hq, cfg.D
    vert = [np.arange(N)] * Hq
    slash = [np.arange(N // 64)] * Hq
    lay = vs.layout("contig", 1, N)
    m = H.gpu_mask(H.upload_lists(vert, slash, N), Hq, 1, lay, 0, 0, H.tile_cap_for(slash, Hq, N // 64))
    q, k, v = (H.to_dev(t[x], "bf16") for x in ("q", "k", "v"))
    o = torch.empty(Hq, N, D, device="cuda")
    lse = torch.empty(Hq, N, device="cuda")
    vs.vs_attn_fwd(q, k, v, m, cfg.scale, o, lse)
    kk = k.float().expand(Hq, N, D).contiguous()
    vv = v.float().expand(Hq, N, D).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(q.float(), kk, vv, is_causal=True)
    torch.cuda.synchronize()
    assert (o - ref).abs().max().item() < 2e-2


def _bwd_case(cfg, vert, slash, kind="contig", P=1, comp=None):
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    comp = comp or cfg.dtype
    t = generate(cfg)
    N, Hq, Hkv, D = cfg.N, cfg.Hq, cfg.Hkv, cfg.D
    lay = vs.layout(kind, P, N)
    QB = N // 64 // P
    lists = H.upload_lists(vert, slash, N)
    cap = H.tile_cap_for(slash, Hq, QB)
    # oracle: full gradients over the global active set
    ref_dq = np.zeros((Hq, N, D))
    ref_dk = np.zeros((Hkv, N, D))
    ref_dv = np.zeros((Hkv, N, D))
    pos = np.arange(N)
    for h in range(Hq):
        g = h * Hkv // Hq
        M, _, _ = om.active(pos, pos, vert[h], slash[h])
        dq, dk, dv = oa.backward_rows(t["q"][h], t["k"][g], t["v"][g], M, cfg.scale, t["do"][h])
        ref_dq[h] += dq
        ref_dk[g] += dk
        ref_dv[g] += dv
    dk_all = {r: torch.zeros(Hkv, QB * 64, D, device="cuda") for r in range(P)}
    dv_all = {r: torch.zeros(Hkv, QB * 64, D, device="cuda") for r in range(P)}
    errs = []
    for rank in range(P):
        q = H.to_dev_comp(H.shard(t["q"], kind, P, rank), comp)
        do = H.to_dev_comp(H.shard(t["do"], kind, P, rank), comp)
        o = torch.zeros(Hq, QB * 64, D, device="cuda")
        lse = torch.full((Hq, QB * 64), -math.inf, device="cuda")
        for step in range(P):
            src = ol.ring_source(rank, step, P)
            k = H.to_dev_comp(H.shard(t["k"], kind, P, src), comp)
            v = H.to_dev_comp(H.shard(t["v"], kind, P, src), comp)
            m = H.gpu_mask(lists, Hq, Hkv, lay, rank, step, cap)
            vs.vs_attn_fwd(q, k, v, m, cfg.scale, o, lse, accumulate=1)
        delta = torch.empty(Hq, QB * 64, device="cuda")
        vs.vs_attn_bwd_prep(o, do, delta)
        dq = torch.zeros(Hq, QB * 64, D, device="cuda")
        for step in range(P):
            src = ol.ring_source(rank, step, P)
            k = H.to_dev_comp(H.shard(t["k"], kind, P, src), comp)
            v = H.to_dev_comp(H.shard(t["v"], kind, P, src), comp)
            m = H.gpu_mask(lists, Hq, Hkv, lay, rank, step, cap)
            vs.vs_attn_bwd(q, k, v, do, lse, delta, m, cfg.scale, dq, dk_all[src], dv_all[src])
        torch.cuda.synchronize()
        rows = ol.shard_positions(kind, N, P, rank)
        errs.append(np.abs(dq.cpu().numpy() - ref_dq[:, rows]).max())
    for r in range(P):
        cols = ol.shard_positions(kind, N, P, r)
        errs.append(np.abs(dk_all[r].cpu().numpy() - ref_dk[:, cols]).max())
        errs.append(np.abs(dv_all[r].cpu().numpy() - ref_dv[:, cols]).max())
    print(f"bwd {comp} D={cfg.D} {kind} P={P}: max errors (dq per rank, then dk, dv per shard) {errs}")
    assert max(errs) <= TOL[comp], errs
    return errs


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 128), ("f32", 64), ("bf16", 64)])
def test_bwd_random_index(dtype, D):
    rng = np.random.default_rng(3)
    cfg = _cfg(dtype, N=64 * 16, Hq=4, Hkv=2, D=D, n_out=4, c=2.0)
    vert, slash = _index(rng, cfg.N, cfg.Hq, 90, 4)
    slash[3] = slash[3][slash[3] != 0]
    _bwd_case(cfg, vert, slash, comp=dtype)


@pytest.mark.parametrize("kind,P,comp", [("striped", 4, "bf16"), ("zigzag", 2, "bf16"), ("zigzag", 2, "f16")])
def test_bwd_ring(kind, P, comp):
    rng = np.random.default_rng(4)
    cfg = config_by_name("qwen32k", N=64 * 16, Hq=2, Hkv=1, n_out=4, c=2.0)
    vert, slash = _index(rng, cfg.N, cfg.Hq, 60, 4)
    _bwd_case(cfg, vert, slash, kind, P, comp=comp)


@pytest.mark.parametrize("P,comp", [(2, "bf16"), (4, "f16"), (8, "f16"), (8, "bf16")])
def test_bwd_stripe1(P, comp):
    rng = np.random.default_rng(40 + P)
    cfg = config_by_name("qwen32k", N=64 * 16 if P <= 4 else 64 * 2 * P, Hq=4, Hkv=2, n_out=4, c=2.0)
    vert, slash = _stripe1_index(rng, cfg.N, cfg.Hq, P)
    _bwd_case(cfg, vert, slash, "striped1", P, comp=comp)


def test_merge_kernel_matches_formula():
    import dynamic_sparse_attention_index_amd as vs
    rng = np.random.default_rng(0)
    Hq, Nq, D = 3, 256, 128
    oa_ = rng.standard_normal((Hq, Nq, D)).astype(np.float32)
    ob_ = rng.standard_normal((Hq, Nq, D)).astype(np.float32)
    la = rng.standard_normal((Hq, Nq)).astype(np.float32) * 3
    lb = rng.standard_normal((Hq, Nq)).astype(np.float32) * 3
    la[0, :10] = -np.inf
    lb[0, 5:15] = -np.inf
    oa_[0, :10] = 0
    ob_[0, 5:15] = 0
    ref_o, ref_l = oa.merge(oa_.astype(np.float64), la.astype(np.float64), ob_.astype(np.float64),
                            lb.astype(np.float64))
    to = torch.tensor(oa_, device="cuda")
    tl = torch.tensor(la, device="cuda")
    vs.vs_merge_lse(to, tl, torch.tensor(ob_, device="cuda"), torch.tensor(lb, device="cuda"))
    torch.cuda.synchronize()
    assert np.abs(to.cpu().numpy() - ref_o).max() < 1e-5
    fin = np.isfinite(ref_l)
    assert np.abs(tl.cpu().numpy()[fin] - ref_l[fin]).max() < 1e-5
    assert (tl.cpu().numpy()[~fin] == -np.inf).all()


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 128), ("f32", 64)])
def test_bwd_overwrite_matches_accumulate(dtype, D):
    """VS_BWD_OVERWRITE on NaN-filled outputs gives what the adding parts give
    on zeroed ones: dq and the slash dk/dv bit for bit (rows without a
    contribution become zero), and after the vertical part (fp32 atomics in
    both runs) to 1e-6. One ring step that leaves many blocks empty."""
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    rng = np.random.default_rng(11)
    kind, P, rank, step = "striped", 4, 1, 2
    cfg = _cfg(dtype, N=64 * 32, Hq=4, Hkv=2, D=D, n_out=4, c=2.0)
    vert, slash = _index(rng, cfg.N, cfg.Hq, 40, 3, band=0)
    t = generate(cfg)
    N, Hq, Hkv = cfg.N, cfg.Hq, cfg.Hkv
    lay = vs.layout(kind, P, N)
    QB = N // 64 // P
    lists = H.upload_lists(vert, slash, N)
    cap = H.tile_cap_for(slash, Hq, QB)
    src = ol.ring_source(rank, step, P)
    q = H.to_dev_comp(H.shard(t["q"], kind, P, rank), dtype)
    do = H.to_dev_comp(H.shard(t["do"], kind, P, rank), dtype)
    k = H.to_dev_comp(H.shard(t["k"], kind, P, src), dtype)
    v = H.to_dev_comp(H.shard(t["v"], kind, P, src), dtype)
    m = H.gpu_mask(lists, Hq, Hkv, lay, rank, step, cap)
    o = torch.zeros(Hq, QB * 64, D, device="cuda")
    lse = torch.full((Hq, QB * 64), -math.inf, device="cuda")
    vs.vs_attn_fwd(q, k, v, m, cfg.scale, o, lse, accumulate=1)
    delta = torch.empty(Hq, QB * 64, device="cuda")
    vs.vs_attn_bwd_prep(o, do, delta)
    shapes = ((Hq, QB * 64, D), (Hkv, QB * 64, D), (Hkv, QB * 64, D))
    ref = [torch.zeros(sh, device="cuda") for sh in shapes]
    got = [torch.full(sh, float("nan"), device="cuda") for sh in shapes]
    vs.vs_attn_bwd_parts(q, k, v, do, lse, delta, m, cfg.scale, *ref, vs.VS_BWD_DQ | vs.VS_BWD_DKDV)
    vs.vs_attn_bwd_parts(q, k, v, do, lse, delta, m, cfg.scale, *got,
                         vs.VS_BWD_DQ | vs.VS_BWD_DKDV | vs.VS_BWD_OVERWRITE)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
    n_zero_rows = int((ref[1].abs().sum(dim=2) == 0).sum().item())
    assert n_zero_rows > 0            # the case has key rows without any contribution
    vs.vs_attn_bwd_parts(q, k, v, do, lse, delta, m, cfg.scale, *ref, vs.VS_BWD_DKDV_VERT)
    vs.vs_attn_bwd_parts(q, k, v, do, lse, delta, m, cfg.scale, *got, vs.VS_BWD_DKDV_VERT)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.allclose(a, b, rtol=1e-6, atol=1e-7)


def test_convert_f16_exact_and_range():
    """vs_convert_f16: bit-exact with round-to-nearest-even (torch's cast), the
    value unchanged wherever fp16 can hold it (2^-17 <= |x| < 65536, and 0),
    and VS_ERR_RANGE in the status word for |x| >= 65536, inf and NaN."""
    import dynamic_sparse_attention_index_amd as vs
    rng = np.random.default_rng(21)
    n = 1 << 20
    mag = np.exp2(rng.uniform(-30, 15.99, n)) * rng.choice([-1.0, 1.0], n)
    mag[:16] = [0.0, -0.0, 65280.0, -65280.0, 2.0 ** -17, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
                1.0, -1.0, 2.0 ** -14, 1e-3, 6e4, -6e4, 2.0 ** -18, 2.0 ** -30]
    x = torch.tensor(mag, dtype=torch.float32).to(torch.bfloat16).cuda()
    out = torch.empty(n, dtype=torch.float16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    vs.vs_convert_f16(x, out, status)
    torch.cuda.synchronize()
    assert int(status.item()) == vs.VS_OK
    ref = x.to(torch.float16)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    xf = x.float()
    held = (xf.abs() >= 2.0 ** -17) | (xf == 0)
    assert torch.equal(out.float()[held], xf[held])
    assert ((out.float() - xf).abs()[~held] <= 2.0 ** -25).all()
    for bad in (65536.0, -1e6, float("inf"), float("nan")):
        y = x.clone()
        y[n // 2 + 3] = bad
        status.zero_()
        vs.vs_convert_f16(y, out, status)
        torch.cuda.synchronize()
        assert int(status.item()) == vs.VS_ERR_RANGE, bad


@pytest.mark.parametrize("D", [128, 64])
def test_bwd_prep_f16_matches_separate_calls(D):
    """vs_attn_bwd_prep_f16 (delta and the fp16 dO copy in one pass): its
    copy equals vs_convert_f16's and its delta vs_attn_bwd_prep's on the same
    dO, bit for bit; range errors reach the status word."""
    import dynamic_sparse_attention_index_amd as vs
    rng = np.random.default_rng(17)
    Hq, Nq = 3, 64 * 5
    o = torch.tensor(rng.standard_normal((Hq, Nq, D)), dtype=torch.float32, device="cuda")
    do = torch.tensor(rng.standard_normal((Hq, Nq, D)) * 3, dtype=torch.float32).to(torch.bfloat16).cuda()
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    do16a = torch.empty(Hq, Nq, D, dtype=torch.float16, device="cuda")
    do16b = torch.empty_like(do16a)
    da, db = torch.empty(Hq, Nq, device="cuda"), torch.empty(Hq, Nq, device="cuda")
    vs.vs_convert_f16(do, do16a, st)
    vs.vs_attn_bwd_prep(o, do, da)              # delta from the bf16 values (the same numbers)
    vs.vs_attn_bwd_prep_f16(o, do, do16b, db, st)
    torch.cuda.synchronize()
    assert int(st.item()) == vs.VS_OK
    assert torch.equal(do16a.view(torch.int16), do16b.view(torch.int16)) and torch.equal(da, db)
    ref = (o.double() * do.double()).sum(-1)
    assert (da.double() - ref).abs().max().item() < 1e-3
    do[1, 7, 5] = 1e6
    vs.vs_attn_bwd_prep_f16(o, do, do16b, db, st)
    torch.cuda.synchronize()
    assert int(st.item()) == vs.VS_ERR_RANGE
