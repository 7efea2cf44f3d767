"""GPU sparse-index build vs the fp64 oracle."""
import numpy as np
import pytest

from oracle import index as oi
from synth import config_by_name, generate

pytestmark = pytest.mark.gpu


def _check_index(cfg, kind="contig", P=1, last_q=64):
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    t = generate(cfg, tensors=("q", "k"), rows=None)
    N = cfg.N
    q_last = t["q"][:, N - last_q:]
    k_store = H.storage_order(t["k"], kind, P)
    lay = vs.layout(kind, P, N)
    out = H.gpu_index(H.to_dev(q_last, cfg.dtype), H.to_dev(k_store, cfg.dtype), lay, cfg.scale, cfg.top_p)
    ref = oi.build_index(q_last, t["k"], cfg.scale, N, cfg.top_p)
    H.check_index(out, ref, cfg.top_p)
    return out, ref


def test_index_tiny_fp32():
    _check_index(config_by_name("tiny"))


@pytest.mark.parametrize("last_q", [64, 40])
def test_index_gqa_bf16(last_q):
    _check_index(config_by_name("qwen32k", N=8192, c=5.0), last_q=last_q)


@pytest.mark.parametrize("kind,P", [("striped", 4), ("zigzag", 2)])
def test_index_layout_storage_order(kind, P):
    _check_index(config_by_name("qwen32k", N=8192, Hq=8, Hkv=2, c=5.0), kind, P)


def test_index_llama_group4_and_budget_edges():
    cfg = config_by_name("llama256k", N=4096, Hq=8, Hkv=2, c=3.0, yarn_scale=32.0)
    _check_index(cfg)
    out, _ = _check_index(config_by_name("llama256k", N=4096, Hq=8, Hkv=2, top_p=1.0))
    assert (out["vcnt"].cpu().numpy() == 4096).all() and (out["scnt"].cpu().numpy() == 64).all()
    out, _ = _check_index(config_by_name("llama256k", N=4096, Hq=8, Hkv=2, top_p=0.0))
    assert (out["vcnt"].cpu().numpy() == 0).all() and (out["scnt"].cpu().numpy() == 0).all()


def test_index_qwen32k_full_size():
    from synth.inputs import CONFIGS
    _check_index(CONFIGS["qwen32k"])


@pytest.mark.parametrize("p", [0.3, 0.55, 0.8, 0.95])
def test_index_ties_at_cutoff(p):
    """Identical key rows give bit-identical vertical scores; with them carrying
    most of the mass, the top-p cutoff falls inside the tie group and the
    selection must keep the lowest-indexed ties first (the oracle's rule
    applied to the GPU's own scores, bit-exact)."""
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    cfg = config_by_name("tiny", top_p=p)
    t = generate(cfg, tensors=("q", "k"))
    k = t["k"].copy()
    k[:, 300:420] = 3.0 * k[:, 300:301]     # 120 identical, dominant columns
    k[:, 900:940] = k[:, 900:901]           # 40 more identical ones
    N = cfg.N
    q_last = t["q"][:, N - 64:]
    lay = vs.layout("contig", 1, N)
    out = H.gpu_index(H.to_dev(q_last, cfg.dtype), H.to_dev(k, cfg.dtype), lay, cfg.scale, p)
    ref = oi.build_index(q_last, k, cfg.scale, N, p)
    vert, _ = H.check_index(out, ref, p)
    gv = out["v"].cpu().numpy()[0]
    assert len(np.unique(gv[300:420])) == 1          # the group really ties
    sel = set(vert[0].tolist())
    inside = [i for i in range(300, 420) if i in sel]
    assert inside == list(range(300, 300 + len(inside)))   # a prefix of the tie group


@pytest.mark.parametrize("kind,P,dtype_cfg", [("striped", 4, "qwen32k"), ("zigzag", 2, "qwen32k"),
                                              ("contig", 4, "qwen32k"), ("striped", 8, "tiny")])
def test_index_distributed_ranks(kind, P, dtype_cfg):
    """The distributed index simulated on one GPU: each rank's pass 1 on its
    own shard, an all-gather of the (max, sum) slots, each rank's pass 2
    writing its score entries, then the selection. Checked against the
    oracle's distributed build (which its CPU tests pin to the global index)
    and against the library's one-pass build on the same device."""
    import torch
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    if dtype_cfg == "tiny":
        cfg = config_by_name("tiny")
    else:
        cfg = config_by_name("qwen32k", N=8192, Hq=8, Hkv=2, c=5.0)
    t = generate(cfg, tensors=("q", "k"), rows=None)
    N, Hq, Hkv, D = cfg.N, cfg.Hq, cfg.Hkv, cfg.D
    q_last = H.to_dev(t["q"][:, N - 64:], cfg.dtype)
    lay = vs.layout(kind, P, N)
    ws = torch.empty(vs.index_workspace_size(Hq, Hkv, N, D, 64), dtype=torch.uint8, device="cuda")
    shards = [H.to_dev(H.shard(t["k"], kind, P, r), cfg.dtype) for r in range(P)]
    all_stats = torch.full((P, Hq, 64, 2), float("nan"), device="cuda")
    for r in range(P):
        vs.vs_index_rank_stats(q_last, shards[r], lay, r, cfg.scale, all_stats[r], ws)
    v = torch.full((Hq, N), float("nan"), device="cuda")
    s = torch.full((Hq, N // 64), float("nan"), device="cuda")
    for r in range(P):
        vs.vs_index_rank_mass(q_last, shards[r], lay, r, cfg.scale, all_stats, v, s, ws)
    out = {"v": v, "s": s,
           "vidx": torch.full((Hq, N), -7, dtype=torch.int32, device="cuda"),
           "vcnt": torch.empty(Hq, dtype=torch.int32, device="cuda"),
           "sidx": torch.full((Hq, N // 64), -7, dtype=torch.int32, device="cuda"),
           "scnt": torch.empty(Hq, dtype=torch.int32, device="cuda")}
    sws = torch.empty(vs.index_select_workspace_size(Hq, N), dtype=torch.uint8, device="cuda")
    vs.vs_index_select(v, s, Hq, N, cfg.top_p, out["vidx"], out["vcnt"], out["sidx"], out["scnt"], sws)
    torch.cuda.synchronize()
    assert not torch.isnan(v).any() and not torch.isnan(s).any()    # every entry written by some rank
    ref = oi.build_index_distributed(t["q"][:, N - 64:], t["k"], cfg.scale, N, cfg.top_p, kind, P)
    H.check_index(out, ref, cfg.top_p)
    one = H.gpu_index(q_last, H.to_dev(H.storage_order(t["k"], kind, P), cfg.dtype), lay, cfg.scale, cfg.top_p)
    for a, b in ((v, one["v"]), (s, one["s"])):
        assert torch.allclose(a, b, rtol=1e-5, atol=1e-9), (a - b).abs().max().item()


def _budget_scores(rng, Hq, N, ties):
    """Seeded score rows shaped like the index's: a heavy-tailed vertical row
    normalised to one, the slash row its 64-wide tile sums (fp32). With
    `ties`, the values are rounded to multiples of 2^-22 so that many are
    equal, zeros included."""
    v = rng.random((Hq, N)) ** 12
    v[:, rng.choice(N, 40, replace=False)] += 0.02
    v /= v.sum(axis=1, keepdims=True)
    if ties:
        v = np.round(v * 2.0 ** 22) / 2.0 ** 22
    s = v.reshape(Hq, N // 64, 64).sum(axis=2)[:, ::-1].copy()   # diagonal j = key tile T-1-j
    return v.astype(np.float32), s.astype(np.float32)


def _run_budget(v, s, budget, p, kv, ks):
    import torch
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    Hq, N = v.shape
    dv, ds = torch.tensor(v, device="cuda"), torch.tensor(s, device="cuda")
    out = {"vidx": torch.full((Hq, N), -7, dtype=torch.int32, device="cuda"),
           "vcnt": torch.full((Hq,), -7, dtype=torch.int32, device="cuda"),
           "sidx": torch.full((Hq, N // 64), -7, dtype=torch.int32, device="cuda"),
           "scnt": torch.full((Hq,), -7, dtype=torch.int32, device="cuda")}
    ws = torch.full((vs.index_select_workspace_size(Hq, N),), 0xAB, dtype=torch.uint8, device="cuda")
    vs.vs_index_select_budget(dv, ds, Hq, N, budget, p, kv, ks, out["vidx"], out["vcnt"], out["sidx"], out["scnt"],
                              ws)
    torch.cuda.synchronize()
    return H.lists_from_gpu(out)


@pytest.mark.parametrize("N,ties", [(32768, True), (131072, False), (4096, True)])
def test_select_budget_top_k(N, ties):
    """Fixed-count budget: bit-exact index lists against the oracle for counts
    from none to more than every element."""
    import dynamic_sparse_attention_index_amd as vs
    rng = np.random.default_rng(N + ties)
    Hq, T = 4, N // 64
    v, s = _budget_scores(rng, Hq, N, ties)
    for kv, ks in ((0, 0), (1, 1), (257, 7), (N // 20, T // 20), (N - 1, T - 1), (N, T), (N + 5, T + 9), (-3, 5)):
        gv, gs = _run_budget(v, s, vs.VS_BUDGET_TOP_K, 0.0, kv, ks)
        for h in range(Hq):
            assert np.array_equal(gv[h], oi.select_top_k(v[h], kv)), (kv, h)
            assert np.array_equal(gs[h], oi.select_top_k(s[h], ks)), (ks, h)


@pytest.mark.parametrize("N,ties", [(32768, True), (131072, False), (4096, True)])
def test_select_budget_joint(N, ties):
    """Joint top-p over the pooled vertical and slash candidates: bit-exact
    against the oracle; the separate top-p through the same entry point equals
    vs_index_select's rule."""
    import dynamic_sparse_attention_index_amd as vs
    rng = np.random.default_rng(7 * N + ties)
    Hq = 4
    v, s = _budget_scores(rng, Hq, N, ties)
    for p in (0.0, 0.05, 0.3, 0.9, 0.95, 0.999, 1.0):
        gv, gs = _run_budget(v, s, vs.VS_BUDGET_JOINT_TOP_P, p, 0, 0)
        for h in range(Hq):
            rv, rs = oi.select_joint_top_p(v[h], s[h], p)
            assert np.array_equal(gv[h], rv) and np.array_equal(gs[h], rs), (p, h)
    gv, gs = _run_budget(v, s, vs.VS_BUDGET_TOP_P, 0.95, 0, 0)
    for h in range(Hq):
        assert np.array_equal(gv[h], oi.select_top_p(v[h], 0.95))
        assert np.array_equal(gs[h], oi.select_top_p(s[h], 0.95))


def test_select_budget_joint_ties_across_directions():
    """Ties at the joint cutoff shared by verticals and slashes: the verticals
    are kept first (in every chunk), then the slashes with the lowest indices."""
    import dynamic_sparse_attention_index_amd as vs
    rng = np.random.default_rng(3)
    Hq, N = 2, 32768
    T = N // 64
    x = np.float32(2.0 ** -12)
    v = np.zeros((Hq, N), dtype=np.float32)
    s = np.zeros((Hq, T), dtype=np.float32)
    for h in range(Hq):
        v[h, rng.choice(N, 100, replace=False)] = x      # spread over every chunk
        s[h, rng.choice(T, 50, replace=False)] = x
        s[h, rng.choice(T, 3, replace=False)] = 4 * x     # above the cutoff
    for p in (0.5, 0.8, 0.9, 0.97):
        gv, gs = _run_budget(v, s, vs.VS_BUDGET_JOINT_TOP_P, p, 0, 0)
        for h in range(Hq):
            rv, rs = oi.select_joint_top_p(v[h], s[h], p)
            assert np.array_equal(gv[h], rv) and np.array_equal(gs[h], rs), (p, h)
    # p = 0.8 of 162 x: 3 big slashes (12 x) then 118 ties -> 100 verticals, 18 slashes
    rv, rs = oi.select_joint_top_p(v[0], s[0], 0.8)
    assert len(rv) == 100 and len(rs) == 3 + 18
