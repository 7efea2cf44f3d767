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
