"""Run-to-run determinism of the HIP path on identical inputs.

Every part of the path except the vertical dK/dV accumulation writes each
output element from one workgroup in a fixed order (no atomics), so two runs
on the same inputs must agree bit for bit: the index (scores and lists), the
active region, the forward (O, LSE), delta, dQ and the dK/dV of the listed
slash tiles. The vertical columns' dK/dV add fp32 partial sums with atomics in
an order that can change between runs; they must agree to the rounding of
that order (relative 1e-5 of the column's magnitude here).
"""
import numpy as np
import pytest
import torch

from synth import config_by_name, generate

pytestmark = pytest.mark.gpu


def _run(vs, H, cfg, comp, lists, lay, q, k, v, do):
    N, Hq, Hkv, D = cfg.N, cfg.Hq, cfg.Hkv, cfg.D
    T = N // 64
    idx = H.gpu_index(q[:, N - cfg.last_q:], k, lay, cfg.scale, cfg.top_p)
    m = H.gpu_mask(lists, Hq, Hkv, lay, 0, 0, Hq * T * (T + 1))
    ops = [H.as_f16(x) for x in (q, k, v, do)] if comp == "f16" else [q, k, v, do]
    o = torch.empty(Hq, N, D, device="cuda")
    lse = torch.empty(Hq, N, device="cuda")
    delta = torch.empty(Hq, N, device="cuda")
    dq = torch.full((Hq, N, D), float("nan"), device="cuda")
    dk = torch.full((Hkv, N, D), float("nan"), device="cuda")
    dv = torch.full((Hkv, N, D), float("nan"), device="cuda")
    vs.vs_attn_fwd(ops[0], ops[1], ops[2], m, cfg.scale, o, lse)
    vs.vs_attn_bwd_prep(o, ops[3], delta)
    vs.vs_attn_bwd_parts(*ops, lse, delta, m, cfg.scale, dq, dk, dv, vs.VS_BWD_DQ | vs.VS_BWD_OVERWRITE)
    vs.vs_attn_bwd_parts(*ops, lse, delta, m, cfg.scale, dq, dk, dv, vs.VS_BWD_DKDV | vs.VS_BWD_OVERWRITE)
    slash_dk, slash_dv = dk.clone(), dv.clone()
    vs.vs_attn_bwd_parts(*ops, lse, delta, m, cfg.scale, dq, dk, dv, vs.VS_BWD_DKDV_VERT)
    torch.cuda.synchronize()
    out = {"v": idx["v"], "s": idx["s"], "vidx": idx["vidx"], "vcnt": idx["vcnt"], "sidx": idx["sidx"],
           "scnt": idx["scnt"], "o": o, "lse": lse, "delta": delta, "dq": dq, "slash_dk": slash_dk,
           "slash_dv": slash_dv, "dk": dk, "dv": dv}
    arr = m.arrays()
    for name in ("tile_ptr", "csc_ptr", "vloc_cnt", "vcum", "vert_end", "slash_bits", "n_active", "status"):
        out["mask_" + name] = arr[name].clone()
    # the list arrays up to their filled lengths (the rest is never written)
    out["mask_tile_col"] = arr["tile_col"][:int(arr["tile_ptr"][-1])].clone()
    out["mask_csc_row"] = arr["csc_row"][:int(arr["csc_ptr"][-1])].clone()
    KB = N // 64
    out["mask_vloc"] = torch.cat([arr["vloc"][h * KB * 64:h * KB * 64 + int(arr["vloc_cnt"][h])] for h in range(Hq)])
    return out


@pytest.mark.parametrize("comp", ["f16", "bf16"])
def test_path_deterministic(comp):
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    from oracle import index as oi
    cfg = config_by_name("qwen32k", N=64 * 128, Hq=4, Hkv=2, n_out=12, c=4.0)
    t = generate(cfg)
    N = cfg.N
    ref = oi.build_index(t["q"][:, N - cfg.last_q:], t["k"], cfg.scale, N, cfg.top_p)
    lists = H.upload_lists(ref["vert"], ref["slash"], N)
    lay = vs.layout("contig", 1, N)
    q, k, v, do = (H.to_dev(t[x], "bf16") for x in ("q", "k", "v", "do"))
    a = _run(vs, H, cfg, comp, lists, lay, q, k, v, do)
    b = _run(vs, H, cfg, comp, lists, lay, q, k, v, do)
    for name in a:
        if name in ("dk", "dv"):
            continue
        x, y = a[name], b[name]
        assert torch.equal(x, y) or (x.is_floating_point() and torch.equal(torch.nan_to_num(x), torch.nan_to_num(y))
                                     and torch.equal(torch.isnan(x), torch.isnan(y))), name
    assert not torch.isnan(a["dq"]).any() and not torch.isnan(a["slash_dk"]).any()
    for name in ("dk", "dv"):
        x, y = a[name], b[name]
        scale = float(x.abs().max())
        diff = float((x - y).abs().max())
        print(f"{comp} {name}: run-to-run max difference {diff:.3e} (max magnitude {scale:.3e})")
        assert diff <= 1e-5 * scale, (name, diff, scale)
