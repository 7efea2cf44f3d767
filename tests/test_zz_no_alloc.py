"""The index build without a caller workspace (vs_index_build_noalloc)
against vs_index_build on the same inputs: scores, lists and counts equal bit
for bit, on two calls in a row, the second with a smaller input (the library's
per-GPU scratch keeps the first call's contents)."""
import numpy as np
import pytest
import torch

from synth import config_by_name, generate

pytestmark = pytest.mark.gpu


def _both(vs, H, cfg):
    t = generate(cfg, tensors=("q", "k"))
    N, Hq, Hkv, D = cfg.N, cfg.Hq, cfg.Hkv, cfg.D
    T = N // 64
    q = H.to_dev(t["q"], cfg.dtype)
    k = H.to_dev(t["k"], cfg.dtype)
    lay = vs.layout("contig", 1, N)
    ref = H.gpu_index(q[:, N - cfg.last_q:], k, lay, cfg.scale, cfg.top_p)
    out = {
        "v": torch.full((Hq, N), float("nan"), device="cuda"), "s": torch.full((Hq, T), float("nan"), device="cuda"),
        "vidx": torch.full((Hq, N), -7, dtype=torch.int32, device="cuda"),
        "vcnt": torch.full((Hq,), -7, dtype=torch.int32, device="cuda"),
        "sidx": torch.full((Hq, T), -7, dtype=torch.int32, device="cuda"),
        "scnt": torch.full((Hq,), -7, dtype=torch.int32, device="cuda"),
    }
    vs.vs_index_build_noalloc(q[:, N - cfg.last_q:], k, lay, cfg.scale, cfg.top_p, out["v"], out["s"], out["vidx"],
                              out["vcnt"], out["sidx"], out["scnt"])
    torch.cuda.synchronize()
    for name in out:
        assert torch.equal(out[name], ref[name]), name
    return int(out["vcnt"].sum()), int(out["scnt"].sum())


def test_index_noalloc_matches_workspace_build():
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    big = config_by_name("qwen32k", N=64 * 256, Hq=8, Hkv=2, n_out=16, c=4.0)
    small = config_by_name("qwen32k", N=64 * 40, Hq=4, Hkv=1, n_out=5, c=3.0, seed=77)
    assert _both(vs, H, big)[0] > 0
    assert _both(vs, H, small)[0] > 0

