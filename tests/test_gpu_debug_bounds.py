"""The bounds-checked debug build (libvsattn_debug.so, VS_DEBUG_BOUNDS).

1. On valid masks it counts no violation and gives the oracle's results
   (the parity cases of the release build rerun through it).
2. On a mask whose list entries were overwritten with out-of-range values
   (a tile past the shard's last key block, a query block past the rank's
   last, a vertical column past the shard) the attention kernels count the
   violations and still finish. The tensors the corrupted values would
   address are views into buffers padded far past those values, so even a
   check that failed to fire would read allocated memory only.
"""
import numpy as np
import pytest
import torch

from synth import config_by_name

pytestmark = pytest.mark.gpu


def _debug():
    import dynamic_sparse_attention_index_amd as vs
    return vs.use_library(vs.DEBUG_LIB_PATH)


@pytest.mark.parametrize("case", ["contig_f16", "contig_bf16", "striped_f16", "zigzag_bf16", "striped1_f16",
                                  "contig_bf16_d64"])
def test_debug_build_parity_without_violations(case):
    import dynamic_sparse_attention_index_amd as vs
    from tests import test_gpu_attention as A
    kind, comp = case.split("_")[0], case.split("_")[1]
    D = 64 if case.endswith("d64") else 128
    P = {"contig": 1, "striped": 2, "zigzag": 2, "striped1": 2}[kind]
    rng = np.random.default_rng(11)
    cfg = A._cfg(comp, N=64 * 16, Hq=4, Hkv=2, D=D, n_out=4, c=2.0)
    vert, slash = A._index(rng, cfg.N, cfg.Hq, 80, 4)
    with _debug():
        assert vs.debug_bounds_enabled()
        vs.debug_bounds_count(reset=True)
        A._fwd_case(cfg, vert, slash, kind, P, accumulate_steps=True, comp=comp)
        A._bwd_case(cfg, vert, slash, kind, P, comp=comp)
        assert vs.debug_bounds_count() == 0


def test_debug_build_resident_ring_without_violations():
    import dynamic_sparse_attention_index_amd as vs
    from tests import test_gpu_ring as R
    with _debug():
        vs.debug_bounds_count(reset=True)
        R._ring_case("striped", 4, "f16", N=64 * 32)
        assert vs.debug_bounds_count() == 0


def test_debug_build_counts_corrupted_mask_entries():
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    N, Hq, Hkv, D, PAD = 64 * 8, 2, 1, 128, 4096
    KB = N // 64
    rng = np.random.default_rng(5)
    cfg = config_by_name("qwen32k", N=N, Hq=Hq, Hkv=Hkv, n_out=2, c=1.0)
    vert = [np.array([3, 70, 200]), np.array([5, 300])]
    slash = [np.array([0, 1, 3]), np.array([0, 2])]

    def padded(shape, last):
        buf = torch.tensor(rng.standard_normal((shape[0], shape[1] + PAD, shape[2])), dtype=torch.bfloat16,
                           device="cuda")
        return buf[:, :shape[1]] if not last else buf

    q = padded((Hq, N, D), False)
    k = padded((Hkv, N, D), False)
    v = padded((Hkv, N, D), False)
    do = padded((Hq, N, D), False)
    lse_buf = torch.zeros(Hq * N + PAD, device="cuda")
    delta_buf = torch.zeros(Hq * N + PAD, device="cuda")
    lse, delta = lse_buf[:Hq * N].view(Hq, N), delta_buf[:Hq * N].view(Hq, N)
    lay = vs.layout("contig", 1, N)
    with _debug():
        vs.debug_bounds_count(reset=True)
        lists = H.upload_lists(vert, slash, N)
        m = H.gpu_mask(lists, Hq, Hkv, lay, 0, 0, H.tile_cap_for(slash, Hq, KB))
        arr = m.arrays()
        assert int(arr["status"].item()) == 0
        # one listed tile past the last key block, one CSC query block past the
        # last query block, one vertical column past the shard
        tp, cp = arr["tile_ptr"], arr["csc_ptr"]
        assert int(tp[-1]) > 0 and int(cp[-1]) > 0 and int(arr["vloc_cnt"][0]) > 0
        arr["tile_col"][int(tp[KB - 1])] = (KB + 3) | (int(arr["tile_col"][int(tp[KB - 1])]) & vs.TILE_DIAG)
        arr["csc_row"][int(cp[1])] = (KB + 2) | (int(arr["csc_row"][int(cp[1])]) & vs.TILE_DIAG)
        arr["vloc"][0] = KB * 64 + 5
        torch.cuda.synchronize()
        o = torch.zeros(Hq, N, D, device="cuda")
        vs.vs_attn_fwd(q, k, v, m, cfg.scale, o, lse)
        n_fwd = vs.debug_bounds_count()
        dq = torch.zeros(Hq, N, D, device="cuda")
        dk = torch.zeros(Hkv, N, D, device="cuda")
        dv = torch.zeros(Hkv, N, D, device="cuda")
        vs.vs_attn_bwd(q, k, v, do, lse, delta, m, cfg.scale, dq, dk, dv)
        n_bwd = vs.debug_bounds_count()
        torch.cuda.synchronize()
        print(f"violations counted: forward {n_fwd}, backward {n_bwd}")
        assert n_fwd > 0 and n_bwd > 0
        assert torch.isfinite(o).all() and torch.isfinite(dq).all() and torch.isfinite(dk).all()
