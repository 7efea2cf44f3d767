"""The longest sequence the kernels take: 2^20 tokens (16384 blocks; the
attention kernels keep a head's slash bitmap, 512 words, in LDS).

One kv group of two q heads at d = 128, bf16 inputs. The GPU index is checked
against the oracle's at this length. The attention path then runs on a sparse
fixed index (the planted outlier keys and 200 random columns as verticals,
diagonals 0-2 and five random ones as slashes; including the sequence's last
key block and first key column), so that the oracle can check every row and
every key of the group (O, LSE, dQ, dK, dV element by element), for fp16 and
bf16 operands.
"""
import numpy as np
import pytest
import torch

from synth import config_by_name, generate
from oracle import index as oi
from oracle import mask as om
from tests import fullsize_group as fg

pytestmark = pytest.mark.gpu

TOL = 2e-2
N_MAX = 1 << 20


def _log(msg):
    import sys
    import time
    print(f"[maxsize {time.strftime('%H:%M:%S')}] {msg}", file=sys.__stderr__, flush=True)


@pytest.mark.timeout(900)
def test_max_sequence_length_index_and_whole_group():
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    cfg = config_by_name("qwen32k", N=N_MAX, Hq=2, Hkv=1, n_out=64, c=2.0)
    N, Hq, Hkv, D = cfg.N, cfg.Hq, cfg.Hkv, cfg.D
    T = N // 64
    _log(f"generating N={N}")
    t = generate(cfg)
    q, k, v, do = (H.to_dev(t[x], cfg.dtype) for x in ("q", "k", "v", "do"))
    lay = vs.layout("contig", 1, N)
    _log("oracle index")
    ref = oi.build_index(t["q"][:, N - cfg.last_q:], t["k"], cfg.scale, N, cfg.top_p)
    _log("GPU index vs oracle index")
    H.check_index(H.gpu_index(q[:, N - cfg.last_q:], k, lay, cfg.scale, cfg.top_p), ref, cfg.top_p)
    rng = np.random.default_rng(cfg.seed + 3)
    vert = [np.unique(np.concatenate([t["outliers"], [0, N - 1], rng.choice(N, 200, replace=False)])).astype(np.int64)
            for _ in range(Hq)]
    slash = [np.unique(np.concatenate([[0, 1, 2, T - 1], rng.choice(T, 5, replace=False)])).astype(np.int64)
             for _ in range(Hq)]
    m = H.gpu_mask(H.upload_lists(vert, slash, N), Hq, Hkv, lay, 0, 0, H.tile_cap_for(slash, Hq, T))
    arr = m.arrays()
    assert int(arr["status"].item()) == 0
    assert int(arr["n_active"].sum().item()) == sum(om.active_count(N, vert[h], slash[h]) for h in range(Hq))
    group = {}
    for comp in ("f16", "bf16"):
        _log(f"GPU forward + backward, {comp} operands")
        ops = [H.as_f16(x) for x in (q, k, v, do)] if comp == "f16" else [q, k, v, do]
        o = torch.empty(Hq, N, D, device="cuda")
        lse = torch.empty(Hq, N, device="cuda")
        delta = torch.empty(Hq, N, device="cuda")
        dq = torch.empty(Hq, N, D, device="cuda")
        dk = torch.empty(Hkv, N, D, device="cuda")
        dv = torch.empty(Hkv, N, D, device="cuda")
        vs.vs_attn_fwd(ops[0], ops[1], ops[2], m, cfg.scale, o, lse)
        vs.vs_attn_bwd_prep(o, ops[3], delta)
        vs.vs_attn_bwd_parts(*ops, lse, delta, m, cfg.scale, dq, dk, dv, vs.VS_BWD_DQ | vs.VS_BWD_OVERWRITE)
        vs.vs_attn_bwd_parts(*ops, lse, delta, m, cfg.scale, dq, dk, dv, vs.VS_BWD_DKDV | vs.VS_BWD_OVERWRITE)
        vs.vs_attn_bwd_parts(*ops, lse, delta, m, cfg.scale, dq, dk, dv, vs.VS_BWD_DKDV_VERT)
        torch.cuda.synchronize()
        del ops
        group[comp] = {"o": o.cpu().numpy(), "lse": lse.cpu().numpy(), "dq": dq.cpu().numpy(),
                       "dk": dk[0].cpu().numpy(), "dv": dv[0].cpu().numpy()}
        del o, lse, delta, dq, dk, dv
    _log(f"whole-group oracle ({Hq} q heads x {N} rows, every key)")
    err, _, _, _, _ = fg.whole_group(t, 0, Hq, Hkv, vert, slash, cfg.scale, group, log=_log)
    for comp, e in err.items():
        _log(f"N = 2^20 [{comp}] whole group: max errors O {e['o']:.3e} LSE {e['lse']:.3e} dQ {e['dq']:.3e} "
             f"dK {e['dk']:.3e} dV {e['dv']:.3e}")
    for comp, e in err.items():
        assert max(e.values()) <= TOL, (comp, e)
