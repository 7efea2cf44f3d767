"""Test harness: runs the HIP path through the binding and the oracle on the
same seeded inputs, and converts both to comparable arrays."""
import numpy as np
import torch

import dynamic_sparse_attention_index_amd as vs
from oracle import attention as oa
from oracle import layout as ol
from oracle import mask as om

DEV = "cuda"


def to_dev(x, dtype):
    t = torch.tensor(x)
    return t.to(device=DEV, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def as_f16(x):
    """Exact fp16 copy of a bf16 device tensor, made by the library's own
    conversion (vs_convert_f16); fails on a range error."""
    out = torch.empty(x.shape, dtype=torch.float16, device=x.device)
    status = torch.zeros(1, dtype=torch.int32, device=x.device)
    vs.vs_convert_f16(x.contiguous(), out, status)
    torch.cuda.synchronize()
    assert int(status.item()) == vs.VS_OK
    return out


def to_dev_comp(x, comp):
    """Device operands for compute format comp: "bf16", "f32", or "f16" (the
    bf16 values converted exactly by the library)."""
    if comp == "f16":
        return as_f16(to_dev(x, "bf16"))
    return to_dev(x, comp)


def gpu_index(q_last, k, lay, scale, top_p):
    """q_last [Hq, L, D], k [Hkv, N, D] device tensors (k in layout storage order)."""
    Hq, Hkv, D, N = q_last.shape[0], k.shape[0], k.shape[2], lay.n_global
    T = N // 64
    out = {
        "v": torch.empty(Hq, N, device=DEV), "s": torch.empty(Hq, T, device=DEV),
        "vidx": torch.full((Hq, N), -7, dtype=torch.int32, device=DEV),
        "vcnt": torch.empty(Hq, dtype=torch.int32, device=DEV),
        "sidx": torch.full((Hq, T), -7, dtype=torch.int32, device=DEV),
        "scnt": torch.empty(Hq, dtype=torch.int32, device=DEV),
    }
    ws = torch.empty(vs.index_workspace_size(Hq, Hkv, N, D, q_last.shape[1]), dtype=torch.uint8, device=DEV)
    vs.vs_index_build(q_last, k, lay, scale, top_p, out["v"], out["s"], out["vidx"], out["vcnt"],
                      out["sidx"], out["scnt"], ws)
    torch.cuda.synchronize()
    return out


def lists_from_gpu(idx):
    vc, sc = idx["vcnt"].cpu().numpy(), idx["scnt"].cpu().numpy()
    vi, si = idx["vidx"].cpu().numpy(), idx["sidx"].cpu().numpy()
    return [vi[h, :vc[h]].astype(np.int64) for h in range(len(vc))], [si[h, :sc[h]].astype(np.int64)
                                                                        for h in range(len(sc))]


def upload_lists(vert, slash, N):
    Hq, T = len(vert), N // 64
    vi = np.zeros((Hq, N), dtype=np.int32)
    si = np.zeros((Hq, T), dtype=np.int32)
    for h in range(Hq):
        vi[h, :len(vert[h])] = vert[h]
        si[h, :len(slash[h])] = slash[h]
    vc = np.array([len(x) for x in vert], dtype=np.int32)
    sc = np.array([len(x) for x in slash], dtype=np.int32)
    return (torch.tensor(vi, device=DEV), torch.tensor(vc, device=DEV), torch.tensor(si, device=DEV),
            torch.tensor(sc, device=DEV))


def tile_cap_for(slash, Hq, QB):
    """Tiles a mask can list: per query block at most one per selected diagonal
    under 64-token layouts and at most two per diagonal under one-position
    stripes (a diagonal j meets block offsets floor(j / P) and ceil(j / P))."""
    return max(1, Hq * QB * (2 * max(len(s) for s in slash) + 1))


def gpu_mask(lists_dev, Hq, Hkv, lay, rank, step, tile_cap):
    m = vs.Mask(Hq, Hkv, lay, tile_cap)
    vs.vs_block_mask(*lists_dev, rank, step, m)
    torch.cuda.synchronize()
    return m


def mask_to_numpy(m):
    return {k: v.cpu().numpy() for k, v in m.arrays().items()}


def shard(x, kind, P, rank):
    """Rows of a global [H, N, D] array held by `rank`, in storage order."""
    return x[:, ol.shard_positions(kind, x.shape[1], P, rank)]


def storage_order(x, kind, P):
    """Concatenate every rank's shard (the key layout the index step reads)."""
    return np.concatenate([shard(x, kind, P, r) for r in range(P)], axis=1)


def oracle_step_forward(q, k, v, vert, slash, kind, P, rank, step, scale, heads=None, blocks=None):
    """Oracle O/LSE of the rank's query blocks against shard (rank-step) mod P.
    q [Hq, N, D], k/v [Hkv, N, D] global order (float32 holding dtype-exact values)."""
    Hq, N, D = q.shape
    Hkv = k.shape[0]
    rows_all = ol.shard_positions(kind, N, P, rank)
    cols = ol.shard_positions(kind, N, P, ol.ring_source(rank, step, P))
    heads = range(Hq) if heads is None else heads
    blocks = range(len(rows_all) // 64) if blocks is None else blocks
    out = {}
    for h in heads:
        g = h * Hkv // Hq
        for I in blocks:
            rows = rows_all[64 * I:64 * I + 64]
            M, _, _ = om.active(rows, cols, vert[h], slash[h])
            used = M.any(axis=0)
            o, lse = oa.forward_rows(q[h, rows], k[g, cols[used]], v[g, cols[used]], M[:, used], scale)
            out[(h, I)] = (o, lse)
    return out


def check_index(out, ref, top_p):
    """GPU index (gpu_index output) against the oracle's build_index result:
    scores within 1e-4 relative (+1e-7 of the row max); the selection equals
    the oracle's top-p rule applied to the GPU's own scores (bit-exact); and
    against the oracle's selection it differs only in positions whose oracle
    score lies within 1e-5 of the cutoff score (ties at the budget edge)."""
    from oracle import index as oi
    gv, gs = out["v"].cpu().numpy(), out["s"].cpu().numpy()
    for g, o in ((gv, ref["v"]), (gs, ref["s"])):
        o64 = o.astype(np.float64)
        tol = 1e-4 * np.abs(o64) + 1e-7 * o64.max(axis=1, keepdims=True)
        assert (np.abs(g - o64) <= tol).all(), np.abs(g - o64).max()
    vert, slash = lists_from_gpu(out)
    for h in range(gv.shape[0]):
        assert np.array_equal(vert[h], oi.select_top_p(gv[h], top_p)), h
        assert np.array_equal(slash[h], oi.select_top_p(gs[h], top_p)), h
        for got, exp, x in ((vert[h], ref["vert"][h], ref["v"][h]), (slash[h], ref["slash"][h], ref["s"][h])):
            diff = np.setxor1d(got, exp)
            if len(diff) and len(exp):
                cut = x[exp].min()
                assert (np.abs(x[diff].astype(np.float64) - cut) <= 1e-5).all(), (h, diff)
    return vert, slash
