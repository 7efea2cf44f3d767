"""GPU active-region compaction vs the oracle's definition (bit-exact)."""
import numpy as np
import torch
import pytest

from oracle import layout as ol
from oracle import mask as om

pytestmark = pytest.mark.gpu


def _random_index(rng, N, Hq, nv, ns, force_diag=None):
    T = N // 64
    vert = [np.sort(rng.choice(N, rng.integers(0, nv + 1), replace=False)) for _ in range(Hq)]
    slash = []
    for h in range(Hq):
        s = set(rng.choice(T, rng.integers(0, ns + 1), replace=False).tolist())
        if force_diag is not None:
            s.discard(0)
            if force_diag[h]:
                s.add(0)
        slash.append(np.array(sorted(s), dtype=np.int64))
    return vert, slash


def _check_mask(vert, slash, Hq, Hkv, kind, P, rank, step, N):
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    lay = vs.layout(kind, P, N)
    QB = N // 64 // P
    m = H.gpu_mask(H.upload_lists(vert, slash, N), Hq, Hkv, lay, rank, step, H.tile_cap_for(slash, Hq, QB))
    a = H.mask_to_numpy(m)
    assert a["status"][0] == 0
    desc = om.step_description(kind, N, P, rank, step, vert, slash)
    src = ol.ring_source(rank, step, P)
    for h in range(Hq):
        vloc = desc["vloc"][h]
        assert a["vloc_cnt"][h] == len(vloc)
        assert np.array_equal(a["vloc"][h * QB * 64: h * QB * 64 + len(vloc)], vloc)
        vcum = np.searchsorted(vloc, np.arange(QB + 1) * 64, side="left")
        assert np.array_equal(a["vcum"][h * (QB + 1):(h + 1) * (QB + 1)], vcum)
        bits = np.zeros(m.desc.W * 32, dtype=np.int64)
        bits[slash[h]] = 1
        words = (bits.reshape(-1, 32) << np.arange(32)).sum(1).astype(np.uint32).view(np.int32)
        assert np.array_equal(a["slash_bits"][h * m.desc.W:(h + 1) * m.desc.W], words)
        csc = om.csc_from_description(desc, h)
        for I in range(QB):
            b = desc["blocks"][(h, I)]
            u = h * QB + I
            got = a["tile_col"][a["tile_ptr"][u]:a["tile_ptr"][u + 1]]
            exp = np.array([J | (0x40000000 if d else 0) for J, d in zip(b["tiles"], b["diag"])], dtype=np.int64)
            assert np.array_equal(got.astype(np.int64), exp), (h, I)
            assert a["vert_end"][u] == b["vert_end"], (h, I)
            assert a["n_active"][u] == b["n_active"], (h, I)
        for J in range(QB):
            u = h * QB + J
            got = a["csc_row"][a["csc_ptr"][u]:a["csc_ptr"][u + 1]]
            exp = np.array([I | (0x40000000 if d else 0) for I, d in csc[J]], dtype=np.int64)
            assert np.array_equal(got.astype(np.int64), exp), (h, J)
    return a


@pytest.mark.parametrize("kind,P", [("contig", 1), ("striped", 2), ("striped", 4), ("zigzag", 2),
                                    ("zigzag", 4), ("contig", 4)])
def test_mask_bitexact_layouts(kind, P):
    rng = np.random.default_rng(P * 7 + len(kind))
    N, Hq, Hkv = 64 * 32, 4, 2
    vert, slash = _random_index(rng, N, Hq, 120, 12, force_diag=[1, 0, 1, 0])
    for rank in range(P):
        for step in range(P):
            _check_mask(vert, slash, Hq, Hkv, kind, P, rank, step, N)


@pytest.mark.parametrize("P", [1, 2, 3, 4, 8, 32])
def test_mask_bitexact_stripe1(P):
    """One-position stripes: every (rank, step) of small rings, and sampled
    (rank, step) pairs at P = 8 and 32, against the oracle's description.
    Slash sets mix sparse diagonals with whole windows of 2P - 1 consecutive
    diagonals (full tiles) and heads without diagonal 0."""
    rng = np.random.default_rng(300 + P)
    N, Hq, Hkv = 64 * P * (24 if P <= 4 else 6), 4, 2
    T = N // 64
    vert, slash = _random_index(rng, N, Hq, 150, 10, force_diag=[1, 0, 1, 0])
    run = min(T - 1, 3 * P)
    slash[2] = np.union1d(slash[2], np.arange(1, run)).astype(np.int64)
    slash[3] = np.union1d(slash[3], np.arange(T - run, T)).astype(np.int64)
    pairs = [(r, s) for r in range(P) for s in range(P)] if P <= 4 else \
        [(0, 0), (P - 1, 0), (1, P - 1), (P // 2, 3), (P - 1, P - 1)]
    for rank, step in pairs:
        _check_mask(vert, slash, Hq, Hkv, "striped1", P, rank, step, N)


def test_mask_edge_cases():
    N, Hq = 64 * 8, 3
    # empty index, full index, and only the diagonal
    vert = [np.zeros(0, dtype=np.int64), np.arange(N), np.array([0, 63, 64, 511])]
    slash = [np.zeros(0, dtype=np.int64), np.arange(N // 64), np.array([0])]
    _check_mask(vert, slash, Hq, 1, "contig", 1, 0, 0, N)
    _check_mask(vert, slash, Hq, 1, "striped", 2, 1, 1, N)
    _check_mask(vert, slash, Hq, 1, "striped1", 2, 1, 1, N)
    _check_mask(vert, slash, Hq, 1, "striped1", 4, 0, 3, N)


def test_mask_capacity_overflow_reported():
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    N, Hq = 64 * 16, 2
    vert = [np.arange(0, N, 5)] * Hq
    slash = [np.arange(N // 64)] * Hq
    lay = vs.layout("contig", 1, N)
    m = H.gpu_mask(H.upload_lists(vert, slash, N), Hq, 1, lay, 0, 0, tile_cap=10)
    a = H.mask_to_numpy(m)
    assert a["status"][0] == vs.VS_ERR_CAPACITY
    # every list reads as empty, so consumers queued behind the mask do nothing
    assert (a["tile_ptr"] == 0).all() and (a["csc_ptr"] == 0).all()
    assert (a["vloc_cnt"] == 0).all() and (a["vert_end"] == 0).all()
    # the exact active counts survive
    for h in range(Hq):
        assert a["n_active"][h * 16:(h + 1) * 16].sum() == om.active_count(N, vert[h], slash[h])
    # a forward and a backward queued behind the overflowed mask compute nothing
    rng = np.random.default_rng(9)
    q = H.to_dev(rng.standard_normal((Hq, N, 128)), "bf16")
    k = H.to_dev(rng.standard_normal((1, N, 128)), "bf16")
    v = H.to_dev(rng.standard_normal((1, N, 128)), "bf16")
    do = H.to_dev(rng.standard_normal((Hq, N, 128)), "bf16")
    o = torch.full((Hq, N, 128), 7.0, device="cuda")
    lse = torch.full((Hq, N), 7.0, device="cuda")
    vs.vs_attn_fwd(q, k, v, m, 0.088, o, lse)
    dq = torch.zeros(Hq, N, 128, device="cuda")
    dk = torch.zeros(1, N, 128, device="cuda")
    dv = torch.zeros(1, N, 128, device="cuda")
    delta = torch.zeros(Hq, N, device="cuda")
    vs.vs_attn_bwd(q, k, v, do, torch.zeros(Hq, N, device="cuda"), delta, m, 0.088, dq, dk, dv)
    torch.cuda.synchronize()
    assert (o == 0).all() and torch.isneginf(lse).all()
    assert (dq == 0).all() and (dk == 0).all() and (dv == 0).all()


def test_mask_full_size_striped_rank_share():
    """Rank share of a 524288-token sequence at P=32 (one step), sampled blocks vs the oracle."""
    import dynamic_sparse_attention_index_amd as vs
    from tests import vs_harness as H
    rng = np.random.default_rng(5)
    N, Hq, Hkv, P = 524288, 16, 2, 32
    vert = [np.sort(rng.choice(N, 3000, replace=False)) for _ in range(Hq)]
    slash = [np.sort(np.unique(np.concatenate([[0, 1, 2], rng.choice(N // 64, 60, replace=False)])))
             for _ in range(Hq)]
    QB = N // 64 // P
    for rank, step in [(0, 0), (31, 5), (7, 20)]:
        m = H.gpu_mask(H.upload_lists(vert, slash, N), Hq, Hkv, vs.layout("striped", P, N), rank, step,
                       H.tile_cap_for(slash, Hq, QB))
        a = H.mask_to_numpy(m)
        assert a["status"][0] == 0
        blocks = sorted(set([0, QB - 1] + rng.choice(QB, 6, replace=False).tolist()))
        desc = om.step_description("striped", N, P, rank, step, vert, slash, heads=[0, 9], blocks=blocks)
        for h in (0, 9):
            assert np.array_equal(a["vloc"][h * QB * 64:h * QB * 64 + a["vloc_cnt"][h]], desc["vloc"][h])
            for I in blocks:
                b = desc["blocks"][(h, I)]
                u = h * QB + I
                got = a["tile_col"][a["tile_ptr"][u]:a["tile_ptr"][u + 1]]
                exp = [J | (0x40000000 if d else 0) for J, d in zip(b["tiles"], b["diag"])]
                assert got.tolist() == exp
                assert a["vert_end"][u] == b["vert_end"] and a["n_active"][u] == b["n_active"]
