"""Pins of the oracle's layouts, active set and per-block description."""
import os

import numpy as np
import pytest

from oracle import layout as ol
from oracle import mask as om
from synth import layout_permutation

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("kind", ["contig", "striped", "zigzag", "striped1"])
@pytest.mark.parametrize("P", [1, 2, 4, 8])
def test_layout_partition_and_agreement(kind, P):
    N = 64 * 32
    parts = [ol.shard_positions(kind, N, P, r) for r in range(P)]
    allpos = np.sort(np.concatenate(parts))
    assert (allpos == np.arange(N)).all()
    for r in range(P):
        assert (parts[r] == layout_permutation(kind, N, P, r)).all()
        assert len(parts[r]) == N // P
        if kind == "striped":
            assert ((parts[r] // 64) % P == r).all()
        if kind == "striped1":
            assert (parts[r] % P == r).all()
        if kind == "zigzag":
            ch = parts[r] // (N // (2 * P))
            assert set(ch.tolist()) == {r, 2 * P - 1 - r}


def test_ring_source_visits_every_shard():
    P = 8
    for r in range(P):
        assert sorted(ol.ring_source(r, s, P) for s in range(P)) == list(range(P))
        assert ol.ring_source(r, 0, P) == r


def _brute_mask(rows, cols, V, S):
    M = np.zeros((len(rows), len(cols)), dtype=bool)
    Vs, Ss = set(int(x) for x in V), set(int(x) for x in S)
    for a, n in enumerate(rows):
        for b, m in enumerate(cols):
            if m <= n and (m in Vs or (n // 64 - m // 64) in Ss):
                M[a, b] = True
    return M


def test_active_matches_bruteforce():
    rng = np.random.default_rng(0)
    N = 256
    V = np.sort(rng.choice(N, 20, replace=False))
    S = np.array([0, 2])
    rows = np.arange(N)
    M, _, _ = om.active(rows, rows, V, S)
    assert (M == _brute_mask(rows, rows, V, S)).all()


def test_golden_tiny_mask():
    V, S = np.array([5, 70]), np.array([0, 2])
    desc = om.step_description("contig", 192, 1, 0, 0, [V], [S])
    for line in open(os.path.join(GOLDEN, "mask_tiny.txt")):
        if line.startswith("#") or not line.strip():
            continue
        blk, tiles, vend, nact = [t.strip() for t in line.split(";")]
        b = desc["blocks"][(0, int(blk))]
        exp_t = [tuple(int(u) for u in t.split(":")) for t in tiles.split()]
        assert [(int(J), int(d)) for J, d in zip(b["tiles"], b["diag"])] == exp_t
        assert b["vert_end"] == int(vend)
        assert b["n_active"] == int(nact)


def _structural_tiles(kind, N, P, r, s, I, S):
    """Tile list from the block-diagonal structure: key block J of the visible
    shard is listed iff G(I) - G'(J) is a selected diagonal (>= 0)."""
    rows = ol.shard_positions(kind, N, P, r)
    cols = ol.shard_positions(kind, N, P, ol.ring_source(r, s, P))
    G = rows[64 * I] // 64
    out = []
    for J in range(len(cols) // 64):
        Gp = cols[64 * J] // 64
        if G - Gp >= 0 and (G - Gp) in set(S.tolist()):
            out.append((J, G == Gp))
    return out


@pytest.mark.parametrize("kind", ["contig", "striped", "zigzag"])
@pytest.mark.parametrize("P", [1, 2, 4])
def test_step_description_partition(kind, P):
    rng = np.random.default_rng(P + len(kind))
    N = 64 * 16
    Hq = 2
    vert = [np.sort(rng.choice(N, 40, replace=False)) for _ in range(Hq)]
    slash = [np.sort(rng.choice(N // 64, 4, replace=False)) for _ in range(Hq)]
    totals = np.zeros(Hq, dtype=np.int64)
    for r in range(P):
        rows = ol.shard_positions(kind, N, P, r)
        for s in range(P):
            desc = om.step_description(kind, N, P, r, s, vert, slash)
            cols = ol.shard_positions(kind, N, P, ol.ring_source(r, s, P))
            for h in range(Hq):
                for I in range(desc["QB"]):
                    b = desc["blocks"][(h, I)]
                    assert [(int(J), bool(d)) for J, d in zip(b["tiles"], b["diag"])] == \
                        _structural_tiles(kind, N, P, r, s, I, slash[h])
                    Mb = _brute_mask(rows[64 * I:64 * I + 64], cols, vert[h], slash[h])
                    assert b["n_active"] == int(Mb.sum())
                    totals[h] += b["n_active"]
    # every active entry of the full causal square lies in exactly one (rank, step) slot
    for h in range(Hq):
        full = _brute_mask(np.arange(N), np.arange(N), vert[h], slash[h]).sum()
        assert totals[h] == full == om.active_count(N, vert[h], slash[h])


def test_active_count_closed_form_vs_dense():
    rng = np.random.default_rng(11)
    for trial in range(10):
        N = 64 * int(rng.integers(1, 9))
        V = np.sort(rng.choice(N, int(rng.integers(0, N // 2 + 1)), replace=False))
        T = N // 64
        S = np.sort(rng.choice(T, int(rng.integers(0, T + 1)), replace=False))
        full = _brute_mask(np.arange(N), np.arange(N), V, S).sum()
        assert om.active_count(N, V, S) == full


def test_csc_is_transpose():
    rng = np.random.default_rng(3)
    N = 64 * 12
    vert = [np.sort(rng.choice(N, 30, replace=False))]
    slash = [np.array([0, 1, 5])]
    desc = om.step_description("striped", N, 2, 1, 1, vert, slash)
    csc = om.csc_from_description(desc, 0)
    pairs_csr = sorted((I, int(J)) for I in range(desc["QB"]) for J in desc["blocks"][(0, I)]["tiles"])
    pairs_csc = sorted((I, J) for J, lst in csc.items() for I, _ in lst)
    assert pairs_csr == pairs_csc


def _golden_cases(fname):
    cases = []
    for line in open(os.path.join(GOLDEN, fname)):
        if line.startswith("#") or not line.strip():
            continue
        if line.startswith("@"):
            head, vloc = line[1:].split(";")
            kind, rank, step = head.split()
            cases.append((kind, int(rank), int(step), [int(x) for x in vloc.split()], []))
            continue
        blk, tiles, vend, nact = [t.strip() for t in line.split(";")]
        exp_t = [tuple(int(u) for u in t.split(":")) for t in tiles.split()]
        cases[-1][4].append((int(blk), exp_t, int(vend), int(nact)))
    return cases


def _check_golden(cases, V, S):
    for kind, rank, step, vloc, blocks in cases:
        desc = om.step_description(kind, 256, 2, rank, step, [V], [S])
        assert desc["vloc"][0].tolist() == vloc, (kind, rank, step)
        assert len(blocks) == desc["QB"] == 2
        for blk, exp_t, vend, nact in blocks:
            b = desc["blocks"][(0, blk)]
            assert [(int(J), int(d)) for J, d in zip(b["tiles"], b["diag"])] == exp_t, (kind, rank, step, blk)
            assert b["vert_end"] == vend, (kind, rank, step, blk)
            assert b["n_active"] == nact, (kind, rank, step, blk)


def test_golden_two_rank_mask():
    """Hand-derived descriptions of a 2-rank ring (striped and zigzag): tile
    lists, LOCAL vertical positions, vertical prefix lengths and counts."""
    cases = _golden_cases("mask_p2.txt")
    assert len(cases) == 5
    _check_golden(cases, np.array([10, 100, 150, 200]), np.array([0, 1]))


def test_golden_one_position_stripes():
    """Hand-derived descriptions under one-position stripes (P = 2): every
    listed tile is partial, counts per query block."""
    cases = _golden_cases("mask_stripe1.txt")
    assert len(cases) == 4
    _check_golden(cases, np.array([10, 77]), np.array([0]))


@pytest.mark.parametrize("P,slash_set", [(2, (0, 1, 5)), (4, (0, 1, 5)),
                                         (2, (0, 1, 2, 3, 4, 5, 9)), (4, tuple(range(12)) + (20,))])
def test_stripe1_description_by_enumeration(P, slash_set):
    """Under one-position stripes, for every (rank, step): a tile is listed
    iff the brute-force active set holds a slash entry in it, flagged iff not
    all of its entries are slash entries, counts per block, and the partition
    of the causal square over all (rank, step). The last two slash sets hold
    whole windows of 2P - 1 consecutive diagonals, so some off-diagonal tiles
    are full (unflagged) and the rest partial."""
    rng = np.random.default_rng(70 + P)
    N = 64 * 8 * P
    vert = [np.sort(rng.choice(N, 25, replace=False))]
    slash = [np.array(slash_set)]
    n_full = 0
    total = 0
    for r in range(P):
        rows = ol.shard_positions("striped1", N, P, r)
        for s_ in range(P):
            cols = ol.shard_positions("striped1", N, P, ol.ring_source(r, s_, P))
            desc = om.step_description("striped1", N, P, r, s_, vert, slash)
            for I in range(desc["QB"]):
                rb = rows[64 * I:64 * I + 64]
                Mb = _brute_mask(rb, cols, vert[0], slash[0])
                Sb = (cols[None, :] <= rb[:, None]) & np.isin(rb[:, None] // 64 - cols[None, :] // 64, slash[0])
                exp = [(J, bool(not Sb[:, 64 * J:64 * J + 64].all())) for J in range(len(cols) // 64)
                       if Sb[:, 64 * J:64 * J + 64].any()]
                b = desc["blocks"][(0, I)]
                assert [(int(J), bool(d)) for J, d in zip(b["tiles"], b["diag"])] == exp
                assert b["n_active"] == int(Mb.sum())
                total += b["n_active"]
                n_full += sum(1 for _, d in exp if not d)
    assert total == om.active_count(N, vert[0], slash[0])
    assert (n_full > 0) == (len(slash_set) > 3)


@pytest.mark.parametrize("kind", ["contig", "striped", "zigzag", "striped1"])
@pytest.mark.parametrize("P", [2, 4])
def test_step_description_verticals_by_enumeration(kind, P):
    """vloc and vert_end against a direct enumeration: vloc[k] is the storage
    index of the k-th visible vertical, and vert_end counts the visible
    verticals with at least one causal row in the query block."""
    rng = np.random.default_rng(40 + P + len(kind))
    N = 64 * 16
    vert = [np.sort(rng.choice(N, 30, replace=False))]
    slash = [np.array([0, 3])]
    for r in range(P):
        rows = ol.shard_positions(kind, N, P, r)
        for s in range(P):
            cols = ol.shard_positions(kind, N, P, ol.ring_source(r, s, P))
            desc = om.step_description(kind, N, P, r, s, vert, slash)
            exp_vloc = [b for b, m in enumerate(cols.tolist()) if m in set(vert[0].tolist())]
            assert desc["vloc"][0].tolist() == exp_vloc
            for I in range(desc["QB"]):
                last_row = int(rows[64 * I + 63])
                exp_end = sum(1 for b in exp_vloc if int(cols[b]) <= last_row)
                assert desc["blocks"][(0, I)]["vert_end"] == exp_end
