"""Pins of the oracle's index step (row statistics, v/s scores, top-p selection)."""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import index as oi
from synth import config_by_name, generate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_lse_matches_library_logsumexp():
    q = _rand((3, 64, 16), 1)
    k = _rand((1, 256, 16), 2)
    zs, lse = oi.row_stats(q, k, 0.25, 256)
    for h in range(3):
        for r in range(64):
            n = 256 - 64 + r
            z = q[h, r] @ k[0, : n + 1].T * 0.25
            assert abs(lse[h, r] - logsumexp(z)) < 1e-12


def test_scores_closed_form_equal_keys():
    # every key equal -> each causal row is uniform: A[n, m] = 1/(n+1)
    N, L = 256, 64
    q = _rand((2, L, 8), 3)
    k = np.tile(_rand((1, 1, 8), 4), (1, N, 1))
    v, s, _ = oi.scores(q, k, 0.3, N)
    for m in range(N):
        exact = sum(Fraction(1, n + 1) for n in range(max(m, N - L), N)) / L
        assert abs(v[0, m] - float(exact)) <= 2e-7 * float(exact)
    T = N // 64
    for j in range(T):
        blk = T - 1 - j
        exact = sum(sum(Fraction(1, n + 1) for n in range(max(m, N - L), N)) for m in range(64 * blk, 64 * blk + 64)) / L
        assert abs(s[0, j] - float(exact)) <= 2e-7 * float(exact)


def test_scores_bruteforce_loops():
    N, L, D = 128, 64, 4
    q = _rand((1, L, D), 5)
    k = _rand((1, N, D), 6)
    scale = 0.5
    v, s, _ = oi.scores(q, k, scale, N)
    vb = [0.0] * N
    sb = [0.0] * (N // 64)
    for r in range(L):
        n = N - L + r
        zs = [sum(q[0, r, d] * k[0, m, d] for d in range(D)) * scale for m in range(n + 1)]
        mx = max(zs)
        tot = sum(math.exp(z - mx) for z in zs)
        for m in range(n + 1):
            a = math.exp(zs[m] - mx) / tot
            vb[m] += a / L
            sb[n // 64 - m // 64] += a / L
    assert np.allclose(v[0], np.float32(vb), rtol=1e-6, atol=0)
    assert np.allclose(s[0], np.float32(sb), rtol=1e-6, atol=0)


def test_scores_invariants():
    N = 1024
    q = _rand((4, 64, 16), 7)
    k = _rand((2, N, 16), 8) * 2
    v, s, _ = oi.scores(q, k, 0.25, N)
    assert (v >= 0).all() and (s >= 0).all()
    assert np.allclose(v.astype(np.float64).sum(1), 1.0, atol=1e-5)
    assert np.allclose(s.astype(np.float64).sum(1), 1.0, atol=1e-5)
    # with last_q = 64 rows in the final block, s(j) is the mass of key block T-1-j
    T = N // 64
    blocks = v.astype(np.float64).reshape(4, T, 64).sum(2)[:, ::-1]
    assert np.allclose(s, blocks, rtol=1e-5, atol=1e-9)


def _read_golden_select():
    cases = []
    for line in open(os.path.join(GOLDEN, "select_top_p.txt")):
        if line.startswith("#") or not line.strip():
            continue
        xs, p, sel = line.split(";")
        cases.append((np.array([float(t) for t in xs.split()], dtype=np.float32), float(p),
                      [int(t) for t in sel.split()]))
    return cases


@pytest.mark.parametrize("x,p,expected", _read_golden_select())
def test_select_golden(x, p, expected):
    assert list(oi.select_top_p(x, p)) == expected


def _brute_select(x_units, p_num, p_den):
    """Exact rational brute force: smallest subset reaching p * total, then the
    largest-mass such subset, then lexicographically smallest sorted indices."""
    n = len(x_units)
    total = sum(x_units)
    tgt = Fraction(p_num, p_den) * total
    for k in range(n + 1):
        best = None
        for comb in itertools.combinations(range(n), k):
            mass = sum(x_units[i] for i in comb)
            if mass >= tgt:
                key = (-mass, comb)
                if best is None or key < best:
                    best = key
        if best is not None:
            return list(best[1])
    return list(range(n))


@pytest.mark.parametrize("seed", range(40))
def test_select_bruteforce(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 11))
    units = rng.integers(0, 6, size=n)           # dyadic scores: units * 2^-20, many ties
    if units.sum() == 0:
        units[0] = 1
    x = (units * 2.0 ** -20).astype(np.float32)
    p_num = int(rng.integers(1, 256))
    got = list(oi.select_top_p(x, p_num / 256.0))
    assert got == _brute_select([int(u) for u in units], p_num, 256)


def test_select_edges_and_monotone():
    x = np.random.default_rng(0).random(500).astype(np.float32)
    assert len(oi.select_top_p(x, 1.0)) == 500
    assert len(oi.select_top_p(x, 1.5)) == 500
    assert len(oi.select_top_p(x, 0.0)) == 0
    assert len(oi.select_top_p(x, -0.2)) == 0
    prev = set()
    for p in np.linspace(0.05, 0.99, 25):
        cur = set(oi.select_top_p(x, p).tolist())
        assert prev <= cur
        prev = cur


def _golden_lines(name):
    for line in open(os.path.join(GOLDEN, name)):
        if not line.startswith("#") and line.strip():
            yield [f.split() for f in line.split(";")]


@pytest.mark.parametrize("x,k,expected", [
    (np.array(xs, dtype=np.float32), int(k[0]), [int(t) for t in sel])
    for xs, k, sel in _golden_lines("select_top_k.txt")])
def test_select_top_k_golden(x, k, expected):
    assert list(oi.select_top_k(x, k)) == expected


def _brute_top_k(x_units, k):
    """Largest-mass subset of size min(k, n), then the lexicographically
    smallest sorted indices."""
    n = len(x_units)
    k = max(0, min(k, n))
    best = None
    for comb in itertools.combinations(range(n), k):
        key = (-sum(x_units[i] for i in comb), comb)
        if best is None or key < best:
            best = key
    return list(best[1])


@pytest.mark.parametrize("seed", range(30))
def test_select_top_k_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 10))
    units = rng.integers(0, 5, size=n)
    x = (units * 2.0 ** -20).astype(np.float32)
    k = int(rng.integers(-1, n + 2))
    assert list(oi.select_top_k(x, k)) == _brute_top_k([int(u) for u in units], k)


@pytest.mark.parametrize("v,s,p,ev,es", [
    (np.array(v, dtype=np.float32), np.array(s, dtype=np.float32), float(p[0]), [int(t) for t in ev],
     [int(t) for t in es]) for v, s, p, ev, es in _golden_lines("select_joint.txt")])
def test_select_joint_golden(v, s, p, ev, es):
    gv, gs = oi.select_joint_top_p(v, s, p)
    assert (list(gv), list(gs)) == (ev, es)


@pytest.mark.parametrize("seed", range(30))
def test_select_joint_bruteforce(seed):
    """Fewest pooled candidates reaching p of the pooled mass (exact rationals;
    candidate order: verticals, then slashes)."""
    rng = np.random.default_rng(200 + seed)
    nv, ns = int(rng.integers(1, 7)), int(rng.integers(1, 5))
    uv, us = rng.integers(0, 6, size=nv), rng.integers(0, 9, size=ns)
    if uv.sum() + us.sum() == 0:
        uv[0] = 1
    v = (uv * 2.0 ** -20).astype(np.float32)
    s = (us * 2.0 ** -20).astype(np.float32)
    p_num = int(rng.integers(1, 256))
    gv, gs = oi.select_joint_top_p(v, s, p_num / 256.0)
    want = _brute_select([int(u) for u in uv] + [int(u) for u in us], p_num, 256)
    assert list(gv) == [i for i in want if i < nv]
    assert list(gs) == [i - nv for i in want if i >= nv]


def test_select_joint_properties():
    rng = np.random.default_rng(5)
    v = rng.random(3000).astype(np.float32) ** 8
    s = rng.random(47).astype(np.float32) ** 4
    for p in (0.3, 0.8, 0.95):
        gv, gs = oi.select_joint_top_p(v, s, p)
        # the separate selections together also reach p of the pooled mass,
        # so the joint count can be no larger than theirs
        assert len(gv) + len(gs) <= len(oi.select_top_p(v, p)) + len(oi.select_top_p(s, p))
        # no slash candidates: the joint budget is the vertical top-p
        jv, js = oi.select_joint_top_p(v, np.zeros_like(s), p)
        assert list(jv) == list(oi.select_top_p(v, p)) and len(js) == 0
    gv, gs = oi.select_joint_top_p(v, s, 1.0)
    assert len(gv) == 3000 and len(gs) == 47
    gv, gs = oi.select_joint_top_p(v, s, 0.0)
    assert len(gv) == 0 and len(gs) == 0


def _index_for(cfg):
    t = generate(cfg, tensors=("q", "k"), rows=None)
    q_last = t["q"][:, cfg.N - cfg.last_q:]
    return oi.build_index(q_last, t["k"], cfg.scale, cfg.N, cfg.top_p), t["outliers"]


@pytest.mark.parametrize("seed", [1001, 7, 8, 9])
def test_planted_outliers_are_top_verticals_literal_inputs(seed):
    # literal tiny workload: N(0,1) inputs, 8 keys scaled x8
    cfg = config_by_name("tiny", seed=seed)
    idx, outl = _index_for(cfg)
    top8 = np.sort(np.argsort(-idx["v"][0].astype(np.float64), kind="stable")[:8])
    assert list(top8) == list(outl)
    assert set(outl.tolist()) <= set(idx["vert"][0].tolist())


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_planted_vertical_and_slash_band(seed):
    # shared mean (slash band) plus moderate outliers (vertical lines)
    cfg = config_by_name("tiny", seed=seed, c=6.0, f_out=3.0)
    idx, outl = _index_for(cfg)
    assert set(outl.tolist()) <= set(idx["vert"][0].tolist())
    assert {0, 1} <= set(idx["slash"][0].tolist())


def test_negative_control_no_structure():
    cfg = config_by_name("tiny", seed=5, n_out=0)
    idx, _ = _index_for(cfg)
    # with no mean and no outliers the mass is spread: most columns are needed
    assert len(idx["vert"][0]) > 0.5 * cfg.N


@pytest.mark.parametrize("kind,P", [("contig", 4), ("striped", 4), ("zigzag", 2), ("striped", 8)])
def test_distributed_index_equals_global(kind, P):
    """Per-rank partial statistics, merged, give the global index (the same
    scores up to fp64 rounding and the same selections)."""
    rng = np.random.default_rng(7 + P)
    Hq, Hkv, L, D, N = 4, 2, 64, 16, 1024
    q = rng.standard_normal((Hq, L, D))
    k = rng.standard_normal((Hkv, N, D))
    k[:, rng.choice(N, 6, replace=False)] *= 5.0
    g = oi.build_index(q, k, 0.25, N, 0.9)
    d = oi.build_index_distributed(q, k, 0.25, N, 0.9, kind, P)
    np.testing.assert_allclose(d["lse"], g["lse"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(d["v"], g["v"], rtol=1e-6, atol=0)
    np.testing.assert_allclose(d["s"], g["s"], rtol=1e-6, atol=0)
    for h in range(Hq):
        assert np.array_equal(d["vert"][h], g["vert"][h])
        assert np.array_equal(d["slash"][h], g["slash"][h])


def test_merge_row_stats_handles_empty_ranks():
    """A rank that holds no causal key of a row contributes (-inf, 0)."""
    m = [np.array([[1.0, -np.inf]]), np.array([[-np.inf, -np.inf]]), np.array([[3.0, -np.inf]])]
    l = [np.array([[2.0, 0.0]]), np.array([[0.0, 0.0]]), np.array([[1.5, 0.0]])]
    lse = oi.merge_row_stats(list(zip(m, l)))
    assert lse[0, 1] == -np.inf
    np.testing.assert_allclose(lse[0, 0], np.log(2.0 * np.exp(1.0) + 1.5 * np.exp(3.0)), rtol=1e-15)


def test_select_group_hand_case():
    """Per-kv-head selection, hand-derived: q heads 0, 1 share kv head 0 and
    q heads 2, 3 kv head 1 (consecutive q heads form a group). Group means:
    [0.4, 0.4, 0.1, 0.1] and [0.1, 0.1, 0.4, 0.4]; at p = 0.75 the two 0.4
    columns (0.8) are the fewest that reach it. Grouping heads h % Hkv
    instead would pair heads 0 and 2 and give other lists."""
    v = np.array([[0.7, 0.1, 0.1, 0.1], [0.1, 0.7, 0.1, 0.1],
                  [0.1, 0.1, 0.1, 0.7], [0.1, 0.1, 0.7, 0.1]], dtype=np.float32)
    s = v.copy()
    vert, slash = oi.select_group_top_p(v, s, 2, 0.75)
    for h, exp in enumerate([[0, 1], [0, 1], [2, 3], [2, 3]]):
        assert vert[h].tolist() == exp and slash[h].tolist() == exp


@pytest.mark.parametrize("seed", range(6))
def test_select_group_reductions(seed):
    """One q head per kv head is the per-head rule; with dyadic scores (exact
    means) the group lists equal the top-p of the group's summed scores, and
    every q head of a group gets the same list."""
    rng = np.random.default_rng(500 + seed)
    Hq, N = 8, 256
    v = (rng.integers(0, 64, (Hq, N)) * rng.integers(0, 2, (Hq, N))).astype(np.float32) / 1024
    s = rng.integers(0, 64, (Hq, N // 4)).astype(np.float32) / 1024
    p = float(rng.uniform(0.3, 0.99))
    vert, slash = oi.select_group_top_p(v, s, Hq, p)
    for h in range(Hq):
        assert np.array_equal(vert[h], oi.select_top_p(v[h], p))
        assert np.array_equal(slash[h], oi.select_top_p(s[h], p))
    for Hkv in (1, 2, 4):
        R = Hq // Hkv
        vert, slash = oi.select_group_top_p(v, s, Hkv, p)
        for g in range(Hkv):
            sv = v[g * R:(g + 1) * R].astype(np.float64).sum(axis=0) / R * (R // 2 if R > 1 else 1)
            # R is a power of two and the scores dyadic: the mean, and the sum
            # scaled by 2^k, are exact in fp32 and select the same set
            sel = oi.select_top_p(np.float32(1.0) * (v[g * R:(g + 1) * R].astype(np.float64).mean(axis=0))
                                  .astype(np.float32), p)
            assert np.array_equal(sel, oi.select_top_p(sv.astype(np.float32), p))
            for h in range(g * R, (g + 1) * R):
                assert np.array_equal(vert[h], sel)
                assert np.array_equal(slash[h], slash[g * R])


def test_select_group_mean_not_max_or_first():
    """The group statistic is the mean of the group's q heads, hand-derived on
    dyadic scores where the mean, the max and the first head disagree:
      head 0 = [1/2, 1/4, 1/4, 0], head 1 = [0, 1/4, 1/4, 1/2] (one kv group)
      mean   = [1/4, 1/4, 1/4, 1/4]: p = 1/2 needs two; ties to the lower index -> {0, 1}
      max    = [1/2, 1/4, 1/4, 1/2]: total 3/2, target 3/4 -> {0, 3}
      head 0 alone: 1/2 reaches 1/2 -> {0}
    so only the mean gives {0, 1}."""
    v = np.array([[0.5, 0.25, 0.25, 0.0], [0.0, 0.25, 0.25, 0.5]], dtype=np.float32)
    assert oi.group_scores(v, 1).tolist() == [[0.25, 0.25, 0.25, 0.25]]
    vert, slash = oi.select_group_top_p(v, v.copy(), 1, 0.5)
    for h in range(2):
        assert vert[h].tolist() == [0, 1] and slash[h].tolist() == [0, 1]
    assert oi.select_top_p(v.max(axis=0), 0.5).tolist() == [0, 3]
    assert oi.select_top_p(v[0], 0.5).tolist() == [0]
