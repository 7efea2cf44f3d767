"""Pins of the oracle's masked attention forward, merge and backward."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import index as oi
from oracle import layout as ol
from oracle import mask as om


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _torch_ref(q, k, v, M, scale, do):
    """Masked attention through torch autograd in fp64 (rows with no key excluded)."""
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    tm = torch.tensor(M)
    nonempty = tm.any(1)
    s = (tq @ tk.T) * scale
    s = s.masked_fill(~tm, float("-inf"))
    p = torch.softmax(s[nonempty], dim=-1)
    o = torch.zeros_like(tq)
    o[nonempty] = p @ tv
    (o * torch.tensor(do)).sum().backward()
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def test_dense_causal_equals_sdpa_library():
    N, D = 192, 16
    q, k, v, do = (_rand((N, D), s) for s in range(4))
    M = np.tril(np.ones((N, N), dtype=bool))
    o, lse = oa.forward_rows(q, k, v, M, 1 / math.sqrt(D))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None], is_causal=True)[0]
    assert np.abs(o - ref.detach().numpy()).max() < 1e-12
    (ref * torch.tensor(do)).sum().backward()
    dq, dk, dv = oa.backward_rows(q, k, v, M, 1 / math.sqrt(D), do)
    assert np.abs(dq - tq.grad.numpy()).max() < 1e-11
    assert np.abs(dk - tk.grad.numpy()).max() < 1e-11
    assert np.abs(dv - tv.grad.numpy()).max() < 1e-11


def test_full_budget_index_gives_dense_mask():
    N = 256
    q = _rand((1, 64, 8), 1)
    k = _rand((1, N, 8), 2)
    idx = oi.build_index(q, k, 0.3, N, 1.0)
    M, _, _ = om.active(np.arange(N), np.arange(N), idx["vert"][0], idx["slash"][0])
    assert (M == np.tril(np.ones((N, N), dtype=bool))).all()


@pytest.mark.parametrize("seed", range(5))
def test_random_mask_vs_torch_autograd(seed):
    rng = np.random.default_rng(seed)
    R, C, D = 40, 70, 8
    q, k, v, do = _rand((R, D), seed), _rand((C, D), seed + 10), _rand((C, D), seed + 20), _rand((R, D), seed + 30)
    M = rng.random((R, C)) < 0.3
    M[3] = False                                  # an empty row
    o, lse = oa.forward_rows(q, k, v, M, 0.4)
    ro, rdq, rdk, rdv = _torch_ref(q, k, v, M, 0.4, do)
    assert np.abs(o - ro).max() < 1e-12
    assert (o[3] == 0).all() and lse[3] == -np.inf
    dq, dk, dv = oa.backward_rows(q, k, v, M, 0.4, do)
    assert np.abs(dq - rdq).max() < 1e-12
    assert np.abs(dk - rdk).max() < 1e-12
    assert np.abs(dv - rdv).max() < 1e-12


def test_bruteforce_loops_tiny():
    R, C, D = 6, 9, 3
    q, k, v = _rand((R, D), 1), _rand((C, D), 2), _rand((C, D), 3)
    M = np.random.default_rng(4).random((R, C)) < 0.5
    M[0] = False
    o, lse = oa.forward_rows(q, k, v, M, 0.7)
    for n in range(R):
        act = [m for m in range(C) if M[n, m]]
        if not act:
            assert lse[n] == -np.inf and (o[n] == 0).all()
            continue
        z = {m: sum(q[n, d] * k[m, d] for d in range(D)) * 0.7 for m in act}
        L = math.log(sum(math.exp(z[m]) for m in act))
        assert abs(lse[n] - L) < 1e-12
        for d in range(D):
            assert abs(o[n, d] - sum(math.exp(z[m] - L) * v[m, d] for m in act)) < 1e-12


def test_special_cases():
    R, C, D = 16, 24, 8
    q, k = _rand((R, D), 1), _rand((C, D), 2)
    M = np.random.default_rng(3).random((R, C)) < 0.4
    M[:, 0] = True
    vconst = np.tile(_rand((1, D), 4), (C, 1))
    o, _ = oa.forward_rows(q, k, vconst, M, 0.5)
    assert np.abs(o - vconst[0]).max() < 1e-12                      # V constant -> O constant
    M1 = np.zeros((R, C), dtype=bool)
    M1[np.arange(R), np.arange(R)] = True                            # one key per row
    v = _rand((C, D), 5)
    o, lse = oa.forward_rows(q, k, v, M1, 0.5)
    assert np.abs(o - v[:R]).max() < 1e-14
    assert np.abs(lse - (q * k[:R]).sum(1) * 0.5).max() < 1e-12


def test_finite_differences():
    R, C, D = 5, 7, 3
    scale = 0.6
    q, k, v, do = _rand((R, D), 1), _rand((C, D), 2), _rand((C, D), 3), _rand((R, D), 4)
    M = np.random.default_rng(5).random((R, C)) < 0.6
    M[:, 0] = True

    def f(q_, k_, v_):
        o, _ = oa.forward_rows(q_, k_, v_, M, scale)
        return (o * do).sum()

    dq, dk, dv = oa.backward_rows(q, k, v, M, scale, do)
    h = 1e-6
    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        for idx in np.ndindex(arr.shape):
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = ap, am
            fd = (f(*args_p) - f(*args_m)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(grad[idx]))


def test_gradient_invariants():
    R, C, D = 30, 50, 8
    q, k, v, do = _rand((R, D), 1), _rand((C, D), 2), _rand((C, D), 3), _rand((R, D), 4)
    M = np.random.default_rng(5).random((R, C)) < 0.3
    M[7] = False
    dq, dk, dv = oa.backward_rows(q, k, v, M, 0.5, do)
    nonempty = M.any(1)
    assert np.abs(dv.sum(0) - do[nonempty].sum(0)).max() < 1e-12
    assert np.abs(dk.sum(0)).max() < 1e-12
    assert (dq[7] == 0).all()
    kconst = np.tile(k[:1], (C, 1))
    dq2, _, _ = oa.backward_rows(q, kconst, v, M, 0.5, do)
    assert np.abs(dq2).max() < 1e-12
    z = oa.backward_rows(q, k, v, M, 0.5, np.zeros_like(do))
    assert all(np.abs(x).max() == 0 for x in z)


def test_merge_chunked_equals_one_shot():
    rng = np.random.default_rng(0)
    R, C, D = 20, 90, 6
    q, k, v = _rand((R, D), 1), _rand((C, D), 2), _rand((C, D), 3)
    M = rng.random((R, C)) < 0.3
    M[2] = False
    o_full, lse_full = oa.forward_rows(q, k, v, M, 0.5)
    cuts = [0, 10, 10, 45, 80, 90]                   # includes an empty chunk
    o_acc, lse_acc = np.zeros((R, D)), np.full(R, -np.inf)
    for a, b in zip(cuts[:-1], cuts[1:]):
        o_c, lse_c = oa.forward_rows(q, k[a:b], v[a:b], M[:, a:b], 0.5)
        o_acc, lse_acc = oa.merge(o_acc, lse_acc, o_c, lse_c)
    assert np.abs(o_acc - o_full).max() < 1e-12
    fin = np.isfinite(lse_full)
    assert np.abs(lse_acc[fin] - lse_full[fin]).max() < 1e-12
    assert (lse_acc[~fin] == -np.inf).all() and (o_acc[~fin] == 0).all()
    # identity and commutativity
    o1, l1 = oa.merge(o_full, lse_full, np.zeros((R, D)), np.full(R, -np.inf))
    assert np.abs(o1 - o_full).max() == 0
    oa_, la_ = oa.forward_rows(q, k[:30], v[:30], M[:, :30], 0.5)
    ob_, lb_ = oa.forward_rows(q, k[30:], v[30:], M[:, 30:], 0.5)
    x1 = oa.merge(oa_, la_, ob_, lb_)
    x2 = oa.merge(ob_, lb_, oa_, la_)
    assert np.abs(x1[0] - x2[0]).max() < 1e-14


@pytest.mark.parametrize("kind", ["striped", "zigzag", "contig"])
def test_ring_steps_reassemble_full(kind):
    rng = np.random.default_rng(1)
    N, D, P = 64 * 8, 8, 4
    q, k, v, do = _rand((N, D), 1), _rand((N, D), 2), _rand((N, D), 3), _rand((N, D), 4)
    V = np.sort(rng.choice(N, 30, replace=False))
    S = np.array([0, 3])
    scale = 0.4
    allp = np.arange(N)
    M_full, _, _ = om.active(allp, allp, V, S)
    o_ref, lse_ref = oa.forward_rows(q, k, v, M_full, scale)
    dq_ref, dk_ref, dv_ref = oa.backward_rows(q, k, v, M_full, scale, do)
    drow = (do * o_ref).sum(1)
    dk_sum, dv_sum = np.zeros_like(k), np.zeros_like(v)
    for r in range(P):
        rows = ol.shard_positions(kind, N, P, r)
        o_acc, lse_acc = np.zeros((len(rows), D)), np.full(len(rows), -np.inf)
        dq_r = np.zeros((len(rows), D))
        for s in range(P):
            cols = ol.shard_positions(kind, N, P, ol.ring_source(r, s, P))
            Ms, _, _ = om.active(rows, cols, V, S)
            o_s, l_s = oa.forward_rows(q[rows], k[cols], v[cols], Ms, scale)
            o_acc, lse_acc = oa.merge(o_acc, lse_acc, o_s, l_s)
            gq, gk, gv = oa.backward_rows(q[rows], k[cols], v[cols], Ms, scale, do[rows],
                                          lse=lse_ref[rows], drow=drow[rows])
            dq_r += gq
            dk_sum[cols] += gk
            dv_sum[cols] += gv
        assert np.abs(o_acc - o_ref[rows]).max() < 1e-12
        assert np.abs(dq_r - dq_ref[rows]).max() < 1e-11
    assert np.abs(dk_sum - dk_ref).max() < 1e-11
    assert np.abs(dv_sum - dv_ref).max() < 1e-11
