"""Pins for the float64 attention oracle (CPU only).

Each check ties the oracle to something it does not compute itself: finite
differences of the scalar loss sum(O * dO), torch's float64 autograd and
scaled_dot_product_attention, an unfused brute-force backward with explicit
softmax Jacobians, closed forms for degenerate inputs, and invariants that
follow from the mathematics. A mutation test at the end plants mistakes in a
copy of the backward and checks that these pins catch each one.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def fwd_bwd(q, k, v, do, causal, scale):
    o, lse = A.forward(q, k, v, causal, scale)
    dq, dk, dv = A.backward(q, k, v, o, do, lse, causal, scale)
    return o, lse, dq, dk, dv


# ------------------------------------------------------------------ finite differences

FD_SHAPES = [(1, 1, 1, 1), (1, 2, 2, 3), (1, 1, 3, 8), (2, 1, 7, 3), (1, 2, 16, 8)]


@pytest.mark.parametrize("shape", FD_SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(shape, causal):
    B, H, S, D = shape
    q, k, v, do = (rnd(shape, s) for s in (1, 2, 3, 4))
    scale = 1.0 / math.sqrt(D) if D > 1 else 0.7
    _, _, dq, dk, dv = fwd_bwd(q, k, v, do, causal, scale)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args = {"q": q, "k": k, "v": v}
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            lp = A.loss(**{**args, name: xp}, do=do, causal=causal, scale=scale)
            lm = A.loss(**{**args, name: xm}, do=do, causal=causal, scale=scale)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-6 * (1 + abs(g[idx])), (name, idx, fd, g[idx])


# ------------------------------------------------------------------ torch float64 library routines

def torch_reference(q, k, v, do, causal, scale):
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = scale * (tq @ tk.transpose(-1, -2))
    if causal:
        S = q.shape[-2]
        s = s.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.softmax(s, dim=-1) @ tv
    o.backward(torch.tensor(do, dtype=torch.float64))
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 3, 37, 16), (1, 2, 130, 64)])
def test_against_torch_autograd(shape, causal):
    q, k, v, do = (rnd(shape, s) for s in (11, 12, 13, 14))
    scale = 1.0 / math.sqrt(shape[-1])
    o, _, dq, dk, dv = fwd_bwd(q, k, v, do, causal, scale)
    to, tdq, tdk, tdv = torch_reference(q, k, v, do, causal, scale)
    for mine, ref in ((o, to), (dq, tdq), (dk, tdk), (dv, tdv)):
        assert np.allclose(mine, ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_forward_against_sdpa(causal):
    shape = (2, 2, 65, 32)
    q, k, v = (rnd(shape, s) for s in (21, 22, 23))
    scale = 0.3
    o, _ = A.forward(q, k, v, causal, scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.tensor(x) for x in (q, k, v)), is_causal=causal, scale=scale).numpy()
    assert np.allclose(o, ref, rtol=1e-11, atol=1e-12)


def test_lse_definition():
    shape = (1, 1, 9, 4)
    q, k, v = (rnd(shape, s) for s in (31, 32, 33))
    for causal in (False, True):
        _, lse = A.forward(q, k, v, causal, 0.5)
        s = 0.5 * (q[0, 0] @ k[0, 0].T)
        for i in range(9):
            keys = range(i + 1) if causal else range(9)
            want = math.log(sum(math.exp(s[i, j]) for j in keys))
            assert abs(lse[0, 0, i] - want) < 1e-13


def test_row_blocking_is_only_memory():
    shape = (1, 2, 300, 8)
    q, k, v, do = (rnd(shape, s) for s in (41, 42, 43, 44))
    for causal in (False, True):
        o1, l1 = A.forward(q, k, v, causal, 0.35, row_block=7)
        o2, l2 = A.forward(q, k, v, causal, 0.35, row_block=1000)
        assert np.allclose(o1, o2, rtol=1e-13, atol=1e-14) and np.allclose(l1, l2, rtol=1e-14)
        g1 = A.backward(q, k, v, o1, do, l1, causal, 0.35, row_block=7)
        g2 = A.backward(q, k, v, o1, do, l1, causal, 0.35, row_block=1000)
        for a, b in zip(g1, g2):
            assert np.allclose(a, b, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ brute force

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S", [1, 2, 5, 33, 64])
def test_bruteforce_jacobian(S, causal):
    D = 8
    q, k, v, do = (rnd((S, D), s) for s in (51, 52, 53, 54))
    scale = 1 / math.sqrt(D)
    o, lse = A.forward_head(q, k, v, causal, scale)
    dq, dk, dv = A.backward_head(q, k, v, o, do, lse, causal, scale)
    bo, bdq, bdk, bdv, _, _ = A.backward_bruteforce_head(q, k, v, do, causal, scale)
    for mine, ref in ((o, bo), (dq, bdq), (dk, bdk), (dv, bdv)):
        assert np.allclose(mine, ref, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ invariants

@pytest.fixture(scope="module")
def head():
    S, D = 48, 16
    return tuple(rnd((S, D), s) for s in (61, 62, 63, 64)) + (1 / math.sqrt(D),)


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(head, causal):
    q, k, v, do, c = head
    S = q.shape[0]
    o, lse = A.forward_head(q, k, v, causal, c)
    p = A.softmax_probs_head(q, k, causal, c)
    # I1 rows of P sum to one
    assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    ds = A.ds_head(q, k, v, o, do, lse, causal, c)
    # I2 masked entries of dS are exactly zero
    if causal:
        assert np.all(ds[np.triu_indices(S, 1)] == 0.0)
    # I3 rows of dS sum to zero when O = P V
    assert np.all(np.abs(ds.sum(axis=1)) <= 1e-10 * np.abs(ds).sum(axis=1) + 1e-300)
    # I4 Delta_i = sum_j P_ij dP_ij
    dp = do @ v.T
    assert np.allclose(A.delta(o, do), (p * dp).sum(axis=1), rtol=1e-12, atol=1e-13)
    dq, dk, dv = A.backward_head(q, k, v, o, do, lse, causal, c)
    # I5 columns of dK sum to zero
    assert np.allclose(dk.sum(axis=0), 0.0, atol=1e-11 * np.abs(dk).sum())
    # I6 columns of dV sum to the columns of dO
    assert np.allclose(dv.sum(axis=0), do.sum(axis=0), rtol=1e-12, atol=1e-11)
    # I7 shifting every key by one vector leaves O, dQ, dK, dV unchanged;
    #    shifting every value shifts O and leaves the gradients unchanged
    u = rnd((1, q.shape[1]), 65)
    o2, l2 = A.forward_head(q, k + u, v, causal, c)
    g2 = A.backward_head(q, k + u, v, o2, do, l2, causal, c)
    assert np.allclose(o2, o, rtol=1e-11, atol=1e-12)
    for a, b in zip(g2, (dq, dk, dv)):
        assert np.allclose(a, b, rtol=1e-10, atol=1e-11)
    o3, l3 = A.forward_head(q, k, v + u, causal, c)
    g3 = A.backward_head(q, k, v + u, o3, do, l3, causal, c)
    assert np.allclose(o3, o + u, rtol=1e-11, atol=1e-12)
    for a, b in zip(g3, (dq, dk, dv)):
        assert np.allclose(a, b, rtol=1e-10, atol=1e-11)


# ------------------------------------------------------------------ closed forms

def test_single_position():
    q, k, v, do = (rnd((1, 5), s) for s in (71, 72, 73, 74))
    for causal in (False, True):
        o, lse = A.forward_head(q, k, v, causal, 0.4)
        assert np.allclose(o, v, rtol=0, atol=1e-15)
        assert abs(lse[0] - 0.4 * float(q[0] @ k[0])) < 1e-15
        dq, dk, dv = A.backward_head(q, k, v, o, do, lse, causal, 0.4)
        assert np.allclose(dv, do, atol=1e-15)
        assert np.allclose(dq, 0, atol=1e-15) and np.allclose(dk, 0, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_uniform(causal):
    S, D = 11, 3
    q = np.zeros((S, D))
    k, v, do = (rnd((S, D), s) for s in (81, 82, 83))
    o, lse = A.forward_head(q, k, v, causal, 0.5)
    dq, dk, dv = A.backward_head(q, k, v, o, do, lse, causal, 0.5)
    for i in range(S):
        n = i + 1 if causal else S
        assert np.allclose(o[i], v[:n].mean(axis=0), atol=1e-14)
        assert abs(lse[i] - math.log(n)) < 1e-14
    for j in range(S):
        rows = range(j, S) if causal else range(S)
        want = sum(do[i] / (i + 1 if causal else S) for i in rows)
        assert np.allclose(dv[j], want, atol=1e-13)


def test_causal_edges():
    S, D = 13, 4
    q, k, v, do = (rnd((S, D), s) for s in (91, 92, 93, 94))
    c = 0.5
    o, lse = A.forward_head(q, k, v, True, c)
    dq, dk, dv = A.backward_head(q, k, v, o, do, lse, True, c)
    # query 0 sees only key 0, so its softmax has no spread: dQ_0 = 0
    assert np.allclose(dq[0], 0, atol=1e-15)
    # the last key is seen only by the last query
    ds = A.ds_head(q, k, v, o, do, lse, True, c)
    assert np.allclose(dk[S - 1], c * ds[S - 1, S - 1] * q[S - 1], atol=1e-14)
    assert np.allclose(dv[S - 1], math.exp(c * q[S - 1] @ k[S - 1] - lse[S - 1]) * do[S - 1], atol=1e-14)


def test_worked_two_by_one():
    # S = 2, D = 1, full mask, scale 1: written out by hand.
    q = np.array([[1.0], [0.0]]); k = np.array([[1.0], [-1.0]])
    v = np.array([[1.0], [2.0]]); do = np.array([[1.0], [0.0]])
    o, lse = A.forward_head(q, k, v, False, 1.0)
    sig = lambda x: 1 / (1 + math.exp(-x))
    # row 0: scores (1, -1) -> probabilities (sig(2), sig(-2)); row 1: scores (0, 0)
    assert abs(o[0, 0] - (sig(2) + 2 * sig(-2))) < 1e-15
    assert abs(o[1, 0] - 1.5) < 1e-15
    assert abs(lse[0] - math.log(math.e + 1 / math.e)) < 1e-15
    dq, dk, dv = A.backward_head(q, k, v, o, do, lse, False, 1.0)
    p0, p1 = sig(2), sig(-2)
    # only row 0 has a nonzero upstream gradient: dP_0 = (1, 2), Delta_0 = O_0
    ds0 = np.array([p0 * (1 - o[0, 0]), p1 * (2 - o[0, 0])])
    assert abs(dq[0, 0] - (ds0 @ k[:, 0])) < 1e-15 and dq[1, 0] == 0.0
    assert np.allclose(dk[:, 0], ds0 * q[0, 0], atol=1e-15)
    assert np.allclose(dv[:, 0], [p0, p1], atol=1e-15)


# ------------------------------------------------------------------ planted mistakes

def _mutant_backward(kind):
    def bwd(q, k, v, o, do, lse, causal, scale):
        S = q.shape[0]
        vis = A._visible(np.arange(S), S, causal)
        p = np.where(vis, np.exp(scale * (q @ k.T) - lse[:, None]), 0.0)
        dp = do @ v.T
        dlt = (do * o).sum(axis=1)
        if kind == "drop_delta":
            dlt = 0 * dlt
        ds = p * (dp - dlt[:, None])
        if kind == "sign":
            ds = -ds
        kk = k[::-1] if kind == "reversed_keys" else k
        dq = scale * (ds @ kk)
        dk = scale * (ds.T @ q)
        dv = (p if kind != "transposed_p" else p.T).T @ do
        if kind == "no_scale":
            dq = dq / scale
        return dq, dk, dv
    return bwd


@pytest.mark.parametrize("kind", ["drop_delta", "sign", "reversed_keys", "transposed_p", "no_scale"])
def test_pins_catch_planted_mistakes(kind):
    S, D = 6, 3
    q, k, v, do = (rnd((S, D), s) for s in (101, 102, 103, 104))
    c = 0.6
    o, lse = A.forward_head(q, k, v, False, c)
    good = A.backward_head(q, k, v, o, do, lse, False, c)
    bad = _mutant_backward(kind)(q, k, v, o, do, lse, False, c)
    # the finite-difference pin on the mutant's gradient must fail somewhere
    h = 1e-6
    failed = False
    for t, (x, g) in enumerate(zip((q, k, v), bad)):
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args = [q, k, v]
            args[t] = xp; lp = A.loss(*[a[None, None] for a in args], do[None, None], False, c)
            args[t] = xm; lm = A.loss(*[a[None, None] for a in args], do[None, None], False, c)
            if abs((lp - lm) / (2 * h) - g[idx]) > 1e-6 * (1 + abs(g[idx])):
                failed = True
    assert failed
    assert any(not np.allclose(a, b) for a, b in zip(good, bad))


@pytest.mark.parametrize("causal", [False, True])
def test_row_sampled_backward_matches_full(causal):
    S, D = 150, 8
    q, k, v, do = (rnd((S, D), s) for s in (111, 112, 113, 114))
    c = 0.4
    o, lse = A.forward_head(q, k, v, causal, c)
    dq, dk, dv = A.backward_head(q, k, v, o, do, lse, causal, c)
    qr = [0, 1, 77, 149]
    kr = [0, 5, 148, 149]
    sq, sk, sv = A.backward_rows_head(q, k, v, o, do, lse, causal, c, qr, kr)
    assert np.allclose(sq, dq[qr], rtol=1e-12, atol=1e-13)
    assert np.allclose(sk, dk[kr], rtol=1e-12, atol=1e-13)
    assert np.allclose(sv, dv[kr], rtol=1e-12, atol=1e-13)
