"""Pins for the grouped-query (shared K/V heads) oracle functions (CPU only).

The grouped backward is tied to things it does not compute itself: finite
differences of sum(O * dO) with respect to the shared K and V, torch's float64
autograd with K and V repeated over each group (a library routine, so the sum
over a group comes from autograd, not from the oracle), the plain oracle when
every query head has its own K/V head, and a planted mistake (dK/dV of one
query head only instead of the group's sum) that the finite differences catch.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def draw(B, H, Hkv, S, D, seed):
    return (rnd((B, H, S, D), seed), rnd((B, Hkv, S, D), seed + 1), rnd((B, Hkv, S, D), seed + 2),
            rnd((B, H, S, D), seed + 3))


def test_group_of():
    assert [A.group_of(8, 2, h) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [A.group_of(6, 6, h) for h in range(6)] == list(range(6))
    with pytest.raises(ValueError):
        A.group_of(6, 4, 0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dims", [(1, 2, 1, 3, 2), (1, 4, 2, 5, 3), (2, 3, 1, 4, 2)])
def test_finite_differences_grouped(dims, causal):
    B, H, Hkv, S, D = dims
    q, k, v, do = draw(B, H, Hkv, S, D, 7)
    scale = 1.0 / math.sqrt(D)
    o, lse = A.forward_grouped(q, k, v, causal, scale)
    dq, dk, dv = A.backward_grouped(q, k, v, o, do, lse, causal, scale)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in np.ndindex(x.shape):
            args = {"q": q, "k": k, "v": v}
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            lp = A.loss_grouped(**{**args, name: xp}, do=do, causal=causal, scale=scale)
            lm = A.loss_grouped(**{**args, name: xm}, do=do, causal=causal, scale=scale)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-6 * (1 + abs(g[idx])), (name, idx, fd, g[idx])


@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_autograd_repeated_kv(causal):
    B, H, Hkv, S, D = 2, 6, 2, 33, 16
    q, k, v, do = draw(B, H, Hkv, S, D, 21)
    scale = 1.0 / math.sqrt(D)
    o, lse = A.forward_grouped(q, k, v, causal, scale)
    dq, dk, dv = A.backward_grouped(q, k, v, o, do, lse, causal, scale)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    G = H // Hkv
    ke, ve = tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1)
    to = torch.nn.functional.scaled_dot_product_attention(tq, ke, ve, is_causal=causal, scale=scale)
    to.backward(torch.tensor(do, dtype=torch.float64))
    assert np.allclose(o, to.detach().numpy(), rtol=1e-11, atol=1e-12)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.allclose(mine, ref.numpy(), rtol=1e-11, atol=1e-12)


def test_one_kv_head_per_query_head_is_the_plain_oracle():
    B, H, S, D = 1, 3, 20, 8
    q, k, v, do = draw(B, H, H, S, D, 31)
    o1, l1 = A.forward_grouped(q, k, v, True, 0.4)
    o2, l2 = A.forward(q, k, v, True, 0.4)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    g1 = A.backward_grouped(q, k, v, o1, do, l1, True, 0.4)
    g2 = A.backward(q, k, v, o2, do, l2, True, 0.4)
    for a, b in zip(g1, g2):
        assert np.array_equal(a, b)


def test_pins_catch_a_missing_group_sum():
    B, H, Hkv, S, D = 1, 4, 2, 4, 2
    q, k, v, do = draw(B, H, Hkv, S, D, 41)
    scale = 0.5
    o, lse = A.forward_grouped(q, k, v, False, scale)
    # planted mistake: each K/V head takes the gradient of its first query head only
    bad_dk = np.zeros_like(k)
    for h in range(0, H, H // Hkv):
        _, dkh, _ = A.backward_head(q[0, h], k[0, A.group_of(H, Hkv, h)], v[0, A.group_of(H, Hkv, h)], o[0, h],
                                    do[0, h], lse[0, h], False, scale)
        bad_dk[0, A.group_of(H, Hkv, h)] = dkh
    h_ = 1e-6
    failed = False
    for idx in np.ndindex(k.shape):
        kp = k.copy(); kp[idx] += h_
        km = k.copy(); km[idx] -= h_
        fd = (A.loss_grouped(q, kp, v, do, False, scale) - A.loss_grouped(q, km, v, do, False, scale)) / (2 * h_)
        if abs(fd - bad_dk[idx]) > 1e-6 * (1 + abs(bad_dk[idx])):
            failed = True
    assert failed
