"""Pins of the oracle's attention backward (CPU only): torch's float64 autograd through a
dense masked softmax attention (library routine), central finite differences on a tiny
case, K=V as one tensor in both roles, the log-sum-exp against its definition, and the
gradient identities (the rows of dS sum to zero, so with q = 0 the key gradient vanishes).

Each check takes the backward callable so the mutant tests can run it on copies of the
oracle with planted mistakes."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import backward as B

RNG = np.random.Generator(np.random.PCG64(31))


def _pack(lens, Hq, Hkv, D, gaps=None):
    gaps = gaps or [0] * (len(lens) + 1)
    starts, t = [], 0
    for L, g in zip(lens, gaps[:-1]):
        t += g
        starts.append(t)
        t += L
    T = t + gaps[-1]
    return (RNG.normal(size=(T, Hq, D)), RNG.normal(size=(T, Hkv, D)), RNG.normal(size=(T, Hkv, D)),
            RNG.normal(size=(T, Hq, D)), np.array(starts), np.array(lens))


def _torch_attention(q, k, v, starts, lens, Hkv, W, scale):
    """Dense masked attention in torch (float64), differentiable."""
    T, Hq, D = q.shape
    G = Hq // Hkv
    out = torch.zeros_like(q)
    for s0, L in zip(starts.tolist(), lens.tolist()):
        i = torch.arange(L)[:, None]
        j = torch.arange(L)[None, :]
        mask = (j <= i) & ((i - j < W) if W > 0 else torch.ones(L, L, dtype=torch.bool))
        qs = q[s0:s0 + L].permute(1, 0, 2)
        ks = k[s0:s0 + L].permute(1, 0, 2).repeat_interleave(G, dim=0)
        vs = v[s0:s0 + L].permute(1, 0, 2).repeat_interleave(G, dim=0)
        s = scale * qs @ ks.transpose(1, 2)
        s = s.masked_fill(~mask, float("-inf"))
        o = torch.softmax(s, dim=-1) @ vs
        out = out.index_put((torch.arange(s0, s0 + L),), o.permute(1, 0, 2))
    return out


def check_against_autograd(bwd):
    """Library pin: torch float64 autograd of the same dense attention, GQA packs with
    padding, sliding and full causal."""
    for (Hq, Hkv, D, W) in [(4, 2, 16, 5), (8, 1, 8, 0), (4, 4, 8, 3)]:
        q, k, v, do, st, ln = _pack([9, 1, 14], Hq, Hkv, D, gaps=[2, 0, 3, 1])
        tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
        o = _torch_attention(tq, tk, tv, st, ln, Hkv, W, 0.3)
        (o * torch.from_numpy(do)).sum().backward()
        out = A.attention(q, k, v, st, ln, Hkv, W, 0.3)
        dq, dk, dv, lse, delta = bwd(q, k, v, out, do, st, ln, Hkv, W, 0.3)
        rows = np.concatenate([np.arange(s, s + L) for s, L in zip(st, ln)])
        for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            assert np.allclose(got[rows], ref.numpy()[rows], rtol=0, atol=1e-11)


def check_k_eq_v_against_autograd(bwd):
    """One tensor as K and V: its gradient is that of both roles (autograd on a shared leaf)."""
    q, k, _, do, st, ln = _pack([11, 6], 8, 2, 8)
    tq, tk = torch.from_numpy(q).requires_grad_(True), torch.from_numpy(k).requires_grad_(True)
    o = _torch_attention(tq, tk, tk, st, ln, 2, 0, 0.4)
    (o * torch.from_numpy(do)).sum().backward()
    out = A.attention(q, k, k, st, ln, 2, 0, 0.4)
    dq, dkv, dv, _, _ = bwd(q, k, None, out, do, st, ln, 2, 0, 0.4, k_eq_v=True)
    assert dv is None
    assert np.allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
    assert np.allclose(dkv, tk.grad.numpy(), rtol=0, atol=1e-11)


def check_finite_differences(bwd):
    """Central differences of sum(dO * out) on a tiny case, a few coordinates of each input."""
    q, k, v, do, st, ln = _pack([7], 2, 1, 4)
    W, sc = 4, 0.7
    f = lambda q_, k_, v_: float(np.sum(do * A.attention(q_, k_, v_, st, ln, 1, W, sc)))
    out = A.attention(q, k, v, st, ln, 1, W, sc)
    dq, dk, dv, _, _ = bwd(q, k, v, out, do, st, ln, 1, W, sc)
    h = 1e-6
    for grad, which in ((dq, 0), (dk, 1), (dv, 2)):
        for idx in [(0, 0, 0), (3, 0, 2), (6, 0, 1)] if which else [(0, 0, 0), (3, 1, 2), (6, 1, 1)]:
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            fp = f(*args)
            args[which][idx] -= 2 * h
            fm = f(*args)
            assert abs((fp - fm) / (2 * h) - grad[idx]) <= 1e-7 * max(1.0, abs(grad[idx]))


def check_lse_and_identities(bwd):
    """lse = log2 sum_j exp(s_ij) over the visible keys; with q = 0 every score is 0, P is
    uniform and dS's rows sum to zero, so dk vanishes; delta = dO . out."""
    q, k, v, do, st, ln = _pack([13], 4, 2, 8)
    out = A.attention(q, k, v, st, ln, 2, 6, 0.25)
    _, _, _, lse, delta = bwd(q, k, v, out, do, st, ln, 2, 6, 0.25)
    for i in range(13):
        lo = max(0, i - 5)
        for h in range(4):
            s = 0.25 * (k[lo:i + 1, h // 2] @ q[i, h])
            assert math.isclose(lse[i, h], np.log2(np.sum(np.exp(s))), rel_tol=0, abs_tol=1e-12)
            assert math.isclose(delta[i, h], float(do[i, h] @ out[i, h]), rel_tol=0, abs_tol=1e-12)
    q0 = np.zeros_like(q)
    out0 = A.attention(q0, k, v, st, ln, 2, 6, 0.25)
    _, dk0, _, _, _ = bwd(q0, k, v, out0, do, st, ln, 2, 6, 0.25)
    assert np.allclose(dk0, 0.0, atol=1e-13)


BACKWARD_CHECKS = [check_against_autograd, check_k_eq_v_against_autograd, check_finite_differences,
                   check_lse_and_identities]


@pytest.mark.parametrize("check", BACKWARD_CHECKS, ids=lambda c: c.__name__)
def test_backward_pin(check):
    check(B.attention_backward)
