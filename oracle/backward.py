"""Gradients of the oracle's attention with respect to q, k and v (float64, dense masks).

Test infrastructure only: the tests and the benchmark's CPU baseline may call it; the
HIP library never does.

Sources (page titles; see the citation key in the design notes):
* RL-Kernel issue #415, Gemma-4-31B-it RFC, section 1 (training and rollout execute the
  same declared arithmetic) and section 5 work item `global_k_eq_v_projection` (the K=V
  parameter mapping's forward identity and backward gradient semantics: the one tensor
  that serves as K and V receives the gradient of both roles).

What is computed is the plain derivative of the attention of oracle.attention, written
out. For each sequence and query head h (KV head g = h // G), with s = scale q k^T over
the visible keys, P = softmax(s) row by row and o = P v:
    dP = dO v^T,   delta_i = sum_d dO_id o_id,   dS = P * (dP - delta[:, None]),
    dq = scale dS k,   dk_g += scale dS^T q,   dv_g += P^T dO   (summed over the group).
With one tensor as K and V its gradient is dk + dv. `out` is the forward output the
caller holds (delta is formed from it, as a trainer's backward forms it from the stored
forward result). Readings (listed in the design notes): lse is reported in log2 units,
log2 of sum_j exp(s_ij); rows of no sequence are NaN.
"""
from __future__ import annotations

import numpy as np

from .attention import visible_mask


def attention_backward(q, k, v, out, dout, seq_start, seq_len, num_kv_heads: int, window: int,
                       scale: float, k_eq_v: bool = False):
    """Packed varlen GQA attention backward.

    q, out, dout [T, Hq, D]; k, v [T, Hkv, D] (v is ignored when k_eq_v: k serves as both).
    Returns (dq [T, Hq, D], dk [T, Hkv, D], dv [T, Hkv, D] or None with k_eq_v (dk then
    holds the sum of both roles), lse [T, Hq] (log2 units), delta [T, Hq]), float64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = k if k_eq_v else np.asarray(v, np.float64)
    out = np.asarray(out, np.float64)
    dout = np.asarray(dout, np.float64)
    T, Hq, D = q.shape
    G = Hq // num_kv_heads
    dq = np.full((T, Hq, D), np.nan)
    dk = np.full((T, num_kv_heads, D), np.nan)
    dv = np.full((T, num_kv_heads, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    delta = np.full((T, Hq), np.nan)
    for s0, L in zip(np.asarray(seq_start).tolist(), np.asarray(seq_len).tolist()):
        if L == 0:
            continue
        rows = slice(s0, s0 + L)
        mask = visible_mask(L, L, window)
        dk[rows] = 0.0
        dv[rows] = 0.0
        for h in range(Hq):
            g = h // G
            qh, kg, vg, oh, doh = q[rows, h], k[rows, g], v[rows, g], out[rows, h], dout[rows, h]
            s = np.where(mask, scale * (qh @ kg.T), -np.inf)
            m = np.max(s, axis=1, keepdims=True)
            e = np.exp(s - m)
            l = np.sum(e, axis=1, keepdims=True)
            P = e / l
            lse[rows, h] = (m[:, 0] + np.log(l[:, 0])) / np.log(2.0)
            dP = doh @ vg.T
            dl = np.sum(doh * oh, axis=1)
            delta[rows, h] = dl
            dS = P * (dP - dl[:, None])
            dq[rows, h] = scale * (dS @ kg)
            dk[rows, g] += scale * (dS.T @ qh)
            dv[rows, g] += P.T @ doh
    if k_eq_v:
        return dq, dk + dv, None, lse, delta
    return dq, dk, dv, lse, delta
