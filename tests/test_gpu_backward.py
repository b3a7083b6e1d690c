"""GPU attention backward (g4attn_prefill_backward) against the float64 oracle's gradients,
and bit-identity of every gradient across batch composition (alone, packed, padded).

Tolerance, from the declared arithmetic: every term summed into a gradient element carries
at most one bf16 rounding (of P or of dS, 2^-9 relative) on top of fp32 products and sums,
and the element is rounded to bf16 once; so |gpu - oracle| <= 2^-8 (sum of |terms|) +
2^-8 |oracle| + 1e-6, with the sum of |terms| formed in float64 from the same inputs
(|dS| |k| for dq, |dS| |q| for dk, P |dO| for dv). lse (log2 units) and delta are fp32 sums:
within 1e-4 (|lse| <= ~20 here) and D 2^-24 <= 4e-5 of sum |dO out| + 1e-6."""
import dataclasses

import numpy as np
import pytest
import torch

import global_gqa_attention_amd as g
import workloads as W
from gpu_helpers import DEV, bits_equal, covered_rows, f64, prefill, to_dev
from oracle.attention import visible_mask
from oracle.backward import attention_backward

pytestmark = pytest.mark.gpu


def term_sums(q, k, v, dout, starts, lens, Hkv, window, scale, k_eq_v):
    """float64 sums of |terms| of each gradient element (the scale of its rounding error)."""
    T, Hq, D = q.shape
    G = Hq // Hkv
    v = k if k_eq_v else v
    mq = np.zeros_like(q)
    mk = np.zeros((T, Hkv, D))
    mv = np.zeros((T, Hkv, D))
    for s0, L in zip(starts, lens):
        rows = slice(s0, s0 + L)
        mask = visible_mask(L, L, window)
        for h in range(Hq):
            gg = h // G
            s = np.where(mask, scale * (q[rows, h] @ k[rows, gg].T), -np.inf)
            P = np.exp(s - s.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            dP = dout[rows, h] @ v[rows, gg].T
            dS = np.abs(P * (dP - np.sum(P * dP, axis=1, keepdims=True))) + P * np.abs(dP) * 2.0 ** -8
            mq[rows, h] = scale * (dS @ np.abs(k[rows, gg]))
            mk[rows, gg] += scale * (dS.T @ np.abs(q[rows, h]))
            mv[rows, gg] += P.T @ np.abs(dout[rows, h])
    if k_eq_v:
        mk = mk + mv
    return mq, mk, mv


def run_backward(spec, q, k, v, out, dout, seq_start, seq_len, max_len):
    layer = g.make_layer(spec)
    sent = lambda t: torch.full(t.shape, 0x7FC0, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    dq, dk = sent(q), sent(k)
    dv = None if spec.k_eq_v else sent(k)
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
    delta = torch.full_like(lse, float("nan"))
    g.g4attn_prefill_backward(layer, q, k, None if spec.k_eq_v else v, out, dout, dq, dk, dv, lse, delta, seq_start,
                              seq_len, max_len)
    return dq, dk, dv, lse, delta


def check_against_oracle(spec, case, seed, what):
    q, k, v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
    ss, sl = to_dev(case.seq_start), to_dev(case.seq_len)
    out, _ = prefill(spec, q, k, v, ss, sl)
    gen = W.make_generator(seed + 1000, DEV)
    dout = W.bf16_normal(gen, q.shape, device=DEV)
    dq, dk, dv, lse, delta = run_backward(spec, q, k, v, out, dout, ss, sl, case.max_seq_len)
    torch.cuda.synchronize()
    rows = covered_rows(case)
    st, ln = case.seq_start.numpy(), case.seq_len.numpy()
    args = (f64(q), f64(k), None if spec.k_eq_v else f64(v), f64(out), f64(dout), st, ln, spec.num_kv_heads,
            spec.window, spec.softmax_scale)
    rq, rk, rv, rlse, rdelta = attention_backward(*args, k_eq_v=spec.k_eq_v)
    mq, mk, mv = term_sums(f64(q), f64(k), None if spec.k_eq_v else f64(v), f64(dout), st.tolist(), ln.tolist(),
                           spec.num_kv_heads, spec.window, spec.softmax_scale, spec.k_eq_v)
    pairs = [("dq", dq, rq, mq), ("dk", dk, rk, mk)]
    if not spec.k_eq_v:
        pairs.append(("dv", dv, rv, mv))
    for name, got, ref, mag in pairs:
        gv = f64(got)[rows]
        err = np.abs(gv - ref[rows])
        bound = 2.0 ** -8 * (mag[rows] + np.abs(ref[rows])) + 1e-6
        assert np.all(np.isfinite(gv)), f"{what} {name}: non-finite"
        worst = float((err / bound).max())
        assert worst <= 1.0, f"{what} {name}: error {worst:.2f} x the bound (max |err| {err.max():.3e})"
    gl = lse.cpu().numpy().astype(np.float64)[rows]
    gd = delta.cpu().numpy().astype(np.float64)[rows]
    assert np.max(np.abs(gl - rlse[rows])) <= 1e-4, f"{what} lse"
    dmag = np.sum(np.abs(f64(dout) * f64(out)), axis=-1)[rows]
    assert np.all(np.abs(gd - rdelta[rows]) <= 4e-5 * dmag + 1e-6), f"{what} delta"
    return out, dout, dq, dk, dv, lse, delta


CASES = [
    ("tiny-sliding", W.TINY_SLIDING, [1, 17, 64, 130], [2, 0, 5, 3, 1], 71),
    ("tiny-global", W.TINY_GLOBAL, [5, 200, 63, 65], [1, 1, 0, 2, 0], 72),
    ("tiny-global-g8", W.TINY_GLOBAL_G8, [100, 33, 257], [0, 3, 1, 2], 73),
    ("31b-sliding", W.SLIDING_31B, [1100, 300], [0, 7, 0], 74),
    ("31b-global", W.GLOBAL_31B, [700, 129], [3, 0, 2], 75),
    ("31b-global-v", W.GLOBAL_31B_V, [600, 65], [0, 1, 0], 76),
]


@pytest.mark.parametrize("name,spec,lens,gaps,seed", CASES, ids=[c[0] for c in CASES])
def test_backward_against_oracle(name, spec, lens, gaps, seed):
    case = W.prefill_case(spec, lens, seed, gaps=gaps)
    layer = g.make_layer(spec)
    q, k = to_dev(case.q), to_dev(case.k)
    g.g4attn_qk_prologue(layer, q, q, k, k, to_dev(case.wq), to_dev(case.wk), to_dev(case.positions))
    case = dataclasses.replace(case, q=q.cpu(), k=k.cpu())
    check_against_oracle(spec, case, seed, name)


@pytest.mark.parametrize("spec", [W.TINY_GLOBAL_G8, W.SLIDING_31B, W.GLOBAL_31B], ids=["tiny-g8", "sliding", "global"])
def test_backward_alone_packed_padded_bitwise(spec):
    """Each sequence's gradients (dq, and dk, dv of its own rows), lse and delta are the same
    bits alone, in the pack and in a pack with N(0,1) padding rows between sequences."""
    lens = [300, 33, 700, 129]
    case = W.prefill_case(spec, lens, 77, gaps=[0, 0, 0, 0, 0])
    q, k, v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
    ss, sl = to_dev(case.seq_start), to_dev(case.seq_len)
    out, _ = prefill(spec, q, k, v, ss, sl)
    dout = W.bf16_normal(W.make_generator(78, DEV), q.shape, device=DEV)
    ref = run_backward(spec, q, k, v, out, dout, ss, sl, max(lens))
    starts = case.seq_start.tolist()
    # padded: gaps of N(0,1) rows between the sequences
    gaps = [5, 17, 1, 40, 3]
    gen = W.make_generator(79, DEV)
    parts = {"q": [], "k": [], "v": [], "out": [], "dout": []}
    pstarts, t = [], 0
    for b, (s0, L) in enumerate(zip(starts, lens)):
        for name, src in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
            if src is None:
                continue
            parts[name] += [W.bf16_normal(gen, (gaps[b],) + tuple(src.shape[1:]), device=DEV), src[s0:s0 + L]]
        pstarts.append(t + gaps[b])
        t += gaps[b] + L
    P = {n: (torch.cat(x) if x else None) for n, x in parts.items()}
    pad = run_backward(spec, P["q"], P["k"], P["v"], P["out"], P["dout"],
                       torch.tensor(pstarts, dtype=torch.int32, device=DEV), sl, max(lens))
    for b, (s0, L) in enumerate(zip(starts, lens)):
        one = torch.tensor([0], dtype=torch.int32, device=DEV)
        ln = torch.tensor([L], dtype=torch.int32, device=DEV)
        sl_ = lambda x: None if x is None else x[s0:s0 + L].contiguous()
        alone = run_backward(spec, sl_(q), sl_(k), sl_(v), sl_(out), sl_(dout), one, ln, L)
        p0 = pstarts[b]
        for i, name in enumerate(["dq", "dk", "dv", "lse", "delta"]):
            if ref[i] is None:
                continue
            a_, r_, p_ = alone[i], ref[i][s0:s0 + L], pad[i][p0:p0 + L]
            if a_.dtype == torch.float32:
                assert torch.equal(a_.view(torch.int32), r_.view(torch.int32)), f"seq {b} {name}: alone != packed"
                assert torch.equal(p_.view(torch.int32), r_.view(torch.int32)), f"seq {b} {name}: padded != packed"
            else:
                assert bits_equal(a_, r_), f"seq {b} {name}: alone != packed"
                assert bits_equal(p_, r_), f"seq {b} {name}: padded != packed"
    torch.cuda.synchronize()
