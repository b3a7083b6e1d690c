"""GPU decode against the oracle, and bit-equality of every decode row with the prefill
row of the same position (sliding layers through a ring cache, global layers through
a linear K=V cache). Cache slots that hold no visible key are filled with NaN: the
kernel must never read them."""
import dataclasses

import numpy as np
import pytest
import torch

import global_gqa_attention_amd as g
import workloads as W
from gpu_helpers import DEV, assert_close, assert_close_peaked, bits_equal, f64, prefill, to_dev
from oracle.attention import decode_rows

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


def build_cache(spec, k, v, starts, lens, slots):
    """Per-sequence regions of `slots` rows; position p of sequence b at row b*slots + p % slots.
    Only the positions the decode row can see are written; everything else is NaN."""
    B = len(lens)
    shape = (B * slots, spec.num_kv_heads, spec.head_dim)
    kc = torch.full(shape, NAN_BF16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    vc = None if spec.k_eq_v else kc.clone()
    for b, (s0, L) in enumerate(zip(starts, lens)):
        lo = max(0, L - spec.window) if spec.window > 0 else 0
        p = torch.arange(lo, L, device=DEV)
        rows = b * slots + p % slots
        kc[rows] = k[s0 + p]
        if vc is not None:
            vc[rows] = v[s0 + p]
    row0 = torch.arange(B, dtype=torch.int64, device=DEV) * slots
    return kc, vc, row0


CASES = [
    ("tiny-sliding", W.TINY_SLIDING, [1, 15, 16, 17, 64, 100, 129], 16, 31),
    ("tiny-sliding-wide-ring", W.TINY_SLIDING, [1, 15, 16, 17, 64, 100, 129], 40, 32),
    ("tiny-global", W.TINY_GLOBAL, [1, 2, 63, 64, 65, 200], None, 33),
    ("tiny-global-g8", W.TINY_GLOBAL_G8, [1, 64, 65, 150], None, 34),
    ("31b-sliding", W.SLIDING_31B, [1, 1023, 1024, 1025, 2000, 3001], 1024, 35),
    ("31b-global", W.GLOBAL_31B, [1, 63, 64, 65, 1500, 3000], None, 36),
    # queries scaled by 24: running maxima jump past the lazy-offset threshold (rescales)
    ("31b-sliding-peaked", W.SLIDING_31B, [1025, 2000], 1024, 37),
    ("31b-global-peaked", W.GLOBAL_31B, [700, 1300], None, 38),
    # windowed rings in the other work-group shapes: one tensor as K and V at head dim 256
    # (one-wave work-groups), and head dim 512 (four-wave work-groups)
    ("windowed-keqv-d256", dataclasses.replace(W.SLIDING_31B, name="windowed-keqv-d256", k_eq_v=True),
     [1, 1025, 2000], 1024, 39),
    ("windowed-keqv-d512", dataclasses.replace(W.SLIDING_31B, name="windowed-keqv-d512", head_dim=512, k_eq_v=True,
                                               rope_dims=512, rope_freq_dim=512, softmax_scale=512 ** -0.5),
     [1, 1025, 2000], 1024, 40),
]


@pytest.mark.parametrize("name,spec,lens,slots,seed", CASES, ids=[c[0] for c in CASES])
def test_decode_equals_prefill_row_and_oracle(name, spec, lens, slots, seed):
    case = W.prefill_case(spec, lens, seed)
    if name.endswith("peaked"):
        case = dataclasses.replace(case, q=(case.q.float() * 24.0).to(torch.bfloat16))
    q, k, v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
    starts = case.seq_start.tolist()
    out_pf, _ = prefill(spec, q, k, v, to_dev(case.seq_start), to_dev(case.seq_len))
    if slots is None:
        slots = max(lens) + 5
    kc, vc, row0 = build_cache(spec, k, v, starts, lens, slots)
    last = torch.tensor([s + L - 1 for s, L in zip(starts, lens)], device=DEV)
    qd = q[last].contiguous()
    out_dec = torch.empty_like(qd)
    ctx = torch.tensor(lens, dtype=torch.int32, device=DEV)
    # serve the longest sequences first; the schedule changes no result
    sched = torch.tensor(np.argsort(-np.array(lens), kind="stable"), dtype=torch.int32, device=DEV)
    prov = g.g4attn_decode(g.make_layer(spec), qd, kc, vc, row0, ctx, slots, out_dec, max(lens), schedule=sched,
                           provenance=True)
    torch.cuda.synchronize()
    for b in range(len(lens)):
        assert bits_equal(out_dec[b], out_pf[last[b]]), f"{name}: decode row {b} (L={lens[b]}) != prefill row"
    vv = case.k if spec.k_eq_v else case.v
    keys = [f64(case.k[s:s + L]) for s, L in zip(starts, lens)]
    vals = [f64(vv[s:s + L]) for s, L in zip(starts, lens)]
    ref = decode_rows(f64(case.q[last.cpu()]), keys, vals, [0] * len(lens), lens, spec.window, spec.softmax_scale)
    if name.endswith("peaked"):
        assert_close_peaked(f64(out_dec), ref, max(float(np.abs(x).max()) for x in vals), name)
    else:
        assert_close(f64(out_dec), ref, name)
    assert prov["split_kv"] == 0


def test_decode_after_prologue_scatter():
    """The whole decode step: the new token's q and k go through the prologue, k lands in
    the ring slot, then decode; equal to prefill of the full sequence after its prologue."""
    spec = W.SLIDING_31B
    L, C = 1300, 1024
    case = W.prefill_case(spec, [L], 41)
    layer = g.make_layer(spec)
    q, k, v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
    wq, wk, pos = to_dev(case.wq), to_dev(case.wk), to_dev(case.positions)
    # reference: prologue over the whole prompt, then prefill
    qp, kp = q.clone(), k.clone()
    g.g4attn_qk_prologue(layer, qp, qp, kp, kp, wq, wk, pos)
    out_pf, _ = prefill(spec, qp, kp, v, to_dev(case.seq_start), to_dev(case.seq_len))
    # cache holds positions [L-C, L-2] already processed; the new token (L-1) comes raw
    kc = torch.full((C, spec.num_kv_heads, spec.head_dim), NAN_BF16, dtype=torch.int16,
                    device=DEV).view(torch.bfloat16)
    vc = kc.clone()
    old = torch.arange(L - C, L - 1, device=DEV)
    kc[old % C] = kp[old]
    vc[old % C] = v[old]
    qn = torch.empty((1, spec.num_q_heads, spec.head_dim), dtype=torch.bfloat16, device=DEV)
    dst = torch.tensor([(L - 1) % C], dtype=torch.int64, device=DEV)
    g.g4attn_qk_prologue(layer, q[L - 1:L], qn, k[L - 1:L], kc, wq, wk, pos[L - 1:L], v_in=v[L - 1:L], v_out=vc,
                         kv_dst_row=dst)
    out = torch.empty_like(qn)
    g.g4attn_decode(layer, qn, kc, vc, torch.zeros(1, dtype=torch.int64, device=DEV),
                    torch.tensor([L], dtype=torch.int32, device=DEV), C, out, L)
    torch.cuda.synchronize()
    assert bits_equal(out[0], out_pf[L - 1])


LONG = [("31b-sliding", W.SLIDING_31B, [4097, 16385, 32768], 51),
        ("31b-global", W.GLOBAL_31B, [8193, 32768], 52)]


@pytest.mark.parametrize("name,spec,lens,seed", LONG, ids=[c[0] for c in LONG])
def test_decode_equals_prefill_at_long_contexts(name, spec, lens, seed):
    """The decode workload's context lengths (up to 32768): the prompt goes through the
    prologue and the prefill; the cache is filled by the prologue's own scatter from the
    same raw prompt (sliding: a ring of `window` slots, global: a linear K=V cache; slots
    outside the visible keys hold NaN); the new token's query goes through the prologue at
    its position. The decode row equals the prefill row bit for bit, and matches the
    oracle (its own prologue of the raw rows, then the token's attention)."""
    from oracle.bf16 import bf16_bits_to_f64
    from oracle.prologue import qk_prologue

    layer = g.make_layer(spec)
    Hq, Hk, D = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    kw = dict(rope_dims=spec.rope_dims, rope_freq_dim=spec.rope_freq_dim, theta=spec.rope_theta, eps=spec.rms_eps)
    for i, L in enumerate(lens):
        print(f"{name}: L={L}", flush=True)
        case = W.prefill_case(spec, [L], seed + i, device=DEV)
        q, k = torch.empty_like(case.q), torch.empty_like(case.k)
        g.g4attn_qk_prologue(layer, case.q, q, case.k, k, case.wq, case.wk, case.positions)
        out_pf, _ = prefill(spec, q, k, case.v, case.seq_start, case.seq_len)
        del q
        slots = spec.window if spec.window > 0 else L + 32
        lo = max(0, L - spec.window) if spec.window > 0 else 0
        kc = torch.full((slots, Hk, D), NAN_BF16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        vc = None if spec.k_eq_v else kc.clone()
        dst = torch.arange(lo, L, dtype=torch.int64, device=DEV) % slots
        g.g4attn_qk_prologue(layer, None, None, case.k[lo:L], kc, None, case.wk, case.positions[lo:L],
                             v_in=None if spec.k_eq_v else case.v[lo:L], v_out=vc, kv_dst_row=dst)
        qd = torch.empty((1, Hq, D), dtype=torch.bfloat16, device=DEV)
        g.g4attn_qk_prologue(layer, case.q[L - 1:L], qd, None, None, case.wq, None, case.positions[L - 1:L])
        out = torch.empty_like(qd)
        g.g4attn_decode(layer, qd, kc, vc, torch.zeros(1, dtype=torch.int64, device=DEV),
                        torch.tensor([L], dtype=torch.int32, device=DEV), slots, out, L)
        torch.cuda.synchronize()
        assert bits_equal(out[0], out_pf[L - 1]), f"{name}: decode at L={L} != prefill row"
        # the oracle, from the raw rows
        _, q1 = qk_prologue(W.bits(case.q[L - 1:L].cpu()), W.bits(case.wq.cpu()), np.array([L - 1]), **kw)
        _, k1 = qk_prologue(W.bits(case.k[lo:L].cpu()), W.bits(case.wk.cpu()), np.arange(lo, L), **kw)
        keys = bf16_bits_to_f64(k1)
        vals = keys if spec.k_eq_v else f64(case.v[lo:L])
        ref = decode_rows(bf16_bits_to_f64(q1), [keys], [vals], [lo], [L], spec.window, spec.softmax_scale)
        assert_close(f64(out), ref, f"{name} L={L}")
        del case, k, kc, vc, out_pf
        torch.cuda.empty_cache()


NEG0 = [("tiny-sliding", W.TINY_SLIDING, [1, 15, 40, 100, 129], 16, 61),
        ("tiny-global", W.TINY_GLOBAL, [1, 2, 40, 65, 200], None, 62),
        ("31b-global", W.GLOBAL_31B, [1, 40, 1500], None, 63)]


@pytest.mark.parametrize("name,spec,lens,slots,seed", NEG0, ids=[c[0] for c in NEG0])
def test_decode_equals_prefill_with_negative_zero_dims(name, spec, lens, slots, seed):
    """Value dims that are -0 for every key (a pruned projection column times negative
    activations gives such a dim). Every product in those output dims is a signed zero;
    the decode meets zero-filled rows (past the context, absent blocks of the last round)
    where prefill meets real rows, and the rows must still agree bit for bit."""
    case = W.prefill_case(spec, lens, seed)
    dims = [0, 3, spec.head_dim - 1]
    neg0 = torch.tensor(-0.0, dtype=torch.bfloat16)
    k, v = case.k.clone(), (case.k if spec.k_eq_v else case.v).clone()
    v[:, :, dims] = neg0
    if spec.k_eq_v:
        k = v
    q, kd = to_dev(case.q), to_dev(k)
    vd = None if spec.k_eq_v else to_dev(v)
    starts = case.seq_start.tolist()
    out_pf, _ = prefill(spec, q, kd, vd if vd is not None else kd, to_dev(case.seq_start), to_dev(case.seq_len))
    if slots is None:
        slots = max(lens) + 5
    kc, vc, row0 = build_cache(spec, kd, vd if vd is not None else kd, starts, lens, slots)
    last = torch.tensor([s + L - 1 for s, L in zip(starts, lens)], device=DEV)
    qd = q[last].contiguous()
    out_dec = torch.empty_like(qd)
    ctx = torch.tensor(lens, dtype=torch.int32, device=DEV)
    g.g4attn_decode(g.make_layer(spec), qd, kc, vc, row0, ctx, slots, out_dec, max(lens))
    torch.cuda.synchronize()
    for b in range(len(lens)):
        assert bits_equal(out_dec[b], out_pf[last[b]]), f"{name}: decode row {b} (L={lens[b]}) != prefill row"
