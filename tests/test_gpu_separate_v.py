"""The global layer at head dim 512 with separate K and V, as the real model forms its
values (TensorFold PR #1186, tf_qk_rows_once commit: v normed by a unit RMS norm at head
dim 512; RL-Kernel issue #415, section 5, global_k_eq_v_projection): one raw projection
goes through the prologue as k (normed with the k weights, rotated) and as v (unit RMS
norm, not rotated), and the attention reads the two tensors separately. Prefill against
the oracle (end to end, through its own prologue and value norm), each sequence alone =
packed bit for bit, decode = the prefill row bit for bit against caches filled by the
prologue's scatter, chunked prefill = whole-sequence prefill bit for bit, and peaked
scores through the second pass."""
import dataclasses

import numpy as np
import pytest
import torch

import global_gqa_attention_amd as g
import workloads as W
from gpu_helpers import DEV, assert_close, assert_close_peaked, bits_equal, covered_rows, f64, prefill, to_dev
from oracle.attention import attention, decode_rows, layer_forward

pytestmark = pytest.mark.gpu

SPEC = W.GLOBAL_31B_V
NAN_BF16 = 0x7FC0


def real_case(lens, seed, gaps=None):
    """A packed case whose raw v rows are its raw k rows (one projection for K and V)."""
    case = W.prefill_case(SPEC, lens, seed, gaps=gaps)
    return dataclasses.replace(case, v=case.k.clone())


def run_prologue(case, spec=SPEC):
    layer = g.make_layer(spec)
    q, k, v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
    qo, ko, vo = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    g.g4attn_qk_prologue(layer, q, qo, k, ko, to_dev(case.wq), to_dev(case.wk), to_dev(case.positions), v_in=v,
                         v_out=vo)
    return qo, ko, vo


def oracle_out(case, spec=SPEC):
    _, _, ref = layer_forward(W.bits(case.q), W.bits(case.k), W.bits(case.v), W.bits(case.wq), W.bits(case.wk),
                              case.positions.numpy(), case.seq_start.numpy(), case.seq_len.numpy(),
                              num_kv_heads=spec.num_kv_heads, window=spec.window, k_eq_v=False,
                              rope_dims=spec.rope_dims, rope_freq_dim=spec.rope_freq_dim, theta=spec.rope_theta,
                              eps=spec.rms_eps, scale=spec.softmax_scale, v_norm=spec.v_norm)
    return ref


def test_prefill_against_oracle_and_alone_equals_packed():
    lens = [1, 31, 32, 33, 300, 700]
    case = real_case(lens, 61, gaps=[3, 0, 5, 1, 2, 7, 4])
    q, k, v = run_prologue(case)
    out, prov = prefill(SPEC, q, k, v, to_dev(case.seq_start), to_dev(case.seq_len))
    torch.cuda.synchronize()
    assert "d512.kv" in prov["kernel_id"]
    rows = covered_rows(case)
    assert_close(f64(out)[rows], oracle_out(case)[rows], SPEC.name)
    pad = np.setdiff1d(np.arange(case.num_tokens), rows)
    assert torch.all(out[torch.from_numpy(pad).to(DEV)].view(torch.int16) == 0x7FC0)  # padding rows untouched
    for b, (s0, L) in enumerate(zip(case.seq_start.tolist(), lens)):
        one = torch.tensor([0], dtype=torch.int32, device=DEV)
        ln = torch.tensor([L], dtype=torch.int32, device=DEV)
        alone, _ = prefill(SPEC, q[s0:s0 + L].contiguous(), k[s0:s0 + L].contiguous(), v[s0:s0 + L].contiguous(),
                           one, ln)
        assert bits_equal(alone, out[s0:s0 + L]), f"seq {b} (L={L}): alone != packed"


def test_raw_separate_v_at_head_dim_512():
    """The same kernels with a raw (unnormed) separate v of its own: against the oracle."""
    spec = dataclasses.replace(SPEC, v_norm=False)
    case = W.prefill_case(spec, [900, 129], 62)
    layer = g.make_layer(spec)
    q, k = to_dev(case.q), to_dev(case.k)
    g.g4attn_qk_prologue(layer, q, q, k, k, to_dev(case.wq), to_dev(case.wk), to_dev(case.positions))
    out, _ = prefill(spec, q, k, to_dev(case.v), to_dev(case.seq_start), to_dev(case.seq_len))
    torch.cuda.synchronize()
    ref = attention(f64(q), f64(k), f64(case.v), case.seq_start.numpy(), case.seq_len.numpy(), spec.num_kv_heads, 0,
                    spec.softmax_scale)
    assert_close(f64(out), ref, "raw v")


@pytest.mark.parametrize("lens,seed", [([1, 2, 33, 64, 65, 700], 63), ([2048, 8193], 64)], ids=["short", "long"])
def test_decode_equals_prefill_row(lens, seed):
    """Linear caches (slots past the keys hold NaN) filled by the prologue's scatter from
    the raw projection (k and v rows), the new tokens' queries through the prologue at
    their positions; every decode row equals its prefill row bit for bit and matches the
    oracle."""
    case = real_case(lens, seed)
    layer = g.make_layer(SPEC)
    q, k, v = run_prologue(case)
    out_pf, _ = prefill(SPEC, q, k, v, to_dev(case.seq_start), to_dev(case.seq_len))
    B, slots = len(lens), max(lens) + 40
    Hq, Hk, D = SPEC.num_q_heads, SPEC.num_kv_heads, SPEC.head_dim
    kc = torch.full((B * slots, Hk, D), NAN_BF16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    vc = kc.clone()
    starts = case.seq_start.tolist()
    rows = torch.cat([torch.arange(s0, s0 + L, device=DEV) for s0, L in zip(starts, lens)])
    dst = torch.cat([b * slots + torch.arange(L, device=DEV) for b, L in enumerate(lens)]).to(torch.int64)
    raw = to_dev(case.k)[rows].contiguous()
    g.g4attn_qk_prologue(layer, None, None, raw, kc, None, to_dev(case.wk), to_dev(case.positions)[rows].contiguous(),
                         v_in=raw, v_out=vc, kv_dst_row=dst)
    last = torch.tensor([s0 + L - 1 for s0, L in zip(starts, lens)], device=DEV)
    qd = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    g.g4attn_qk_prologue(layer, to_dev(case.q)[last].contiguous(), qd, None, None, to_dev(case.wq), None,
                         to_dev(case.positions)[last].contiguous())
    od = torch.empty_like(qd)
    prov = g.g4attn_decode(layer, qd, kc, vc, torch.arange(B, dtype=torch.int64, device=DEV) * slots,
                           torch.tensor(lens, dtype=torch.int32, device=DEV), slots, od, max(lens), provenance=True)
    torch.cuda.synchronize()
    assert "d512.kv" in prov["kernel_id"]
    for b, L in enumerate(lens):
        assert bits_equal(od[b], out_pf[last[b]]), f"decode row {b} (L={L}) != prefill row"
    keys = [f64(k[s0:s0 + L]) for s0, L in zip(starts, lens)]
    vals = [f64(v[s0:s0 + L]) for s0, L in zip(starts, lens)]
    ref = decode_rows(f64(qd), keys, vals, [0] * B, lens, 0, SPEC.softmax_scale)
    assert_close(f64(od), ref, "decode")


def test_chunked_prefill_equals_whole():
    """Chunks of a sequence (ragged, two sequences per call) through the prologue's scatter
    into linear K and V caches, then g4attn_prefill_cached: the chunk rows equal the
    whole-sequence prefill bit for bit."""
    lens = [1300, 700]
    case = real_case(lens, 65)
    layer = g.make_layer(SPEC)
    q, k, v = run_prologue(case)
    out_w, _ = prefill(SPEC, q, k, v, to_dev(case.seq_start), to_dev(case.seq_len))
    B, slots = len(lens), 1344
    Hq, Hk, D = SPEC.num_q_heads, SPEC.num_kv_heads, SPEC.head_dim
    kc = torch.full((B * slots, Hk, D), NAN_BF16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    vc = kc.clone()
    row0 = torch.arange(B, dtype=torch.int64, device=DEV) * slots
    starts = case.seq_start.tolist()
    out = torch.full(q.shape, NAN_BF16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    P = [0, 0]
    for c in [512, 129, 300, 512, 512]:
        grp = [b for b in range(B) if P[b] < lens[b]]
        if not grp:
            break
        cl = [min(c, lens[b] - P[b]) for b in grp]
        rows = torch.cat([torch.arange(starts[b] + P[b], starts[b] + P[b] + n, device=DEV) for b, n in zip(grp, cl)])
        pos = torch.cat([torch.arange(P[b], P[b] + n, dtype=torch.int32, device=DEV) for b, n in zip(grp, cl)])
        dst = torch.cat([row0[b] + torch.arange(P[b], P[b] + n, device=DEV) for b, n in zip(grp, cl)])
        raw = to_dev(case.k)[rows].contiguous()
        qc = torch.empty((len(rows), Hq, D), dtype=torch.bfloat16, device=DEV)
        g.g4attn_qk_prologue(layer, to_dev(case.q)[rows].contiguous(), qc, raw, kc, to_dev(case.wq), to_dev(case.wk),
                             pos, v_in=raw, v_out=vc, kv_dst_row=dst.to(torch.int64))
        oc = torch.empty_like(qc)
        g.g4attn_prefill_cached(layer, qc, kc, vc, oc, torch.tensor(np.concatenate([[0], np.cumsum(cl)[:-1]]),
                                                                    dtype=torch.int32, device=DEV),
                                torch.tensor([P[b] for b in grp], dtype=torch.int32, device=DEV),
                                torch.tensor(cl, dtype=torch.int32, device=DEV), row0[grp].contiguous(), slots, max(cl),
                                max(P[b] + n for b, n in zip(grp, cl)))
        out[rows] = oc
        for b, n in zip(grp, cl):
            P[b] += n
    torch.cuda.synchronize()
    assert P == lens
    assert bits_equal(out, out_w), "chunked rows differ from the whole-sequence prefill"


def test_peaked_scores_second_pass():
    """Queries x 24 after the prologue: the second pass from the final offsets; decode row
    = prefill row bit for bit, and the output matches the oracle within the peaked bound."""
    lens = [900, 1500]
    case = real_case(lens, 66)
    layer = g.make_layer(SPEC)
    q, k, v = run_prologue(case)
    q = (q.float() * 24.0).to(torch.bfloat16)
    out, _ = prefill(SPEC, q, k, v, to_dev(case.seq_start), to_dev(case.seq_len))
    starts = case.seq_start.tolist()
    for s0, L in zip(starts, lens):
        od = torch.empty((1, SPEC.num_q_heads, SPEC.head_dim), dtype=torch.bfloat16, device=DEV)
        g.g4attn_decode(layer, q[s0 + L - 1:s0 + L].contiguous(), k[s0:s0 + L].contiguous(), v[s0:s0 + L].contiguous(),
                        torch.zeros(1, dtype=torch.int64, device=DEV), torch.tensor([L], dtype=torch.int32, device=DEV),
                        L, od, L)
        torch.cuda.synchronize()
        assert bits_equal(od[0], out[s0 + L - 1])
    ref = attention(f64(q), f64(k), f64(v), case.seq_start.numpy(), case.seq_len.numpy(), SPEC.num_kv_heads, 0,
                    SPEC.softmax_scale)
    assert_close_peaked(f64(out), ref, float(np.abs(f64(v)).max()), "peaked")
