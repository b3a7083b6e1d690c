"""The prefill with the q prologue inside (g4attn_prefill_qp) against the two calls it
replaces: g4attn_qk_prologue on q and k, then g4attn_prefill. The outputs must be equal bit
for bit (the work-groups norm and rotate the raw rows with the prologue's arithmetic in its
order), and, through that, within the oracle's tolerance of the float64 layer."""
import dataclasses

import pytest
import torch

import global_gqa_attention_amd as g
import workloads as W
from gpu_helpers import DEV, bits_equal, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    ("31b-global-varlen", W.GLOBAL_31B, [1, 15, 16, 17, 300, 1500], 0, 1.0, 51),
    ("31b-global-far-positions", W.GLOBAL_31B, [700, 64], 100_000, 1.0, 52),
    # q_norm_w scaled by 24 (a scale of the raw rows would be normed away): peaked scores, so
    # most work-groups take the second pass from the final offsets, with the transformed
    # fragments still in registers
    ("31b-global-peaked", W.GLOBAL_31B, [900, 130], 0, 24.0, 53),
    # the softmax scale transformers' Gemma 4 uses (1.0): the second pass again
    ("31b-global-scale1", dataclasses.replace(W.GLOBAL_31B, name="scale1", softmax_scale=1.0), [900, 130], 0, 1.0, 57),
    # rotation partners half a head apart instead of half the rotated dims
    ("31b-global-half-head-pairs", dataclasses.replace(W.GLOBAL_31B, name="half-head-pairs"), [513, 40], 0, 1.0, 54),
    ("31b-global-8192", W.GLOBAL_31B, [8192], 0, 1.0, 55),
]


@pytest.mark.parametrize("name,spec,lens,pos_shift,w_scale,seed", CASES, ids=[c[0] for c in CASES])
def test_prefill_qp_equals_prologue_then_prefill(name, spec, lens, pos_shift, w_scale, seed):
    case = W.prefill_case(spec, lens, seed)
    layer = g.make_layer(spec)
    if name.endswith("half-head-pairs"):
        layer.rope_pairing = g.G4ATTN_ROPE_PAIRS_HALF_HEAD
    q = to_dev(case.q)
    k = to_dev(case.k)
    wq, wk = to_dev((case.wq.float() * w_scale).to(torch.bfloat16)), to_dev(case.wk)
    pos = to_dev(case.positions) + pos_shift
    start, slen = to_dev(case.seq_start), to_dev(case.seq_len)
    # the two calls
    qp, kp = torch.empty_like(q), torch.empty_like(k)
    g.g4attn_qk_prologue(layer, q, qp, k, kp, wq, wk, pos)
    ref = torch.empty_like(q)
    g.g4attn_prefill(layer, qp, kp, None, ref, start, slen, max(lens))
    # the fused call (k through the prologue alone)
    k2 = torch.empty_like(k)
    g.g4attn_qk_prologue(layer, None, None, k, k2, None, wk, pos)
    out = torch.full_like(q, float("nan"))
    prov = g.g4attn_prefill_qp(layer, q, wq, pos, k2, None, out, start, slen, max(lens), provenance=True)
    torch.cuda.synchronize()
    assert bits_equal(k2, kp)
    rows = torch.cat([torch.arange(s, s + L) for s, L in zip(case.seq_start.tolist(), lens)]).to(DEV)
    assert bits_equal(out[rows], ref[rows]), f"{name}: fused q prologue differs from prologue + prefill"
    assert prov["kernel_id"].endswith("qprologue")


def test_prefill_qp_rejects_other_layers():
    spec = W.SLIDING_31B
    case = W.prefill_case(spec, [64], 56)
    layer = g.make_layer(spec)
    q, k, v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
    out = torch.empty_like(q)
    with pytest.raises(g.G4AttnError) as e:
        g.g4attn_prefill_qp(layer, q, to_dev(case.wq), to_dev(case.positions), k, v, out, to_dev(case.seq_start),
                            to_dev(case.seq_len), 64)
    assert e.value.status == g.G4ATTN_ERR_UNSUPPORTED
