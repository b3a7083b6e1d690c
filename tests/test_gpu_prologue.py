"""GPU prologue (RMSNorm + RoPE + bf16 rounding) against the oracle.

The oracle rounds its float64 result once; the GPU computes in fp32 (angles in fp64)
and rounds once, so every value must be within one bf16 ulp and almost all equal."""
import numpy as np
import pytest
import torch

import global_gqa_attention_amd as g
import workloads as W
from gpu_helpers import DEV, to_dev
from oracle.prologue import qk_prologue

pytestmark = pytest.mark.gpu


def ordered(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def check_bits(gpu_bits, ref_bits, what):
    d = np.abs(ordered(gpu_bits) - ordered(ref_bits))
    frac_equal = float(np.mean(d == 0))
    assert d.max() <= 1, f"{what}: {int(d.max())} ulp"
    assert frac_equal >= 0.999, f"{what}: only {frac_equal:.5f} bit-equal"
    return frac_equal


def _pairing_spec(spec, pairing):
    import dataclasses

    class S:
        pass

    s = S()
    for f in dataclasses.fields(spec):
        setattr(s, f.name, getattr(spec, f.name))
    s.rope_pairing = pairing
    return s


@pytest.mark.parametrize("name", ["tiny-sliding", "tiny-global", "gemma4-31b-sliding", "gemma4-31b-global"])
@pytest.mark.parametrize("pairing", [0, 1])
def test_prologue_matches_oracle(name, pairing):
    spec = W.SPECS[name]
    T = 300
    case = W.prefill_case(spec, [T], seed=21)
    rng = np.random.Generator(np.random.PCG64(5))
    pos = np.concatenate([[0, 1, 2, 1023, 1024, 8191, 32767, 262143],
                          rng.integers(0, 262144, size=T - 8)]).astype(np.int32)
    sp = _pairing_spec(spec, pairing)
    layer = g.make_layer(sp)
    q, k = to_dev(case.q), to_dev(case.k)
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    g.g4attn_qk_prologue(layer, q, qo, k, ko, to_dev(case.wq), to_dev(case.wk), torch.from_numpy(pos).to(DEV))
    torch.cuda.synchronize()
    P = spec.head_dim // 2 if pairing else None
    kw = dict(rope_dims=spec.rope_dims, rope_freq_dim=spec.rope_freq_dim, theta=spec.rope_theta,
              eps=spec.rms_eps, pair_offset=P)
    _, qref = qk_prologue(W.bits(case.q), W.bits(case.wq), pos, **kw)
    _, kref = qk_prologue(W.bits(case.k), W.bits(case.wk), pos, **kw)
    check_bits(W.bits(qo.cpu()), qref, f"{name} q")
    check_bits(W.bits(ko.cpu()), kref, f"{name} k")
    # inputs untouched when out of place
    assert torch.equal(q.cpu().view(torch.int16), case.q.view(torch.int16))


def test_prologue_in_place_equals_out_of_place():
    spec = W.SLIDING_31B
    case = W.prefill_case(spec, [77], seed=3)
    layer = g.make_layer(spec)
    q, k = to_dev(case.q), to_dev(case.k)
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    pos = to_dev(case.positions)
    g.g4attn_qk_prologue(layer, q, qo, k, ko, to_dev(case.wq), to_dev(case.wk), pos)
    g.g4attn_qk_prologue(layer, q, q, k, k, to_dev(case.wq), to_dev(case.wk), pos)
    torch.cuda.synchronize()
    assert torch.equal(q.view(torch.int16), qo.view(torch.int16))
    assert torch.equal(k.view(torch.int16), ko.view(torch.int16))


def test_prologue_scatter_into_ring():
    """k rows go to kv_dst_row (negative = skipped), v rows are copied raw with the same
    map, q stays in token order; untouched cache rows keep their contents."""
    spec = W.TINY_SLIDING
    T, C = 40, 16
    case = W.prefill_case(spec, [T], seed=8)
    layer = g.make_layer(spec)
    pos = np.arange(T, dtype=np.int32)
    dst = np.where(pos >= T - C, 100 + pos % C, -1).astype(np.int64)  # last C positions into a ring at row 100
    kc = torch.full((100 + C + 5, spec.num_kv_heads, spec.head_dim), 77, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    vc = kc.clone()
    q, k, v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
    qo = torch.empty_like(q)
    kref_full = torch.empty_like(k)
    g.g4attn_qk_prologue(layer, q, qo, k, kc, to_dev(case.wq), to_dev(case.wk), torch.from_numpy(pos).to(DEV),
                         v_in=v, v_out=vc, kv_dst_row=torch.from_numpy(dst).to(DEV))
    g.g4attn_qk_prologue(layer, None, None, k, kref_full, None, to_dev(case.wk), torch.from_numpy(pos).to(DEV))
    torch.cuda.synchronize()
    for t in range(T):
        if dst[t] >= 0:
            assert torch.equal(kc[dst[t]].view(torch.int16), kref_full[t].view(torch.int16))
            assert torch.equal(vc[dst[t]].view(torch.int16), v[t].view(torch.int16))
    untouched = [r for r in range(kc.shape[0]) if r not in set(dst[dst >= 0].tolist())]
    assert torch.all(kc[untouched].view(torch.int16) == 77) and torch.all(vc[untouched].view(torch.int16) == 77)
