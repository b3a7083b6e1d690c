"""GPU prologue (RMSNorm + RoPE + bf16 rounding) against the oracle.

The oracle rounds its exact float64 result once; the GPU computes in fp32 (angles in
fp64) and rounds once. Bound: |gpu - exact| <= 1 bf16 ulp of the exact value plus the
fp32 error of the rotation, which scales with the pair's magnitude, not the result's:
a few fp32 roundings of |y_i| + |y_partner| (2^-21 of it covers them). Where the
rotation does not cancel that second term is far below an ulp, so almost every value
is bit-equal to the oracle's rounding (>= 99.9 % required)."""
import numpy as np
import pytest
import torch

import global_gqa_attention_amd as g
import workloads as W
from gpu_helpers import DEV, to_dev
from oracle.bf16 import bf16_bits_to_f64
from oracle.prologue import qk_prologue, rms_norm

pytestmark = pytest.mark.gpu


def ordered(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def check_bits(gpu_bits, exact, scale, what):
    """gpu_bits: GPU bf16 bits; exact: oracle float64 before rounding; scale: per-value
    magnitude of the inputs of its last operation (|y_i| + |y_partner|, or |y_i|)."""
    from oracle.bf16 import f64_to_bf16_bits
    ref_bits = f64_to_bf16_bits(exact)
    got = bf16_bits_to_f64(gpu_bits)
    a = np.abs(exact)
    ulp = np.where(a > 0, np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - 7), 2.0 ** -133)
    err = np.abs(got - exact)
    bound = ulp + 2.0 ** -21 * scale
    worst = float(np.max(err / bound))
    frac_equal = float(np.mean(gpu_bits == ref_bits))
    assert worst <= 1.0, f"{what}: error {worst:.2f} x the bound"
    assert frac_equal >= 0.999, f"{what}: only {frac_equal:.5f} bit-equal"
    return frac_equal


def magnitude(x_bits, w_bits, eps, R, P):
    """|y_d| + |y_partner(d)| of the normalised values (before rotation) per element."""
    y = np.abs(rms_norm(bf16_bits_to_f64(x_bits), bf16_bits_to_f64(w_bits), eps))
    m = y.copy()
    h = R // 2
    if h:
        m[..., :h] += y[..., P:P + h]
        m[..., P:P + h] += y[..., :h]
    return m


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
    qex, _ = qk_prologue(W.bits(case.q), W.bits(case.wq), pos, **kw)
    kex, _ = qk_prologue(W.bits(case.k), W.bits(case.wk), pos, **kw)
    Pd = P if P is not None else spec.rope_dims // 2
    check_bits(W.bits(qo.cpu()), qex, magnitude(W.bits(case.q), W.bits(case.wq), spec.rms_eps, spec.rope_dims, Pd),
               f"{name} q")
    check_bits(W.bits(ko.cpu()), kex, magnitude(W.bits(case.k), W.bits(case.wk), spec.rms_eps, spec.rope_dims, Pd),
               f"{name} k")
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


@pytest.mark.parametrize("name", ["tiny-sliding", "gemma4-31b-sliding", "gemma4-31b-global"])
def test_prologue_value_norm_matches_oracle(name):
    """With the layer's v_norm set, the v rows are stored as their unit RMS norm (no weight,
    no rotation), rounded once: against the oracle's v_prologue at the prologue's bound
    (one bf16 ulp plus 2^-21 of |y|), at varied row magnitudes. The global layer takes its
    one raw projection as both k and v (separate K and V, as the real model forms them);
    k is unchanged by the value norm."""
    import dataclasses

    from oracle.prologue import v_prologue

    spec = dataclasses.replace(W.SPECS[name], k_eq_v=False, v_norm=True)
    T = 200
    case = W.prefill_case(dataclasses.replace(spec, k_eq_v=False), [T], seed=23)
    gen = W.make_generator(24)
    scale = torch.exp(torch.randn((T, spec.num_kv_heads, 1), generator=gen) * 2.0)
    raw_v = (case.v.float() * scale).to(torch.bfloat16)
    layer = g.make_layer(spec)
    pos = torch.from_numpy(np.arange(T, dtype=np.int32) * 37).to(DEV)
    ko, vo = torch.empty_like(to_dev(case.k)), torch.empty_like(to_dev(raw_v))
    g.g4attn_qk_prologue(layer, None, None, to_dev(case.k), ko, None, to_dev(case.wk), pos, v_in=to_dev(raw_v),
                         v_out=vo)
    # the global layer's form: the same projection as k and as v
    ko2, vo2 = torch.empty_like(ko), torch.empty_like(ko)
    g.g4attn_qk_prologue(layer, None, None, to_dev(case.k), ko2, None, to_dev(case.wk), pos, v_in=to_dev(case.k),
                         v_out=vo2)
    torch.cuda.synchronize()
    for src, got in ((raw_v, vo), (case.k, vo2)):
        exact, _ = v_prologue(W.bits(src), eps=spec.rms_eps)
        check_bits(W.bits(got.cpu()), exact, np.abs(exact), f"{name} v")
    assert torch.equal(ko.view(torch.int16), ko2.view(torch.int16))
    plain = torch.empty_like(ko)
    g.g4attn_qk_prologue(g.make_layer(dataclasses.replace(spec, v_norm=False)), None, None, to_dev(case.k), plain,
                         None, to_dev(case.wk), pos)
    torch.cuda.synchronize()
    assert torch.equal(ko.view(torch.int16), plain.view(torch.int16))
