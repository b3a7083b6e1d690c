"""Pins of the oracle's q/k prologue (RMSNorm, RoPE, one bf16 rounding). CPU only.

Independent checks: closed forms of the norm, group and relative-position properties
of the rotation, hand-worked values, and library routines from the installed HF
transformers Gemma 4 model code (its RMSNorm, its proportional RoPE frequencies and
its rotate-half application).
"""
import math

import numpy as np
import pytest
import torch

from oracle.bf16 import bf16_bits_to_f64, f64_to_bf16_bits
from oracle.prologue import qk_prologue, rms_norm, rope, rope_inv_freq, v_prologue

RNG = np.random.Generator(np.random.PCG64(7))

# (head dim, rotated dims R, frequency dim F, theta) of the two 31B layer types
SLIDING = (256, 256, 256, 1e4)
GLOBAL = (512, 128, 512, 1e6)


# ----------------------------------------------------------------------- RMSNorm
def check_rmsnorm_unit_weight_closed_form(rms_norm=rms_norm):
    """With w = 1, mean(y^2) = ms / (ms + eps)."""
    x = RNG.normal(size=(50, 256)) * RNG.uniform(0.0005, 10, size=(50, 1))
    eps = 1e-6
    y = rms_norm(x, np.ones(256), eps)
    ms = np.mean(x * x, axis=1)
    assert np.allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-13, atol=0)


def test_rmsnorm_constant_vector():
    """A constant row c gives c / sqrt(c^2 + eps) in every dim, times that dim's weight."""
    w = RNG.normal(1.0, 0.1, size=64)
    for c in (1e-4, 0.3, -2.0, 1e3):
        y = rms_norm(np.full((1, 64), c), w, 1e-6)
        assert np.allclose(y[0], w * c / math.sqrt(c * c + 1e-6), rtol=1e-14, atol=0)


def test_rmsnorm_scale_invariance_and_weight_per_dim():
    x = RNG.normal(size=(4, 128))
    w = RNG.normal(1.0, 0.1, size=128)
    y = rms_norm(x, w, 0.0)
    assert np.allclose(rms_norm(1e5 * x, w, 0.0), y, rtol=1e-13, atol=1e-15)
    w2 = w.copy()
    w2[17] *= 3.0
    y2 = rms_norm(x, w2, 0.0)
    assert np.allclose(y2[:, 17], 3.0 * y[:, 17], rtol=1e-14)
    keep = np.arange(128) != 17
    assert np.array_equal(y2[:, keep], y[:, keep])


def check_rmsnorm_matches_transformers_gemma4(rms_norm=rms_norm):
    """Library pin: transformers' Gemma4RMSNorm (float32 arithmetic) agrees to float32
    precision; its weight multiplies directly."""
    from transformers.models.gemma4.modeling_gemma4 import Gemma4RMSNorm
    for D in (256, 512):
        x = RNG.normal(size=(16, 3, D))
        w = RNG.normal(1.0, 0.1, size=D)
        mod = Gemma4RMSNorm(D, eps=1e-6)
        with torch.no_grad():
            mod.weight.copy_(torch.from_numpy(w))
            ref = mod(torch.from_numpy(x).float()).double().numpy()
        assert np.allclose(rms_norm(x, w, 1e-6), ref, rtol=2e-6, atol=2e-6)


def test_rmsnorm_unit_weight_closed_form():
    check_rmsnorm_unit_weight_closed_form()


def test_rmsnorm_matches_transformers_gemma4():
    check_rmsnorm_matches_transformers_gemma4()


# -------------------------------------------------------------------------- RoPE
def _rand_heads(T, H, D):
    return RNG.normal(size=(T, H, D))


@pytest.mark.parametrize("geom", [SLIDING, GLOBAL, (64, 64, 64, 1e4), (64, 16, 64, 1e6)])
def test_rope_position_zero_is_identity(geom):
    D, R, F, th = geom
    y = _rand_heads(5, 2, D)
    assert np.array_equal(rope(y, np.zeros(5, np.int64), R, F, th), y)


@pytest.mark.parametrize("geom", [SLIDING, GLOBAL])
def test_rope_preserves_pair_norms(geom):
    D, R, F, th = geom
    y = _rand_heads(7, 2, D)
    pos = RNG.integers(0, 262144, size=7)
    z = rope(y, pos, R, F, th)
    h = R // 2
    n0 = y[..., :h] ** 2 + y[..., h:R] ** 2
    n1 = z[..., :h] ** 2 + z[..., h:R] ** 2
    assert np.allclose(n0, n1, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("geom", [SLIDING, GLOBAL])
def test_rope_relative_position(geom):
    """<R_m q, R_n k> depends only on m - n."""
    D, R, F, th = geom
    q = _rand_heads(1, 1, D)
    k = _rand_heads(1, 1, D)
    for m, n, s in [(10, 3, 100), (1000, 999, 30000), (5, 4000, 12345)]:
        a = np.sum(rope(q, [m], R, F, th) * rope(k, [n], R, F, th))
        b = np.sum(rope(q, [m + s], R, F, th) * rope(k, [n + s], R, F, th))
        assert abs(a - b) <= 1e-10 * max(1.0, abs(a))


@pytest.mark.parametrize("geom", [SLIDING, GLOBAL])
def test_rope_composes(geom):
    D, R, F, th = geom
    y = _rand_heads(3, 2, D)
    a = np.array([3, 70, 1000])
    b = np.array([11, 5, 2048])
    assert np.allclose(rope(rope(y, a, R, F, th), b, R, F, th), rope(y, a + b, R, F, th),
                       rtol=1e-10, atol=1e-12)


def check_rope_hand_example_direction_and_speed(rope=rope, rope_inv_freq=rope_inv_freq):
    """Unit vector on dim i of pair (i, i + R/2) at position p turns to
    (cos p f_i, sin p f_i), f_i = theta^(-2 i / F)."""
    D, R, F, th = GLOBAL
    for i in (0, 1, 17, 63):
        e = np.zeros((1, 1, D))
        e[0, 0, i] = 1.0
        p = 37
        z = rope(e, [p], R, F, th)[0, 0]
        f = th ** (-2.0 * i / F)
        assert np.isclose(z[i], math.cos(p * f), atol=1e-15)
        assert np.isclose(z[i + R // 2], math.sin(p * f), atol=1e-15)
        others = np.ones(D, bool)
        others[[i, i + R // 2]] = False
        assert np.all(z[others] == 0)
    # lowest rotated frequency of the global layer: pair 63 at 1e6^(-126/512)
    assert np.isclose(rope_inv_freq(R, F, th)[-1], 1e6 ** (-126 / 512), rtol=1e-15)
    assert np.isclose(rope_inv_freq(R, F, th)[-1], 0.0333762469, rtol=1e-8)


def test_rope_hand_example_direction_and_speed():
    check_rope_hand_example_direction_and_speed()


def test_rope_global_rotates_exactly_first_quarter():
    D, R, F, th = GLOBAL
    y = _rand_heads(4, 3, D)
    z = rope(y, [1, 50, 999, 8191], R, F, th)
    assert np.array_equal(z[..., 128:], y[..., 128:])
    moved = np.any(z[..., :128] != y[..., :128], axis=(0, 1))
    assert moved.all()


class _RopeCfg:
    """Minimal config carrying what transformers' rope initialiser reads."""

    def __init__(self, head_dim, theta, partial):
        self.head_dim = head_dim
        self.rope_parameters = {"rope_type": "proportional", "rope_theta": theta,
                                "partial_rotary_factor": partial}

    def standardize_rope_params(self):
        pass


@pytest.mark.parametrize("geom,partial", [(SLIDING, 1.0), (GLOBAL, 0.25)])
def test_rope_frequencies_match_transformers(geom, partial, rope_inv_freq=rope_inv_freq):
    """Library pin: transformers' proportional RoPE initialiser (float32) gives the same
    frequencies for the first R/2 pairs and zero for the rest of the head."""
    from transformers.modeling_rope_utils import _compute_proportional_rope_parameters
    D, R, F, th = geom
    inv, _ = _compute_proportional_rope_parameters(_RopeCfg(D, th, partial), "cpu")
    inv = inv.double().numpy()
    assert inv.shape == (D // 2,)
    assert np.allclose(rope_inv_freq(R, F, th), inv[:R // 2], rtol=3e-7, atol=0)
    assert np.all(inv[R // 2:] == 0)


@pytest.mark.parametrize("geom", [SLIDING, GLOBAL])
def test_rope_full_head_layout_matches_transformers(geom, rope=rope, rope_inv_freq=rope_inv_freq):
    """Library pin: with pair offset D/2 the rotation equals transformers'
    apply_rotary_pos_emb (rotate-half over the whole head) fed the same angles."""
    from transformers.models.gemma4.modeling_gemma4 import apply_rotary_pos_emb
    D, R, F, th = geom
    T, H = 6, 3
    y = _rand_heads(T, H, D)
    pos = np.array([0, 1, 7, 1023, 8191, 32767])
    inv = np.zeros(D // 2)
    inv[:R // 2] = rope_inv_freq(R, F, th)
    freqs = pos[:, None].astype(np.float64) * inv[None, :]
    emb = np.concatenate([freqs, freqs], axis=-1)
    ref = apply_rotary_pos_emb(torch.from_numpy(y), torch.from_numpy(np.cos(emb)),
                               torch.from_numpy(np.sin(emb)), unsqueeze_dim=1).numpy()
    got = rope(y, pos, R, F, th, pair_offset=D // 2)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_rope_block_layout_is_full_head_layout_on_permuted_dims():
    """The default pairing (i, i + R/2) equals the full-head layout after moving dims
    [R/2, R) to [D/2, D/2 + R/2): the same rotation, so both are pinned by the library."""
    D, R, F, th = GLOBAL
    h = R // 2
    perm = np.arange(D)  # perm[new] = old
    perm[h:D // 2] = np.concatenate([np.arange(R, D // 2 + h)])
    perm[D // 2:D // 2 + h] = np.arange(h, R)
    perm[D // 2 + h:] = np.arange(D // 2 + h, D)
    assert sorted(perm.tolist()) == list(range(D))
    y = _rand_heads(4, 2, D)
    pos = np.array([3, 99, 4096, 30000])
    a = rope(y, pos, R, F, th)
    b = rope(y[..., perm], pos, R, F, th, pair_offset=D // 2)
    inv = np.empty(D, np.int64)
    inv[perm] = np.arange(D)
    assert np.array_equal(a, b[..., inv])


# ----------------------------------------------------------------- whole prologue
def transformers_prologue(x_bits, w_bits, positions, D, R, F, theta, eps=1e-6):
    """Reference q/k prologue from the library modules: transformers' Gemma4RMSNorm
    (float32, the weight multiplying the normalised row), then its apply_rotary_pos_emb
    (rotate-half over the whole head, i.e. pairs (i, i + D/2), the pairs past R/2 at
    frequency zero) fed float64 angles position * theta^(-2i/F). Float64 result."""
    from transformers.models.gemma4.modeling_gemma4 import Gemma4RMSNorm, apply_rotary_pos_emb
    mod = Gemma4RMSNorm(D, eps=eps)
    with torch.no_grad():
        mod.weight.copy_(torch.from_numpy(bf16_bits_to_f64(w_bits)))
        normed = mod(torch.from_numpy(bf16_bits_to_f64(x_bits)).float()).double()
    inv = np.zeros(D // 2)
    inv[:R // 2] = np.power(float(theta), -2.0 * np.arange(R // 2) / float(F))
    ang = np.asarray(positions, np.float64)[:, None] * inv[None, :]
    emb = np.concatenate([ang, ang], axis=-1)
    return apply_rotary_pos_emb(normed, torch.from_numpy(np.cos(emb)), torch.from_numpy(np.sin(emb)),
                                unsqueeze_dim=1).numpy()


def check_prologue_norm_then_rope_matches_transformers(qk_prologue=qk_prologue):
    """Library pin of the composition at nonzero positions, rotated dims included: the
    norm (with its weight) comes first, the rotation second (TensorFold PR #1186, qk-rows
    commit). The two orders differ because the weight is not constant over a pair."""
    for D, R, F, th in (SLIDING, GLOBAL):
        xb = f64_to_bf16_bits(RNG.normal(size=(6, 3, D)))
        wb = f64_to_bf16_bits(RNG.normal(1.0, 0.1, size=D))
        pos = np.array([1, 5, 77, 1000, 4097, 30001])
        vals, bits = qk_prologue(xb, wb, pos, rope_dims=R, rope_freq_dim=F, theta=th, eps=1e-6,
                                 pair_offset=D // 2)
        ref = transformers_prologue(xb, wb, pos, D, R, F, th)
        assert np.allclose(vals, ref, rtol=0, atol=2e-5)
        assert np.array_equal(bits, f64_to_bf16_bits(vals))


def test_prologue_norm_then_rope_matches_transformers():
    check_prologue_norm_then_rope_matches_transformers()


def test_prologue_single_rounding_and_position_zero():
    D, R, F, th = GLOBAL
    x = f64_to_bf16_bits(RNG.normal(size=(5, 4, D)))
    w = f64_to_bf16_bits(RNG.normal(1.0, 0.1, size=D))
    pos = np.array([0, 1, 2, 500, 8000])
    vals, bits = qk_prologue(x, w, pos, rope_dims=R, rope_freq_dim=F, theta=th, eps=1e-6)
    assert np.array_equal(bits, f64_to_bf16_bits(vals))
    normed = rms_norm(bf16_bits_to_f64(x), bf16_bits_to_f64(w), 1e-6)
    assert np.array_equal(vals[0], normed[0])
    assert np.array_equal(vals[:, :, 128:], normed[:, :, 128:])


# ------------------------------------------------------------------- value norm
def check_v_prologue_matches_transformers(v_prologue=v_prologue):
    """Library pin: transformers' Gemma4RMSNorm without a weight (its v_norm, float32)
    agrees to float32 precision, and the closed form with unit weight holds: mean(y^2) =
    ms / (ms + eps). No rotation: the result does not depend on the token's position."""
    from transformers.models.gemma4.modeling_gemma4 import Gemma4RMSNorm
    for D in (256, 512):
        xb = f64_to_bf16_bits(RNG.normal(size=(12, 3, D)) * RNG.uniform(0.01, 30.0, size=(12, 3, 1)))
        vals, bits = v_prologue(xb, eps=1e-6)
        mod = Gemma4RMSNorm(D, eps=1e-6, with_scale=False)
        ref = mod(torch.from_numpy(bf16_bits_to_f64(xb)).float()).double().numpy()
        assert np.allclose(vals, ref, rtol=2e-6, atol=2e-6)
        x = bf16_bits_to_f64(xb)
        ms = np.mean(x * x, axis=-1)
        assert np.allclose(np.mean(vals * vals, axis=-1), ms / (ms + 1e-6), rtol=1e-12, atol=0)
        assert np.array_equal(bits, f64_to_bf16_bits(vals))


def test_v_prologue_matches_transformers():
    check_v_prologue_matches_transformers()
