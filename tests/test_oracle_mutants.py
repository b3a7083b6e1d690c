"""Planted mistakes in copies of the oracle must each fail at least one pin (CPU only).

This shows the pins are strong enough to catch the plausible slips named for the
oracle: a dropped term, a wrong sign or index, an operand in the wrong place.
The real oracle is never modified: attention mutants wrap it or swap one of its
helpers for the duration of one check (pytest's monkeypatch restores it).
"""
import numpy as np
import pytest

import oracle.attention as A
from oracle.prologue import rms_norm as real_rms_norm
from oracle.prologue import rope as real_rope
from oracle.prologue import rope_inv_freq as real_inv_freq

import test_oracle_attention as TA
import test_oracle_prologue as TP


def _fails_some(checks) -> bool:
    for chk in checks:
        try:
            chk()
        except AssertionError:
            return True
    return False


# ------------------------------------------------------------------ attention mutants
def _mask_window_inclusive(nq, nk, window, query_pos0=0, key_pos0=0):
    i = query_pos0 + np.arange(nq)[:, None]
    j = key_pos0 + np.arange(nk)[None, :]
    m = j <= i
    if window > 0:
        m &= (i - j) <= window
    return m


def _mask_no_self(nq, nk, window, query_pos0=0, key_pos0=0):
    i = query_pos0 + np.arange(nq)[:, None]
    j = key_pos0 + np.arange(nk)[None, :]
    m = (j < i) | ((i == 0) & (j == 0))
    if window > 0:
        m &= (i - j) < window
    return m


def _mask_not_causal(nq, nk, window, query_pos0=0, key_pos0=0):
    i = query_pos0 + np.arange(nq)[:, None]
    j = key_pos0 + np.arange(nk)[None, :]
    m = np.ones((nq, nk), bool)
    if window > 0:
        m &= np.abs(i - j) < window
    return m


def _weights_normalised_over_all(q_rows, k_rows, mask, scale):
    s = scale * (q_rows @ k_rows.T)
    m = np.max(np.where(mask, s, -np.inf), axis=1, keepdims=True)
    p = np.exp(s - m)
    return np.where(mask, p, 0.0) / np.sum(p, axis=1, keepdims=True)


def _attn_gqa_modulo(q, k, v, st, ln, Hkv, W, scale):
    Hq = q.shape[1]
    idx = np.arange(Hq) % Hkv
    return A.attention(q, k[:, idx], v[:, idx], st, ln, Hq, W, scale)


def _attn_no_scale(q, k, v, st, ln, Hkv, W, scale):
    return A.attention(q, k, v, st, ln, Hkv, W, 1.0)


def _attn_v_is_k(q, k, v, st, ln, Hkv, W, scale):
    return A.attention(q, k, k, st, ln, Hkv, W, scale)


HELPER_MUTANTS = {
    "window_inclusive": ("visible_mask", _mask_window_inclusive),
    "self_not_visible": ("visible_mask", _mask_no_self),
    "not_causal": ("visible_mask", _mask_not_causal),
    "normaliser_over_hidden_keys": ("attention_weights", _weights_normalised_over_all),
}
WRAPPER_MUTANTS = {"gqa_modulo": _attn_gqa_modulo, "scale_dropped": _attn_no_scale, "v_is_k": _attn_v_is_k}


@pytest.mark.parametrize("name", sorted(HELPER_MUTANTS))
def test_attention_helper_mutant_is_caught(name, monkeypatch):
    attr, fn = HELPER_MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    assert _fails_some([lambda c=c: c(A.attention) for c in TA.ATTENTION_CHECKS])


@pytest.mark.parametrize("name", sorted(WRAPPER_MUTANTS))
def test_attention_wrapper_mutant_is_caught(name):
    fn = WRAPPER_MUTANTS[name]
    assert _fails_some([lambda c=c: c(fn) for c in TA.ATTENTION_CHECKS])


# ------------------------------------------------------------ per-row last-key mutants
def _lk_mask_exclusive(nq, nk, window, query_pos0=0, key_pos0=0, last_key=None):
    """An image row misses the image's last row (j < last instead of j <= last)."""
    i = query_pos0 + np.arange(nq)[:, None]
    j = key_pos0 + np.arange(nk)[None, :]
    m = j <= i
    if last_key is not None:
        m |= j < np.asarray(last_key)[:, None]
    if window > 0:
        m &= (i - j) < window
    return m


def _lk_mask_window_ignored(nq, nk, window, query_pos0=0, key_pos0=0, last_key=None):
    """Image rows escape the window."""
    i = query_pos0 + np.arange(nq)[:, None]
    j = key_pos0 + np.arange(nk)[None, :]
    causal = j <= i
    if window > 0:
        causal &= (i - j) < window
    if last_key is None:
        return causal
    img = np.asarray(last_key)[:, None] > i
    return np.where(img, j <= np.asarray(last_key)[:, None], causal)


def _lk_mask_dropped(nq, nk, window, query_pos0=0, key_pos0=0, last_key=None):
    """The last keys are ignored (every row stays causal)."""
    return A.__dict__["_real_visible_mask"](nq, nk, window, query_pos0, key_pos0)


LAST_KEY_MUTANTS = {"last_key_exclusive": _lk_mask_exclusive, "window_ignored_for_images": _lk_mask_window_ignored,
                    "last_key_dropped": _lk_mask_dropped}


@pytest.mark.parametrize("name", sorted(LAST_KEY_MUTANTS))
def test_last_key_mutant_is_caught(name, monkeypatch):
    monkeypatch.setitem(A.__dict__, "_real_visible_mask", A.visible_mask)
    monkeypatch.setattr(A, "visible_mask", LAST_KEY_MUTANTS[name])
    assert _fails_some([lambda c=c: c(TA._attention_with_last_key) for c in TA.LAST_KEY_CHECKS])


# ------------------------------------------------------------------- prologue mutants
def _rms_one_plus_w(x, w, eps):
    return real_rms_norm(x, 1.0 + np.asarray(w), eps)


def _rms_eps_outside(x, w, eps):
    x = np.asarray(x, np.float64)
    return np.asarray(w) * x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps)


def _inv_freq_half_exponent(R, F, theta):
    i = np.arange(R // 2, dtype=np.float64)
    return np.power(float(theta), -i / float(F))


def _rope_backwards(y, positions, R, F, theta, pair_offset=None):
    return real_rope(y, -np.asarray(positions), R, F, theta, pair_offset)


def _rope_interleaved(y, positions, R, F, theta, pair_offset=None):
    y = np.asarray(y, np.float64)
    ang = np.asarray(positions, np.float64)[:, None] * real_inv_freq(R, F, theta)[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    out = y.copy()
    a, b = y[..., 0:R:2], y[..., 1:R:2]
    out[..., 0:R:2] = a * c - b * s
    out[..., 1:R:2] = b * c + a * s
    return out


def test_rmsnorm_mutants_are_caught():
    for fn in (_rms_one_plus_w, _rms_eps_outside):
        assert _fails_some([lambda: TP.check_rmsnorm_unit_weight_closed_form(fn),
                            lambda: TP.check_rmsnorm_matches_transformers_gemma4(fn)])


def test_rope_mutants_are_caught():
    geoms = [(TP.SLIDING, 1.0), (TP.GLOBAL, 0.25)]
    for rope_fn, freq_fn in ((real_rope, _inv_freq_half_exponent), (_rope_backwards, real_inv_freq),
                             (_rope_interleaved, real_inv_freq)):
        checks = [lambda: TP.check_rope_hand_example_direction_and_speed(rope_fn, freq_fn)]
        for g, part in geoms:
            checks.append(lambda g=g, part=part: TP.test_rope_frequencies_match_transformers(g, part, freq_fn))
            checks.append(lambda g=g: TP.test_rope_full_head_layout_matches_transformers(g, rope_fn, freq_fn))
        assert _fails_some(checks)


# ------------------------------------------------------------- composition mutants
def _prologue_rope_before_norm(x_bits, w_bits, positions, *, rope_dims, rope_freq_dim, theta, eps,
                               pair_offset=None):
    """RoPE applied before the RMSNorm."""
    from oracle.bf16 import bf16_bits_to_f64, f64_to_bf16_bits
    x = bf16_bits_to_f64(x_bits)
    y = real_rms_norm(real_rope(x, positions, rope_dims, rope_freq_dim, theta, pair_offset),
                      bf16_bits_to_f64(w_bits), eps)
    return y, f64_to_bf16_bits(y)


def _layer_forward_k_with_q_weights(q, k, v, wq, wk, *args, **kw):
    """k normed with the q weights."""
    return A.layer_forward(q, k, v, wq, wq, *args, **kw)


def _layer_forward_q_with_k_weights(q, k, v, wq, wk, *args, **kw):
    """q normed with the k weights."""
    return A.layer_forward(q, k, v, wk, wk, *args, **kw)


def test_prologue_order_mutant_is_caught():
    assert _fails_some([lambda: TP.check_prologue_norm_then_rope_matches_transformers(_prologue_rope_before_norm)])


@pytest.mark.parametrize("fn", [_layer_forward_k_with_q_weights, _layer_forward_q_with_k_weights],
                         ids=["k_with_wq", "q_with_wk"])
def test_layer_forward_weight_mutant_is_caught(fn):
    assert _fails_some([lambda: TA.check_layer_forward_routes_weights(fn)])


# --------------------------------------------------------------- value-norm mutants
def _v_prologue_weighted(x_bits, *, eps):
    """v normed with a weight of 1.1 (a stray weight)."""
    from oracle.bf16 import bf16_bits_to_f64, f64_to_bf16_bits
    x = bf16_bits_to_f64(x_bits)
    y = real_rms_norm(x, np.full(x.shape[-1], 1.1), eps)
    return y, f64_to_bf16_bits(y)


def _v_prologue_eps_outside(x_bits, *, eps):
    from oracle.bf16 import bf16_bits_to_f64, f64_to_bf16_bits
    x = bf16_bits_to_f64(x_bits)
    y = x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps)
    return y, f64_to_bf16_bits(y)


@pytest.mark.parametrize("fn", [_v_prologue_weighted, _v_prologue_eps_outside], ids=["weighted", "eps_outside"])
def test_v_prologue_mutant_is_caught(fn):
    assert _fails_some([lambda: TP.check_v_prologue_matches_transformers(fn)])


def _layer_forward_v_rotated(q, k, v, wq, wk, positions, *args, v_norm=False, **kw):
    """V taken as the rotated, weighted k (the K=V reading) instead of the unit-normed v."""
    if v_norm:
        return A.layer_forward(q, k, v, wq, wk, positions, *args, k_eq_v=True,
                               **{x: y for x, y in kw.items() if x != "k_eq_v"})
    return A.layer_forward(q, k, v, wq, wk, positions, *args, **kw)


def _layer_forward_v_raw(q, k, v, wq, wk, positions, *args, v_norm=False, **kw):
    """The v norm dropped (raw v)."""
    return A.layer_forward(q, k, v, wq, wk, positions, *args, **kw)


@pytest.mark.parametrize("fn", [_layer_forward_v_rotated, _layer_forward_v_raw], ids=["v_rotated", "v_raw"])
def test_layer_forward_v_norm_mutant_is_caught(fn):
    assert _fails_some([lambda: TA.check_layer_forward_v_norm(fn)])


# ------------------------------------------------------------------- backward mutants
import oracle.backward as BW  # noqa: E402
import test_oracle_backward as TB  # noqa: E402


def _bwd_no_scale_in_dq(*a, **kw):
    dq, dk, dv, lse, delta = BW.attention_backward(*a, **kw)
    return dq / a[9], dk, dv, lse, delta


def _bwd_no_delta(q, k, v, out, dout, st, ln, Hkv, W, scale, k_eq_v=False):
    """delta dropped: dS = P * dP."""
    return BW.attention_backward(q, k, v, np.zeros_like(np.asarray(out, np.float64)), dout, st, ln, Hkv, W, scale,
                                 k_eq_v=k_eq_v)


def _bwd_first_head_only(q, k, v, out, dout, st, ln, Hkv, W, scale, k_eq_v=False):
    """dk and dv from the group's first query head only."""
    G = q.shape[1] // Hkv
    res = list(BW.attention_backward(q, k, v, out, dout, st, ln, Hkv, W, scale, k_eq_v=k_eq_v))
    mask = (np.arange(q.shape[1]) % G == 0)[None, :, None]
    sub = BW.attention_backward(q * mask, k, v, out * mask, dout * mask, st, ln, Hkv, W, scale, k_eq_v=k_eq_v)
    res[1], res[2] = sub[1], sub[2]
    return tuple(res)


def _bwd_keqv_drops_v_role(q, k, v, out, dout, st, ln, Hkv, W, scale, k_eq_v=False):
    dq, dk, dv, lse, delta = BW.attention_backward(q, k, k if k_eq_v else v, out, dout, st, ln, Hkv, W, scale)
    return dq, dk, (None if k_eq_v else dv), lse, delta


@pytest.mark.parametrize("fn", [_bwd_no_scale_in_dq, _bwd_no_delta, _bwd_first_head_only, _bwd_keqv_drops_v_role],
                         ids=["dq_scale_dropped", "delta_dropped", "group_sum_dropped", "keqv_v_role_dropped"])
def test_backward_mutant_is_caught(fn):
    assert _fails_some([lambda c=c: c(fn) for c in TB.BACKWARD_CHECKS])


# ------------------------------------------------------------------- split-form mutants
import oracle.split as S  # noqa: E402
import test_oracle_split as TS  # noqa: E402

_real_merge = S.merge_partials
_real_partials = S.chunk_partials


def _merge_unweighted(parts):
    """The chunk partials summed without their weights exp(m_c - M)."""
    return sum(p[5] for p in parts) / sum(p[4] for p in parts)


def _merge_weight_sign(parts):
    """exp(M - m_c) in place of exp(m_c - M)."""
    M = max(p[3] for p in parts)
    return (sum(np.exp(M - p[3]) * p[5] for p in parts) / sum(np.exp(M - p[3]) * p[4] for p in parts))


def _merge_den_unweighted(parts):
    """The weighted O over an unweighted sum of l."""
    M = max(p[3] for p in parts)
    return sum(np.exp(p[3] - M) * p[5] for p in parts) / sum(p[4] for p in parts)


def _partials_shifted_boundary(q_row, k_rows, v_rows, key_pos0, visible, scale, chunk):
    """Chunks one position late (c C + 1 .. c C + C)."""
    return _real_partials(q_row, k_rows, v_rows, key_pos0 - 1, visible, scale, chunk)


SPLIT_MUTANTS = {"merge_unweighted": ("merge_partials", _merge_unweighted),
                 "merge_weight_sign": ("merge_partials", _merge_weight_sign),
                 "merge_den_unweighted": ("merge_partials", _merge_den_unweighted),
                 "chunk_boundary_shifted": ("chunk_partials", _partials_shifted_boundary)}


@pytest.mark.parametrize("name", sorted(SPLIT_MUTANTS))
def test_split_mutant_is_caught(name, monkeypatch):
    attr, fn = SPLIT_MUTANTS[name]
    monkeypatch.setattr(S, attr, fn)
    checks = [TS.test_chunks_cover_the_visible_keys_in_order, TS.test_closed_form_two_chunks,
              TS.test_split_equals_unsplit_softmax, TS.test_split_with_peaked_scores]
    assert _fails_some(checks)
