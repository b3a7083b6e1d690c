"""Pins of the oracle's attention (CPU only).

Independent checks: pure-Python brute force on tiny packs, torch's float64
scaled_dot_product_attention with an explicit boolean mask (library routine), and
closed-form properties (rows of weights sum to 1, convex combinations, the first row
equals v_0, q = 0 gives the mean of the visible values, the visible set of each row,
GQA head mapping, sequence independence, sliding = full when the sequence fits in
the window, decode row = last prefill row).

Each check takes the attention callable so the mutant test can run the same checks
against copies of the oracle with planted mistakes.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle.bf16 import bf16_bits_to_f64, f64_to_bf16_bits

RNG = np.random.Generator(np.random.PCG64(11))


def _pack(lens, gaps, Hq, Hkv, D, rng):
    starts, t = [], 0
    for L, g in zip(lens, gaps[:-1]):
        t += g
        starts.append(t)
        t += L
    T = t + gaps[-1]
    q = rng.normal(size=(T, Hq, D))
    k = rng.normal(size=(T, Hkv, D))
    v = rng.normal(size=(T, Hkv, D))
    return q, k, v, np.array(starts), np.array(lens)


def brute_force(q, k, v, starts, lens, Hkv, W, scale):
    """Pure-Python loops: for every row, list its visible keys, exponentiate, divide."""
    T, Hq, D = q.shape
    G = Hq // Hkv
    out = np.full((T, Hq, D), np.nan)
    for s0, L in zip(starts, lens):
        for i in range(L):
            vis = [j for j in range(L) if j <= i and (W == 0 or i - j < W)]
            for h in range(Hq):
                g = h // G
                sc = [scale * sum(q[s0 + i, h, d] * k[s0 + j, g, d] for d in range(D)) for j in vis]
                mx = max(sc)
                e = [math.exp(s - mx) for s in sc]
                tot = sum(e)
                for d in range(D):
                    out[s0 + i, h, d] = sum(e[n] * v[s0 + j, g, d] for n, j in enumerate(vis)) / tot
    return out


# ------------------------------------------------------------------ checks
def check_brute_force(attn):
    for W in (0, 5):
        q, k, v, st, ln = _pack([13, 1, 20], [2, 0, 3, 1], 4, 2, 8, RNG)
        ref = brute_force(q, k, v, st, ln, 2, W, 0.35)
        got = attn(q, k, v, st, ln, 2, W, 0.35)
        rows = np.concatenate([np.arange(s, s + L) for s, L in zip(st, ln)])
        assert np.allclose(got[rows], ref[rows], rtol=0, atol=1e-12)
        pad = np.setdiff1d(np.arange(q.shape[0]), rows)
        assert np.all(np.isnan(got[pad]))


def check_library_sdpa(attn):
    """torch SDPA in float64 with an explicit boolean mask and KV repeated per group."""
    for (Hq, Hkv, D, W, L) in [(4, 2, 64, 16, 64), (4, 1, 64, 0, 64), (16, 2, 32, 0, 40), (8, 8, 16, 7, 50)]:
        q, k, v, st, ln = _pack([L], [0, 0], Hq, Hkv, D, RNG)
        scale = 1.0 / math.sqrt(D)
        got = attn(q, k, v, st, ln, Hkv, W, scale)
        G = Hq // Hkv
        qt = torch.from_numpy(q).permute(1, 0, 2)[None]
        kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        i = torch.arange(L)[:, None]
        j = torch.arange(L)[None, :]
        mask = (j <= i) & ((i - j < W) if W > 0 else torch.ones(L, L, dtype=torch.bool))
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
        ref = ref[0].permute(1, 0, 2).numpy()
        assert np.allclose(got, ref, rtol=0, atol=1e-12)


def check_visible_sets(attn):
    """One-hot values reveal each row's visible keys: with q = 0 the output of row i
    is 1/n on exactly the keys j with j <= i and i - j < W."""
    L = 40
    for W in (0, 1, 7, 39, 40):
        q = np.zeros((L, 1, L))
        k = RNG.normal(size=(L, 1, L))
        v = np.eye(L)[:, None, :]
        out = attn(q, k, v, [0], [L], 1, W, 1.0)[:, 0, :]
        for i in range(L):
            vis = [j for j in range(L) if j <= i and (W == 0 or i - j < W)]
            expect = np.zeros(L)
            expect[vis] = 1.0 / len(vis)
            assert np.allclose(out[i], expect, rtol=0, atol=1e-15), (W, i)


def check_gqa_mapping(attn):
    """KV head g holds the constant value g + 1: query head h must return
    floor(h / G) + 1."""
    Hq, Hkv, L, D = 16, 4, 9, 8
    q = RNG.normal(size=(L, Hq, D))
    k = RNG.normal(size=(L, Hkv, D))
    v = np.broadcast_to((np.arange(Hkv) + 1.0)[None, :, None], (L, Hkv, D)).copy()
    out = attn(q, k, v, [0], [L], Hkv, 0, 0.5)
    for h in range(Hq):
        assert np.allclose(out[:, h, :], h // (Hq // Hkv) + 1.0, rtol=0, atol=1e-14)


def check_scale(attn):
    """Doubling the scale equals doubling q; the scale is applied exactly once."""
    q, k, v, st, ln = _pack([12], [0, 0], 2, 1, 4, RNG)
    a = attn(q, k, v, st, ln, 1, 0, 0.7)
    b = attn(2 * q, k, v, st, ln, 1, 0, 0.35)
    assert np.allclose(a, b, rtol=0, atol=1e-13)
    # two keys with scores s0, s1: weight of key 1 for row 1 = sigmoid(s1 - s0)
    q = np.array([[[1.0, 0.0]], [[0.5, 2.0]]])
    k = np.array([[[0.3, -1.0]], [[1.5, 0.25]]])
    v = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    scale = 0.8
    s0 = scale * (0.5 * 0.3 + 2.0 * -1.0)
    s1 = scale * (0.5 * 1.5 + 2.0 * 0.25)
    w1 = 1.0 / (1.0 + math.exp(s0 - s1))
    out = attn(q, k, v, [0], [2], 1, 0, scale)
    assert np.allclose(out[1, 0], [1 - w1, w1], rtol=0, atol=1e-15)


def check_properties(attn):
    q, k, v, st, ln = _pack([30, 17], [1, 2, 0], 4, 2, 16, RNG)
    for W in (0, 8):
        out = attn(q, k, v, st, ln, 2, W, 0.25)
        for s0, L in zip(st, ln):
            # the first row sees only itself: its output is v_0 exactly
            assert np.array_equal(out[s0, 0], v[s0, 0]) and np.array_equal(out[s0, 3], v[s0, 1])
            for i in range(L):
                lo = 0 if W == 0 else max(0, i - W + 1)
                for h in range(4):
                    vv = v[s0 + lo:s0 + i + 1, h // 2]
                    assert np.all(out[s0 + i, h] <= vv.max(axis=0) + 1e-12)
                    assert np.all(out[s0 + i, h] >= vv.min(axis=0) - 1e-12)
    # q = 0: uniform weights -> mean of visible values
    q0 = np.zeros_like(q)
    out = attn(q0, k, v, st, ln, 2, 8, 0.25)
    s0, L = st[1], ln[1]
    for i in range(L):
        lo = max(0, i - 7)
        assert np.allclose(out[s0 + i, 2], v[s0 + lo:s0 + i + 1, 1].mean(axis=0), rtol=0, atol=1e-14)


def check_sliding_equals_full_within_window(attn):
    W = 16
    for L, same in ((16, True), (17, False)):
        q, k, v, st, ln = _pack([L], [0, 0], 2, 1, 8, RNG)
        a = attn(q, k, v, st, ln, 1, W, 0.3)
        b = attn(q, k, v, st, ln, 1, 0, 0.3)
        assert np.array_equal(a[:W], b[:W])
        if not same:
            assert not np.allclose(a[W], b[W])


def check_sequences_independent(attn):
    """Permuting and re-padding the sequences of a pack permutes the outputs bitwise."""
    lens = [5, 11, 3, 8]
    q, k, v, st, ln = _pack(lens, [1, 0, 2, 0, 1], 4, 1, 8, RNG)
    out = attn(q, k, v, st, ln, 1, 4, 0.4)
    order = [2, 0, 3, 1]
    rows = [np.arange(st[b], st[b] + lens[b]) for b in order]
    gap = 3
    q2 = np.concatenate([np.concatenate([RNG.normal(size=(gap, 4, 8)), q[r]]) for r in rows])
    k2 = np.concatenate([np.concatenate([RNG.normal(size=(gap, 1, 8)), k[r]]) for r in rows])
    v2 = np.concatenate([np.concatenate([RNG.normal(size=(gap, 1, 8)), v[r]]) for r in rows])
    st2, t = [], 0
    for b in order:
        st2.append(t + gap)
        t += gap + lens[b]
    out2 = attn(q2, k2, v2, st2, [lens[b] for b in order], 1, 4, 0.4)
    for n, b in enumerate(order):
        assert np.array_equal(out2[st2[n]:st2[n] + lens[b]], out[st[b]:st[b] + lens[b]])


ATTENTION_CHECKS = [check_brute_force, check_library_sdpa, check_visible_sets, check_gqa_mapping,
                    check_scale, check_properties, check_sliding_equals_full_within_window,
                    check_sequences_independent]


# ------------------------------------------------------------------ per-row last keys
# (the rows of an image see every row of that image; TensorFold PR #1186, the vision
# commit of the native Gemma 4 engine). Each check takes attn(q, k, v, st, ln, Hkv, W,
# scale, last_key) so the mutant test can plant mistakes in the mask.

def _image_last_keys(T, starts, images):
    """last_key [T]: -1 for text rows, the image's last position for its rows.
    images: per sequence, a list of (first position, number of rows)."""
    lk = np.full(T, -1, np.int64)
    for s0, imgs in zip(starts, images):
        for a, n in imgs:
            lk[s0 + a:s0 + a + n] = a + n - 1
    return lk


def brute_force_images(q, k, v, starts, lens, images, Hkv, W, scale):
    """Pure-Python loops, visibility stated the pages' way: key j is visible to row i
    if j <= i or both lie in the same image, and always i - j < W for a sliding layer."""
    T, Hq, D = q.shape
    G = Hq // Hkv
    out = np.full((T, Hq, D), np.nan)
    for s0, L, imgs in zip(starts, lens, images):
        img_of = {}
        for n_img, (a, n) in enumerate(imgs):
            for p in range(a, a + n):
                img_of[p] = n_img
        for i in range(L):
            vis = [j for j in range(L)
                   if (j <= i or (i in img_of and img_of.get(j) == img_of[i])) and (W == 0 or i - j < W)]
            for h in range(Hq):
                g = h // G
                sc = [scale * sum(q[s0 + i, h, d] * k[s0 + j, g, d] for d in range(D)) for j in vis]
                mx = max(sc)
                e = [math.exp(x - mx) for x in sc]
                tot = sum(e)
                for d in range(D):
                    out[s0 + i, h, d] = sum(e[n] * v[s0 + j, g, d] for n, j in enumerate(vis)) / tot
    return out


def check_images_brute_force(attn):
    images = [[(3, 5)], [], [(0, 5), (10, 8)]]
    for W in (0, 5):
        q, k, v, st, ln = _pack([13, 1, 20], [2, 0, 3, 1], 4, 2, 8, RNG)
        lk = _image_last_keys(q.shape[0], st, images)
        ref = brute_force_images(q, k, v, st, ln, images, 2, W, 0.35)
        got = attn(q, k, v, st, ln, 2, W, 0.35, lk)
        rows = np.concatenate([np.arange(s, s + L) for s, L in zip(st, ln)])
        assert np.allclose(got[rows], ref[rows], rtol=0, atol=1e-12)


def check_whole_sequence_image_is_unmasked_attention(attn):
    """One image spanning the whole sequence, no window: every row sees every key, i.e.
    torch's float64 attention with no mask at all."""
    for (Hq, Hkv, D, L) in [(4, 2, 16, 24), (8, 1, 8, 9)]:
        q, k, v, st, ln = _pack([L], [1, 2], Hq, Hkv, D, RNG)
        lk = _image_last_keys(q.shape[0], st, [[(0, L)]])
        got = attn(q, k, v, st, ln, Hkv, 0, 0.3, lk)[st[0]:st[0] + L]
        G = Hq // Hkv
        qt = torch.from_numpy(q[st[0]:st[0] + L]).permute(1, 0, 2)[None]
        kt = torch.from_numpy(k[st[0]:st[0] + L]).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        vt = torch.from_numpy(v[st[0]:st[0] + L]).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.3)[0].permute(1, 0, 2).numpy()
        assert np.allclose(got, ref, rtol=0, atol=1e-12)


def check_text_rows_and_causal_last_keys_unchanged(attn):
    """Rows outside images, and last keys at or below the row's own position, give the
    plain causal result; a last key past the sequence is clipped to its end."""
    q, k, v, st, ln = _pack([17, 11], [0, 2, 0], 4, 2, 8, RNG)
    T = q.shape[0]
    for W in (0, 4):
        base = A.attention(q, k, v, st, ln, 2, W, 0.5)
        lk = _image_last_keys(T, st, [[(6, 4)], [(0, 3)]])
        got = attn(q, k, v, st, ln, 2, W, 0.5, lk)
        text = np.concatenate([np.r_[st[0]:st[0] + 6, st[0] + 10:st[0] + 17], np.r_[st[1] + 3:st[1] + 11]])
        assert np.array_equal(got[text], base[text])
        own = np.full(T, -1, np.int64)
        for s0, L in zip(st, ln):
            own[s0:s0 + L] = np.arange(L) - (np.arange(L) % 3)  # at or below the row's position
        assert np.array_equal(attn(q, k, v, st, ln, 2, W, 0.5, own)[text], base[text])
        far = lk.copy()
        far[st[1]:st[1] + 3] = 1000
        assert np.array_equal(attn(q, k, v, st, ln, 2, W, 0.5, far)[st[1]:st[1] + 11],
                              attn(q, k, v, st, ln, 2, W, 0.5, np.where(far == 1000, 10, far))[st[1]:st[1] + 11])


LAST_KEY_CHECKS = [check_images_brute_force, check_whole_sequence_image_is_unmasked_attention,
                   check_text_rows_and_causal_last_keys_unchanged]


def _attention_with_last_key(q, k, v, st, ln, Hkv, W, scale, last_key):
    return A.attention(q, k, v, st, ln, Hkv, W, scale, last_key=last_key)


@pytest.mark.parametrize("check", LAST_KEY_CHECKS, ids=lambda c: c.__name__)
def test_last_key_pin(check):
    check(_attention_with_last_key)


@pytest.mark.parametrize("check", ATTENTION_CHECKS, ids=lambda c: c.__name__)
def test_attention_pin(check):
    check(A.attention)


def test_weights_rows_sum_to_one_and_vanish_on_hidden_keys():
    q = RNG.normal(size=(50, 32))
    k = RNG.normal(size=(50, 32))
    for W in (0, 10):
        m = A.visible_mask(50, 50, W)
        w = A.attention_weights(q, k, m, 0.2)
        assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        assert np.all(w[~m] == 0) and np.all(w[m] > 0)


def test_decode_rows_equal_last_prefill_row():
    Hq, Hkv, D = 8, 2, 16
    for W in (0, 6):
        lens = [1, 5, 23]
        q, k, v, st, ln = _pack(lens, [0, 0, 0, 0], Hq, Hkv, D, RNG)
        full = A.attention(q, k, v, st, ln, Hkv, W, 0.25)
        qn = np.stack([q[s + L - 1] for s, L in zip(st, ln)])
        # keys handed over from the position of the first visible key (as a ring keeps them)
        p0 = [0 if W == 0 else max(0, L - W) for L in lens]
        keys = [k[s + a:s + L] for s, L, a in zip(st, ln, p0)]
        vals = [v[s + a:s + L] for s, L, a in zip(st, ln, p0)]
        dec = A.decode_rows(qn, keys, vals, p0, ln, W, 0.25)
        for b, (s, L) in enumerate(zip(st, ln)):
            assert np.allclose(dec[b], full[s + L - 1], rtol=0, atol=1e-13)


def test_layer_forward_k_eq_v_uses_rotated_k_as_values():
    D, R, F, th = 16, 4, 16, 1e6
    T = 9
    qb = f64_to_bf16_bits(RNG.normal(size=(T, 4, D)))
    kb = f64_to_bf16_bits(RNG.normal(size=(T, 1, D)))
    w = f64_to_bf16_bits(RNG.normal(1, 0.1, size=D))
    pos = np.arange(T)
    kw = dict(num_kv_heads=1, window=0, rope_dims=R, rope_freq_dim=F, theta=th, eps=1e-6, scale=0.25)
    q1, k1, out = A.layer_forward(qb, kb, None, w, w, pos, [0], [T], k_eq_v=True, **kw)
    ref = A.attention(bf16_bits_to_f64(q1), bf16_bits_to_f64(k1), bf16_bits_to_f64(k1), [0], [T], 1, 0, 0.25)
    assert np.array_equal(out, ref)
    junk = f64_to_bf16_bits(RNG.normal(size=(T, 1, D)))
    _, _, out2 = A.layer_forward(qb, kb, junk, w, w, pos, [0], [T], k_eq_v=True, **kw)
    assert np.array_equal(out, out2)
    _, _, out3 = A.layer_forward(qb, kb, junk, w, w, pos, [0], [T], k_eq_v=False, **kw)
    assert not np.allclose(out, out3)


def check_layer_forward_routes_weights(layer_forward):
    """q goes through the q weights and k through the k weights (distinct draws), each
    against the library prologue (transformers' norm then rotation), at positions past
    0; the output is torch's float64 SDPA over those bits, with V = the post-prologue k
    for a K=V layer and the raw v otherwise."""
    from test_oracle_prologue import transformers_prologue
    D, R, F, th, Hq, Hkv, T = 64, 16, 64, 1e6, 4, 2, 40
    qb = f64_to_bf16_bits(RNG.normal(size=(T, Hq, D)))
    kb = f64_to_bf16_bits(RNG.normal(size=(T, Hkv, D)))
    vb = f64_to_bf16_bits(RNG.normal(size=(T, Hkv, D)))
    wq = f64_to_bf16_bits(RNG.normal(1.0, 0.1, size=D))
    wk = f64_to_bf16_bits(RNG.normal(1.0, 0.1, size=D))
    pos = np.arange(T)
    for k_eq_v in (True, False):
        q1, k1, out = layer_forward(qb, kb, vb, wq, wk, pos, [0], [T], num_kv_heads=Hkv, window=0, k_eq_v=k_eq_v,
                                    rope_dims=R, rope_freq_dim=F, theta=th, eps=1e-6, scale=0.125, pair_offset=D // 2)
        for got, x, w in ((q1, qb, wq), (k1, kb, wk)):
            ref = transformers_prologue(x, w, pos, D, R, F, th)
            # one bf16 rounding of a float32-accurate value: within 2^-8 relative
            assert np.all(np.abs(bf16_bits_to_f64(got) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)
        vals = k1 if k_eq_v else vb
        G = Hq // Hkv
        qt = torch.from_numpy(bf16_bits_to_f64(q1)).permute(1, 0, 2)[None]
        kt = torch.from_numpy(bf16_bits_to_f64(k1)).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        vt = torch.from_numpy(bf16_bits_to_f64(vals)).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        mask = torch.arange(T)[None, :] <= torch.arange(T)[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.125)
        assert np.allclose(out, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_layer_forward_routes_weights():
    check_layer_forward_routes_weights(A.layer_forward)


def check_layer_forward_v_norm(layer_forward):
    """The real model's global layer: K and V come from the same raw projection; K is
    normed with the k weights and rotated, V is the projection's unit RMS norm (no weight,
    not rotated). Against torch's float64 SDPA with V from transformers' weightless
    Gemma4RMSNorm of the raw rows, K from the library prologue."""
    from transformers.models.gemma4.modeling_gemma4 import Gemma4RMSNorm

    from test_oracle_prologue import transformers_prologue
    D, R, F, th, Hq, Hkv, T = 64, 16, 64, 1e6, 4, 1, 33
    qb = f64_to_bf16_bits(RNG.normal(size=(T, Hq, D)))
    kb = f64_to_bf16_bits(RNG.normal(size=(T, Hkv, D)) * 3.0)
    wq = f64_to_bf16_bits(RNG.normal(1.0, 0.1, size=D))
    wk = f64_to_bf16_bits(RNG.normal(1.0, 0.1, size=D))
    pos = np.arange(T) + 5
    q1, k1, out = layer_forward(qb, kb, kb, wq, wk, pos, [0], [T], num_kv_heads=Hkv, window=0, k_eq_v=False,
                                rope_dims=R, rope_freq_dim=F, theta=th, eps=1e-6, scale=0.125, pair_offset=D // 2,
                                v_norm=True)
    kref = transformers_prologue(kb, wk, pos, D, R, F, th)
    assert np.all(np.abs(bf16_bits_to_f64(k1) - kref) <= 2.0 ** -8 * np.abs(kref) + 1e-6)
    vref = Gemma4RMSNorm(D, eps=1e-6, with_scale=False)(torch.from_numpy(bf16_bits_to_f64(kb)).float()).double()
    vbits = f64_to_bf16_bits(vref.numpy())
    G = Hq // Hkv
    qt = torch.from_numpy(bf16_bits_to_f64(q1)).permute(1, 0, 2)[None]
    kt = torch.from_numpy(bf16_bits_to_f64(k1)).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    vt = torch.from_numpy(bf16_bits_to_f64(vbits)).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    mask = torch.arange(T)[None, :] <= torch.arange(T)[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.125)
    # V bits from float32 library arithmetic may differ from the float64 rounding by one
    # bf16 ulp here and there: allow that much in the weighted mean
    assert np.allclose(out, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=2.0 ** -8 * 6)
    with pytest.raises(ValueError):
        layer_forward(qb, kb, kb, wq, wk, pos, [0], [T], num_kv_heads=Hkv, window=0, k_eq_v=True, rope_dims=R,
                      rope_freq_dim=F, theta=th, eps=1e-6, scale=0.125, v_norm=True)


def test_layer_forward_v_norm():
    check_layer_forward_v_norm(A.layer_forward)
