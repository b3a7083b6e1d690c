"""Pins of the oracle's split form (CPU only): what its chunks hold, a closed-form case,
and agreement with the unsplit softmax, which it equals in exact arithmetic."""
import numpy as np

import oracle.attention as A
import oracle.split as S


def _seqs(rng, lens, hq=4, hkv=2, d=16):
    T = sum(lens) + 3
    q = rng.standard_normal((T, hq, d))
    k = rng.standard_normal((T, hkv, d))
    v = rng.standard_normal((T, hkv, d))
    starts = np.cumsum([1] + list(lens))[:-1]  # one padding row in front
    return q, k, v, starts, np.array(lens)


def test_chunks_cover_the_visible_keys_in_order():
    rng = np.random.default_rng(1)
    d, n = 8, 700
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    q = rng.standard_normal(d)
    for i, C in [(0, 256), (255, 256), (256, 256), (699, 256), (699, 100), (300, 1024)]:
        vis = np.arange(n) <= i
        parts = S.chunk_partials(q, k, v, 0, vis, 0.3, C)
        assert [p[0] for p in parts] == list(range(i // C + 1))
        for c, lo, hi, m, l, o in parts:
            assert lo == c * C and hi == min(i, c * C + C - 1)
            s = 0.3 * (k[lo:hi + 1] @ q)
            assert m == np.max(s)
            np.testing.assert_allclose(l, np.sum(np.exp(s - m)), rtol=1e-14)
            np.testing.assert_allclose(o, np.exp(s - m) @ v[lo:hi + 1], rtol=1e-13, atol=1e-13)
    # a window: the first chunk starts at the window's first key
    vis = (np.arange(n) <= 650) & (650 - np.arange(n) < 300)
    parts = S.chunk_partials(q, k, v, 0, vis, 0.3, 256)
    assert [(p[0], p[1], p[2]) for p in parts] == [(1, 351, 511), (2, 512, 650)]


def test_closed_form_two_chunks():
    # scores 0 and ln 3 in chunks of one key: weights 1/4 and 3/4
    q = np.array([1.0, 0.0])
    k = np.array([[0.0, 5.0], [np.log(3.0), -2.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    parts = S.chunk_partials(q, k, v, 0, np.array([True, True]), 1.0, 1)
    assert len(parts) == 2
    np.testing.assert_allclose(S.merge_partials(parts), [0.25, 0.75], rtol=1e-15)
    # merged in the other order is refused (the tree is fixed)
    try:
        S.merge_partials(parts[::-1])
    except AssertionError:
        pass
    else:
        raise AssertionError("a merge out of chunk order was accepted")


def test_split_equals_unsplit_softmax():
    rng = np.random.default_rng(2)
    q, k, v, st, ln = _seqs(rng, [600, 1, 257, 300])
    ref = A.attention(q, k, v, st, ln, 2, 0, 0.25)
    for C in (256, 512, 64):
        got = S.split_attention(q, k, v, st, ln, 2, 0, 0.25, C)
        rows = ~np.isnan(ref[:, 0, 0])
        assert np.array_equal(rows, ~np.isnan(got[:, 0, 0]))
        np.testing.assert_allclose(got[rows], ref[rows], rtol=1e-11, atol=1e-12)


def test_split_with_peaked_scores():
    # scores far apart (offsets of chunks differ by hundreds): the weights exp(m_c - M)
    # carry the whole difference
    rng = np.random.default_rng(3)
    q, k, v, st, ln = _seqs(rng, [520], hq=2, hkv=1, d=8)
    q *= 40.0
    ref = A.attention(q, k, v, st, ln, 1, 0, 1.0)
    got = S.split_attention(q, k, v, st, ln, 1, 0, 1.0, 128)
    rows = ~np.isnan(ref[:, 0, 0])
    np.testing.assert_allclose(got[rows], ref[rows], rtol=1e-10, atol=1e-12)


def test_split_decode_rows_equal_the_prefill_rows():
    rng = np.random.default_rng(4)
    L = [1, 256, 257, 700]
    hq, hkv, d = 4, 1, 8
    keys = [rng.standard_normal((n, hkv, d)) for n in L]
    vals = [rng.standard_normal((n, hkv, d)) for n in L]
    q = rng.standard_normal((len(L), hq, d))
    got = S.split_decode_rows(q, keys, vals, [0] * len(L), L, 0, 0.5, 256)
    ref = A.decode_rows(q, keys, vals, [0] * len(L), L, 0, 0.5)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    # and the last row of a whole-sequence split prefill
    b = 3
    qq = np.zeros((L[b], hq, d))
    qq[-1] = q[b]
    pre = S.split_attention(qq, keys[b], vals[b], [0], [L[b]], hkv, 0, 0.5, 256)
    np.testing.assert_allclose(pre[-1], got[b], rtol=1e-12, atol=1e-13)
