"""The split form of the attention: a row's keys in fixed chunks, merged in chunk order.

Test infrastructure only: the tests, the smoke check and the benchmark's CPU
baseline may call it; the HIP library never does.

Sources (page titles; see the citation key in the design notes):
* RL-Kernel issue #415, Gemma-4-31B-it RFC, section 4 (numerical contract), rule 3:
  a split of the key range is allowed only when the split and its merge tree are
  fixed by the contract.
* TensorFold PR #1186, the window-rows commits: decode runs over fixed key chunks
  whose partial results are merged in chunk order (at head dims 256 and 512).

Readings taken where the pages are silent (listed in the design notes):
* chunk c of a sequence is the C consecutive positions c C .. c C + C - 1 (aligned to
  position 0, C fixed by the caller); a row takes the chunks that hold its visible
  keys, in ascending order;
* a chunk's partial result over the row's visible keys k in it is the triple
  m_c = max_k s_k, l_c = sum_k exp(s_k - m_c), O_c = sum_k exp(s_k - m_c) v_k;
* the merge: M = max_c m_c, w_c = exp(m_c - M), out = (sum_c w_c O_c) / (sum_c w_c l_c),
  both sums taken in ascending c.
In exact arithmetic this is the softmax over all of the row's keys (the form changes
only where the rounding happens); here everything is float64.
"""
from __future__ import annotations

import numpy as np

from .attention import visible_mask


def chunk_partials(q_row, k_rows, v_rows, key_pos0: int, visible, scale: float, chunk: int):
    """Partial results of one query row over each chunk that holds visible keys.

    q_row [D]; k_rows, v_rows [n, D] hold key positions key_pos0 .. key_pos0 + n - 1;
    visible: bool [n]. Returns a list, in ascending chunk order, of
    (c, first_pos, last_pos, m_c, l_c, O_c [D]) with first/last the chunk's visible key
    positions.
    """
    q = np.asarray(q_row, np.float64)
    k = np.asarray(k_rows, np.float64)
    v = np.asarray(v_rows, np.float64)
    vis = np.asarray(visible, bool)
    pos = key_pos0 + np.arange(k.shape[0])
    s = scale * (k @ q)
    parts = []
    for c in np.unique(pos[vis] // chunk):
        sel = vis & (pos // chunk == c)
        sc = s[sel]
        m = np.max(sc)
        e = np.exp(sc - m)
        parts.append((int(c), int(pos[sel][0]), int(pos[sel][-1]), m, np.sum(e), e @ v[sel]))
    return parts


def merge_partials(parts) -> np.ndarray:
    """The row's output from its chunk partials, merged in ascending chunk order."""
    assert [p[0] for p in parts] == sorted(p[0] for p in parts), "chunks in ascending order"
    M = max(p[3] for p in parts)
    num = np.zeros_like(parts[0][5])
    den = 0.0
    for _, _, _, m, l, o in parts:
        w = np.exp(m - M)
        num = num + w * o
        den = den + w * l
    return num / den


def split_attention(q, k, v, seq_start, seq_len, num_kv_heads: int, window: int, scale: float,
                    chunk: int) -> np.ndarray:
    """Packed varlen GQA attention in the split form (layout as attention.attention).

    q [T, Hq, D], k and v [T, Hkv, D]. Returns float64 [T, Hq, D]; rows of no sequence
    are NaN.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, Hq, D = q.shape
    G = Hq // num_kv_heads
    out = np.full((T, Hq, D), np.nan)
    for s0, L in zip(np.asarray(seq_start).tolist(), np.asarray(seq_len).tolist()):
        if L == 0:
            continue
        mask = visible_mask(L, L, window)
        for i in range(L):
            for h in range(Hq):
                g = h // G
                parts = chunk_partials(q[s0 + i, h], k[s0:s0 + L, g], v[s0:s0 + L, g], 0, mask[i], scale, chunk)
                out[s0 + i, h] = merge_partials(parts)
    return out


def split_decode_rows(q, keys, values, key_pos0, ctx_len, window: int, scale: float, chunk: int) -> np.ndarray:
    """One new token per sequence in the split form (arguments as attention.decode_rows)."""
    q = np.asarray(q, np.float64)
    B, Hq, D = q.shape
    out = np.empty((B, Hq, D))
    for b in range(B):
        L = int(ctx_len[b])
        kb = np.asarray(keys[b], np.float64)
        vb = np.asarray(values[b], np.float64)
        p0 = int(key_pos0[b])
        G = Hq // kb.shape[1]
        vis = visible_mask(1, kb.shape[0], window, query_pos0=L - 1, key_pos0=p0)[0]
        for h in range(Hq):
            parts = chunk_partials(q[b, h], kb[:, h // G], vb[:, h // G], p0, vis, scale, chunk)
            out[b, h] = merge_partials(parts)
    return out
