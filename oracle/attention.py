"""Attention of the oracle: exact softmax GQA attention with explicit dense masks.

Test infrastructure only: the tests, the smoke check and the benchmark's CPU
baseline may call it; the HIP library never does.

Sources (page titles; see the citation key in the design notes):
* RL-Kernel issue #415, Gemma-4-31B-it RFC, section 5 work items
  `sliding_attention_core` (causal local attention, window 1024, Q32/KV16, D256),
  `global_attention_core` (full attention, Q32/KV4, D512, K=V),
  `global_k_eq_v_projection` (one tensor is both K and V) and
  `hybrid_kv_cache_contract` (prefill -> decode handoff of the same rows);
  section 2 fingerprint table (window 1024, attention_k_eq_v=true).
* TensorFold PR #1186, commit message for the native Gemma 4 engine: a prompt-cache
  state keeps each sliding layer's last 1023 keys, i.e. with the new row a sliding
  query sees 1024 keys including itself.
* TensorFold PR #1186, commit message for the vision path of that engine: an image's
  rows each see all of that image's rows, through a per-row last key of the sliding
  attention; RL-Kernel #415 section 2 (use_bidirectional_attention = "vision") and
  section 5 (multimodal_bidirectional_mask).

Readings taken where the pages are silent (listed in the design notes):
* key j is visible to query i of the same sequence iff j <= i and, for a sliding
  layer with window W, i - j < W; sequences never see one another or padding rows;
* query head h reads KV head floor(h / G), G = Hq / Hkv (contiguous groups);
* scores are scale * <q_i, k_j> with scale 1/sqrt(D) (passed in); no logit softcap;
* the global layer's V is the same post-prologue tensor as its K; the sliding
  layer's V is the raw v input;
* a decode row is the prefill row of the sequence's last position;
* with per-row last keys, row i sees key j iff j <= max(i, last_i) and the window rule
  i - j < W holds (the window still bounds the keys before the row); last_i is clipped
  to the sequence's last position.

Everything is float64; the result is not rounded (the comparison rounds nothing).
"""
from __future__ import annotations

import numpy as np

from .bf16 import bf16_bits_to_f64
from .prologue import qk_prologue, v_prologue


def visible_mask(num_queries: int, num_keys: int, window: int, query_pos0: int = 0,
                 key_pos0: int = 0, last_key=None) -> np.ndarray:
    """Boolean [Lq, Lk]: query at position query_pos0 + a sees key at key_pos0 + b.

    last_key (optional, int [Lq]): position of each query's last visible key; a query
    sees the keys up to the later of its own position and last_key (the rows of an
    image see the whole image); the window rule is unchanged.
    """
    i = query_pos0 + np.arange(num_queries)[:, None]
    j = key_pos0 + np.arange(num_keys)[None, :]
    hi = i if last_key is None else np.maximum(i, np.asarray(last_key, np.int64)[:, None])
    m = j <= hi
    if window > 0:
        m &= (i - j) < window
    return m


def attention_weights(q_rows: np.ndarray, k_rows: np.ndarray, mask: np.ndarray,
                      scale: float) -> np.ndarray:
    """Softmax over the visible keys of scale * q k^T; zero on hidden keys.

    q_rows [Lq, D], k_rows [Lk, D], mask [Lq, Lk]; every row must see >= 1 key.
    """
    s = scale * (np.asarray(q_rows, np.float64) @ np.asarray(k_rows, np.float64).T)
    s = np.where(mask, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    p = np.exp(s - m)  # exp(-inf) = 0 on hidden keys
    return p / np.sum(p, axis=1, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, seq_start, seq_len,
              num_kv_heads: int, window: int, scale: float, last_key=None) -> np.ndarray:
    """Packed varlen GQA attention.

    q [T, Hq, D], k and v [T, Hkv, D] (float64 values). Sequence b owns rows
    [seq_start[b], seq_start[b] + seq_len[b]) with positions 0..seq_len[b]-1.
    last_key (optional, int [T], indexed by packed row): each row's last visible key
    position, clipped to its sequence's last position (see visible_mask).
    Returns float64 [T, Hq, D]; rows of no sequence are NaN.
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
        if last_key is None:
            mask = visible_mask(L, L, window)
        else:
            lk = np.minimum(np.asarray(last_key, np.int64)[s0:s0 + L], L - 1)
            mask = visible_mask(L, L, window, last_key=lk)
        for h in range(Hq):
            g = h // G
            w = attention_weights(q[s0:s0 + L, h, :], k[s0:s0 + L, g, :], mask, scale)
            out[s0:s0 + L, h, :] = w @ v[s0:s0 + L, g, :]
    return out


def decode_rows(q: np.ndarray, keys, values, key_pos0, ctx_len, window: int,
                scale: float) -> np.ndarray:
    """One new token per sequence against its cached keys.

    q [B, Hq, D] (the new tokens, already through the prologue); keys[b], values[b]
    [n_b, Hkv, D] hold sequence b's keys at logical positions key_pos0[b] ..
    key_pos0[b] + n_b - 1, which must cover every key the row can see. The query sits
    at position ctx_len[b] - 1. Returns float64 [B, Hq, D].
    """
    q = np.asarray(q, np.float64)
    B, Hq, D = q.shape
    out = np.empty((B, Hq, D))
    for b in range(B):
        L = int(ctx_len[b])
        kb = np.asarray(keys[b], np.float64)
        vb = np.asarray(values[b], np.float64)
        p0 = int(key_pos0[b])
        first_visible = max(0, L - window) if window > 0 else 0
        assert p0 <= first_visible and p0 + kb.shape[0] >= L, "keys must cover the visible range"
        Hkv = kb.shape[1]
        G = Hq // Hkv
        mask = visible_mask(1, kb.shape[0], window, query_pos0=L - 1, key_pos0=p0)
        for h in range(Hq):
            w = attention_weights(q[b, h:h + 1, :], kb[:, h // G, :], mask, scale)
            out[b, h, :] = (w @ vb[:, h // G, :])[0]
    return out


def layer_forward(q_bits, k_bits, v_bits, wq_bits, wk_bits, positions, seq_start, seq_len,
                  *, num_kv_heads: int, window: int, k_eq_v: bool, rope_dims: int,
                  rope_freq_dim: int, theta: float, eps: float, scale: float,
                  pair_offset: int | None = None, v_norm: bool = False):
    """Prologue on q and k, then attention; returns (q bits, k bits, float64 output).

    With k_eq_v the post-prologue k tensor is also V and v_bits is ignored; otherwise
    V is the raw v input, or with v_norm its unit RMS norm (v_prologue: no weight, no
    rotation). The real model's global layer is k_eq_v False, v_norm True, with v_bits
    the same raw projection as k_bits (K normed and rotated, V only normed).
    """
    if k_eq_v and v_norm:
        raise ValueError("v_norm needs a separate V (k_eq_v False)")
    kw = dict(rope_dims=rope_dims, rope_freq_dim=rope_freq_dim, theta=theta, eps=eps,
              pair_offset=pair_offset)
    _, qb = qk_prologue(q_bits, wq_bits, positions, **kw)
    _, kb = qk_prologue(k_bits, wk_bits, positions, **kw)
    if k_eq_v:
        vb = kb
    elif v_norm:
        _, vb = v_prologue(v_bits, eps=eps)
    else:
        vb = np.asarray(v_bits, np.uint16)
    out = attention(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb),
                    seq_start, seq_len, num_kv_heads, window, scale)
    return qb, kb, out
