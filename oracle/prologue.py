"""q/k prologue of the oracle: per-head RMSNorm, then RoPE, then one bf16 rounding.

Test infrastructure only: the tests, the smoke check and the benchmark's CPU
baseline may call it; the HIP library never does.

Sources (page titles; see the citation key in the design notes):
* RL-Kernel issue #415, Gemma-4-31B-it RFC, section 5 work items
  `qk_rmsnorm_d256_d512` (per-head q/k RMSNorm at head dim 256 and 512),
  `sliding_rope_d256` (standard RoPE, theta 10000) and `global_proportional_p_rope`
  (partial proportional p-RoPE, factor 0.25, theta 1e6); section 2 fingerprint table.
* TensorFold PR #1186, commit message for tf_qk_rows_once / tf_qk_rows_round: the
  norm multiplies by the weight (w * (x * inv)) and comes before RoPE; at head dim 512
  the same rows can norm v by a unit RMS norm (no weight, and v is not rotated).

Readings taken where the pages are silent (listed in the design notes):
* weight form y = w * x / sqrt(mean(x^2) + eps) (weights multiply directly, eps 1e-6);
* RoPE pairs are rotate-half pairs (i, i + R/2) inside the rotated block [0, R)
  (pair_offset R/2); the layout with pairs (i, i + D/2) over the whole head, the rest
  of the pairs at frequency zero, is the same rotation on permuted dims and is
  available as pair_offset D/2;
* pair i turns by position * theta^(-2 i / F); sliding layers R = F = D, global layers
  R = D/4 (the partial factor) and F = D ("proportional": frequencies keep the full
  head dim's spacing), so the global layer rotates exactly dims 0..127 of 512;
* one bf16 rounding, straight from the float64 result.
"""
from __future__ import annotations

import numpy as np

from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """y = w * x / sqrt(mean(x^2) + eps) over the last axis (the head dim), float64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return w * (x / np.sqrt(ms + eps))


def rope_inv_freq(rope_dims: int, rope_freq_dim: int, theta: float) -> np.ndarray:
    """Angular speed of pair i, i in [0, R/2): theta^(-2 i / F)."""
    i = np.arange(rope_dims // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / float(rope_freq_dim))


def rope(y: np.ndarray, positions: np.ndarray, rope_dims: int, rope_freq_dim: int,
         theta: float, pair_offset: int | None = None) -> np.ndarray:
    """Rotate pairs (i, i + P) of y[t, h, :], i in [0, R/2), by positions[t] * inv_freq[i].

    y: float64 [T, H, D]; positions: integer [T]; P = pair_offset, default R/2.
    (y_i, y_{i+P}) -> (y_i cos a - y_{i+P} sin a, y_{i+P} cos a + y_i sin a).
    Dims outside the R rotated ones pass through unchanged.
    """
    y = np.asarray(y, dtype=np.float64)
    half = rope_dims // 2
    P = half if pair_offset is None else int(pair_offset)
    assert P >= half and P + half <= y.shape[-1]
    ang = np.asarray(positions, dtype=np.float64)[:, None] * rope_inv_freq(rope_dims, rope_freq_dim, theta)[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a = y[..., :half]
    b = y[..., P:P + half]
    out = y.copy()
    out[..., :half] = a * c - b * s
    out[..., P:P + half] = b * c + a * s
    return out


def qk_prologue(x_bits: np.ndarray, w_bits: np.ndarray, positions: np.ndarray, *,
                rope_dims: int, rope_freq_dim: int, theta: float, eps: float,
                pair_offset: int | None = None):
    """Norm then rotate one bf16 tensor [T, H, D]; returns (float64 values, bf16 bits).

    The float64 values are the exact result before the single rounding; the bits are
    what the layer stores (they are also the KV-cache contents for k).
    """
    x = bf16_bits_to_f64(x_bits)
    w = bf16_bits_to_f64(w_bits)
    y = rope(rms_norm(x, w, eps), positions, rope_dims, rope_freq_dim, theta, pair_offset)
    return y, f64_to_bf16_bits(y)


def v_prologue(x_bits: np.ndarray, *, eps: float):
    """The value rows' unit RMS norm: y = x / sqrt(mean(x^2) + eps) over the head dim, no
    weight and no rotation, then one bf16 rounding; returns (float64 values, bf16 bits).
    (TensorFold PR #1186, tf_qk_rows_once commit: v normed by a unit RMS norm.)"""
    x = bf16_bits_to_f64(x_bits)
    y = rms_norm(x, np.ones(x.shape[-1]), eps)
    return y, f64_to_bf16_bits(y)
