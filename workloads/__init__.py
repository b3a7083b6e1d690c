"""Seeded synthetic inputs shared by the oracle checks, the GPU tests and the benchmark.

This module draws numbers and describes shapes; it holds none of the attention,
norm or rotary arithmetic. Both sides of every parity test (the CPU oracle and the
HIP library) receive the same arrays from here.

Layer geometry follows the Gemma-4-31B-it checkpoint fingerprint table (RL-Kernel
issue #415, "[RFC][Gemma-4-31B-it] WS1/WS2 kernel roadmap", section 2): 32 query
heads; sliding layers with 16 KV heads of dim 256, window 1024 and standard RoPE at
theta 1e4; global layers with 4 KV heads of dim 512, K=V, and proportional p-RoPE
with partial factor 0.25 at theta 1e6.

Values: bf16 tensors are drawn as float32 N(mean, std) by torch's seeded generator
and converted to bf16 by torch (round to nearest even). Sequence lengths come from
numpy's PCG64 generator.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np
import torch

SLIDING = 0
GLOBAL = 1


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    """Geometry of one attention layer type (mirrors the C struct g4attn_layer)."""

    name: str
    kind: int  # SLIDING or GLOBAL
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    window: int  # > 0: key j visible to query i iff 0 <= i - j < window; 0: full causal
    k_eq_v: bool  # one tensor serves as both K and V
    rope_dims: int  # rotated dims [0, rope_dims)
    rope_freq_dim: int  # pair i turns at theta ** (-2 i / rope_freq_dim)
    rope_theta: float
    softmax_scale: float
    rms_eps: float = 1e-6
    v_norm: bool = False  # the prologue stores v's unit RMS norm (needs a separate V)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def _scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


# Gemma-4-31B sliding layer: Q32/KV16, D256, window 1024, RoPE theta 1e4 on all dims.
SLIDING_31B = LayerSpec("gemma4-31b-sliding", SLIDING, 32, 16, 256, 1024, False, 256, 256, 1e4, _scale(256))
# Gemma-4-31B global layer: Q32/KV4, D512, K=V, p-RoPE on the first quarter (128 dims), theta 1e6.
GLOBAL_31B = LayerSpec("gemma4-31b-global", GLOBAL, 32, 4, 512, 0, True, 128, 512, 1e6, _scale(512))
# Tiny sliding layer (correctness size): Q4/KV2, D64, window 16, theta 1e4.
TINY_SLIDING = LayerSpec("tiny-sliding", SLIDING, 4, 2, 64, 16, False, 64, 64, 1e4, _scale(64))
# Tiny global twin: Q4/KV1, D64, K=V, a quarter of the dims rotated, theta 1e6.
TINY_GLOBAL = LayerSpec("tiny-global", GLOBAL, 4, 1, 64, 0, True, 16, 64, 1e6, _scale(64))
# Tiny global layer with the 31B grouping (8 query heads per KV head).
TINY_GLOBAL_G8 = LayerSpec("tiny-global-g8", GLOBAL, 16, 2, 64, 0, True, 16, 64, 1e6, _scale(64))

# Gemma-4-31B global layer with its values formed as the real model forms them: K and V are
# separate tensors of head dim 512 from one projection, K normed and rotated, V only normed
# (unit RMS, no weight, no rotation); the caller passes the raw projection as both k and v.
GLOBAL_31B_V = LayerSpec("gemma4-31b-global-v", GLOBAL, 32, 4, 512, 0, False, 128, 512, 1e6, _scale(512), v_norm=True)

SPECS = {s.name: s for s in (SLIDING_31B, GLOBAL_31B, GLOBAL_31B_V, TINY_SLIDING, TINY_GLOBAL, TINY_GLOBAL_G8)}


def bf16_normal(gen: torch.Generator, shape, mean: float = 0.0, std: float = 1.0,
                device: str = "cpu") -> torch.Tensor:
    """bf16 tensor of N(mean, std) draws (float32 draw, then torch's bf16 conversion)."""
    x = torch.randn(tuple(shape), generator=gen, dtype=torch.float32, device=device)
    if std != 1.0:
        x = x * std
    if mean != 0.0:
        x = x + mean
    return x.to(torch.bfloat16)


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor, on the host."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def from_bits(b: np.ndarray, device: str = "cpu") -> torch.Tensor:
    """bf16 tensor from uint16 bit patterns."""
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(device)


def make_generator(seed: int, device: str = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


@dataclasses.dataclass
class PrefillCase:
    """Packed varlen batch: rows [seq_start[b], seq_start[b] + seq_len[b]) belong to sequence b.

    Rows that belong to no sequence are padding (random values, never read as keys).
    Tensors are bf16 [T, H, D] on `device`; index arrays are int32 tensors on `device`.
    """

    spec: LayerSpec
    q: torch.Tensor
    k: torch.Tensor
    v: Optional[torch.Tensor]
    wq: torch.Tensor
    wk: torch.Tensor
    positions: torch.Tensor
    seq_start: torch.Tensor
    seq_len: torch.Tensor

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def batch(self) -> int:
        return int(self.seq_len.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_len.max().item()) if self.batch else 0


def prefill_case(spec: LayerSpec, seq_lens: Sequence[int], seed: int,
                 gaps: Optional[Sequence[int]] = None, device: str = "cpu") -> PrefillCase:
    """Draw order: q, k, then v (omitted when K=V), then the q and k norm weights.

    gaps[b] padding rows are placed before sequence b (and gaps[B] after the last one).
    """
    seq_lens = [int(x) for x in seq_lens]
    B = len(seq_lens)
    if gaps is None:
        gaps = [0] * (B + 1)
    gaps = [int(x) for x in gaps]
    assert len(gaps) == B + 1
    starts: List[int] = []
    t = 0
    for b in range(B):
        t += gaps[b]
        starts.append(t)
        t += seq_lens[b]
    T = t + gaps[B]
    g = make_generator(seed, device)
    H, Hk, D = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    q = bf16_normal(g, (T, H, D), device=device)
    k = bf16_normal(g, (T, Hk, D), device=device)
    v = None if spec.k_eq_v else bf16_normal(g, (T, Hk, D), device=device)
    wq = bf16_normal(g, (D,), 1.0, 0.1, device=device)
    wk = bf16_normal(g, (D,), 1.0, 0.1, device=device)
    pos = np.zeros(T, dtype=np.int32)
    for b in range(B):
        pos[starts[b]:starts[b] + seq_lens[b]] = np.arange(seq_lens[b], dtype=np.int32)
    return PrefillCase(
        spec, q, k, v, wq, wk,
        torch.from_numpy(pos).to(device),
        torch.tensor(starts, dtype=torch.int32, device=device),
        torch.tensor(seq_lens, dtype=torch.int32, device=device),
    )


def decode_ctx_lens(batch: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Context lengths uniform over the integers [lo, hi] (numpy PCG64)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi + 1, size=batch).astype(np.int32)


def log_uniform_lens(n: int, lo: int, hi: int, total: int, seed: int) -> np.ndarray:
    """n lengths log-uniform in [lo, hi]; if their sum exceeds `total`, all are scaled
    by total / sum, floored and clamped to >= lo (the pack then leaves the remainder
    as padding)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = np.exp(rng.uniform(np.log(lo), np.log(hi), size=n))
    lens = np.floor(x).astype(np.int64)
    lens = np.clip(lens, lo, hi)
    s = int(lens.sum())
    if s > total:
        lens = np.maximum(np.floor(lens * (total / s)).astype(np.int64), lo)
        while int(lens.sum()) > total:  # clamping can overshoot by a few rows
            lens[int(np.argmax(lens))] -= 1
    return lens.astype(np.int32)


def random_gaps(n_seqs: int, max_gap: int, seed: int) -> List[int]:
    rng = np.random.Generator(np.random.PCG64(seed))
    return [int(x) for x in rng.integers(0, max_gap + 1, size=n_seqs + 1)]


def image_last_keys(seq_start, seq_len, images, num_tokens: int) -> torch.Tensor:
    """int32 [num_tokens] per-row last keys for sequences that carry images: -1 on text and
    padding rows, and on the rows of an image the position of that image's last row.
    images: per sequence, a list of (first position, number of rows), inside the sequence
    and not overlapping."""
    lk = np.full(num_tokens, -1, np.int32)
    for s0, L, imgs in zip(np.asarray(seq_start).tolist(), np.asarray(seq_len).tolist(), images):
        for a, n in imgs:
            assert 0 <= a and n >= 1 and a + n <= L, (a, n, L)
            lk[s0 + a:s0 + a + n] = a + n - 1
    return torch.from_numpy(lk)


def image_spans(seq_lens: Sequence[int], rows_per_image: int, images_per_seq: int, seed: int) -> List[List[tuple]]:
    """Seeded, non-overlapping image placements: images_per_seq images of rows_per_image
    rows in each sequence, each starting at a position drawn uniformly among the free
    stretches (a stand-in for image soft tokens inside a prompt)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for L in seq_lens:
        n = min(images_per_seq, L // rows_per_image)
        text = L - n * rows_per_image  # text rows to spread around the images
        cuts = np.sort(rng.integers(0, text + 1, size=n))
        out.append([(c + i * rows_per_image, rows_per_image) for i, c in enumerate(cuts.tolist())])
    return out


@dataclasses.dataclass
class DecodeCase:
    """Raw inputs of a decode step: one new token per sequence against a KV cache.

    ctx[b] = L_b counts the new token (position L_b - 1). The cache of sequence b holds
    the keys of positions lo_b .. L_b - 1 (lo_b = max(0, L_b - window) for a sliding ring,
    0 for a linear cache); key position p lives in cache row row0[b] + p % slots. The
    raw (pre-prologue) rows of those keys are k_raw (and v_raw) in sequence order, with
    their positions in `positions` and their cache rows in `dst_row`; the new tokens' raw
    queries are q_raw [B, Hq, D] at positions ctx - 1.
    """

    spec: LayerSpec
    ctx: np.ndarray       # int32 [B]
    slots: int            # ring size (sliding) or per-sequence region (global): position p at p % slots
    row0: np.ndarray      # int64 [B] first cache row of each sequence's region
    cache_rows: int       # rows of the whole cache
    key_start: np.ndarray  # int64 [B] first k_raw row of each sequence
    key_lo: np.ndarray    # int64 [B] position of each sequence's first cached key
    q_raw: torch.Tensor   # bf16 [B, Hq, D]
    k_raw: torch.Tensor   # bf16 [N, Hkv, D]
    v_raw: Optional[torch.Tensor]
    wq: torch.Tensor
    wk: torch.Tensor
    positions: torch.Tensor  # int32 [N]
    dst_row: torch.Tensor    # int64 [N]


def decode_case(spec: LayerSpec, batch: int, lo: int, hi: int, seed: int, device: str = "cpu") -> DecodeCase:
    """Context lengths uniform over [lo, hi] (numpy PCG64, `seed`); then, from torch's
    generator seeded with `seed`: q (the new tokens), k of every cached position (and v for
    separate K and V), then the q and k norm weights. Sliding layers keep a ring of
    `window` slots per sequence (the last `window` positions), global layers a linear
    region as long as the sequence."""
    ctx = decode_ctx_lens(batch, lo, hi, seed)
    W_ = spec.window
    if W_ > 0:
        slots = W_
        region = [slots] * batch
        key_lo = np.array([max(0, int(L) - W_) for L in ctx], np.int64)
    else:
        slots = int(ctx.max())
        region = [int(L) for L in ctx]
        key_lo = np.zeros(batch, np.int64)
    row0 = np.concatenate([[0], np.cumsum(region)[:-1]]).astype(np.int64)
    nkeys = ctx.astype(np.int64) - key_lo
    key_start = np.concatenate([[0], np.cumsum(nkeys)[:-1]]).astype(np.int64)
    N = int(nkeys.sum())
    pos = np.concatenate([np.arange(a, L, dtype=np.int64) for a, L in zip(key_lo.tolist(), ctx.tolist())])
    seq = np.repeat(np.arange(batch), nkeys)
    dst = row0[seq] + pos % slots
    g = make_generator(seed, device)
    H, Hk, D = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    q = bf16_normal(g, (batch, H, D), device=device)
    k = bf16_normal(g, (N, Hk, D), device=device)
    v = None if spec.k_eq_v else bf16_normal(g, (N, Hk, D), device=device)
    wq = bf16_normal(g, (D,), 1.0, 0.1, device=device)
    wk = bf16_normal(g, (D,), 1.0, 0.1, device=device)
    return DecodeCase(spec, ctx, slots, row0, int(sum(region)), key_start, key_lo, q, k, v, wq, wk,
                      torch.from_numpy(pos.astype(np.int32)).to(device), torch.from_numpy(dst).to(device))
