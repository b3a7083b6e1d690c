"""The synthetic-input module: geometry against the page's fingerprint table, and
determinism of the seeded draws (CPU only)."""
import os

import numpy as np
import torch

import workloads as W


def _golden(golden_dir):
    out = {}
    with open(os.path.join(golden_dir, "gemma4_31b_attention_geometry.txt")) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                k, v = (x.strip() for x in line.split("=", 1))
                out[k] = v
    return out


def test_31b_geometry_matches_fingerprint(golden_dir):
    g = _golden(golden_dir)
    s, gl = W.SLIDING_31B, W.GLOBAL_31B
    assert s.num_q_heads == gl.num_q_heads == int(g["q_heads"])
    assert (s.num_kv_heads, s.head_dim) == (int(g["sliding_kv_heads"]), int(g["sliding_head_dim"]))
    assert (gl.num_kv_heads, gl.head_dim) == (int(g["global_kv_heads"]), int(g["global_head_dim"]))
    assert s.window == int(g["sliding_window"]) and gl.window == 0
    assert s.rope_theta == float(g["sliding_rope_theta"]) and gl.rope_theta == float(g["global_rope_theta"])
    assert gl.rope_dims == int(float(g["global_rope_partial_factor"]) * gl.head_dim)
    assert s.rope_dims == s.head_dim
    assert gl.k_eq_v and g["global_k_eq_v"] == "true" and not s.k_eq_v
    for spec in W.SPECS.values():
        assert spec.num_q_heads % spec.num_kv_heads == 0
        assert abs(spec.softmax_scale - spec.head_dim ** -0.5) < 1e-15


def test_prefill_case_layout_and_determinism():
    a = W.prefill_case(W.TINY_SLIDING, [5, 9], seed=3, gaps=[1, 2, 3])
    b = W.prefill_case(W.TINY_SLIDING, [5, 9], seed=3, gaps=[1, 2, 3])
    assert a.num_tokens == 1 + 5 + 2 + 9 + 3
    assert a.seq_start.tolist() == [1, 8] and a.seq_len.tolist() == [5, 9]
    assert a.positions[1:6].tolist() == list(range(5)) and a.positions[8:17].tolist() == list(range(9))
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v), (a.wq, b.wq)):
        assert x.dtype == torch.bfloat16 and torch.equal(x.view(torch.int16), y.view(torch.int16))
    c = W.prefill_case(W.TINY_GLOBAL, [7], seed=3)
    assert c.v is None and c.k.shape == (7, 1, 64)
    bits = W.bits(a.q)
    assert bits.dtype == np.uint16 and torch.equal(W.from_bits(bits), a.q)


def test_length_generators():
    L = W.decode_ctx_lens(64, 1024, 32768, seed=3)
    assert L.shape == (64,) and L.min() >= 1024 and L.max() <= 32768
    lens = W.log_uniform_lens(24, 128, 16384, 65536, seed=4)
    assert lens.shape == (24,) and lens.min() >= 128 and lens.sum() <= 65536
    assert np.array_equal(lens, W.log_uniform_lens(24, 128, 16384, 65536, seed=4))
