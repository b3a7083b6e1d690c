"""Batch invariance on the GPU: a sequence's output rows are bit-identical whether it
runs alone, packed with unrelated sequences, in another order, or with padding between
sequences, and from run to run (RL-Kernel #415 section 4, rule 6; the acceptance of
RL-Kernel #428 section 4 is exact equality)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import DEV, bits_equal, prefill, to_dev

pytestmark = pytest.mark.gpu


def _run_pack(spec, seqs, order, gaps, seed_pad):
    """seqs: list of (q, k, v) device tensors per sequence; returns per-sequence outputs."""
    gen = W.make_generator(seed_pad, DEV)
    H, Hk, D = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    qs, ks, vs, starts, lens = [], [], [], [], []
    t = 0
    for n, b in enumerate(order):
        q, k, v = seqs[b]
        gq = W.bf16_normal(gen, (gaps[n], H, D), device=DEV)
        gk = W.bf16_normal(gen, (gaps[n], Hk, D), device=DEV)
        qs += [gq, q]
        ks += [gk, k]
        if v is not None:
            vs += [W.bf16_normal(gen, (gaps[n], Hk, D), device=DEV), v]
        starts.append(t + gaps[n])
        lens.append(q.shape[0])
        t += gaps[n] + q.shape[0]
    Q, K = torch.cat(qs), torch.cat(ks)
    V = torch.cat(vs) if vs else None
    out, _ = prefill(spec, Q, K, V, torch.tensor(starts, dtype=torch.int32, device=DEV),
                     torch.tensor(lens, dtype=torch.int32, device=DEV))
    res = {}
    for n, b in enumerate(order):
        res[b] = out[starts[n]:starts[n] + lens[n]].clone()
    return res


@pytest.mark.parametrize("spec,qscale", [(W.TINY_SLIDING, 1.0), (W.TINY_GLOBAL_G8, 1.0), (W.SLIDING_31B, 1.0),
                                         (W.GLOBAL_31B, 1.0), (W.SLIDING_31B, 24.0), (W.GLOBAL_31B, 24.0)],
                         ids=["tiny-sliding", "tiny-global-g8", "31b-sliding", "31b-global", "31b-sliding-peaked",
                              "31b-global-peaked"])
def test_alone_packed_padded_permuted_are_bit_identical(spec, qscale):
    """qscale 24 spreads the scores so that rows rescale O: the rescaling pass of some
    work-groups must give bit-identical rows."""
    lens = [int(x) for x in W.log_uniform_lens(6, 1, 2500 if spec.head_dim >= 256 else 300, 10 ** 9, seed=4)]
    lens[0] = 1
    gen = W.make_generator(99, DEV)
    seqs = []
    for L in lens:
        q = W.bf16_normal(gen, (L, spec.num_q_heads, spec.head_dim), device=DEV, std=qscale)
        k = W.bf16_normal(gen, (L, spec.num_kv_heads, spec.head_dim), device=DEV)
        v = None if spec.k_eq_v else W.bf16_normal(gen, (L, spec.num_kv_heads, spec.head_dim), device=DEV)
        seqs.append((q, k, v))
    B = len(lens)
    alone = {b: _run_pack(spec, seqs, [b], [0], 1)[b] for b in range(B)}
    packed = _run_pack(spec, seqs, list(range(B)), [0] * B, 2)
    rng = np.random.Generator(np.random.PCG64(3))
    order = [int(x) for x in rng.permutation(B)]
    padded = _run_pack(spec, seqs, order, [int(x) for x in rng.integers(0, 97, size=B)], 3)
    again = _run_pack(spec, seqs, order, [int(x) for x in rng.integers(0, 97, size=B)], 4)
    torch.cuda.synchronize()
    for b in range(B):
        assert bits_equal(alone[b], packed[b]), f"seq {b} (L={lens[b]}): alone != packed"
        assert bits_equal(alone[b], padded[b]), f"seq {b} (L={lens[b]}): alone != padded/permuted"
        assert bits_equal(padded[b], again[b]), f"seq {b}: run-to-run difference"
