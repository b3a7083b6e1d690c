"""The allocation-free split decode (g4attn_decode_split_noalloc: partial results in the
library's own device array, no workspace argument) against g4attn_decode_split with a
caller workspace: the same bits, on two calls in a row, the second smaller (the array
keeps the first call's partials; none of them may be read)."""
import numpy as np
import pytest
import torch

import global_gqa_attention_amd as g
import workloads as W
from gpu_helpers import DEV, bits_equal
from test_gpu_decode import build_cache

pytestmark = pytest.mark.gpu


def _run(spec, lens, keys, seed):
    case = W.prefill_case(spec, lens, seed, device=DEV)
    starts = case.seq_start.tolist()
    slots = max(lens) + 32
    kc, vc, row0 = build_cache(spec, case.k, case.v, starts, lens, slots)
    last = torch.tensor([s + L - 1 for s, L in zip(starts, lens)], device=DEV)
    qd = case.q[last].contiguous()
    ctx = torch.tensor(lens, dtype=torch.int32, device=DEV)
    layer = g.make_layer(spec)
    nbytes = g.g4attn_split_workspace_bytes(layer, len(lens), 1, max(lens), keys)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=DEV)
    ref = torch.empty_like(qd)
    g.g4attn_decode_split(layer, qd, kc, vc, row0, ctx, slots, ref, max(lens), keys, ws)
    out = torch.full_like(qd, float("nan"))
    prov = g.g4attn_decode_split_noalloc(layer, qd, kc, vc, row0, ctx, slots, out, max(lens), keys, provenance=True)
    torch.cuda.synchronize()
    assert prov["split_kv"] == keys
    return out, ref


def test_decode_split_noalloc_equals_decode_split():
    spec, keys = W.GLOBAL_31B, 4096
    rng = np.random.default_rng(5)
    big = [int(x) for x in rng.integers(4097, 20000, size=12)] + [1, 4096]
    out, ref = _run(spec, big, keys, 101)
    assert bits_equal(out, ref), "first call"
    small = [4097, 9000, 300]
    out, ref = _run(spec, small, keys, 102)
    assert bits_equal(out, ref), "second, smaller call"
