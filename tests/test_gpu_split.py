"""GPU tests of the split form (global layers): a row's keys in fixed chunks whose
partial results are merged in ascending order, the same in prefill and decode.

Checked: the split prefill against the oracle (its split form and the plain softmax,
which it equals up to rounding); rows whose keys lie in one chunk equal the plain
prefill bit for bit; every decode row equals the split prefill row of its position bit
for bit (caches hold NaN outside the visible keys, the workspace starts as NaN); a row's
bits do not depend on what else is in the batch; provenance reports the split."""
import dataclasses

import numpy as np
import pytest
import torch

import global_gqa_attention_amd as g
import workloads as W
from gpu_helpers import DEV, assert_close, assert_close_peaked, bits_equal, covered_rows, f64, prefill, to_dev
from oracle.attention import attention, decode_rows
from oracle.split import split_attention
from test_gpu_decode import build_cache

pytestmark = pytest.mark.gpu


def workspace(nbytes: int):
    """A NaN-filled workspace: a partial read before it is written shows up as NaN."""
    if nbytes == 0:
        return None
    return torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=DEV)


def split_prefill(spec, q, k, v, seq_start, seq_len, keys, max_len=None):
    layer = g.make_layer(spec)
    out = torch.full(q.shape, 0x7FC0, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    if max_len is None:
        max_len = int(seq_len.max().item())
    nbytes = g.g4attn_split_workspace_bytes(layer, int(seq_len.shape[0]), max_len, max_len, keys)
    prov = g.g4attn_prefill_split(layer, q, k, None if spec.k_eq_v else v, out, seq_start, seq_len, max_len, keys,
                                  workspace(nbytes), provenance=True)
    return out, prov


def split_decode(spec, qd, kc, vc, row0, ctx, slots, max_ctx, keys, schedule=None):
    layer = g.make_layer(spec)
    out = torch.full(qd.shape, 0x7FC0, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    nbytes = g.g4attn_split_workspace_bytes(layer, int(ctx.shape[0]), 1, max_ctx, keys)
    prov = g.g4attn_decode_split(layer, qd, kc, vc, row0, ctx, slots, out, max_ctx, keys, workspace(nbytes),
                                 schedule=schedule, provenance=True)
    return out, prov


CASES = [
    # name, spec, sequence lengths, chunk size, seed
    ("tiny-global", W.TINY_GLOBAL, [1, 255, 256, 257, 700, 1100], 256, 61),
    ("tiny-global-g8", W.TINY_GLOBAL_G8, [300, 511, 512, 513, 1030], 256, 62),
    ("31b-global", W.GLOBAL_31B, [255, 256, 257, 700, 1300], 256, 63),
    ("31b-global-c512", W.GLOBAL_31B, [1, 511, 512, 513, 1800], 512, 64),
    ("31b-global-v", W.GLOBAL_31B_V, [256, 600, 1025], 256, 65),
    # queries scaled by 24: chunk offsets far apart, and offsets that move inside a chunk
    ("31b-global-peaked", W.GLOBAL_31B, [900, 1300], 256, 66),
]


@pytest.mark.parametrize("name,spec,lens,keys,seed", CASES, ids=[c[0] for c in CASES])
def test_split_prefill_and_decode(name, spec, lens, keys, seed):
    print(f"split {name}: lens={lens} keys={keys}", flush=True)
    case = W.prefill_case(spec, lens, seed, gaps=[3] + [1] * len(lens))
    if name.endswith("peaked"):
        case = dataclasses.replace(case, q=(case.q.float() * 24.0).to(torch.bfloat16))
    q, k, v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
    st, ln = to_dev(case.seq_start), to_dev(case.seq_len)
    out_sp, prov = split_prefill(spec, q, k, v, st, ln, keys)
    out_pf, _ = prefill(spec, q, k, v, st, ln)
    torch.cuda.synchronize()
    assert prov["split_kv"] == keys and prov["kernel_id"].endswith(".split")
    starts = case.seq_start.tolist()
    rows = covered_rows(case)
    # padding rows are not written
    pad = np.setdiff1d(np.arange(case.q.shape[0]), rows)
    assert torch.all(out_sp[torch.as_tensor(pad, device=DEV)].view(torch.int16) == 0x7FC0)
    # positions below the chunk size: one chunk, the plain prefill's bits
    pos = case.positions.numpy()
    one = rows[pos[rows] < keys]
    assert bits_equal(out_sp[torch.as_tensor(one, device=DEV)], out_pf[torch.as_tensor(one, device=DEV)])
    # against the oracle (its split form; the plain softmax on the biggest case)
    vv = case.k if spec.k_eq_v else case.v
    qf, kf, vf = f64(case.q), f64(case.k), f64(vv)
    ref = split_attention(qf, kf, vf, case.seq_start, case.seq_len, spec.num_kv_heads, 0, spec.softmax_scale, keys) \
        if spec.head_dim <= 64 else attention(qf, kf, vf, case.seq_start, case.seq_len, spec.num_kv_heads, 0,
                                              spec.softmax_scale)
    got = f64(out_sp)
    if name.endswith("peaked"):
        assert_close_peaked(got[rows], ref[rows], float(np.abs(vf).max()), name)
    else:
        assert_close(got[rows], ref[rows], name)
    # decode rows at every sequence's last position equal the split prefill rows
    slots = max(lens) + 40
    kc, vc, row0 = build_cache(spec, k, v, starts, lens, slots)
    last = torch.tensor([s + L - 1 for s, L in zip(starts, lens)], device=DEV)
    qd = q[last].contiguous()
    ctx = torch.tensor(lens, dtype=torch.int32, device=DEV)
    sched = torch.tensor(np.argsort(-np.array(lens), kind="stable"), dtype=torch.int32, device=DEV)
    out_dec, dprov = split_decode(spec, qd, kc, vc, row0, ctx, slots, max(lens), keys, schedule=sched)
    torch.cuda.synchronize()
    assert dprov["split_kv"] == keys
    for b in range(len(lens)):
        assert bits_equal(out_dec[b], out_sp[last[b]]), f"{name}: decode row {b} (L={lens[b]}) != split prefill row"


CHUNKED = [
    # name, spec, lengths, prompt-chunk pattern (repeated), sequences per call, key-chunk size, seed
    ("31b-global-512-c256", W.GLOBAL_31B, [1200], [512], 1, 256, 111),
    ("31b-global-ragged-c512", W.GLOBAL_31B, [700, 1100], [129, 512, 33], 2, 512, 112),
    ("31b-global-v-c256", W.GLOBAL_31B_V, [900], [300, 512], 1, 256, 113),
    ("tiny-global-g8-c256", W.TINY_GLOBAL_G8, [600, 333], [100, 7], 2, 256, 114),
]


@pytest.mark.parametrize("name,spec,lens,chunks,per_call,keys,seed", CHUNKED, ids=[c[0] for c in CHUNKED])
def test_split_chunked_prefill_equals_split_prefill(name, spec, lens, chunks, per_call, keys, seed):
    """Prompts prefilled chunk by chunk (prompt chunks that start anywhere, so a work-group's
    rows can straddle a key-chunk boundary) in the split form: every row equals the
    whole-sequence split prefill bit for bit."""
    from test_gpu_chunked import _chunked

    print(f"split chunked {name}", flush=True)
    case = W.prefill_case(spec, lens, seed)
    out_c, qpost, kpost = _chunked(spec, case, chunks, per_call, split_keys=keys)
    torch.cuda.synchronize()
    v = None
    if not spec.k_eq_v:
        # the value-norm layer's V as the prologue left it in the cache: rebuild it whole
        layer = g.make_layer(spec)
        v = torch.empty_like(to_dev(case.v))
        g.g4attn_qk_prologue(layer, None, None, to_dev(case.k), torch.empty_like(kpost), to_dev(case.wq),
                             to_dev(case.wk), to_dev(case.positions), v_in=to_dev(case.v), v_out=v)
    out_w, _ = split_prefill(spec, qpost, kpost, v, to_dev(case.seq_start), to_dev(case.seq_len), keys)
    torch.cuda.synchronize()
    assert bits_equal(out_c, out_w), f"{name}: chunked split rows differ from the whole-sequence split prefill"


def test_split_rows_do_not_depend_on_the_batch():
    """A sequence alone, and packed among others with gaps (a different partial layout
    and grid), gives the same bits."""
    spec, keys = W.GLOBAL_31B, 256
    lens = [700, 40, 1200, 257]
    case = W.prefill_case(spec, lens, 71, gaps=[5, 2, 0, 7, 1])
    q, k = to_dev(case.q), to_dev(case.k)
    out_all, _ = split_prefill(spec, q, k, None, to_dev(case.seq_start), to_dev(case.seq_len), keys)
    for b in (0, 2):
        s0, L = int(case.seq_start[b]), lens[b]
        one = torch.tensor([0], dtype=torch.int32, device=DEV)
        n = torch.tensor([L], dtype=torch.int32, device=DEV)
        out_one, _ = split_prefill(spec, q[s0:s0 + L].contiguous(), k[s0:s0 + L].contiguous(), None, one, n, keys,
                                   max_len=L + 100)
        torch.cuda.synchronize()
        assert bits_equal(out_one, out_all[s0:s0 + L]), f"sequence {b}"


def test_split_decode_against_prefill_at_long_contexts():
    """Context lengths of the decode workload (up to 32768) with 4096-key chunks: the
    decode row equals the split prefill row bit for bit and matches the oracle."""
    spec, keys = W.GLOBAL_31B, 4096
    for i, L in enumerate([8193, 32768]):
        print(f"split long: L={L}", flush=True)
        case = W.prefill_case(spec, [L], 81 + i, device=DEV)
        out_sp, _ = split_prefill(spec, case.q, case.k, None, case.seq_start, case.seq_len, keys)
        kc = case.k.clone()
        qd = case.q[L - 1:L].contiguous()
        ctx = torch.tensor([L], dtype=torch.int32, device=DEV)
        row0 = torch.zeros(1, dtype=torch.int64, device=DEV)
        out_dec, _ = split_decode(spec, qd, kc, None, row0, ctx, L, L, keys)
        torch.cuda.synchronize()
        assert bits_equal(out_dec[0], out_sp[L - 1])
        ref = decode_rows(f64(qd), [f64(case.k)], [f64(case.k)], [0], [L], 0, spec.softmax_scale)
        assert_close(f64(out_dec), ref, f"L={L}")
        del case, out_sp, kc
        torch.cuda.empty_cache()


@pytest.mark.parametrize("keys", [2048, 6144], ids=["c2048", "c6144-bench"])
def test_split_decode_full_size_against_oracle(keys):
    """The global decode workload as bench.py builds it (64 sequences, contexts uniform in
    [1024, 32768], caches filled by the prologue's scatter) in the split form with
    2048-key chunks and with bench.py's 6144: every row against the oracle over the cached
    keys; rows whose keys lie in one chunk equal the plain decode bit for bit."""
    import bench

    spec = W.GLOBAL_31B
    if keys != 2048:
        assert keys == bench.SPLIT_KEYS
    case = W.decode_case(spec, 64, 1024, 32768, seed=3, device=DEV)
    qd, kc, vc = bench.fill_decode_cache(torch, g, case)
    row0 = torch.from_numpy(case.row0).to(DEV)
    ctx = torch.from_numpy(case.ctx).to(DEV)
    order = torch.from_numpy(np.argsort(-case.ctx, kind="stable").astype(np.int32)).to(DEV)
    out, prov = split_decode(spec, qd, kc, vc, row0, ctx, case.slots, int(case.ctx.max()), keys, schedule=order)
    plain = torch.empty_like(qd)
    g.g4attn_decode(g.make_layer(spec), qd, kc, vc, row0, ctx, case.slots, plain, int(case.ctx.max()), schedule=order)
    torch.cuda.synchronize()
    assert prov["split_kv"] == keys
    got, qf = f64(out), f64(qd)
    for b in range(64):
        L = int(case.ctx[b])
        rows = torch.from_numpy(case.row0[b] + np.arange(L)).to(DEV)
        kb = f64(kc[rows])
        ref = decode_rows(qf[b:b + 1], [kb], [kb], [0], [L], 0, spec.softmax_scale)
        assert_close(got[b:b + 1], ref, f"row {b} (L={L})")
        if L <= keys:
            assert bits_equal(out[b], plain[b]), f"row {b} (L={L}): one chunk, not the plain decode's bits"
