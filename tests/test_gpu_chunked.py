"""Chunked prefill against the KV cache (g4attn_prefill_cached) on the GPU: a sequence
prefilled chunk by chunk through the prologue's cache scatter gives, row for row, the
same bits as the whole-sequence prefill (the key blocks are aligned to position 0
whatever the chunking), and matches the float64 oracle. Sliding layers use a ring of
window + 512 slots, global layers a linear K=V cache whose slots past the keys hold NaN
(never read)."""
import numpy as np
import pytest
import torch

import global_gqa_attention_amd as g
import workloads as W
from gpu_helpers import DEV, assert_close, bits_equal, f64, prefill, to_dev
from oracle.attention import attention

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


def _chunked(spec, case, chunks, seqs_per_call=1, last_key=None, split_keys=0):
    """Prologue + g4attn_prefill_cached over `chunks` (lengths summing to each sequence's
    length; every sequence of the case is cut the same way where it is long enough), or
    g4attn_prefill_cached_masked with the chunk rows' entries of `last_key` (int32 [T]), or
    with split_keys > 0 g4attn_prefill_cached_split (a NaN-filled workspace per call).
    Returns the output rows of every sequence in packed order and the post-prologue
    (q, k) of the whole pack (for the unchunked reference)."""
    layer = g.make_layer(spec)
    B = case.seq_len.numel()
    lens = case.seq_len.tolist()
    starts = case.seq_start.tolist()
    H, Hk, D = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    if spec.window > 0:
        slots = -(-(spec.window + 512) // 32) * 32  # window + the longest chunk, a multiple of 32
        fill = 0  # a ring region starts zero-filled (finite in every slot)
    else:
        slots = -(-max(lens) // 32) * 32 + 64
        fill = NAN_BF16  # slots past the keys are never read
    kc = torch.full((B * slots, Hk, D), fill, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    vc = None if spec.k_eq_v else torch.full_like(kc.view(torch.int16), fill).view(torch.bfloat16)
    row0 = torch.arange(B, dtype=torch.int64, device=DEV) * slots
    q_in, k_in = to_dev(case.q), to_dev(case.k)
    v_in = to_dev(case.v) if case.v is not None else None
    wq, wk = to_dev(case.wq), to_dev(case.wk)
    out = torch.full(q_in.shape, NAN_BF16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    qpost = torch.empty_like(q_in)
    kpost = torch.empty_like(k_in)
    P = [0] * B
    while any(P[b] < lens[b] for b in range(B)):
        for c in chunks:
            act = [b for b in range(B) if P[b] < lens[b]]
            if not act:
                break
            for i in range(0, len(act), seqs_per_call):
                grp = act[i:i + seqs_per_call]
                cl = [min(c, lens[b] - P[b]) for b in grp]
                # the chunk's rows, gathered into a packed chunk batch
                rows = torch.cat([torch.arange(starts[b] + P[b], starts[b] + P[b] + n, device=DEV)
                                  for b, n in zip(grp, cl)])
                pos = torch.cat([torch.arange(P[b], P[b] + n, dtype=torch.int32, device=DEV)
                                 for b, n in zip(grp, cl)])
                dst = torch.cat([row0[b] + torch.arange(P[b], P[b] + n, device=DEV) % slots
                                 for b, n in zip(grp, cl)]).to(torch.int64)
                qc = torch.empty((len(rows), H, D), dtype=torch.bfloat16, device=DEV)
                g.g4attn_qk_prologue(layer, q_in[rows].contiguous(), qc, k_in[rows].contiguous(), kc, wq, wk, pos,
                                     v_in=v_in[rows].contiguous() if v_in is not None else None, v_out=vc,
                                     kv_dst_row=dst)
                oc = torch.full_like(qc.view(torch.int16), NAN_BF16).view(torch.bfloat16)
                qr = torch.tensor(np.concatenate([[0], np.cumsum(cl)[:-1]]), dtype=torch.int32, device=DEV)
                qp = torch.tensor([P[b] for b in grp], dtype=torch.int32, device=DEV)
                clt = torch.tensor(cl, dtype=torch.int32, device=DEV)
                r0 = row0[grp].contiguous()
                maxkey = max(P[b] + n for b, n in zip(grp, cl))
                if split_keys:
                    nb = g.g4attn_split_workspace_bytes(layer, len(grp), max(cl), maxkey, split_keys)
                    ws = torch.full((nb // 4,), float("nan"), dtype=torch.float32, device=DEV) if nb else None
                    g.g4attn_prefill_cached_split(layer, qc, kc, vc, oc, qr, qp, clt, r0, slots, max(cl), maxkey,
                                                  split_keys, ws)
                elif last_key is None:
                    g.g4attn_prefill_cached(layer, qc, kc, vc, oc, qr, qp, clt, r0, slots, max(cl), maxkey)
                else:
                    g.g4attn_prefill_cached_masked(layer, qc, kc, vc, oc, qr, qp, clt, to_dev(last_key)[rows].contiguous(),
                                                   r0, slots, max(cl), max(P[b] + n for b, n in zip(grp, cl)))
                out[rows] = oc
                qpost[rows] = qc
                for b, n in zip(grp, cl):
                    P[b] += n
    # the unchunked reference reads k after the prologue: run it on the whole pack
    g.g4attn_qk_prologue(layer, q_in, qpost, k_in, kpost, wq, wk, to_dev(case.positions))
    return out, qpost, kpost


CASES = [
    # name, spec, lengths, chunk pattern (repeated), sequences per call, seed
    ("31b-sliding-512", W.SLIDING_31B, [1800], [512], 1, 41),
    ("31b-sliding-ragged", W.SLIDING_31B, [1300, 2100], [300, 512, 77, 1], 2, 42),
    ("31b-global-512", W.GLOBAL_31B, [1200], [512], 1, 43),
    ("31b-global-ragged", W.GLOBAL_31B, [700, 1100], [129, 512, 33], 2, 44),
    ("tiny-sliding-chunks", W.TINY_SLIDING, [64, 130], [16, 5, 1], 2, 45),
    ("tiny-global-g8-chunks", W.TINY_GLOBAL_G8, [100, 33], [32, 7], 2, 46),
]


@pytest.mark.parametrize("name,spec,lens,chunks,per_call,seed", CASES, ids=[c[0] for c in CASES])
def test_chunked_prefill_equals_whole_prefill_and_oracle(name, spec, lens, chunks, per_call, seed):
    case = W.prefill_case(spec, lens, seed)
    out_c, qpost, kpost = _chunked(spec, case, chunks, per_call)
    torch.cuda.synchronize()
    v = to_dev(case.v) if case.v is not None else None
    out_w, _ = prefill(spec, qpost, kpost, v, to_dev(case.seq_start), to_dev(case.seq_len))
    torch.cuda.synchronize()
    assert bits_equal(out_c, out_w), f"{name}: chunked rows differ from the whole-sequence prefill"
    vv = kpost if spec.k_eq_v else v
    ref = attention(f64(qpost), f64(kpost), f64(vv), case.seq_start.numpy(), case.seq_len.numpy(),
                    spec.num_kv_heads, spec.window, spec.softmax_scale)
    assert_close(f64(out_c), ref, name)


def _boundaries(L, chunks):
    """Chunk start positions of a sequence of length L cut by the repeated pattern."""
    cuts, p = [], 0
    while p < L:
        for c in chunks:
            if p >= L:
                break
            cuts.append(p)
            p += min(c, L - p)
    return cuts + [L]


IMAGE_CASES = [
    # name, spec, lengths, chunk pattern, sequences per call, images per sequence, seed
    ("31b-sliding-512", W.SLIDING_31B, [1800], [512], 1, [[(100, 256), (600, 280), (1600, 150)]], 51),
    ("31b-global-512", W.GLOBAL_31B, [1200], [512], 1, [[(0, 256), (700, 256)]], 52),
    ("tiny-sliding-chunks", W.TINY_SLIDING, [64, 130], [16, 5, 1], 2, [[(22, 16), (44, 16)], [(66, 16), (88, 16)]], 53),
]


@pytest.mark.parametrize("name,spec,lens,chunks,per_call,images,seed", IMAGE_CASES, ids=[c[0] for c in IMAGE_CASES])
def test_chunked_prefill_with_images_equals_whole_masked_prefill(name, spec, lens, chunks, per_call, images, seed):
    """Images that no chunk cuts (TensorFold PR #1186, vision commit): the chunk rows carry
    the bits of g4attn_prefill_masked over the whole sequence, and match the oracle."""
    for L, imgs in zip(lens, images):
        cuts = _boundaries(L, chunks)
        for a, n in imgs:
            assert all(not (a < c < a + n) for c in cuts), f"image {(a, n)} crosses a chunk boundary"
    case = W.prefill_case(spec, lens, seed)
    lk = W.image_last_keys(case.seq_start, case.seq_len, images, case.num_tokens)
    out_c, qpost, kpost = _chunked(spec, case, chunks, per_call, last_key=lk)
    torch.cuda.synchronize()
    v = to_dev(case.v) if case.v is not None else None
    layer = g.make_layer(spec)
    out_w = torch.full(qpost.shape, NAN_BF16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    g.g4attn_prefill_masked(layer, qpost, kpost, None if spec.k_eq_v else v, out_w, to_dev(case.seq_start),
                            to_dev(case.seq_len), to_dev(lk), max(lens))
    torch.cuda.synchronize()
    assert bits_equal(out_c, out_w), f"{name}: chunked rows differ from the whole-sequence masked prefill"
    vv = kpost if spec.k_eq_v else v
    ref = attention(f64(qpost), f64(kpost), f64(vv), case.seq_start.numpy(), case.seq_len.numpy(),
                    spec.num_kv_heads, spec.window, spec.softmax_scale, last_key=lk.numpy())
    assert_close(f64(out_c), ref, name)
