"""GPU prefill with per-row last keys — the rows of an image see every row of that image
(TensorFold PR #1186, the vision commit of the native Gemma 4 engine; RL-Kernel #415
section 5, multimodal_bidirectional_mask) — against the float64 oracle; its text rows
and causal last keys against g4attn_prefill bit for bit; and batch invariance."""
import numpy as np
import pytest
import torch

import global_gqa_attention_amd as g
import workloads as W
from gpu_helpers import DEV, assert_close, bits_equal, covered_rows, f64, prefill, to_dev
from oracle.attention import attention

pytestmark = pytest.mark.gpu

CASES = [
    # name, spec, lengths, gaps, images per sequence (first position, rows), seed
    ("tiny-sliding", W.TINY_SLIDING, [64, 130], [2, 3, 1], [[(5, 9)], [(0, 20), (40, 7), (100, 30)]], 21),
    ("tiny-global", W.TINY_GLOBAL, [200, 63], [1, 0, 2], [[(10, 40), (150, 50)], [(62, 1)]], 22),
    ("tiny-global-g8", W.TINY_GLOBAL_G8, [100], None, [[(30, 33)]], 23),
    ("31b-sliding", W.SLIDING_31B, [1500, 700], [3, 5, 7], [[(100, 256), (1200, 256)], [(0, 256), (444, 256)]], 24),
    ("31b-global", W.GLOBAL_31B, [1100], None, [[(200, 256), (700, 280)]], 25),
]


def masked(spec, q, k, v, seq_start, seq_len, last_key, sentinel=0x7FC0):
    layer = g.make_layer(spec)
    out = torch.full(q.shape, sentinel, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    max_len = int(seq_len.max().item())
    prov = g.g4attn_prefill_masked(layer, q, k, None if spec.k_eq_v else v, out, seq_start, seq_len, last_key,
                                   max_len, provenance=True)
    return out, prov


def _text_rows(case, images):
    rows = []
    for s0, L, imgs in zip(case.seq_start.tolist(), case.seq_len.tolist(), images):
        img = np.zeros(L, bool)
        for a, n in imgs:
            img[a:a + n] = n > 1
        rows.append(s0 + np.nonzero(~img)[0])
    return np.concatenate(rows)


@pytest.mark.parametrize("name,spec,lens,gaps,images,seed", CASES, ids=[c[0] for c in CASES])
def test_masked_prefill_matches_oracle(name, spec, lens, gaps, images, seed):
    case = W.prefill_case(spec, lens, seed, gaps)
    lk = W.image_last_keys(case.seq_start, case.seq_len, images, case.num_tokens)
    q, k, v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
    out, prov = masked(spec, q, k, v, to_dev(case.seq_start), to_dev(case.seq_len), to_dev(lk))
    torch.cuda.synchronize()
    vv = case.k if spec.k_eq_v else case.v
    ref = attention(f64(case.q), f64(case.k), f64(vv), case.seq_start.numpy(), case.seq_len.numpy(),
                    spec.num_kv_heads, spec.window, spec.softmax_scale, last_key=lk.numpy())
    rows = covered_rows(case)
    mx, mean = assert_close(f64(out)[rows], ref[rows], name)
    pad = np.setdiff1d(np.arange(case.num_tokens), rows)
    assert np.all(W.bits(out.cpu())[pad] == 0x7FC0), "padding rows were written"
    assert prov["split_kv"] == 0 and prov["fallback"] == 0
    print(f"{name}: max {mx:.2e} mean {mean:.2e} kernel {prov['kernel_id']}")


@pytest.mark.parametrize("name,spec,lens,gaps,images,seed", CASES, ids=[c[0] for c in CASES])
def test_text_rows_and_causal_last_keys_equal_plain_prefill(name, spec, lens, gaps, images, seed):
    """Rows outside images see exactly the causal keys, so they carry g4attn_prefill's
    bits; last keys at or below every row's position give its whole output."""
    case = W.prefill_case(spec, lens, seed, gaps)
    lk = W.image_last_keys(case.seq_start, case.seq_len, images, case.num_tokens)
    q, k, v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
    st, ln = to_dev(case.seq_start), to_dev(case.seq_len)
    plain, _ = prefill(spec, q, k, v, st, ln)
    with_images, _ = masked(spec, q, k, v, st, ln, to_dev(lk))
    causal = torch.full_like(lk, -1)
    causal[::3] = 0  # at or below the row's own position
    all_causal, _ = masked(spec, q, k, v, st, ln, to_dev(causal))
    torch.cuda.synchronize()
    text = torch.from_numpy(_text_rows(case, images)).to(DEV)
    assert bits_equal(with_images[text], plain[text]), "text rows differ from g4attn_prefill"
    assert bits_equal(all_causal, plain), "causal last keys differ from g4attn_prefill"
    assert not bits_equal(with_images, plain), "the images changed nothing"


@pytest.mark.parametrize("spec,images", [
    (W.TINY_SLIDING, [[(3, 30)], [(0, 9), (50, 14)], [(70, 60)]]),
    (W.SLIDING_31B, [[(30, 256)], [(0, 300)], [(900, 256)]]),
    (W.GLOBAL_31B, [[(10, 256)], [(200, 280)], [(0, 64), (500, 200)]]),
], ids=["tiny-sliding", "31b-sliding", "31b-global"])
def test_images_alone_packed_reordered_are_bit_identical(spec, images):
    lens = [300, 520, 1200] if spec.head_dim > 64 else [40, 80, 130]
    cases = [W.prefill_case(spec, [L], 40 + n) for n, L in enumerate(lens)]
    seqs = [(to_dev(c.q), to_dev(c.k), to_dev(c.v)) for c in cases]
    lks = [W.image_last_keys(c.seq_start, c.seq_len, [imgs], c.num_tokens) for c, imgs in zip(cases, images)]

    def run(order, gaps):
        qs, ks, vs, ls, starts, t = [], [], [], [], [], 0
        H, Hk, D = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
        for n, b in enumerate(order):
            q, k, v = seqs[b]
            qs += [torch.zeros(gaps[n], H, D, dtype=torch.bfloat16, device=DEV), q]
            ks += [torch.zeros(gaps[n], Hk, D, dtype=torch.bfloat16, device=DEV), k]
            if v is not None:
                vs += [torch.zeros(gaps[n], Hk, D, dtype=torch.bfloat16, device=DEV), v]
            ls += [torch.full((gaps[n],), 7, dtype=torch.int32), lks[b]]
            starts.append(t + gaps[n])
            t += gaps[n] + q.shape[0]
        st = torch.tensor(starts, dtype=torch.int32, device=DEV)
        ln = torch.tensor([lens[b] for b in order], dtype=torch.int32, device=DEV)
        out, _ = masked(spec, torch.cat(qs), torch.cat(ks), torch.cat(vs) if vs else None, st, ln,
                        to_dev(torch.cat(ls)))
        return {b: out[starts[n]:starts[n] + lens[b]].clone() for n, b in enumerate(order)}

    alone = {b: run([b], [0])[b] for b in range(3)}
    packed = run([0, 1, 2], [0, 0, 0])
    shuffled = run([2, 0, 1], [5, 33, 1])
    torch.cuda.synchronize()
    for b in range(3):
        assert bits_equal(alone[b], packed[b]), f"sequence {b}: packed differs from alone"
        assert bits_equal(alone[b], shuffled[b]), f"sequence {b}: reordered / padded differs from alone"


@pytest.mark.parametrize("spec,lens,images,seed", [
    (W.TINY_SLIDING, [90, 40], [[(10, 30), (60, 20)], [(0, 17)]], 61),
    (W.SLIDING_31B, [900, 500], [[(100, 256)], [(200, 280)]], 62),
    (W.GLOBAL_31B, [700], [[(64, 256)]], 63),
], ids=["tiny-sliding", "31b-sliding", "31b-global"])
def test_peaked_images_take_the_rescale_path(spec, lens, images, seed):
    """Queries scaled by 24 move the rows' offsets by more than the lazy threshold, so the
    work-groups run the rescaling pass of the last-key kernels: the result still matches the
    oracle (the peaked-input bound), its text rows equal g4attn_prefill's on the same
    inputs bit for bit, and each sequence's rows are the same alone and packed."""
    from gpu_helpers import assert_close_peaked

    case = W.prefill_case(spec, lens, seed)
    q = (case.q.float() * 24.0).to(torch.bfloat16)
    lk = W.image_last_keys(case.seq_start, case.seq_len, images, case.num_tokens)
    st, ln = to_dev(case.seq_start), to_dev(case.seq_len)
    out, _ = masked(spec, to_dev(q), to_dev(case.k), to_dev(case.v), st, ln, to_dev(lk))
    plain, _ = prefill(spec, to_dev(q), to_dev(case.k), to_dev(case.v), st, ln)
    torch.cuda.synchronize()
    vv = case.k if spec.k_eq_v else case.v
    ref = attention(f64(q), f64(case.k), f64(vv), case.seq_start.numpy(), case.seq_len.numpy(),
                    spec.num_kv_heads, spec.window, spec.softmax_scale, last_key=lk.numpy())
    rows = covered_rows(case)
    assert_close_peaked(f64(out)[rows], ref[rows], float(np.abs(f64(vv)).max()), spec.name)
    text = torch.from_numpy(_text_rows(case, images)).to(DEV)
    assert bits_equal(out[text], plain[text]), "text rows differ from g4attn_prefill"
    # the first sequence alone
    s0, L0 = int(case.seq_start[0]), lens[0]
    one = lambda t: None if t is None else to_dev(t)[s0:s0 + L0].contiguous()
    st1 = torch.zeros(1, dtype=torch.int32, device=DEV)
    ln1 = torch.tensor([L0], dtype=torch.int32, device=DEV)
    alone, _ = masked(spec, one(q), one(case.k), one(case.v), st1, ln1, one(lk))
    torch.cuda.synchronize()
    assert bits_equal(alone, out[s0:s0 + L0]), "first sequence alone differs from packed"
