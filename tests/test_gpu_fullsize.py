"""Parity at the benchmark's full sizes, in the launch configuration bench.py times:
the sliding-layer step (2 x 4096, prologue + attention), the global-layer 8k prefill
and the 64-sequence decode on both layer types, on the benchmark's own seeded inputs.
The oracle computes sampled tokens one by one (all heads of a token: the token's row
against the keys it sees, oracle.attention.decode_rows) and sampled prologue rows.
The batch-invariance stress packs 24 log-uniform sequences into 65536 tokens and
checks every sequence's rows bit for bit alone, packed and padded, on both layers."""
import numpy as np
import pytest
import torch

import global_gqa_attention_amd as g
import workloads as W
from gpu_helpers import DEV, MAX_ABS, MEAN_ABS, bits_equal, f64, prefill
from oracle.attention import decode_rows
from oracle.prologue import qk_prologue
from test_gpu_prologue import check_bits, magnitude

pytestmark = pytest.mark.gpu


def sample_positions(L, window, seed, n=12):
    """Edges of the 32-key blocks and of the window, the ends, and seeded random ones."""
    fixed = [0, 1, 31, 32, 33, L // 2, L - 2, L - 1]
    if window > 0:
        fixed += [window - 1, window, window + 1]
    rng = np.random.Generator(np.random.PCG64(seed))
    extra = rng.integers(0, L, size=n).tolist()
    return sorted({p for p in fixed + extra if 0 <= p < L})


def oracle_token_rows(spec, q, k, v, s0, positions):
    """The oracle's output rows of the given positions of the sequence starting at row s0."""
    W_ = spec.window
    out = []
    for P in positions:
        lo = max(0, P - W_ + 1) if W_ > 0 else 0
        keys = f64(k[s0 + lo:s0 + P + 1])
        vals = keys if spec.k_eq_v else f64(v[s0 + lo:s0 + P + 1])
        out.append(decode_rows(f64(q[s0 + P:s0 + P + 1]), [keys], [vals], [lo], [P + 1], W_, spec.softmax_scale)[0])
    return np.stack(out)


def check_rows(got, ref, what):
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), what
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, f"{what}: max {err.max():.3e} mean {err.mean():.3e}"


@pytest.mark.parametrize("which", ["sliding-2x4096", "global-1x8192"])
def test_full_size_prefill_sampled_against_oracle(which):
    if which.startswith("sliding"):
        spec, lens, seed, maxlen = W.SLIDING_31B, [4096, 4096], 1, 4096
    else:
        spec, lens, seed, maxlen = W.GLOBAL_31B, [8192], 2, 8192
    case = W.prefill_case(spec, lens, seed=seed, device=DEV)  # the benchmark's inputs
    layer = g.make_layer(spec)
    q, k = torch.empty_like(case.q), torch.empty_like(case.k)
    g.g4attn_qk_prologue(layer, case.q, q, case.k, k, case.wq, case.wk, case.positions)
    out, prov = prefill(spec, q, k, case.v, case.seq_start, case.seq_len, maxlen)
    torch.cuda.synchronize()
    assert prov["block_q"] == (128 if spec.head_dim >= 512 else 256)  # the benchmark's (wide) launch form
    kw = dict(rope_dims=spec.rope_dims, rope_freq_dim=spec.rope_freq_dim, theta=spec.rope_theta, eps=spec.rms_eps)
    for b, (s0, L) in enumerate(zip(case.seq_start.tolist(), lens)):
        pos = sample_positions(L, spec.window, seed * 100 + b)
        ref = oracle_token_rows(spec, q, k, case.v, s0, pos)
        got = np.stack([f64(out[s0 + P]) for P in pos])
        check_rows(got, ref, f"{which} seq {b}")
        # prologue of the same tokens (q and k rows) against the oracle's prologue
        rows = [s0 + P for P in pos]
        p_np = np.array(pos, dtype=np.int32)
        for x_raw, x_gpu, w in ((case.q, q, case.wq), (case.k, k, case.wk)):
            xb, wb = W.bits(x_raw[rows].cpu()), W.bits(w.cpu())
            exact, _ = qk_prologue(xb, wb, p_np, **kw)
            mag = magnitude(xb, wb, spec.rms_eps, spec.rope_dims, spec.rope_dims // 2)
            check_bits(W.bits(x_gpu[rows].cpu()), exact, mag, f"{which} prologue seq {b}")


@pytest.mark.parametrize("spec", [W.SLIDING_31B, W.GLOBAL_31B], ids=["sliding", "global"])
def test_full_size_decode_against_oracle(spec):
    """The benchmark's decode workload as bench.py builds and launches it: 64 sequences,
    context lengths uniform in [1024, 32768] (seed 3), caches filled by the prologue's
    scatter at the keys' true positions, longest-first schedule. Every one of the 64
    decode rows against the oracle's attention over the cached keys (the prologue's
    output), three sequences end to end from the raw rows through the oracle's own
    prologue, and sampled cache rows against the oracle's prologue."""
    import bench
    from oracle.bf16 import bf16_bits_to_f64

    case = W.decode_case(spec, 64, 1024, 32768, seed=3, device=DEV)
    order = np.argsort(-case.ctx, kind="stable").astype(np.int32)
    qd, kc, vc = bench.fill_decode_cache(torch, g, case)
    od = torch.empty_like(qd)
    g.g4attn_decode(g.make_layer(spec), qd, kc, vc, torch.from_numpy(case.row0).to(DEV),
                    torch.from_numpy(case.ctx).to(DEV), case.slots, od, int(case.ctx.max()),
                    schedule=torch.from_numpy(order).to(DEV))
    torch.cuda.synchronize()
    got = f64(od)
    assert np.all(np.isfinite(got))
    kw = dict(rope_dims=spec.rope_dims, rope_freq_dim=spec.rope_freq_dim, theta=spec.rope_theta, eps=spec.rms_eps)
    qf = f64(qd)
    errs = []
    for b in range(64):
        lo, L = int(case.key_lo[b]), int(case.ctx[b])
        rows = torch.from_numpy(case.row0[b] + np.arange(lo, L) % case.slots).to(DEV)
        keys = f64(kc[rows])
        vals = keys if spec.k_eq_v else f64(vc[rows])
        ref = decode_rows(qf[b:b + 1], [keys], [vals], [lo], [L], spec.window, spec.softmax_scale)
        errs.append(np.abs(got[b:b + 1] - ref))
        del keys, vals
    err = np.concatenate(errs)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, f"attention: max {err.max():.3e} mean {err.mean():.3e}"
    for b in sorted({int(order[0]), int(order[-1]), 7}):
        lo, L = int(case.key_lo[b]), int(case.ctx[b])
        a = int(case.key_start[b])
        _, q1 = qk_prologue(W.bits(case.q_raw[b:b + 1].cpu()), W.bits(case.wq.cpu()), np.array([L - 1]), **kw)
        kraw = W.bits(case.k_raw[a:a + L - lo].cpu())
        exact, k1 = qk_prologue(kraw, W.bits(case.wk.cpu()), np.arange(lo, L), **kw)
        keys = bf16_bits_to_f64(k1)
        vals = keys if spec.k_eq_v else f64(case.v_raw[a:a + L - lo])
        ref = decode_rows(bf16_bits_to_f64(q1), [keys], [vals], [lo], [L], spec.window, spec.softmax_scale)
        check_rows(got[b:b + 1], ref, f"end to end, seq {b} (L={L})")
        # the prologue's cache rows of this sequence (a sample of positions)
        pick = np.unique(np.r_[0, L - lo - 1, np.linspace(0, L - lo - 1, 40).astype(np.int64)])
        rows = torch.from_numpy(case.row0[b] + (lo + pick) % case.slots).to(DEV)
        mag = magnitude(kraw[pick], W.bits(case.wk.cpu()), spec.rms_eps, spec.rope_dims, spec.rope_dims // 2)
        check_bits(W.bits(kc[rows].cpu()), exact[pick], mag, f"cache rows, seq {b}")
    print(f"decode {spec.name}: 64 rows max {err.max():.2e} mean {err.mean():.2e}")


@pytest.mark.parametrize("spec", [W.SLIDING_31B, W.GLOBAL_31B], ids=["sliding", "global"])
def test_stress_65536_alone_packed_padded_bitwise(spec):
    """24 sequences, lengths log-uniform in [128, 16384] fitted to 65536 tokens (seed 4);
    each sequence's rows alone, in the pack, and in a pack with N(0,1) padding between
    sequences are the same bits."""
    lens = W.log_uniform_lens(24, 128, 16384, 65536, seed=4).tolist()
    tail = 65536 - sum(lens)
    packed = W.prefill_case(spec, lens, seed=4, gaps=[0] * len(lens) + [tail], device=DEV)
    v = packed.v
    out_p, _ = prefill(spec, packed.q, packed.k, v, packed.seq_start, packed.seq_len)
    gaps = W.random_gaps(len(lens), 96, seed=5)
    gen = W.make_generator(6, DEV)
    qs, ks, vs, starts = [], [], [], []
    t = 0
    for b, (s0, L) in enumerate(zip(packed.seq_start.tolist(), lens)):
        H, Hk, D = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
        qs += [W.bf16_normal(gen, (gaps[b], H, D), device=DEV), packed.q[s0:s0 + L]]
        ks += [W.bf16_normal(gen, (gaps[b], Hk, D), device=DEV), packed.k[s0:s0 + L]]
        if v is not None:
            vs += [W.bf16_normal(gen, (gaps[b], Hk, D), device=DEV), v[s0:s0 + L]]
        starts.append(t + gaps[b])
        t += gaps[b] + L
    Qp, Kp = torch.cat(qs), torch.cat(ks)
    Vp = torch.cat(vs) if vs else None
    out_g, _ = prefill(spec, Qp, Kp, Vp, torch.tensor(starts, dtype=torch.int32, device=DEV), packed.seq_len)
    for b, (s0, L) in enumerate(zip(packed.seq_start.tolist(), lens)):
        one = torch.tensor([0], dtype=torch.int32, device=DEV)
        ln = torch.tensor([L], dtype=torch.int32, device=DEV)
        out_a, _ = prefill(spec, packed.q[s0:s0 + L].contiguous(), packed.k[s0:s0 + L].contiguous(),
                           v[s0:s0 + L].contiguous() if v is not None else None, one, ln)
        assert bits_equal(out_a, out_p[s0:s0 + L]), f"seq {b} (L={L}): alone != packed"
        assert bits_equal(out_g[starts[b]:starts[b] + L], out_p[s0:s0 + L]), f"seq {b} (L={L}): padded != packed"
    torch.cuda.synchronize()


def test_full_size_images_against_oracle():
    """The benchmark's image measurement at its own size and launch: the sliding step's
    inputs (2 x 4096, seed 1) through the prologue, four 256-row images per sequence (seed
    5), g4attn_prefill_masked; every output row against the oracle with the same last
    keys (float64 over the whole step, a few seconds), and the text rows bit for bit
    against g4attn_prefill."""
    from oracle.attention import attention

    spec = W.SLIDING_31B
    lens = [4096, 4096]
    case = W.prefill_case(spec, lens, seed=1, device=DEV)
    images = W.image_spans(lens, 256, 4, seed=5)
    lk = W.image_last_keys(case.seq_start.cpu(), case.seq_len.cpu(), images, case.num_tokens)
    layer = g.make_layer(spec)
    q, k = torch.empty_like(case.q), torch.empty_like(case.k)
    g.g4attn_qk_prologue(layer, case.q, q, case.k, k, case.wq, case.wk, case.positions)
    out = torch.empty_like(q)
    g.g4attn_prefill_masked(layer, q, k, case.v, out, case.seq_start, case.seq_len, lk.to(DEV), 4096)
    plain, _ = prefill(spec, q, k, case.v, case.seq_start, case.seq_len, 4096)
    torch.cuda.synchronize()
    ref = attention(f64(q), f64(k), f64(case.v), case.seq_start.cpu().numpy(), case.seq_len.cpu().numpy(),
                    spec.num_kv_heads, spec.window, spec.softmax_scale, last_key=lk.numpy())
    err = np.abs(f64(out) - ref)
    assert np.all(np.isfinite(f64(out)))
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (err.max(), err.mean())
    text = torch.from_numpy(np.nonzero(lk.numpy() < 0)[0]).to(DEV)
    assert bits_equal(out[text], plain[text])
    print(f"images full size: max {err.max():.2e} mean {err.mean():.2e}")
