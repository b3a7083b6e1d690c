"""The benchmark's host-side arithmetic (CPU only): the visible (query, key) pairs that
bench.py credits, against a brute-force count of the oracle's visibility mask, and the
per-launch timing statistics it reports."""
import numpy as np
import pytest

import bench
import workloads as W
from oracle.attention import visible_mask


@pytest.mark.parametrize("L,window", [(1, 0), (17, 0), (100, 16), (100, 100), (100, 150), (1000, 1024), (3000, 1024)])
def test_masked_pairs_equals_mask_count(L, window):
    assert bench.masked_pairs(L, window) == int(visible_mask(L, L, window).sum())


@pytest.mark.parametrize("lens,window,images", [
    ([64, 130], 16, [[(5, 9)], [(0, 20), (40, 7), (100, 30)]]),
    ([200], 0, [[(10, 40), (150, 50)]]),
    ([3000], 1024, [[(100, 256), (2000, 280)]]),
])
def test_image_pairs_equals_mask_count(lens, window, images):
    brute = 0
    for L, imgs in zip(lens, images):
        lk = W.image_last_keys([0], [L], [imgs], L).numpy()
        brute += int(visible_mask(L, L, window, last_key=lk).sum())
    assert bench.image_pairs(np, lens, images, window) == brute


def test_image_pairs_without_images_is_the_causal_count():
    assert bench.image_pairs(np, [4096, 4096], [[], []], 1024) == 2 * bench.masked_pairs(4096, 1024)


def test_bench_image_spans_fit_and_do_not_overlap():
    spans = W.image_spans([4096, 4096], 256, 4, seed=5)
    for L, s in zip([4096, 4096], spans):
        assert len(s) == 4
        ends = [(a, a + n) for a, n in s]
        assert all(ends[i][1] <= ends[i + 1][0] for i in range(len(ends) - 1)) and ends[-1][1] <= L


class _FakeEvent:
    def __init__(self, t):
        self.t = t

    def elapsed_time(self, other):
        return other.t - self.t


def test_kernel_timer_mean_median_min():
    """The benchmark's per-launch statistics: mean (the rates), median and minimum."""
    from bench import KernelTimer
    t = KernelTimer(None)
    for start, dur in [(0.0, 0.30), (1.0, 0.25), (2.0, 0.40), (3.0, 0.27)]:
        t.pairs.append((_FakeEvent(start), _FakeEvent(start + dur)))
    assert abs(t.mean_ms() - 0.305) < 1e-12
    sp = t.spread()
    assert sp["kernel_ms_median"] == round(0.5 * (0.27 + 0.30), 4)
    assert sp["kernel_ms_min"] == 0.25
    t.pairs.pop()
    assert t.spread()["kernel_ms_median"] == 0.3
    assert KernelTimer(None).spread() == {}


@pytest.mark.parametrize("spec", [W.TINY_SLIDING, W.TINY_GLOBAL])
def test_decode_kv_bytes_equals_visible_keys_of_the_oracle_mask(spec):
    """The decode measurement's credited bytes: every key the new token sees (the oracle's
    visibility of the row at position L - 1), per KV head, K and V or the one K=V tensor."""
    case = W.decode_case(spec, 9, 1, 70, seed=12)
    brute = 0
    for L in case.ctx.tolist():
        brute += int(visible_mask(1, L, spec.window, query_pos0=L - 1).sum())
    per_key = spec.num_kv_heads * spec.head_dim * 2 * (1 if spec.k_eq_v else 2)
    assert bench.decode_kv_bytes(spec, case.ctx, case.key_lo) == brute * per_key
    # the case caches exactly those keys
    assert int(case.k_raw.shape[0]) == brute


def test_rerun_estimate_zero_and_one_moved_row():
    """The peaked measurement's estimate: flat scores move no offset; one row whose later
    block jumps far above its first block's maximum makes exactly its work-group re-run."""
    import torch
    spec = W.TINY_GLOBAL_G8  # 16 q heads over 2 KV heads (G = 8), head dim 64
    L, D = 300, spec.head_dim
    q = torch.zeros((L, spec.num_q_heads, D))
    k = torch.zeros((L, spec.num_kv_heads, D))
    assert bench.rerun_fraction(torch, spec, q, k, [L], [0], 0.125, 128) == 0.0
    # row (position 200, head 3 of KV head 0): keys of block 6 (positions 192..223) score 1000 log2 units
    q[200, 3, 0] = 1.0
    k[192:200, 0, 0] = 1000.0 / 0.125 * 0.6931471805599453  # 1000 log2 units after the scale
    groups = 2 * ((L + 15) // 16)  # 128 rows / 8 heads = 16 positions per work-group, 2 KV heads
    assert bench.rerun_fraction(torch, spec, q, k, [L], [0], 0.125, 128) == 1.0 / groups
