"""The benchmark's FLOP counts (CPU only): the visible (query, key) pairs that bench.py
credits, against a brute-force count of the oracle's visibility mask."""
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
