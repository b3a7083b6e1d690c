"""Shared plumbing for the GPU tests: running the library on synthetic cases and
comparing with the oracle. Not collected as tests."""
from __future__ import annotations

import numpy as np
import torch

import global_gqa_attention_amd as g
import workloads as W
from oracle.bf16 import bf16_bits_to_f64

DEV = "cuda"
MAX_ABS = 1.5e-2  # tolerance of the GPU bf16 output against the float64 oracle
MEAN_ABS = 2e-3


def to_dev(t):
    return None if t is None else t.to(DEV)


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a bf16 tensor."""
    return bf16_bits_to_f64(W.bits(t.cpu()))


def covered_rows(case: W.PrefillCase) -> np.ndarray:
    return np.concatenate([np.arange(s, s + L) for s, L in zip(case.seq_start.tolist(), case.seq_len.tolist())])


def assert_close(got: np.ndarray, ref: np.ndarray, what: str = "") -> tuple:
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{what}: max |err| {mx:.3e} (<= {MAX_ABS}), mean {mean:.3e} (<= {MEAN_ABS})"
    return mx, mean


def assert_close_peaked(got: np.ndarray, ref: np.ndarray, vmax: float, what: str = "") -> None:
    """Tolerance for queries scaled far beyond N(0,1). Sharp rows put most weight on one
    value row, so outputs reach a few units, where a bf16 ulp is 2^-6 .. 2^-5. On top of
    the N(0,1) bound this allows the two bf16 roundings of the arithmetic, each at most
    2^-8 relative: of P (an error of at most 2^-8 max|v| in the weighted mean) and of the
    output (at most 2^-8 |out|)."""
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    bound = MAX_ABS + 2.0 ** -8 * (np.abs(ref) + vmax)
    assert np.all(err <= bound), f"{what}: max excess over the bound {(err - bound).max():.3e}"
    assert err.mean() <= MEAN_ABS, f"{what}: mean |err| {err.mean():.3e} (<= {MEAN_ABS})"


def prefill(spec, q, k, v, seq_start, seq_len, max_len=None, sentinel=0x7FC0):
    """Run g4attn_prefill on device tensors; padding rows of `out` keep `sentinel`."""
    layer = g.make_layer(spec)
    out = torch.full(q.shape, sentinel, dtype=torch.int16, device=DEV).view(torch.bfloat16) if sentinel is not None \
        else torch.empty_like(q)
    if max_len is None:
        max_len = int(seq_len.max().item()) if seq_len.numel() else 0
    prov = g.g4attn_prefill(layer, q, k, None if spec.k_eq_v else v, out, seq_start, seq_len, max_len,
                            provenance=True)
    return out, prov


def prologue(spec, case: W.PrefillCase):
    """In-place prologue of case.q and case.k on the device; returns (q, k, v) device tensors."""
    layer = g.make_layer(spec)
    q, k, v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
    g.g4attn_qk_prologue(layer, q, q, k, k, to_dev(case.wq), to_dev(case.wk), to_dev(case.positions))
    return q, k, v


def bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))
