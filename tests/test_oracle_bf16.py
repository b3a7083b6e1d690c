"""Pins of the oracle's bf16 codec against the format's definition, the page's printed
case and a library conversion (CPU only)."""
import os

import numpy as np
import torch

from oracle.bf16 import bf16_bits_to_f64, f64_to_bf16_bits

ALL = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
NAN_MASK = ((ALL & 0x7FFF) > 0x7F80)


def test_exhaustive_round_trip():
    """Every non-NaN bf16 value is a fixed point: widen, round, same 16 bits."""
    vals = ALL[~NAN_MASK]
    assert np.array_equal(f64_to_bf16_bits(bf16_bits_to_f64(vals)), vals)


def test_widening_matches_format():
    """Widening follows sign / exponent / fraction from the bit layout directly."""
    b = ALL[~NAN_MASK].astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    f = b & 0x7F
    val = np.where(e == 0, f * 2.0 ** -133, (1 + f / 128.0) * np.power(2.0, (e - 127).astype(np.float64)))
    val = np.where(e == 0xFF, np.inf, val) * sign
    got = bf16_bits_to_f64(b.astype(np.uint16))
    assert np.array_equal(got, val)
    assert np.array_equal(np.signbit(got), np.signbit(val))


def test_midpoints_round_to_even():
    """Exact midpoints of adjacent positive finite values go to the even neighbour;
    a nudge either way goes to the nearer one."""
    lo = np.arange(0x0000, 0x7F7F, dtype=np.uint16)
    hi = (lo + 1).astype(np.uint16)
    a = bf16_bits_to_f64(lo)
    b = bf16_bits_to_f64(hi)
    mid = (a + b) / 2  # exact in float64
    even = np.where(lo % 2 == 0, lo, hi)
    assert np.array_equal(f64_to_bf16_bits(mid), even)
    assert np.array_equal(f64_to_bf16_bits(-mid), even | np.uint16(0x8000))
    eps = (b - a) * 2.0 ** -20
    assert np.array_equal(f64_to_bf16_bits(mid - eps), lo)
    assert np.array_equal(f64_to_bf16_bits(mid + eps), hi)


def test_golden_cases(golden_dir):
    path = os.path.join(golden_dir, "bf16_rounding_cases.txt")
    n = 0
    with open(path) as fh:
        for line in fh:
            if not line.strip() or line.startswith("#"):
                continue
            x_hex, bits_hex = line.split()[:2]
            got = int(f64_to_bf16_bits(np.array([float.fromhex(x_hex)]))[0])
            assert got == int(bits_hex, 16), line
            n += 1
    assert n >= 20


def test_nan():
    assert int(f64_to_bf16_bits(np.array([np.nan]))[0]) == 0x7FC0


def test_matches_library_float32_conversion():
    """For float32-representable inputs direct rounding equals torch's float32 -> bf16
    conversion (round to nearest even), including subnormals and signed zeros."""
    rng = np.random.Generator(np.random.PCG64(123))
    raw = rng.integers(0, 1 << 32, size=400_000, dtype=np.uint64).astype(np.uint32)
    raw = np.concatenate([raw, np.arange(0, 1 << 17, dtype=np.uint32),  # subnormal region
                          np.arange(0x7F7F0000, 0x7F800000, dtype=np.uint32)])  # overflow edge
    f32 = raw.view(np.float32)
    keep = ~np.isnan(f32)
    f32 = f32[keep]
    lib = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f64_to_bf16_bits(f32.astype(np.float64)), lib)


def test_direct_rounding_differs_from_double_rounding():
    """1 + 2^-8 + 2^-40 lies just above a bf16 tie: direct rounding goes up, while
    rounding to float32 first lands on the tie and then rounds to even."""
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert int(f64_to_bf16_bits(np.array([x]))[0]) == 0x3F81
    via32 = torch.tensor([x], dtype=torch.float64).to(torch.float32).to(torch.bfloat16)
    assert int(via32.view(torch.int16).item()) & 0xFFFF == 0x3F80
