"""Pins for the oracle's bf16 rounding (round to nearest, ties to even)."""

from fractions import Fraction

import numpy as np
import torch

from oracle.bf16 import from_bits, round_bf16, to_bits


def _torch_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(x32.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_matches_torch_on_fp32_inputs():
    # torch's float -> bfloat16 conversion is RNE; for fp32 inputs one rounding
    # from fp64 must give the same bits.
    rng = np.random.default_rng(1)
    raw = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = raw.view(np.float32)
    x = x[np.isfinite(x)]
    specials = np.array([0.0, -0.0, 1.0, -1.0, 1e-45, -1e-45, 3.4e38, -3.4e38, 1.0 + 2**-8,
                         1.0 + 3 * 2**-8, 2.0**-126, 2.0**-133, 2.0**-134, 1.5 * 2**-134],
                        dtype=np.float32)
    x = np.concatenate([x, specials])
    assert np.array_equal(to_bits(x.astype(np.float64)), _torch_bits(x))


def _exact_rne_bf16(v: Fraction) -> Fraction:
    """Reference rounding of an exact rational to bf16 (normal range, 8 significant bits)."""
    if v == 0:
        return Fraction(0)
    s = -1 if v < 0 else 1
    a = abs(v)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    scaled = a * 128  # [128, 256)
    q = scaled.numerator // scaled.denominator
    rem = scaled - q
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and q % 2 == 1):
        q += 1
    return s * Fraction(q) * Fraction(2) ** (e - 7)


def test_single_rounding_from_fp64():
    # Values just above a bf16 tie that an fp32 detour would round onto the tie
    # (double rounding) must round up from fp64.
    cases = [1.0 + 2**-8 + 2**-30, 1.0 + 2**-8 - 2**-30, 1.0 + 3 * 2**-8 + 2**-40, -(1.0 + 2**-8 + 2**-31),
             0.1, 1 / 3, 2.0**-100 * (1 + 2**-8 + 2**-35), 12345.678]
    for c in cases:
        want = float(_exact_rne_bf16(Fraction(c)))
        assert round_bf16(np.array([c]))[0] == want, c


def test_overflow_underflow_and_bits_roundtrip():
    big = np.array([3.5e38, -3.5e38, 2.0**128, 3.3895e38])
    r = round_bf16(big)
    assert np.isinf(r[0]) and r[0] > 0 and np.isinf(r[1]) and r[1] < 0 and np.isinf(r[2])
    assert np.isfinite(r[3])  # bf16 max is about 3.3895e38
    assert round_bf16(np.array([2.0**-134]))[0] == 0.0  # exact tie to the even subnormal 0
    assert round_bf16(np.array([1.5 * 2.0**-133]))[0] == 2.0**-132
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = from_bits(allbits)
    fin = np.isfinite(vals)
    assert np.array_equal(to_bits(vals[fin]), allbits[fin])
