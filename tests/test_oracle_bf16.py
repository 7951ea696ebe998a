"""Pins for the oracle's bf16 conversions: exhaustive round trip, agreement
with torch's float32 -> bfloat16 rounding (single rounding, ties to even), and
hand-derived tie / overflow / subnormal cases."""

import numpy as np
import torch

from oracle.bf16 import bf16_to_f64, f64_to_bf16


def test_roundtrip_every_bf16_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16_to_f64(bits)
    back = f64_to_bf16(vals)
    nan = np.isnan(vals)
    assert np.array_equal(back[~nan], bits[~nan])
    assert np.all(np.isnan(bf16_to_f64(back[nan])))


def test_decode_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
    mine = bf16_to_f64(bits)
    ok = np.isnan(mine) == np.isnan(t.numpy())
    assert ok.all()
    fin = ~np.isnan(mine)
    assert np.array_equal(mine[fin], t.numpy()[fin])


def test_rounding_matches_torch_from_float32():
    # float32 -> float64 is exact, so one rounding to bf16 must equal torch's
    # round-to-nearest-even float32 -> bfloat16 conversion.
    rng = np.random.default_rng(7)
    parts = [
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(50000) * 1e-39).astype(np.float32),   # subnormal
        np.clip(rng.standard_normal(50000) * 1e38, -3.3e38, 3.3e38).astype(np.float32),  # near overflow
        rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ]
    x = np.concatenate(parts)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mine = f64_to_bf16(x.astype(np.float64))
    assert np.array_equal(mine, ref)


def test_ties_overflow_subnormal_by_hand():
    one = 1.0
    cases = [
        (one, 0x3F80),
        (one + 2.0 ** -8, 0x3F80),  # tie between 1 and 1+2^-7 -> even (1)
        (one + 3 * 2.0 ** -8, 0x3F82),  # tie between 1+2^-7 and 1+2^-6 -> even
        (one + 2.0 ** -8 + 2.0 ** -40, 0x3F81),  # just above the tie -> up
        (-2.5, 0xC020),
        ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),  # largest finite bf16
        (2.0 ** 128 - 2.0 ** 119, 0x7F80),  # tie above max -> even -> inf
        (2.0 ** -133, 0x0001),  # smallest subnormal
        (2.0 ** -134, 0x0000),  # tie -> even (zero)
        (1.5 * 2.0 ** -134, 0x0001),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (float("inf"), 0x7F80),
        (float("-inf"), 0xFF80),
    ]
    for x, want in cases:
        got = int(f64_to_bf16(np.array([x]))[0])
        assert got == want, (x, hex(got), hex(want))
    assert int(f64_to_bf16(np.array([np.nan]))[0]) == 0x7FC0
