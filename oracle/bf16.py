"""Exact bf16 <-> fp64 conversions for the oracle (test infrastructure).

bf16 is the top half of an IEEE binary32: 1 sign bit, 8 exponent bits, 7
stored mantissa bits.  The pages hold K/V/q in bf16 ("qwen-engine" README,
benchmark table: Qwen3-0.6B bf16; "qvllm" README, Scope: bf16 activations and
KV cache) and round intermediate results back to the input dtype with
``.to(orig_dtype)`` ("nano-vLLM learning note", ``RMSNorm.rms_forward`` and
``apply_rotary_emb`` blocks).

Decoding is exact.  Encoding rounds an fp64 value to the nearest bf16 with
ties to even, in one rounding step (no detour through float32), including
bf16 subnormals and overflow to infinity.
"""

import numpy as np

BF16_NAN_BITS = np.uint16(0x7FC0)
F32_NAN_BITS = np.uint32(0x7FC00000)


def bf16_to_f64(bits):
    """uint16 bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f32_bits_to_f64(bits):
    """uint32 binary32 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x):
    """float64 values -> uint16 bf16 bit patterns, round-to-nearest-even.

    A finite nonzero |x| = m * 2**e with m in [0.5, 1) has unbiased exponent
    E = e - 1.  A bf16 with that exponent is an integer multiple of the
    quantum 2**(E - 7); below the smallest normal exponent (-126) the quantum
    stays 2**-133 (subnormals).  Dividing by a power of two is exact in
    float64, so ``rint`` (ties-to-even) of |x| / quantum is the single
    correctly rounded step.  Results of magnitude 2**128 or more are
    infinite.  NaN maps to the canonical quiet NaN 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    finite = np.isfinite(ax)
    safe = np.where(finite, ax, 0.0)
    _, e = np.frexp(safe)
    exp_unbiased = np.maximum(e.astype(np.int64) - 1, -126)
    quantum = np.ldexp(1.0, (exp_unbiased - 7).astype(np.int32))
    y = np.rint(safe / quantum) * quantum
    y = np.where(finite, y, ax)           # +inf stays +inf, NaN stays NaN
    y = np.where(y >= 2.0 ** 128, np.inf, y)
    with np.errstate(over="ignore", invalid="ignore"):
        y32 = y.astype(np.float32)        # exact: y is a bf16 value (or inf)
    bits = (y32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.signbit(x), bits | np.uint16(0x8000), bits).astype(np.uint16)
    bits = np.where(np.isnan(x), BF16_NAN_BITS, bits).astype(np.uint16)
    return bits


def round_bf16(x):
    """float64 -> nearest bf16 value, returned as float64."""
    return bf16_to_f64(f64_to_bf16(x))


def to_f64(bits, dtype):
    """Raw element bits ('bf16' uint16 / 'f32' uint32) -> float64 values."""
    if dtype == "bf16":
        return bf16_to_f64(bits)
    if dtype == "f32":
        return f32_bits_to_f64(bits)
    raise ValueError(f"unknown dtype {dtype!r}")
