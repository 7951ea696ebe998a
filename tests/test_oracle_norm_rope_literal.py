"""Pin of the oracle's fused norm + RoPE rounding sequence against a literal
transcription of the page's own code, run by torch on the CPU.

"nano-vLLM learning note", RMSNorm.rms_forward block: the row is widened to
float, var = mean(x^2) over the last axis, x is multiplied in place by
rsqrt(var + eps), cast back to the input dtype, and multiplied in place by the
weight (a bf16 tensor times a bf16 tensor, i.e. the exact product rounded to
bf16).  apply_rotary_emb block: the row is widened to float and split into
halves x1, x2; y1 = x1 cos - x2 sin and y2 = x2 cos + x1 sin are formed in
float and the concatenation is cast back to the input dtype.

torch runs those steps in float32, the oracle in float64; both round to bf16
at the same three points.  So the two can disagree only where a value lies
within float32 error of a bf16 rounding boundary:
  * after the normalisation, y = bf16(x r) can come out one bf16 ulp apart
    (at most 2^-7 |y| relative);
  * the weight product is exact before its rounding, so that ulp becomes at
    most 2^-7 |y w| and the rounding of the product can add one more ulp of
    the result: the weighted row differs by at most 2^-6 |y w| per element;
  * the rotation carries a difference d_a, d_b of the two halves into the
    output as |d_a cos| + |d_b sin| <= 2^-6 (|y_a cos| + |y_b sin|), and its
    float32 evaluation (two products and a sum, each rounded) adds at most
    2^-23 (|y_a cos| + |y_b sin|), inside the same term;
  * the final rounding to bf16 adds at most one output ulp.
Bar: every element within one output ulp plus 2^-6 (|y_a cos| + |y_b sin|),
and at least 99.9 % of the elements bit-exact.  Dropping either of the
oracle's bf16 roundings before the rotation (planted below, on the CPU) moves
a large share of the elements and fails the exact-fraction bar.
"""

import numpy as np
import pytest
import torch

from oracle import norm_rope as o_nr
from oracle.bf16 import bf16_to_f64, round_bf16
from workloads import bf16_from_f32

ROWS = 100_000
EPS = 1e-6


def literal_rms_forward(x, weight, eps):
    """The page's rms_forward, step for step, on a bf16 tensor."""
    orig_dtype = x.dtype
    x = x.float()
    var = x.pow(2).mean(dim=-1, keepdim=True)
    x.mul_(torch.rsqrt(var + eps))
    x = x.to(orig_dtype).mul_(weight)
    return x


def literal_apply_rotary_emb(x, cos, sin):
    """The page's apply_rotary_emb, step for step (cos, sin float32)."""
    x1, x2 = torch.chunk(x.float(), 2, dim=-1)
    y1 = x1 * cos - x2 * sin
    y2 = x2 * cos + x1 * sin
    return torch.cat((y1, y2), dim=-1).to(x.dtype)


def bits_to_bf16_tensor(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16)


def bf16_tensor_to_bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def draw_rows(seed, rows=ROWS):
    """bf16 rows at several scales (N(0,1) times 10^U(-2, 1.5)), a bf16
    weight U(0.5, 1.5), fp32 table rows at random positions below 8192."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, 128)).astype(np.float32)
    x *= (10.0 ** rng.uniform(-2, 1.5, (rows, 1))).astype(np.float32)
    w = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    table = o_nr.rope_table(8192, 128, 1.0e6)
    pos = rng.integers(0, 8192, rows)
    return bf16_from_f32(x), bf16_from_f32(w), table[pos]


def literal_bits(x_bits, w_bits, tab_rows):
    x = bits_to_bf16_tensor(x_bits)
    w = bits_to_bf16_tensor(w_bits)
    cos = torch.from_numpy(np.ascontiguousarray(tab_rows[:, :64]))
    sin = torch.from_numpy(np.ascontiguousarray(tab_rows[:, 64:]))
    return bf16_tensor_to_bits(literal_apply_rotary_emb(literal_rms_forward(x, w, EPS), cos, sin))


def compare(oracle_bits, lit_bits, x_bits, w_bits, tab_rows):
    """(fraction not bit-exact, worst |diff| / bound) of the oracle against the
    literal transcription, with the bound stated in the module docstring."""
    tab = tab_rows.astype(np.float64)
    c, s = np.abs(tab[:, :64]), np.abs(tab[:, 64:])
    y = round_bf16(round_bf16(o_nr.rms_normalize(bf16_to_f64(x_bits), EPS)) * bf16_to_f64(w_bits))
    ya, yb = np.abs(y[:, :64]), np.abs(y[:, 64:])
    rot = 2.0 ** -6 * np.concatenate([ya * c + yb * s, yb * c + ya * s], axis=1)
    got, ref = bf16_to_f64(oracle_bits), bf16_to_f64(lit_bits)
    bound = np.maximum(np.abs(ref), 2.0 ** -126) * 2.0 ** -7 + rot
    return float(np.mean(oracle_bits != lit_bits)), float(np.max(np.abs(got - ref) / bound))


def oracle_bits(x_bits, w_bits, tab_rows):
    tab = tab_rows.astype(np.float64)
    return o_nr.qk_norm_rope(x_bits, w_bits, EPS, tab[:, :64], tab[:, 64:])


def test_oracle_matches_literal_page_code():
    x, w, tab = draw_rows(11)
    lit = literal_bits(x, w, tab)
    inexact, worst = compare(oracle_bits(x, w, tab), lit, x, w, tab)
    print(f"oracle vs literal page code over {ROWS} rows: non-exact fraction {inexact:.2e}, "
          f"worst |diff|/bound {worst:.3f}")
    assert inexact < 1e-3
    assert worst <= 1.0


def test_literal_transcription_is_not_the_oracle():
    """The transcription is an independent evaluation: float32 steps, not the
    oracle's float64, so some elements do differ (else the pin would be a
    re-run of the same arithmetic)."""
    x, w, tab = draw_rows(12, rows=20_000)
    lit = literal_bits(x, w, tab)
    assert np.any(oracle_bits(x, w, tab) != lit)


@pytest.mark.parametrize("skip_call", [0, 1], ids=["no-round-after-normalise", "no-round-after-weight"])
def test_planted_dropped_rounding_is_caught(monkeypatch, skip_call):
    """Drop one of the two bf16 roundings ahead of the rotation inside the
    oracle itself: the literal-code pin must fail."""
    x, w, tab = draw_rows(13, rows=20_000)
    lit = literal_bits(x, w, tab)
    real = o_nr.round_bf16
    calls = {"n": 0}

    def planted(v):
        i = calls["n"]
        calls["n"] += 1
        return np.asarray(v, dtype=np.float64) if i == skip_call else real(v)

    monkeypatch.setattr(o_nr, "round_bf16", planted)
    bad = oracle_bits(x, w, tab)
    assert calls["n"] == 2, "qk_norm_rope rounds twice ahead of the rotation"
    monkeypatch.setattr(o_nr, "round_bf16", real)
    inexact, worst = compare(bad, lit, x, w, tab)
    print(f"planted slip {skip_call}: non-exact fraction {inexact:.2e}, worst {worst:.3f}")
    assert inexact >= 1e-3 or worst > 1.0
