"""Pins for the oracle's per-head RMSNorm, RoPE table and rotation, and the
fused norm + RoPE + scatter write: torch float64 rms_norm, closed forms,
complex-number rotation, norm preservation, the relative-position property,
and the identity at position 0."""

import numpy as np
import torch

from oracle import norm_rope, paged
from oracle.bf16 import bf16_to_f64, f64_to_bf16, round_bf16
from workloads import bf16_from_f32, sentinel_pool


def test_rms_normalize_matches_torch_rms_norm():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 128)) * rng.uniform(0.01, 30, (64, 1))
    mine = norm_rope.rms_normalize(x, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), eps=1e-6).numpy()
    np.testing.assert_allclose(mine, ref, rtol=1e-14, atol=1e-15)


def test_constant_row_closed_form():
    # x = c * ones, w = 1: x / sqrt(c^2 + eps); at position 0 RoPE is identity
    for c in (0.5, 1.0, -3.0, 2.0 ** -10):
        x = f64_to_bf16(np.full(128, c))
        w = f64_to_bf16(np.ones(128))
        cos, sin = np.ones(64), np.zeros(64)
        out = bf16_to_f64(norm_rope.qk_norm_rope(x, w, 1e-6, cos, sin))
        want = round_bf16(np.array([c / np.sqrt(c * c + 1e-6)]))[0]
        assert np.all(out == want), (c, out[:2], want)


def test_table_closed_forms():
    t = norm_rope.rope_table(4096, 128, 1.0e6).astype(np.float64)
    assert t.shape == (4096, 128)
    assert np.all(t[0, :64] == 1.0) and np.all(t[0, 64:] == 0.0)
    pos = np.arange(4096)
    # j = 0: inv_freq = 1, angle = pos
    assert np.array_equal(t[:, 0], np.cos(pos).astype(np.float32).astype(np.float64))
    assert np.array_equal(t[:, 64], np.sin(pos).astype(np.float32).astype(np.float64))
    # j = 32: inv_freq = theta^(-1/2) = 1e-3
    np.testing.assert_allclose(norm_rope.rope_inv_freq(128, 1.0e6)[32], 1e-3, rtol=1e-15)
    np.testing.assert_allclose(t[:, 32], np.cos(pos * 1e-3), atol=1e-7)


def test_rotation_is_complex_multiplication():
    rng = np.random.default_rng(2)
    y = rng.standard_normal((10, 128))
    ang = rng.uniform(-50, 50, (10, 64))
    got = norm_rope.rope_rotate(y, np.cos(ang), np.sin(ang))
    z = (y[:, :64] + 1j * y[:, 64:]) * np.exp(1j * ang)
    np.testing.assert_allclose(got[:, :64], z.real, atol=1e-12)
    np.testing.assert_allclose(got[:, 64:], z.imag, atol=1e-12)
    # each (d, d + 64) pair keeps its length
    np.testing.assert_allclose(got[:, :64] ** 2 + got[:, 64:] ** 2,
                               y[:, :64] ** 2 + y[:, 64:] ** 2, rtol=1e-12)


def test_relative_position_property():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    inv = norm_rope.rope_inv_freq(128, 1.0e6)

    def rot(x, p):
        return norm_rope.rope_rotate(x, np.cos(p * inv), np.sin(p * inv))

    base = rot(q, 100) @ rot(k, 37)
    for shift in (1, 250, 3000):
        np.testing.assert_allclose(rot(q, 100 + shift) @ rot(k, 37 + shift), base, rtol=1e-9)
    assert abs(rot(q, 100) @ rot(k, 38) - base) > 1e-6


def test_fused_write_places_normed_k_and_raw_v():
    rng = np.random.default_rng(4)
    T, hq, hkv, d, page, pages = 6, 4, 2, 128, 4, 5
    q = bf16_from_f32(rng.standard_normal((T, hq, d)).astype(np.float32))
    k = bf16_from_f32(rng.standard_normal((T, hkv, d)).astype(np.float32))
    v = bf16_from_f32(rng.standard_normal((T, hkv, d)).astype(np.float32))
    wq = bf16_from_f32(rng.uniform(0.5, 1.5, d).astype(np.float32))
    wk = bf16_from_f32(rng.uniform(0.5, 1.5, d).astype(np.float32))
    table = norm_rope.rope_table(64, d, 1.0e6)
    pos = np.array([0, 5, 9, 63, 1, 2], np.int32)
    slots = np.array([3, -1, 17, 0, 19, 8], np.int32)
    kp = sentinel_pool(pages, hkv, page, d, "bf16")
    vp = sentinel_pool(pages, hkv, page, d, "bf16")
    before_k = kp.copy()
    q_out = norm_rope.fused_kv_write(kp, vp, q, k, v, slots, pos, wq, wk, 1e-6, table, page)
    tab = table.astype(np.float64)
    for t in range(T):
        c, s = tab[pos[t], :64], tab[pos[t], 64:]
        assert np.array_equal(q_out[t], norm_rope.qk_norm_rope(q[t], wq, 1e-6, c, s))
        if slots[t] < 0:
            continue
        pg, off = divmod(int(slots[t]), page)
        assert np.array_equal(kp[pg, :, off], norm_rope.qk_norm_rope(k[t], wk, 1e-6, c, s))
        assert np.array_equal(vp[pg, :, off], v[t])
    # position 0 rotates nothing: q_out equals the bf16-rounded normalised row times w
    y = round_bf16(round_bf16(norm_rope.rms_normalize(bf16_to_f64(q[0]), 1e-6)) * bf16_to_f64(wq))
    assert np.array_equal(bf16_to_f64(q_out[0]), y)
    # untouched slots keep the sentinel
    written = {int(s) for s in slots if s >= 0}
    for s in range(pages * page):
        if s not in written:
            pg, off = divmod(s, page)
            assert np.array_equal(kp[pg, :, off], before_k[pg, :, off])


def test_planted_sign_error_is_caught(monkeypatch):
    rng = np.random.default_rng(5)
    y = rng.standard_normal((4, 128))
    ang = rng.uniform(-3, 3, (4, 64))
    real = norm_rope.rope_rotate

    def flipped(y_, c, s):  # y1*c + y2*s instead of y1*c - y2*s
        return real(y_, c, -s)
    z = (y[:, :64] + 1j * y[:, 64:]) * np.exp(1j * ang)
    monkeypatch.setattr(norm_rope, "rope_rotate", flipped)
    got = norm_rope.rope_rotate(y, np.cos(ang), np.sin(ang))
    assert not np.allclose(got[:, :64], z.real, atol=1e-6)
