"""Pins for the oracle's merged QKV projection: brute-force exact dot
products on a tiny case, one-hot activations (the output is a weight
column), the [Q | K | V] column layout of the "nano-vLLM learning note"
QKVParallelLinear block, a single rounding from the exact product, and the
reduction of project-then-write to the already pinned fused write when the
weight is an identity."""

import math

import numpy as np

from oracle import norm_rope, projection
from oracle.bf16 import bf16_to_f64, f64_to_bf16
from workloads import bf16_from_f32, sentinel_pool


def test_brute_force_exact_dot_products():
    # exact sums of exact products (math.fsum), rounded to bf16 once
    rng = np.random.default_rng(7)
    x = bf16_from_f32(rng.standard_normal((5, 64)).astype(np.float32))
    w = bf16_from_f32(rng.standard_normal((3 * 128, 64)).astype(np.float32))
    xf, wf = bf16_to_f64(x), bf16_to_f64(w)
    want = np.empty((5, 3 * 128), dtype=np.uint16)
    for t in range(5):
        for n in range(3 * 128):
            s = math.fsum(float(xf[t, k]) * float(wf[n, k]) for k in range(64))
            want[t, n] = f64_to_bf16(np.array([s]))[0]
    assert np.array_equal(projection.qkv_projection(x, w), want)


def test_one_hot_rows_pick_weight_columns():
    # x[t] = 2^s * e_j: the output row is weight column j times 2^s, exactly
    rng = np.random.default_rng(8)
    w = bf16_from_f32(rng.standard_normal((6 * 128, 96)).astype(np.float32))
    js, ss = [0, 5, 95, 40], [0, 3, -2, 1]
    x = np.zeros((4, 96))
    for t, (j, s) in enumerate(zip(js, ss)):
        x[t, j] = 2.0 ** s
    out = bf16_to_f64(projection.qkv_projection(f64_to_bf16(x), w))
    for t, (j, s) in enumerate(zip(js, ss)):
        assert np.array_equal(out[t], bf16_to_f64(w[:, j]) * 2.0 ** s)


def test_column_layout_q_then_k_then_v():
    # weight column 0 holds the output head's index + 1, column 1 the dim
    hq, hkv, d = 32, 8, 128
    n = (hq + 2 * hkv) * d
    w = np.zeros((n, 16))
    w[:, 0] = np.arange(n) // d + 1
    w[:, 1] = np.arange(n) % d
    x = np.zeros((2, 16))
    x[0, 0] = 1.0
    x[1, 1] = 1.0
    qkv = projection.qkv_projection(f64_to_bf16(x), f64_to_bf16(w))
    q, k, v = (bf16_to_f64(a) for a in projection.split_qkv(qkv, hq, hkv))
    assert q.shape == (2, hq, d) and k.shape == (2, hkv, d) and v.shape == (2, hkv, d)
    for h in range(hq):
        assert np.all(q[0, h] == h + 1)
    for g in range(hkv):
        assert np.all(k[0, g] == hq + g + 1)
        assert np.all(v[0, g] == hq + hkv + g + 1)
    for a in (q, k, v):
        assert np.all(a[1] == np.arange(d))


def test_rounded_once_from_the_exact_product():
    # 1 + 2^-8 + 2^-30 lies just above the tie between the bf16 neighbours 1
    # and 1 + 2^-7, so it rounds up; a float32 running sum drops 2^-30, lands
    # on the tie and rounds to even (down)
    x = f64_to_bf16(np.array([[1.0, 2.0 ** -8, 2.0 ** -30, 0.0]]))
    w = f64_to_bf16(np.ones((1, 4)))
    got = bf16_to_f64(projection.qkv_projection(x, w))[0, 0]
    assert got == 1.0 + 2.0 ** -7
    f32 = np.float32(1.0) + np.float32(2.0 ** -8) + np.float32(2.0 ** -30)
    assert bf16_to_f64(bf16_from_f32(np.array([f32])))[0] == 1.0


def test_identity_weight_reduces_to_the_fused_write():
    rng = np.random.default_rng(9)
    hq, hkv, d, page = 4, 2, 128, 16
    n = (hq + 2 * hkv) * d
    t = 7
    x = bf16_from_f32(rng.standard_normal((t, n)).astype(np.float32))
    eye = f64_to_bf16(np.eye(n))
    slots = np.array([3, 17, -1, 40, 5, 63, 22], dtype=np.int32)
    pos = np.array([0, 9, 4, 100, 31, 7, 64], dtype=np.int32)
    qw = bf16_from_f32(rng.uniform(0.5, 1.5, d).astype(np.float32))
    kw = bf16_from_f32(rng.uniform(0.5, 1.5, d).astype(np.float32))
    table = norm_rope.rope_table(128, d, 1.0e6)
    kp1, vp1 = sentinel_pool(4, hkv, page, d, "bf16"), sentinel_pool(4, hkv, page, d, "bf16")
    q_out, qkv = projection.qkv_proj_write(kp1, vp1, x, eye, hq, hkv, slots, pos, qw, kw, 1e-6,
                                           table, page)
    assert np.array_equal(qkv, x)
    kp2, vp2 = sentinel_pool(4, hkv, page, d, "bf16"), sentinel_pool(4, hkv, page, d, "bf16")
    q, k, v = x[:, :hq * d], x[:, hq * d:(hq + hkv) * d], x[:, (hq + hkv) * d:]
    q_ref = norm_rope.fused_kv_write(kp2, vp2, q.reshape(t, hq, d), k.reshape(t, hkv, d),
                                     v.reshape(t, hkv, d), slots, pos, qw, kw, 1e-6, table, page)
    assert np.array_equal(q_out, q_ref)
    assert np.array_equal(kp1, kp2) and np.array_equal(vp1, vp2)
