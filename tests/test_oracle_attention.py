"""Pins for the oracle's paged attention: a library routine (torch float64
scaled_dot_product_attention with an explicit bottom-right causal mask and
enable_gqa), hand-derived closed forms, GQA head mapping 16:8 and 32:8, page
permutation invariance, chunking invariance, and NaN sentinels in every
unwritten slot."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import attention, paged
from oracle.bf16 import bf16_to_f64
from workloads import bf16_from_f32, sentinel_pool

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def build_paged(rng, lengths, hkv, d, page, extra_pages=3):
    """Random logical K/V (bf16 bits) for each request, scattered into
    sentinel pools through a random page placement."""
    need = [-(-L // page) for L in lengths]
    num_pages = sum(need) + extra_pages
    perm = rng.permutation(num_pages)
    stride = max(need)
    bt = np.full((len(lengths), stride), -1, np.int32)
    at = 0
    for r, k in enumerate(need):
        bt[r, :k] = perm[at:at + k]
        at += k
    kp = sentinel_pool(num_pages, hkv, page, d, "bf16")
    vp = sentinel_pool(num_pages, hkv, page, d, "bf16")
    logical = []
    for r, L in enumerate(lengths):
        k = bf16_from_f32(rng.standard_normal((L, hkv, d)).astype(np.float32))
        v = bf16_from_f32(rng.standard_normal((L, hkv, d)).astype(np.float32))
        slots = [paged.logical_slot(bt[r], j, page) for j in range(L)]
        paged.kv_write(kp, vp, k, v, np.array(slots), page)
        logical.append((k, v))
    return kp, vp, bt, logical


def sdpa_reference(q, k, v, scale):
    """torch float64 SDPA with an explicit bottom-right causal mask."""
    n, hq, d = q.shape
    L = k.shape[0]
    qi = torch.from_numpy(q).permute(1, 0, 2)[None]       # [1, Hq, n, D]
    ki = torch.from_numpy(k).permute(1, 0, 2)[None]       # [1, Hkv, L, D]
    vi = torch.from_numpy(v).permute(1, 0, 2)[None]
    pos = L - n + torch.arange(n)
    mask = torch.arange(L)[None, :] <= pos[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        qi, ki, vi, attn_mask=mask, scale=float(scale), enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("hq,hkv,page", [(4, 2, 4), (16, 8, 16), (32, 8, 16), (8, 8, 2), (8, 1, 8)])
def test_matches_torch_sdpa(hq, hkv, page):
    rng = np.random.default_rng(100 + hq + page)
    d = 128
    lengths = [1, 7, 33, 50]
    new = [1, 3, 33, 17]
    kp, vp, bt, logical = build_paged(rng, lengths, hkv, d, page)
    q = bf16_from_f32(rng.standard_normal((sum(new), hq, d)).astype(np.float32))
    cu = np.concatenate([[0], np.cumsum(new)])
    scale = np.float32(1 / np.sqrt(d))
    out = attention.paged_attention(q, kp, vp, bt, cu, np.array(lengths), scale, page, "bf16")
    for r in range(len(lengths)):
        k, v = logical[r]
        ref = sdpa_reference(bf16_to_f64(q[cu[r]:cu[r + 1]]), bf16_to_f64(k), bf16_to_f64(v), scale)
        np.testing.assert_allclose(out[cu[r]:cu[r + 1]], ref, rtol=1e-12, atol=1e-12)


def test_golden_closed_forms():
    with open(os.path.join(GOLDEN, "attention_closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"], np.float64)
        k = np.array(c["keys"], np.float64)
        v = np.array(c["values"], np.float64)
        out = attention.attend(q, k, v, c["scale"], k.shape[1])
        np.testing.assert_allclose(out, np.array(c["expected"]), rtol=0, atol=c["atol"] + 1e-300,
                                   err_msg=c["name"])


def test_single_key_returns_v_exactly():
    rng = np.random.default_rng(3)
    kp, vp, bt, logical = build_paged(rng, [1, 1], 8, 128, 16)
    q = bf16_from_f32(rng.standard_normal((2, 16, 128)).astype(np.float32))
    out = attention.paged_decode(q, kp, vp, bt, np.array([1, 1]), np.float32(0.088388346), 16, "bf16")
    for r in range(2):
        v = bf16_to_f64(logical[r][1][0])            # [Hkv][D]
        for h in range(16):
            assert np.array_equal(out[r, h], v[h // 2])


def test_equal_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(4)
    L, n, hkv, hq, d, page = 40, 9, 2, 4, 128, 8
    kp, vp, bt, logical = build_paged(rng, [L], hkv, d, page)
    same_k = np.broadcast_to(logical[0][0][:1], (L, hkv, d)).copy()
    slots = [paged.logical_slot(bt[0], j, page) for j in range(L)]
    paged.kv_write(kp, vp, same_k, logical[0][1], np.array(slots), page)
    q = bf16_from_f32(rng.standard_normal((n, hq, d)).astype(np.float32))
    out = attention.paged_attention(q, kp, vp, bt, np.array([0, n]), np.array([L]), 0.1, page, "bf16")
    v = bf16_to_f64(logical[0][1])
    for i in range(n):
        vis = L - n + i + 1
        for h in range(hq):
            np.testing.assert_allclose(out[i, h], v[:vis, h // 2].mean(axis=0), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("hq,hkv", [(16, 8), (32, 8)])
def test_gqa_head_mapping(hq, hkv):
    rng = np.random.default_rng(5)
    L, page, d = 37, 16, 128
    kp, vp, bt, logical = build_paged(rng, [L], hkv, d, page)
    const_v = np.zeros((L, hkv, d), np.uint16)
    for g in range(hkv):
        const_v[:, g, :] = bf16_from_f32(np.full(d, g + 1, np.float32))
    slots = [paged.logical_slot(bt[0], j, page) for j in range(L)]
    paged.kv_write(kp, vp, logical[0][0], const_v, np.array(slots), page)
    q = bf16_from_f32(rng.standard_normal((1, hq, d)).astype(np.float32))
    out = attention.paged_decode(q, kp, vp, bt, np.array([L]), 0.088, page, "bf16")
    group = hq // hkv
    for h in range(hq):
        np.testing.assert_allclose(out[0, h], h // group + 1, rtol=1e-14)


def test_page_permutation_invariance():
    rng = np.random.default_rng(6)
    lengths, page = [70, 5, 129], 16
    kp, vp, bt, _ = build_paged(rng, lengths, 8, 128, page)
    q = bf16_from_f32(rng.standard_normal((3, 16, 128)).astype(np.float32))
    base = attention.paged_decode(q, kp, vp, bt, np.array(lengths), 0.088, page, "bf16")
    perm = rng.permutation(kp.shape[0])        # physical page p moves to perm[p]
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    moved = attention.paged_decode(q, kp2, vp2, bt2, np.array(lengths), 0.088, page, "bf16")
    assert np.array_equal(base, moved)


def test_chunking_invariance():
    """Full prefill == token-by-token decode == irregular chunks (the
    qwen-inference-lab validation section compares exactly these three)."""
    rng = np.random.default_rng(8)
    L, hq, hkv, d, page = 45, 4, 2, 128, 4
    kp, vp, bt, _ = build_paged(rng, [L], hkv, d, page)
    q = bf16_from_f32(rng.standard_normal((L, hq, d)).astype(np.float32))
    full = attention.paged_attention(q, kp, vp, bt, np.array([0, L]), np.array([L]), 0.09, page, "bf16")
    step = np.stack([attention.paged_decode(q[j:j + 1], kp, vp, bt, np.array([j + 1]), 0.09, page, "bf16")[0]
                     for j in range(L)])
    np.testing.assert_allclose(step, full, rtol=1e-12, atol=1e-12)
    cuts = [0, 1, 8, 9, 30, L]
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        parts.append(attention.paged_attention(q[a:b], kp, vp, bt, np.array([0, b - a]), np.array([b]),
                                               0.09, page, "bf16"))
    np.testing.assert_allclose(np.concatenate(parts), full, rtol=1e-12, atol=1e-12)


def test_never_reads_unwritten_slots():
    # every unwritten slot (tails of partial pages, spare pages) is NaN
    rng = np.random.default_rng(9)
    lengths, page = [17, 31, 2], 16
    kp, vp, bt, _ = build_paged(rng, lengths, 8, 128, page)
    assert np.isnan(bf16_to_f64(kp[bt[0, 1], 0, 1])).all()      # a tail slot is poisoned
    q = bf16_from_f32(rng.standard_normal((sum(lengths), 16, 128)).astype(np.float32))
    cu = np.concatenate([[0], np.cumsum(lengths)])
    out = attention.paged_attention(q, kp, vp, bt, cu, np.array(lengths), 0.088, page, "bf16")
    assert np.isfinite(out).all()


def test_planted_mistakes_are_caught(monkeypatch):
    """Each plausible slip in the oracle trips one of the pins above."""
    rng = np.random.default_rng(10)
    lengths, new, hq, hkv, page = [20, 9], [4, 9], 4, 2, 4
    kp, vp, bt, logical = build_paged(rng, lengths, hkv, 128, page)
    q = bf16_from_f32(rng.standard_normal((sum(new), hq, 128)).astype(np.float32))
    cu = np.concatenate([[0], np.cumsum(new)])

    def agrees():
        out = attention.paged_attention(q, kp, vp, bt, cu, np.array(lengths), 0.088, page, "bf16")
        for r in range(2):
            k, v = logical[r]
            ref = sdpa_reference(bf16_to_f64(q[cu[r]:cu[r + 1]]), bf16_to_f64(k), bf16_to_f64(v), 0.088)
            if not np.allclose(out[cu[r]:cu[r + 1]], ref, rtol=1e-10, atol=1e-10):
                return False
        return True

    assert agrees()
    real_attend = attention.attend

    def wrong_head_map(q_, keys, values, scale, nkv):   # h % Hkv instead of h // G
        perm = [h % nkv * (q_.shape[1] // nkv) + h // nkv for h in range(q_.shape[1])]
        return real_attend(q_[:, perm], keys, values, scale, nkv)[:, np.argsort(perm)]
    monkeypatch.setattr(attention, "attend", wrong_head_map)
    assert not agrees()

    def top_left_mask(q_, keys, values, scale, nkv):    # causal mask anchored at key 0
        return real_attend(q_, keys[:q_.shape[0]], values[:q_.shape[0]], scale, nkv)
    monkeypatch.setattr(attention, "attend", top_left_mask)
    assert not agrees()

    def no_scale(q_, keys, values, scale, nkv):
        return real_attend(q_, keys, values, 1.0, nkv)
    monkeypatch.setattr(attention, "attend", no_scale)
    assert not agrees()
    monkeypatch.setattr(attention, "attend", real_attend)

    real_logical = paged.gather_request

    def off_by_one_page(pool, row, length, p):           # reads the next logical page
        return real_logical(pool, np.roll(row[:-(-length // p)], 1), length, p)
    monkeypatch.setattr(attention, "gather_request", off_by_one_page)
    assert not agrees()
