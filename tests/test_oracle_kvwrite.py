"""Pins for the oracle's plain scatter write and block-table addressing: the
slot formula of the decode step worked by hand, -1 skipping, bit-exact
placement with every other slot untouched, and write -> gather round trip."""

import json
import os

import numpy as np

from oracle import paged
from workloads import bf16_from_f32, sentinel_pool

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_slot_formula_golden():
    with open(os.path.join(GOLDEN, "slot_formula.json")) as f:
        g = json.load(f)
    bt, bs, n = g["block_table"], g["block_size"], g["seq_len"]
    last_block_tokens = n - (len(bt) - 1) * bs
    assert paged.logical_slot(bt, n - 1, bs) == g["decode_slot"]
    assert bt[-1] * bs + last_block_tokens - 1 == g["decode_slot"]
    assert paged.slot_to_page_offset(g["decode_slot"], bs) == (g["decode_page"], g["decode_offset"])
    assert -(-n // bs) == g["pages_needed"]


def test_write_is_exact_and_skips_minus_one():
    rng = np.random.default_rng(11)
    pages, hkv, page, d = 6, 3, 4, 128
    for dtype in ("bf16", "f32"):
        kp = sentinel_pool(pages, hkv, page, d, dtype)
        vp = sentinel_pool(pages, hkv, page, d, dtype)
        T = 9
        x = rng.standard_normal((2, T, hkv, d)).astype(np.float32)
        k, v = (bf16_from_f32(x[0]), bf16_from_f32(x[1])) if dtype == "bf16" else (x[0].view(np.uint32), x[1].view(np.uint32))
        slots = np.array([5, -1, 0, 23, 12, -1, 7, 8, 22], np.int32)
        kp0, vp0 = kp.copy(), vp.copy()
        paged.kv_write(kp, vp, k, v, slots, page)
        touched = np.zeros((pages, page), bool)
        for t, s in enumerate(slots):
            if s < 0:
                continue
            pg, off = s // page, s % page
            touched[pg, off] = True
            assert np.array_equal(kp[pg, :, off], k[t]) and np.array_equal(vp[pg, :, off], v[t])
        for pg in range(pages):
            for off in range(page):
                if not touched[pg, off]:
                    assert np.array_equal(kp[pg, :, off], kp0[pg, :, off])
                    assert np.array_equal(vp[pg, :, off], vp0[pg, :, off])


def test_flat_index_matches_layout_statement():
    # element (slot s, head g, dim d) at ((s // P * Hkv + g) * P + s % P) * D + d
    pages, hkv, page, d = 5, 2, 8, 128
    flat = np.arange(pages * hkv * page * d, dtype=np.uint32)
    view = paged.pool_view(flat, pages, hkv, page, d)
    for s, g, e in [(0, 0, 0), (13, 1, 77), (39, 0, 127), (8, 1, 5)]:
        assert view[s // page, g, s % page, e] == ((s // page * hkv + g) * page + s % page) * d + e


def test_write_then_gather_roundtrip():
    rng = np.random.default_rng(12)
    page, hkv, d, L = 16, 8, 128, 50
    bt = np.array([9, 2, 5, 0], np.int32)
    kp = sentinel_pool(10, hkv, page, d, "bf16")
    vp = sentinel_pool(10, hkv, page, d, "bf16")
    k = bf16_from_f32(rng.standard_normal((L, hkv, d)).astype(np.float32))
    v = bf16_from_f32(rng.standard_normal((L, hkv, d)).astype(np.float32))
    order = rng.permutation(L)                     # write order does not matter
    slots = np.array([paged.logical_slot(bt, j, page) for j in order])
    paged.kv_write(kp, vp, k[order], v[order], slots, page)
    assert np.array_equal(paged.gather_request(kp, bt, L, page), k)
    assert np.array_equal(paged.gather_request(vp, bt, L, page), v)
