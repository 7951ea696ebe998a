"""Seeded sweeps of qil_paged_prefill (whole tiles, split over keys, fp32),
qil_paged_decode and qil_paged_decode_append over drawn shapes:
GQA group size, KV heads, page size, batch, cached prefix and chunk lengths
(edge values such as 1, the 64-key tile and page multiples drawn more often),
each case against the fp64 oracle at the bf16 / fp32 tolerance.  The shapes
are a fixed function of the case index, so every run checks the same cases."""

import numpy as np
import pytest
import torch

from tests import harness as H
from workloads import make_custom

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

GROUPS = (1, 2, 4, 5, 8, 16)
KV_HEADS = (1, 2, 4, 8)
PAGES = (16, 32, 64, 128, 256)
EDGES = (1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257)


def draw_len(rng, hi):
    """A length in [1, hi]: an edge value a third of the time."""
    if rng.random() < 1 / 3:
        e = [v for v in EDGES if v <= hi]
        return int(rng.choice(e))
    return int(rng.integers(1, hi + 1))


def draw_heads(rng):
    g = int(rng.choice(GROUPS))
    hkv = int(rng.choice(KV_HEADS))
    while g * hkv > 64:
        hkv //= 2
    return g * hkv, hkv


@pytest.mark.parametrize("case", range(12))
def test_prefill_sweep(qil, case):
    rng = np.random.default_rng(9000 + case)
    hq, hkv = draw_heads(rng)
    page = int(rng.choice(PAGES))
    batch = int(rng.integers(1, 6))
    new = [draw_len(rng, 300) for _ in range(batch)]
    prefix = [0 if rng.random() < 0.3 else draw_len(rng, 300) for _ in range(batch)]
    ctx = [p + n for p, n in zip(prefix, new)]
    print(f"prefill sweep {case}: hq={hq} hkv={hkv} page={page} new={new} ctx={ctx}", flush=True)
    got, ref = H.run_small_prefill(DEV, ctx, new, hq, hkv, page, seed=500 + case)
    print(f"  max abs err {np.max(np.abs(got - ref)):.3e}", flush=True)
    assert H.excess(got, ref, "bf16") <= 0


@pytest.mark.parametrize("case", range(12))
def test_decode_sweep(qil, case):
    rng = np.random.default_rng(9100 + case)
    hq, hkv = draw_heads(rng)
    page = int(rng.choice(PAGES))
    dtype = "f32" if case % 3 == 2 else "bf16"
    batch = int(rng.integers(1, 41))
    ctx = [draw_len(rng, 2000) for _ in range(batch)]
    split = int(rng.choice([0, 64, 256]))
    print(f"decode sweep {case}: {dtype} hq={hq} hkv={hkv} page={page} batch={batch} "
          f"max ctx={max(ctx)} keys_per_split={split}", flush=True)
    w = make_custom(ctx, [1] * batch, hq=hq, hkv=hkv, page=page, dtype=dtype, seed=600 + case,
                    decode=True)
    got, ref = H.run_decode_case(w, DEV, keys_per_split=split)
    print(f"  max abs err {np.max(np.abs(got - ref)):.3e}", flush=True)
    assert H.excess(got, ref, dtype) <= 0


@pytest.mark.parametrize("case", range(8))
def test_split_prefill_sweep(qil, case):
    # drawn shapes with long cached prefixes, split over keys: automatic or a
    # drawn piece length; fp32 cases (G <= 8, contexts <= 4,096) every fourth
    rng = np.random.default_rng(9200 + case)
    hq, hkv = draw_heads(rng)
    dtype = "f32" if case % 4 == 3 else "bf16"
    while dtype == "f32" and hq // hkv > 8:
        hq //= 2
    page = int(rng.choice(PAGES))
    batch = int(rng.integers(1, 4))
    new = [draw_len(rng, 300) for _ in range(batch)]
    prefix = [int(rng.integers(1000, 3500)) for _ in range(batch)]
    ctx = [p + n for p, n in zip(prefix, new)]
    kps = int(rng.choice([0, 128, 512, 1024]))
    print(f"split prefill sweep {case}: {dtype} hq={hq} hkv={hkv} page={page} new={new} "
          f"ctx={ctx} keys_per_split={kps}", flush=True)
    w = make_custom(ctx, new, hq=hq, hkv=hkv, page=page, dtype=dtype, seed=700 + case)
    case_ = H.DeviceCase(w, DEV)
    got = H.to_f64(case_.prefill(keys_per_split=kps))
    ref = H.OracleCase(w, case_.data, range(w.batch)).attention(range(w.batch))
    print(f"  max abs err {np.max(np.abs(got - ref)):.3e}", flush=True)
    assert H.excess(got, ref, dtype) <= 0


@pytest.mark.parametrize("case", range(6))
def test_decode_append_sweep(qil, case):
    # the fused write + decode against the two calls, bit for bit, on drawn shapes
    import paged_kv_attention_16_amd as qil_
    rng = np.random.default_rng(9300 + case)
    hq, hkv = draw_heads(rng)
    page = int(rng.choice(PAGES))
    batch = int(rng.integers(1, 41))
    ctx = [draw_len(rng, 2000) for _ in range(batch)]
    split = int(rng.choice([0, 64, 256]))
    print(f"decode append sweep {case}: hq={hq} hkv={hkv} page={page} batch={batch} "
          f"max ctx={max(ctx)} keys_per_split={split}", flush=True)
    w = make_custom(ctx, [1] * batch, hq=hq, hkv=hkv, page=page, seed=800 + case, decode=True)
    sep = H.DeviceCase(w, DEV)
    app = H.DeviceCase(w, DEV, data=sep.data, write_new=False)
    out_sep = sep.decode(keys_per_split=split)
    out_app = torch.empty_like(app.q_all)
    qil_.paged_decode_append(out_app, app.q_all, app.k_new, app.v_new, app.new_slots, app.kp,
                             app.vp, app.bt, app.ctx, int(w.context_lens.max()), float(w.scale),
                             keys_per_split=split)
    torch.cuda.synchronize()
    assert np.array_equal(H.to_bits(out_app), H.to_bits(out_sep))
    assert np.array_equal(H.to_bits(app.kp), H.to_bits(sep.kp))
    assert np.array_equal(H.to_bits(app.vp), H.to_bits(sep.vp))
