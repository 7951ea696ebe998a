"""qil_paged_prefill on the GPU against the oracle: the varlen workload in
full, ragged and degenerate chunks, every GQA group size, several page
sizes, decode == prefill with one query token, and chunking invariance."""

import numpy as np
import pytest
import torch

from tests import harness as H
from workloads import make_workload, make_custom

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_cfg4_full(qil):
    w = make_workload(4)
    print("cfg4 chunks", w.new_lens.tolist(), "prefix", w.cached_lens.tolist(), flush=True)
    case = H.DeviceCase(w, DEV)
    out = H.to_f64(case.prefill())
    ref = H.OracleCase(w, case.data, range(w.batch)).attention(range(w.batch))
    print("cfg4 max abs err", np.max(np.abs(out - ref)), flush=True)
    assert H.excess(out, ref, "bf16") <= 0


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (32, 8), (16, 2), (40, 8), (64, 4)])
def test_group_sizes_ragged(qil, hq, hkv):
    # chunk lengths straddle the query tile (128 / G tokens) and key tile (64)
    ctx = [1, 65, 200, 129, 700, 33]
    new = [1, 1, 200, 64, 131, 17]
    got, ref = H.run_small_prefill(DEV, ctx, new, hq, hkv, 16, seed=hq * 10 + hkv)
    assert H.excess(got, ref, "bf16") <= 0


@pytest.mark.parametrize("hq,hkv", [(16, 8), (32, 8), (40, 8), (64, 4)])
def test_loose_context_bound_is_invisible(qil, hq, hkv):
    """max_context_len is a host bound on the contexts; any value at least the
    longest context gives the same output bit for bit.  A bound of 4,096 keys
    (block tables padded with -1 columns to fit it) also switches the whole-
    tile kernel from workgroups of 128 query rows (two per CU) to 256, so both
    shapes run on the same inputs, and both match the oracle."""
    ctx = [1, 65, 200, 129, 700, 33, 2000]
    new = [1, 1, 200, 64, 131, 17, 1500]
    w = make_custom(ctx, new, hq=hq, hkv=hkv, page=16, seed=hq + hkv)
    case = H.DeviceCase(w, DEV)
    tight = case.prefill()
    reqs = np.asarray(w.prefill_idx)
    rows = torch.from_numpy(case.rows_of(reqs)).to(DEV)
    q = case.q_all.index_select(0, rows).contiguous()
    bt = case.bt.index_select(0, torch.from_numpy(reqs).to(DEV))
    pad = torch.full((bt.shape[0], 4096 // 16 - bt.shape[1]), -1, dtype=bt.dtype, device=DEV)
    bt = torch.cat([bt, pad], dim=1).contiguous()
    ctx_d = case.ctx.index_select(0, torch.from_numpy(reqs).to(DEV)).contiguous()
    cu = H.i32(w.cu_seqlens(reqs), DEV)
    loose = torch.empty_like(q)
    qil.paged_prefill(loose, q, case.kp, case.vp, bt, cu, ctx_d, int(w.new_lens.max()), 4096,
                      float(w.scale))
    torch.cuda.synchronize()
    assert torch.equal(tight.view(torch.int16), loose.view(torch.int16))
    ref = H.OracleCase(w, case.data, range(w.batch)).attention(range(w.batch))
    assert H.excess(H.to_f64(loose), ref, "bf16") <= 0


@pytest.mark.parametrize("page", [32, 64, 256])
def test_page_sizes(qil, page):
    got, ref = H.run_small_prefill(DEV, [300, 1000, 90], [100, 257, 90], 16, 8, page, seed=page)
    assert H.excess(got, ref, "bf16") <= 0


def test_decode_equals_prefill_one_token(qil):
    w = make_custom([1, 17, 300, 1024, 77], [1] * 5, page=16, seed=21, decode=True)
    case = H.DeviceCase(w, DEV)
    dec = H.to_f64(case.decode())
    pre = H.to_f64(case.prefill(requests=np.arange(5)))
    assert np.max(np.abs(dec - pre)) < 1e-2


def test_chunking_invariance(qil):
    # the whole prompt as one chunk vs three irregular chunks over the same pool
    L = 777
    w = make_custom([L], [L], page=16, seed=22)
    case = H.DeviceCase(w, DEV)
    full = H.to_f64(case.prefill())
    parts = []
    for a, b in [(0, 100), (100, 101), (101, L)]:
        q = case.q_all[a:b].contiguous()
        out = torch.empty_like(q)
        qil.paged_prefill(out, q, case.kp, case.vp, case.bt, H.i32([0, b - a], DEV),
                          H.i32([b], DEV), b - a, b, float(w.scale))
        parts.append(H.to_f64(out))
    assert np.max(np.abs(np.concatenate(parts) - full)) < 1e-2
    ref = H.OracleCase(w, case.data, [0]).attention([0])
    assert H.excess(full, ref, "bf16") <= 0


def test_zero_length_request_is_skipped(qil):
    w = make_custom([50, 20, 64], [10, 1, 64], page=16, seed=23)
    case = H.DeviceCase(w, DEV)
    # request 1 gets no new tokens in this call
    reqs = np.array([0, 1, 2])
    rows = torch.from_numpy(np.concatenate([case.rows_of([0]), case.rows_of([2])])).to(DEV)
    q = case.q_all.index_select(0, rows).contiguous()
    cu = H.i32([0, 10, 10, 74], DEV)
    ctx = H.i32([50, 19, 64], DEV)
    out = torch.empty_like(q)
    qil.paged_prefill(out, q, case.kp, case.vp, case.bt, cu, ctx, 64, 64, float(w.scale))
    got = H.to_f64(out)
    ref = H.OracleCase(w, case.data, [0, 2]).attention([0, 2])
    assert H.excess(got, ref, "bf16") <= 0
    del reqs


def test_run_twice_bitwise(qil):
    w = make_workload(4)
    case = H.DeviceCase(w, DEV)
    a = H.to_bits(case.prefill())
    b = H.to_bits(case.prefill())
    assert np.array_equal(a, b)


def spiked_case(seed, hq=16, cached=0):
    """One 300-token context (the first `cached` tokens already in the pool)
    whose keys at positions 40, 105, 170 and 235 (each in the second 32-key
    half of a 64-key tile) carry a growing component along dim 0, while every
    query carries +4 there: each spike lifts the row maximum of the scores by
    about 10 in base 2, past the kernels' 2^8 rescale threshold.  Values are
    bf16 and finite."""
    from workloads import bf16_from_f32
    from oracle import bf16 as obf
    w = make_custom([300], [300 - cached], hq=hq, hkv=8, page=16, seed=seed)
    d = w.gather()
    kc = obf.bf16_to_f64(d["k_cached"]).astype(np.float32)
    kn = obf.bf16_to_f64(d["k_new"]).astype(np.float32)
    q = obf.bf16_to_f64(d["q"]).astype(np.float32)
    for pos, mag in ((40, 10.0), (105, 30.0), (170, 50.0), (235, 70.0)):
        if pos < cached:
            kc[pos, :, 0] = mag
        else:
            kn[pos - cached, :, 0] = mag
    q[:, :, 0] = 4.0
    d["k_cached"] = bf16_from_f32(kc)
    d["k_new"] = bf16_from_f32(kn)
    d["q"] = bf16_from_f32(q)
    return w, d


@pytest.mark.parametrize("hq,cached", [(16, 0), (32, 0), (64, 0), (16, 100)])
def test_max_jump_inside_a_tile(qil, hq, cached):
    # A row maximum that jumps inside the second half of a key tile must
    # rescale everything accumulated before it, including the first half.
    w, d = spiked_case(31, hq, cached)
    case = H.DeviceCase(w, DEV, data=d)
    got = H.to_f64(case.prefill())
    ref = H.OracleCase(w, d, [0]).attention([0])
    print(f"spiked prefill hq={hq} cached={cached} max abs err", np.max(np.abs(got - ref)), flush=True)
    assert H.excess(got, ref, "bf16") <= 0


@pytest.mark.parametrize("hq,hkv,page", [(16, 8, 16), (32, 8, 16), (8, 8, 64), (64, 8, 32), (16, 2, 256)])
def test_fp32_ragged(qil, hq, hkv, page):
    # fp32 prefill (the fp32 decode kernel, one row per new token) at the fp32 bar
    ctx = [1, 65, 200, 129, 700, 33, 4000]
    new = [1, 1, 200, 64, 131, 17, 300]
    w = make_custom(ctx, new, hq=hq, hkv=hkv, page=page, dtype="f32", seed=hq + page + 3)
    case = H.DeviceCase(w, DEV)
    got = H.to_f64(case.prefill())
    ref = H.OracleCase(w, case.data, range(w.batch)).attention(range(w.batch))
    print(f"fp32 prefill hq={hq} hkv={hkv} page={page} max abs err", np.max(np.abs(got - ref)),
          flush=True)
    assert H.excess(got, ref, "f32") <= 0


def test_fp32_decode_equals_prefill_and_chunking(qil):
    # one query token per request: prefill rows equal decode rows (one split
    # each); a prompt as one chunk equals the same prompt in irregular chunks
    w = make_custom([1, 17, 300, 1024, 77], [1] * 5, page=16, dtype="f32", seed=27, decode=True)
    case = H.DeviceCase(w, DEV)
    dec = H.to_bits(case.decode(keys_per_split=1024))
    pre = H.to_bits(case.prefill(requests=np.arange(5)))
    assert np.array_equal(dec, pre)
    L = 777
    w = make_custom([L], [L], page=16, dtype="f32", seed=28)
    case = H.DeviceCase(w, DEV)
    full = H.to_bits(case.prefill())
    parts = []
    for a, b in [(0, 100), (100, 101), (101, L)]:
        q = case.q_all[a:b].contiguous()
        out = torch.empty_like(q)
        qil.paged_prefill(out, q, case.kp, case.vp, case.bt, H.i32([0, b - a], DEV),
                          H.i32([b], DEV), b - a, b, float(w.scale))
        parts.append(H.to_bits(out))
    assert np.array_equal(np.concatenate(parts), full)
