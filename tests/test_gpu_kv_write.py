"""qil_kv_write on the GPU against the oracle: bit-exact over the whole pool
(every unwritten slot keeps its NaN sentinel), -1 slots skipped, strided
views into a fused QKV buffer."""

import numpy as np
import pytest
import torch

from tests import harness as H
from oracle import paged as o_paged
from workloads import make_workload, make_custom, sentinel_pool

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def oracle_pools_all(w, data):
    kp = sentinel_pool(w.num_pages, w.num_kv_heads, w.page_size, w.head_dim, w.dtype)
    vp = sentinel_pool(w.num_pages, w.num_kv_heads, w.page_size, w.head_dim, w.dtype)
    o_paged.kv_write(kp, vp, data["k_cached"], data["v_cached"], data["cached_slots"], w.page_size)
    o_paged.kv_write(kp, vp, data["k_new"], data["v_new"], data["new_slots"], w.page_size)
    return kp, vp


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_whole_pool_bit_exact(qil, cfg):
    w = make_workload(cfg)
    print(f"kv_write cfg{cfg} pages={w.num_pages}", flush=True)
    case = H.DeviceCase(w, DEV)
    torch.cuda.synchronize()
    kp, vp = oracle_pools_all(w, case.data)
    assert np.array_equal(H.to_bits(case.kp), kp)
    assert np.array_equal(H.to_bits(case.vp), vp)


def test_skip_and_strided_views(qil):
    w = make_custom([40, 17, 5], [40, 17, 5], hq=16, hkv=8, page=16, seed=3)
    data = w.gather()
    T = data["k_new"].shape[0]
    slots = data["new_slots"].copy()
    slots[[1, 7, T - 1]] = -1                          # skipped tokens
    # k and v live inside one [T][Hq + 2 Hkv][D] buffer, as after a fused QKV GEMM
    qkv = torch.zeros(T, 16 + 16, 128, dtype=torch.bfloat16, device=DEV)
    qkv[:, 16:24] = H.to_dev(data["k_new"], "bf16", DEV)
    qkv[:, 24:32] = H.to_dev(data["v_new"], "bf16", DEV)
    kp, vp = H.device_pools(w, DEV)
    qil.kv_write(qkv[:, 16:24], qkv[:, 24:32], kp, vp, H.i32(slots, DEV))
    torch.cuda.synchronize()
    okp = sentinel_pool(w.num_pages, 8, 16, 128, "bf16")
    ovp = sentinel_pool(w.num_pages, 8, 16, 128, "bf16")
    o_paged.kv_write(okp, ovp, data["k_new"], data["v_new"], slots, 16)
    assert np.array_equal(H.to_bits(kp), okp)
    assert np.array_equal(H.to_bits(vp), ovp)


@pytest.mark.parametrize("page", [32, 64, 128, 256])
def test_page_sizes_bit_exact(qil, page):
    w = make_custom([300, 1, 257, 64], [300, 1, 257, 64], hq=8, hkv=2, page=page, seed=page)
    case = H.DeviceCase(w, DEV)
    torch.cuda.synchronize()
    kp, vp = oracle_pools_all(w, case.data)
    assert np.array_equal(H.to_bits(case.kp), kp)
    assert np.array_equal(H.to_bits(case.vp), vp)


def test_empty_write_is_noop(qil):
    w = make_custom([16], [16], seed=9)
    kp, vp = H.device_pools(w, DEV)
    before = H.to_bits(kp).copy()
    e = torch.empty(0, 8, 128, dtype=torch.bfloat16, device=DEV)
    qil.kv_write(e, e, kp, vp, torch.empty(0, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert np.array_equal(H.to_bits(kp), before)
