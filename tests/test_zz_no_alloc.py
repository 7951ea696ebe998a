"""qil_paged_decode_no_alloc (the decode with the library's fixed scratch
array as its workspace) against qil_paged_decode with a workspace of its
own and against the oracle: two calls in a row, the second with a smaller
input, each equal bit for bit to the workspace call (same kernels, same
split plan) and within the bf16 bar of the oracle."""

import numpy as np
import pytest
import torch

from tests import harness as H
from workloads import make_custom, make_workload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def both(qil, w, case, keys_per_split):
    q = case.q_all.contiguous()
    maxl = int(w.context_lens.max())
    with_ws = case.decode(keys_per_split=keys_per_split)
    fixed = torch.empty_like(q)
    qil.paged_decode_no_alloc(fixed, q, case.kp, case.vp, case.bt, case.ctx, maxl, float(w.scale),
                              keys_per_split=keys_per_split)
    torch.cuda.synchronize()
    return with_ws, fixed


def test_no_alloc_two_calls(qil):
    # call 1: the decode part of the Qwen3-8B-shaped step (64 requests,
    # contexts to 8,192: three splits per long request and the ordering pass)
    w5 = make_workload(5)
    dec = np.asarray(w5.decode_idx)
    w1 = make_custom(w5.context_lens[dec], np.ones(len(dec), np.int64), hq=32, hkv=8, page=16,
                     seed=401, decode=True)
    need = qil.paged_decode_workspace_size(w1.batch, 32, 8, int(w1.context_lens.max()), 16, 0)
    print(f"no-alloc call 1: batch {w1.batch}, workspace {need} bytes", flush=True)
    assert need > 0
    c1 = H.DeviceCase(w1, DEV)
    a1, b1 = both(qil, w1, c1, 0)
    assert np.array_equal(H.to_bits(a1), H.to_bits(b1))
    ref1 = H.OracleCase(w1, c1.data, range(w1.batch)).attention(range(w1.batch))
    assert H.excess(H.to_f64(b1), ref1, "bf16") <= 0
    del c1
    # call 2, smaller: 5 requests, forced 256-key splits (partials in the
    # same scratch, no ordering pass)
    w2 = make_custom([700, 33, 1, 260, 1500], [1] * 5, hq=16, hkv=8, page=16, seed=402, decode=True)
    print("no-alloc call 2: batch 5, 256-key splits", flush=True)
    c2 = H.DeviceCase(w2, DEV)
    a2, b2 = both(qil, w2, c2, 256)
    assert np.array_equal(H.to_bits(a2), H.to_bits(b2))
    ref2 = H.OracleCase(w2, c2.data, range(w2.batch)).attention(range(w2.batch))
    assert H.excess(H.to_f64(b2), ref2, "bf16") <= 0
