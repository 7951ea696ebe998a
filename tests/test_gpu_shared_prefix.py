"""Shared-prefix pages (prefix caching): requests whose block tables point
at the same read-only physical pages for a common prompt prefix.  The
"nano-vLLM learning note" BlockManager shares whole blocks of identical
token prefixes between sequences by reference count (its Block and
hash_blocks / allocate blocks); only full blocks are shared, and a request's
own tokens go to its own pages.  The kernels need nothing new for it: the
results over shared pages must equal, bit for bit, the results over private
copies of the same prefix, and both must match the oracle."""

import numpy as np
import pytest
import torch

from tests import harness as H
from workloads import bf16_from_f32, sentinel_pool
from oracle import attention as o_attn
from oracle import paged as o_paged

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
P, HQ, HKV, D = 16, 16, 8, 128
SCALE = np.float32(1.0 / np.sqrt(128.0))


def bits(rng, *shape):
    return bf16_from_f32(rng.standard_normal(shape).astype(np.float32))


def build(shared, prefix_pages, tails, new, seed=71):
    """Pools and tables for requests with `prefix_pages` full shared pages,
    then `tails[r]` private tokens of which the last `new[r]` are queries.
    shared=False gives every request a private copy of the prefix."""
    rng = np.random.default_rng(seed)
    B = len(tails)
    Lp = prefix_pages * P
    k_pre, v_pre = bits(rng, Lp, HKV, D), bits(rng, Lp, HKV, D)
    k_tail = [bits(rng, t, HKV, D) for t in tails]
    v_tail = [bits(rng, t, HKV, D) for t in tails]
    q = [bits(rng, n, HQ, D) for n in new]
    ctx = np.array([Lp + t for t in tails])
    tail_pages = [-(-t // P) for t in tails]
    n_pages = (prefix_pages if shared else B * prefix_pages) + sum(tail_pages) + 3
    perm = np.random.default_rng(seed + 1).permutation(n_pages).astype(np.int32)
    at = 0
    stride = prefix_pages + max(tail_pages)
    bt = np.full((B, stride), -1, np.int32)
    if shared:
        common = perm[at:at + prefix_pages]
        at += prefix_pages
    for r in range(B):
        if shared:
            bt[r, :prefix_pages] = common
        else:
            bt[r, :prefix_pages] = perm[at:at + prefix_pages]
            at += prefix_pages
        bt[r, prefix_pages:prefix_pages + tail_pages[r]] = perm[at:at + tail_pages[r]]
        at += tail_pages[r]
    # writes: the prefix once per distinct page set, the tails per request
    ks, vs, slots = [], [], []
    for r in range(B):
        if r == 0 or not shared:
            j = np.arange(Lp)
            ks.append(k_pre); vs.append(v_pre)
            slots.append(bt[r, j // P] * P + j % P)
        j = Lp + np.arange(tails[r])
        ks.append(k_tail[r]); vs.append(v_tail[r])
        slots.append(bt[r, j // P] * P + j % P)
    k_all, v_all = np.concatenate(ks), np.concatenate(vs)
    slot_all = np.concatenate(slots).astype(np.int32)
    return dict(bt=bt, ctx=ctx, new=np.array(new), q=np.concatenate(q), k=k_all, v=v_all,
                slots=slot_all, n_pages=n_pages)


def device_run(c, decode):
    import paged_kv_attention_16_amd as qil
    kp = torch.full((c["n_pages"], HKV, P, D), 0x7FC0, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    vp = kp.clone()
    qil.kv_write(H.to_dev(c["k"], "bf16", DEV), H.to_dev(c["v"], "bf16", DEV), kp, vp,
                 H.i32(c["slots"], DEV))
    q = H.to_dev(c["q"], "bf16", DEV)
    out = torch.empty_like(q)
    bt, ctx = H.i32(c["bt"], DEV), H.i32(c["ctx"], DEV)
    if decode:
        qil.paged_decode(out, q, kp, vp, bt, ctx, int(c["ctx"].max()), float(SCALE))
    else:
        cu = H.i32(np.concatenate([[0], np.cumsum(c["new"])]), DEV)
        qil.paged_prefill(out, q, kp, vp, bt, cu, ctx, int(c["new"].max()), int(c["ctx"].max()),
                          float(SCALE))
    torch.cuda.synchronize()
    return H.to_bits(out)


def oracle_run(c):
    kp = sentinel_pool(c["n_pages"], HKV, P, D, "bf16")
    vp = sentinel_pool(c["n_pages"], HKV, P, D, "bf16")
    o_paged.kv_write(kp, vp, c["k"], c["v"], c["slots"], P)
    cu = np.concatenate([[0], np.cumsum(c["new"])])
    return o_attn.paged_attention(c["q"], kp, vp, c["bt"], cu, c["ctx"], SCALE, P, "bf16")


@pytest.mark.parametrize("decode", [True, False])
def test_shared_equals_private_copies(qil, decode):
    tails = [5, 40, 77, 130]
    new = [1, 1, 1, 1] if decode else [5, 17, 64, 130]
    sh = build(True, 18, tails, new)
    pr = build(False, 18, tails, new)
    got_sh = device_run(sh, decode)
    got_pr = device_run(pr, decode)
    assert np.array_equal(got_sh, got_pr)
    ref = oracle_run(sh)
    got = got_sh.astype(np.uint32) << 16
    assert H.excess(got.view(np.float32).astype(np.float64), ref, "bf16") <= 0
