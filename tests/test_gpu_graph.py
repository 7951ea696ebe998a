"""Decode step captured into a HIP graph at a padded batch bucket, with the
write fused into decode and as two calls: every replay equals the eager
write + decode launches bit for bit (same split plan),
with eager work and synchronisations between replays; a smaller batch padded
into the same graph gives the same rows; and the graph's output matches the
oracle."""

import numpy as np
import pytest
import torch

from tests import harness as H
from workloads import make_custom

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def layer_cases(ctx, layers, hq=16, hkv=8, page=16, seed=51):
    """Per-layer pools over one page placement (the block tables, slots and
    lengths are shared by all layers of a step): layer l > 0 holds layer 0's
    data with K and V swapped and, for odd l, q negated.  The new token is
    written by the step itself."""
    w = make_custom(ctx, [1] * len(ctx), hq=hq, hkv=hkv, page=page, seed=seed, decode=True)
    d0 = w.gather()
    out = []
    for l in range(layers):
        d = dict(d0)
        if l > 0:
            d["k_cached"], d["v_cached"] = d0["v_cached"], d0["k_cached"]
            d["k_new"], d["v_new"] = d0["v_new"], d0["k_new"]
            if l % 2:
                d["q"] = d0["q"] ^ np.uint16(0x8000)
        out.append((w, H.DeviceCase(w, DEV, data=d, write_new=False)))
    return out


def eager_decode(case, w, max_l, keys_per_split):
    q = case.q_all.contiguous()
    out = torch.empty_like(q)
    from paged_kv_attention_16_amd import paged_decode
    paged_decode(out, q, case.kp, case.vp, case.bt, case.ctx, max_l, float(w.scale),
                 keys_per_split=keys_per_split)
    return out


@pytest.mark.parametrize("fused_write", [True, False])
def test_graph_replays_equal_eager(qil, fused_write):
    from paged_kv_attention_16_amd.graph import DecodeStepGraph, bucket_for
    ctx = [7, 300, 1025, 64, 513]
    cases = layer_cases(ctx, 2)
    w0 = cases[0][0]
    bucket = bucket_for(len(ctx))
    assert bucket == 8
    max_l, S = 2048, 256   # a fixed split size: the eager reference has the same plan
    g = DecodeStepGraph([(c.kp, c.vp) for _, c in cases], bucket, w0.num_q_heads,
                        w0.block_tables.shape[1] + 64, max_l, float(w0.scale), pad_page=0,
                        keys_per_split=S, fused_write=fused_write)
    g.update(cases[0][1].new_slots, cases[0][1].bt, cases[0][1].ctx,
             q=[c.q_all for _, c in cases], k_new=[c.k_new for _, c in cases],
             v_new=[c.v_new for _, c in cases])
    g.capture()   # its warm-up already wrote the new rows; rewriting them is idempotent
    # eager reference: the same write + decode, same max_context_len (same split plan)
    refs = []
    for w, c in cases:
        qil.kv_write(c.k_new, c.v_new, c.kp, c.vp, c.new_slots)
        # same split size, so the same split boundaries as in the graph
        refs.append(H.to_bits(eager_decode(c, w, max(ctx), S)))
    for rep in range(3):
        for o in g.out:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for l, ref in enumerate(refs):
            got = H.to_bits(g.out[l][:len(ctx)])
            assert np.array_equal(got, ref), f"replay {rep} layer {l}"
        # unrelated eager work between replays
        x = torch.randn(1 << 20, device=DEV)
        _ = (x * 2).sum().item()
        eager_decode(cases[1][1], cases[1][0], max(ctx), 0)
        torch.cuda.synchronize()
    # the graph's rows against the oracle
    for l, (w, c) in enumerate(cases):
        got = H.to_f64(g.out[l][:len(ctx)])
        ref = H.OracleCase(w, c.data, range(len(ctx))).attention(range(len(ctx)))
        assert H.excess(got, ref, "bf16") <= 0


def test_smaller_batch_in_same_graph(qil):
    from paged_kv_attention_16_amd.graph import DecodeStepGraph
    ctx = [100, 2000, 33, 700, 5, 1500]
    cases = layer_cases(ctx, 1, seed=61)
    w, c = cases[0]
    max_l = 2048
    g = DecodeStepGraph([(c.kp, c.vp)], 16, w.num_q_heads, 128, max_l,
                        float(w.scale), pad_page=int(w.block_tables[0, 0]))
    g.update(c.new_slots, c.bt, c.ctx, q=[c.q_all], k_new=[c.k_new], v_new=[c.v_new]).capture()
    full = H.to_bits(g.out[0][:6])
    # now only requests 1 and 4 are running: padded to 16 in the same graph
    sel = torch.tensor([1, 4], device=DEV)
    g.update(c.new_slots.index_select(0, sel), c.bt.index_select(0, sel),
             c.ctx.index_select(0, sel), q=[c.q_all.index_select(0, sel)],
             k_new=[c.k_new.index_select(0, sel)], v_new=[c.v_new.index_select(0, sel)])
    g.replay()
    torch.cuda.synchronize()
    got = H.to_bits(g.out[0][:2])
    assert np.array_equal(got, full[[1, 4]])
    assert g.context_lens[2:].eq(1).all() and g.slots[2:].eq(-1).all()
