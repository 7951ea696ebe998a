"""qil_paged_prefill_append: a prefill step's write and attention in one
call.  It must leave the pools and the outputs bit for bit as
qil_kv_write followed by qil_paged_prefill, on the one-kernel path (bf16,
whole query tiles, both workgroup shapes) and on the two-call paths (a call
split over keys, fp32), and match the oracle."""

import numpy as np
import pytest
import torch

from tests import harness as H
from workloads import make_workload, make_custom

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def run_both(qil, w, keys_per_split=0, k_view=None, v_view=None):
    """(two-call case, its output, append case, its output) on the same inputs;
    the append case's pools hold only the cached rows before the call."""
    two = H.DeviceCase(w, DEV)
    out_two = two.prefill(keys_per_split=keys_per_split)
    app = H.DeviceCase(w, DEV, data=two.data, write_new=False)
    reqs = np.asarray(w.prefill_idx)
    rows = torch.from_numpy(app.rows_of(reqs)).to(DEV)
    q = app.q_all.index_select(0, rows).contiguous()
    sel = torch.from_numpy(reqs).to(DEV)
    bt = app.bt.index_select(0, sel).contiguous()
    ctx = app.ctx.index_select(0, sel).contiguous()
    cu = H.i32(w.cu_seqlens(reqs), DEV)
    k_new = app.k_new if k_view is None else k_view(app.k_new)
    v_new = app.v_new if v_view is None else v_view(app.v_new)
    out_app = torch.empty_like(q)
    qil.paged_prefill_append(out_app, q, k_new, v_new, app.new_slots, app.kp, app.vp, bt, cu, ctx,
                             int(w.new_lens[reqs].max()), int(w.context_lens[reqs].max()),
                             float(w.scale), keys_per_split=keys_per_split)
    torch.cuda.synchronize()
    return two, out_two, app, out_app


def same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.int16 if a.element_size() == 2 else torch.int32),
                       b.contiguous().view(torch.int16 if b.element_size() == 2 else torch.int32))


def test_cfg4_matches_write_then_prefill(qil):
    w = make_workload(4)
    two, out_two, app, out_app = run_both(qil, w)
    assert same_bits(app.kp, two.kp) and same_bits(app.vp, two.vp), "pools differ"
    assert same_bits(out_app, out_two), "outputs differ"
    ref = H.OracleCase(w, app.data, range(w.batch)).attention(range(w.batch))
    assert H.excess(H.to_f64(out_app), ref, "bf16") <= 0


@pytest.mark.parametrize("hq,hkv,page,long", [(16, 8, 16, False), (32, 8, 16, True),
                                               (8, 8, 64, False), (40, 8, 16, True),
                                               (64, 4, 256, False), (16, 2, 32, True)])
def test_ragged_shapes(qil, hq, hkv, page, long):
    """Chunks that straddle query and key tiles, prefixes of 0 and of several
    tiles; `long` adds a 3,000-key context, so whole tiles run as 256-row
    workgroups instead of 128-row ones."""
    ctx = [1, 65, 200, 129, 700, 33] + ([3000] if long else [])
    new = [1, 1, 200, 64, 131, 17] + ([900] if long else [])
    w = make_custom(ctx, new, hq=hq, hkv=hkv, page=page, seed=hq + hkv + page)
    two, out_two, app, out_app = run_both(qil, w)
    assert same_bits(app.kp, two.kp) and same_bits(app.vp, two.vp)
    assert same_bits(out_app, out_two)
    ref = H.OracleCase(w, app.data, range(w.batch)).attention(range(w.batch))
    assert H.excess(H.to_f64(out_app), ref, "bf16") <= 0


def test_split_call_runs_two_kernels(qil):
    """One 512-token chunk over a 7,680-key prefix is split over keys: the
    call writes, then runs the split prefill; same bits as the two calls."""
    w = make_custom([8192], [512], hq=32, hkv=8, page=16, seed=77)
    two, out_two, app, out_app = run_both(qil, w)
    assert same_bits(app.kp, two.kp) and same_bits(app.vp, two.vp)
    assert same_bits(out_app, out_two)


def test_fp32_runs_two_kernels(qil):
    w = make_custom([300, 40, 1000], [100, 40, 257], page=32, dtype="f32", seed=78)
    two, out_two, app, out_app = run_both(qil, w)
    assert same_bits(app.kp, two.kp) and same_bits(app.vp, two.vp)
    assert same_bits(out_app, out_two)


def test_strided_rows(qil):
    """k_new / v_new as views into a wider per-token buffer (a fused QKV
    output): token strides above the row length."""
    w = make_custom([200, 700, 64], [200, 131, 64], page=16, seed=79)

    def widen(x):
        t = x.shape[0]
        buf = torch.full((t, 3 * x.shape[1] * x.shape[2]), float("nan"), dtype=x.dtype, device=DEV)
        view = buf[:, 128:128 + x.shape[1] * x.shape[2]]
        view.copy_(x.reshape(t, -1))
        return view
    two, out_two, app, out_app = run_both(qil, w, k_view=widen, v_view=widen)
    assert same_bits(app.kp, two.kp) and same_bits(app.vp, two.vp)
    assert same_bits(out_app, out_two)


def test_skipped_slots_are_not_written(qil):
    """slot -1 stores nothing: those pool rows keep their sentinel bits, and
    every other new row lands as in kv_write."""
    w = make_custom([300, 90], [100, 90], page=16, seed=80)
    app = H.DeviceCase(w, DEV, write_new=False)
    before_k = app.kp.clone()
    slots = app.new_slots.clone()
    skip = torch.arange(0, slots.numel(), 7, device=DEV)
    slots[skip] = -1
    reqs = np.asarray(w.prefill_idx)
    q = app.q_all.contiguous()
    out = torch.empty_like(q)
    qil.paged_prefill_append(out, q, app.k_new, app.v_new, slots, app.kp, app.vp, app.bt,
                             H.i32(w.cu_seqlens(reqs), DEV), app.ctx, int(w.new_lens.max()),
                             int(w.context_lens.max()), float(w.scale))
    torch.cuda.synchronize()
    ref = H.DeviceCase(w, DEV, data=app.data, write_new=False)
    qil.kv_write(ref.k_new, ref.v_new, ref.kp, ref.vp, slots)
    torch.cuda.synchronize()
    assert same_bits(app.kp, ref.kp) and same_bits(app.vp, ref.vp)
    assert not same_bits(app.kp, before_k)
    assert bool(torch.isfinite(out).all())
