"""Debug mode (QIL_DEBUG / qil_set_debug): every precondition on the
device-resident metadata that include/qil.h states is checked on the device
before the launch and reported as QIL_EINVAL with the first violation; valid
metadata gives the same results as without the checks."""

import numpy as np
import pytest
import torch

import paged_kv_attention_16_amd as qil_mod
from tests import harness as H
from workloads import make_custom

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture
def debug(qil):
    qil.set_debug(True)
    yield qil
    qil.set_debug(False)


def small_case(prefix=(40, 0, 70), new=(8, 20, 1), page=16):
    ctx = [p + n for p, n in zip(prefix, new)]
    w = make_custom(ctx, list(new), page=page, seed=81)
    return w, H.DeviceCase(w, DEV, write_new=False)


def expect_einval(fn, text):
    with pytest.raises(qil_mod.QilError) as ei:
        fn()
    assert ei.value.code == 1, str(ei.value)
    assert text in str(ei.value), str(ei.value)


def test_kv_write_slots(debug):
    qil = debug
    w, c = small_case()
    bad = c.new_slots.clone()
    bad[2] = w.num_pages * w.page_size          # one past the pool
    expect_einval(lambda: qil.kv_write(c.k_new, c.v_new, c.kp, c.vp, bad), "slot_mapping[2]")
    bad = c.new_slots.clone()
    bad[5] = -7
    expect_einval(lambda: qil.kv_write(c.k_new, c.v_new, c.kp, c.vp, bad), "slot_mapping[5]")
    dup = c.new_slots.clone()
    dup[9] = dup[3]
    expect_einval(lambda: qil.kv_write(c.k_new, c.v_new, c.kp, c.vp, dup), "are both")
    ok = c.new_slots.clone()
    ok[4] = -1                                  # -1 is a skip, not a violation
    qil.kv_write(c.k_new, c.v_new, c.kp, c.vp, ok)
    torch.cuda.synchronize()


def test_fused_positions(debug):
    qil = debug
    w, c = small_case()
    T = int(c.new_slots.shape[0])
    q = torch.zeros(T, w.num_q_heads, 128, dtype=torch.bfloat16, device=DEV)
    wts = torch.ones(128, dtype=torch.bfloat16, device=DEV)
    table = torch.zeros(64, 128, dtype=torch.float32, device=DEV)
    pos = torch.arange(T, dtype=torch.int32, device=DEV)
    pos[T - 1] = 64                             # == max_position
    fz = qil.QKNormRope(q, torch.empty_like(q), wts, wts, pos, table)
    expect_einval(lambda: qil.kv_write(c.k_new, c.v_new, c.kp, c.vp, c.new_slots, fuse=fz),
                  f"positions[{T - 1}]")


def test_decode_tables(debug):
    qil = debug
    w = make_custom([40, 300, 17], [1, 1, 1], page=16, seed=82, decode=True)
    c = H.DeviceCase(w, DEV)
    maxl = int(w.context_lens.max())
    q = c.q_all.contiguous()
    out = torch.empty_like(q)
    base = H.to_bits(c.decode())                # debug on, valid metadata
    qil.set_debug(False)
    assert np.array_equal(base, H.to_bits(c.decode()))
    qil.set_debug(True)
    bt = c.bt.clone()
    bt[1, 5] = -1                               # inside request 1's 300 keys
    expect_einval(lambda: qil.paged_decode(out, q, c.kp, c.vp, bt, c.ctx, maxl, float(w.scale)),
                  "block_tables[1][5]")
    bt = c.bt.clone()
    bt[0, 1] = w.num_pages                      # request 0 reads 3 pages
    expect_einval(lambda: qil.paged_decode(out, q, c.kp, c.vp, bt, c.ctx, maxl, float(w.scale)),
                  "block_tables[0][1]")
    ctx = c.ctx.clone()
    ctx[2] = 0
    expect_einval(lambda: qil.paged_decode(out, q, c.kp, c.vp, c.bt, ctx, maxl, float(w.scale)),
                  "context_lens[2] = 0")
    ctx = c.ctx.clone()
    ctx[0] = maxl + 1                           # above the host bound
    expect_einval(lambda: qil.paged_decode(out, q, c.kp, c.vp, c.bt, ctx, maxl, float(w.scale)),
                  "context_lens[0]")


def test_decode_append_context_past_table(debug):
    """A context past the host bound is reported by the debug checks of the
    fused decode step, and the slot check reads no block-table entry past the
    request's row (it stops at min(max_context_len, stride * page_size))."""
    qil = debug
    w = make_custom([40, 300, 17], [1, 1, 1], page=16, seed=83, decode=True)
    c = H.DeviceCase(w, DEV, write_new=False)
    q = c.q_all.contiguous()
    out = torch.empty_like(q)
    stride = int(c.bt.shape[1])
    maxl = stride * w.page_size                 # the largest host bound the table allows
    ctx = c.ctx.clone()
    ctx[0] = maxl + 1                           # row 0: one key past its block-table row
    expect_einval(lambda: qil.paged_decode_append(out, q, c.k_new, c.v_new, c.new_slots, c.kp, c.vp,
                                                  c.bt, ctx, maxl, float(w.scale)),
                  "context_lens[0]")
    # valid metadata still runs under the checks
    qil.paged_decode_append(out, q, c.k_new, c.v_new, c.new_slots, c.kp, c.vp, c.bt, c.ctx, maxl,
                            float(w.scale))
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()


def test_prefill_cu_seqlens(debug):
    qil = debug
    w, c = small_case()
    c_new = H.DeviceCase(w, DEV)
    q = c_new.q_all.contiguous()
    out = torch.empty_like(q)
    maxq, maxk = int(w.new_lens.max()), int(w.context_lens.max())
    cu = H.i32(w.cu_seqlens(np.arange(w.batch)), DEV)   # [0, 8, 28, 29]

    def run(cu_, ctx_=None, maxq_=maxq):
        qil.paged_prefill(out, q, c_new.kp, c_new.vp, c_new.bt, cu_,
                          c_new.ctx if ctx_ is None else ctx_, maxq_, maxk, float(w.scale))
    run(cu)                                     # valid
    torch.cuda.synchronize()
    # each case breaks exactly one condition, so the first violation is known
    expect_einval(lambda: run(H.i32([0, 10, 9, 29], DEV)), "cu_seqlens_q[2]")
    expect_einval(lambda: run(H.i32([1, 8, 28, 29], DEV)), "cu_seqlens_q[0]")
    ctx = c_new.ctx.clone()
    ctx[1] = 10                                 # 20 new tokens, context 10
    expect_einval(lambda: run(cu, ctx), "request 1 has 20 new tokens but context_len 10")
    expect_einval(lambda: run(cu, None, 16), "above max_seqlen_q 16")


def test_debug_refuses_under_capture(debug):
    qil = debug
    w = make_custom([40], [1], page=16, seed=83, decode=True)
    c = H.DeviceCase(w, DEV)
    q = c.q_all.contiguous()
    out = torch.empty_like(q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        with pytest.raises(qil_mod.QilError) as ei:
            qil.paged_decode(out, q, c.kp, c.vp, c.bt, c.ctx, 40, float(w.scale))
    assert "capture" in str(ei.value)


def test_qkv_proj_slots_and_positions(debug):
    """The projection checks the same metadata as the fused write, before
    either of its paths runs: slots in range and distinct, positions in
    [0, max_position)."""
    qil = debug
    w, c = small_case()
    T = int(c.new_slots.shape[0])
    hq, hkv = w.num_q_heads, w.num_kv_heads
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    x = torch.randn(T, 256, device=DEV, generator=g).to(torch.bfloat16)
    wt = (torch.randn((hq + 2 * hkv) * 128, 256, device=DEV, generator=g) / 16).to(torch.bfloat16)
    q_out = torch.empty(T, hq, 128, dtype=torch.bfloat16, device=DEV)
    wn = torch.ones(128, dtype=torch.bfloat16, device=DEV)
    table = torch.zeros(64, 128, dtype=torch.float32, device=DEV)
    pos = torch.arange(T, dtype=torch.int32, device=DEV)
    run = lambda slots, p: qil.qkv_proj_write(x, wt, c.kp, c.vp, slots, q_out, hq, wn, wn, p, table)
    bad = c.new_slots.clone()
    bad[1] = w.num_pages * w.page_size
    expect_einval(lambda: run(bad, pos), "slot_mapping[1]")
    dup = c.new_slots.clone()
    dup[6] = dup[2]
    expect_einval(lambda: run(dup, pos), "are both")
    badp = pos.clone()
    badp[3] = 64                                # == max_position
    expect_einval(lambda: run(c.new_slots, badp), "positions[3]")
    run(c.new_slots, pos)                       # valid metadata runs
    torch.cuda.synchronize()
