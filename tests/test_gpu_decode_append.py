"""qil_paged_decode_append (the decode step's write and decode in one call)
against the two calls it replaces and against the oracle: the outputs and
the whole pools bitwise, at the decode workloads' shapes, with forced splits
that put the new token in every wavefront and group position, GQA group
sizes, fp32, and the debug-mode check of the slot precondition."""

import numpy as np
import pytest
import torch

import paged_kv_attention_16_amd as qil
from tests import harness as H
from workloads import make_custom, make_workload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def append_case(w, keys_per_split=0):
    """(append output, append pools, separate output, separate pools)."""
    sep = H.DeviceCase(w, DEV)                      # cached rows, then the new rows written
    app = H.DeviceCase(w, DEV, data=sep.data, write_new=False)
    reqs = np.asarray(w.decode_idx)
    assert np.array_equal(reqs, np.arange(w.batch))
    maxl = int(w.context_lens.max())
    out_sep = sep.decode(keys_per_split=keys_per_split)
    out_app = torch.empty_like(app.q_all)
    qil.paged_decode_append(out_app, app.q_all, app.k_new, app.v_new, app.new_slots, app.kp, app.vp,
                            app.bt, app.ctx, maxl, float(w.scale), keys_per_split=keys_per_split)
    torch.cuda.synchronize()
    return out_app, app, out_sep, sep


def check_identical(w, keys_per_split=0):
    out_app, app, out_sep, sep = append_case(w, keys_per_split)
    assert np.array_equal(H.to_bits(out_app), H.to_bits(out_sep)), "outputs differ"
    assert np.array_equal(H.to_bits(app.kp), H.to_bits(sep.kp)), "K pools differ"
    assert np.array_equal(H.to_bits(app.vp), H.to_bits(sep.vp)), "V pools differ"
    ref = H.OracleCase(w, sep.data, range(w.batch)).attention(range(w.batch))
    assert H.excess(H.to_f64(out_app), ref, w.dtype) <= 0


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_decode_workloads(qil, cfg):
    w = make_workload(cfg)
    print(f"decode append, workload {cfg}: batch {w.batch}", flush=True)
    check_identical(w)


@pytest.mark.parametrize("kps", [64, 128, 256])
def test_new_token_in_every_position(qil, kps):
    # contexts whose last key falls in each 16-key group of each of the four
    # wavefronts of a split, at the start, middle and end of a split
    lens = [1, 2, 15, 16, 17, 31, 32, 33, 48, 63, 64, 65, 100, 127, 128, 129, 255, 256, 257, 700]
    w = make_custom(lens, [1] * len(lens), page=16, seed=kps, decode=True)
    print(f"decode append, keys_per_split {kps}", flush=True)
    check_identical(w, kps)


@pytest.mark.parametrize("hq,hkv,page", [(32, 8, 16), (64, 4, 64), (40, 8, 256), (4, 1, 32)])
def test_group_sizes_and_pages(qil, hq, hkv, page):
    w = make_custom([700, 33, 4096, 5, 129, 1], [1] * 6, hq=hq, hkv=hkv, page=page,
                    seed=hq + page, decode=True)
    print(f"decode append hq={hq} hkv={hkv} page={page}", flush=True)
    check_identical(w)


def test_fp32(qil):
    w = make_custom([1, 63, 64, 65, 300, 1024], [1] * 6, page=16, dtype="f32", seed=11, decode=True)
    check_identical(w, 64)


def test_debug_mode_checks_the_slot(qil):
    w = make_custom([40, 70], [1, 1], page=16, seed=12, decode=True)
    app = H.DeviceCase(w, DEV, write_new=False)
    out = torch.empty_like(app.q_all)
    # request 1's last position (69) sits at offset 5 of its page: offset 6
    # is a free slot of the pool, but not that position's
    wrong = app.new_slots.clone()
    wrong[1] += 1
    qil.set_debug(True)
    try:
        with pytest.raises(qil.QilError) as err:
            qil.paged_decode_append(out, app.q_all, app.k_new, app.v_new, wrong, app.kp, app.vp,
                                    app.bt, app.ctx, 70, float(w.scale))
        assert "last position" in str(err.value)
        qil.paged_decode_append(out, app.q_all, app.k_new, app.v_new, app.new_slots, app.kp,
                                app.vp, app.bt, app.ctx, 70, float(w.scale))
    finally:
        qil.set_debug(False)
    torch.cuda.synchronize()


def test_debug_mode_context_past_the_table_row(qil):
    """A context length past its block-table row (and past max_context_len)
    is reported as a bad context, and the slot check that runs after the
    table check reads no block-table entry for that request (the last row of
    the table is the one whose read would leave the table)."""
    w = make_custom([40, 300, 17], [1, 1, 1], page=16, seed=13, decode=True)
    app = H.DeviceCase(w, DEV, write_new=False)
    out = torch.empty_like(app.q_all)
    stride = int(app.bt.shape[1])
    ctx = app.ctx.clone()
    ctx[2] = stride * 16 + 1                    # one key past request 2's table row
    qil.set_debug(True)
    try:
        # max_context_len itself may not exceed the table row (checked on the host)
        for maxl in (int(w.context_lens.max()), stride * 16):
            with pytest.raises(qil.QilError) as err:
                qil.paged_decode_append(out, app.q_all, app.k_new, app.v_new, app.new_slots, app.kp,
                                        app.vp, app.bt, ctx, maxl, float(w.scale))
            assert err.value.code == 1 and "context_lens[2]" in str(err.value), str(err.value)
    finally:
        qil.set_debug(False)
    torch.cuda.synchronize()
