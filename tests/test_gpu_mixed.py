"""qil_paged_attention_mixed: the decode batch and the prefill batch of a step
in one launch.  Prefill tiles run the same device code as qil_paged_prefill's
whole query tiles, and decode splits the same code and split plan as
qil_paged_decode, so both must match the separate calls bit for bit, and the
oracle within the bf16 tolerance.  Either batch may be absent."""

import numpy as np
import pytest
import torch

from tests import harness as H
from workloads import make_workload, make_custom

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def split_step(w, case, dec_reqs, pre_reqs):
    """Device tensors of the decode part and the prefill part of a workload."""
    def part(reqs):
        sel = torch.from_numpy(np.asarray(reqs)).to(DEV)
        rows = torch.from_numpy(case.rows_of(reqs)).to(DEV)
        q = case.q_all.index_select(0, rows).contiguous()
        return dict(q=q, out=torch.empty_like(q), block_tables=case.bt.index_select(0, sel).contiguous(),
                    context_lens=case.ctx.index_select(0, sel).contiguous(),
                    max_context_len=int(w.context_lens[reqs].max()))
    dec = part(dec_reqs) if len(dec_reqs) else None
    pre = None
    if len(pre_reqs):
        pre = part(pre_reqs)
        pre["cu_seqlens_q"] = H.i32(w.cu_seqlens(np.asarray(pre_reqs)), DEV)
        pre["max_seqlen_q"] = int(w.new_lens[pre_reqs].max())
    return dec, pre


def separate(qil, w, case, dec, pre):
    out_d = out_p = None
    if dec is not None:
        out_d = torch.empty_like(dec["q"])
        qil.paged_decode(out_d, dec["q"], case.kp, case.vp, dec["block_tables"], dec["context_lens"],
                         dec["max_context_len"], float(w.scale))
    if pre is not None:
        # the single launch runs whole query tiles: so does this call (one
        # piece spans every context), which makes the two bitwise comparable
        out_p = torch.empty_like(pre["q"])
        whole = (pre["max_context_len"] + 63) // 64 * 64
        qil.paged_prefill(out_p, pre["q"], case.kp, case.vp, pre["block_tables"], pre["cu_seqlens_q"],
                          pre["context_lens"], pre["max_seqlen_q"], pre["max_context_len"],
                          float(w.scale), keys_per_split=whole)
    torch.cuda.synchronize()
    return out_d, out_p


def test_mixed_step_8b_layer(qil):
    w = make_workload(5, 0)
    case = H.DeviceCase(w, DEV)
    dec_reqs, pre_reqs = list(range(64)), [64, 65, 66, 67]
    dec, pre = split_step(w, case, dec_reqs, pre_reqs)
    qil.paged_attention_mixed(case.kp, case.vp, float(w.scale), decode=dec, prefill=pre)
    sep_d, sep_p = separate(qil, w, case, dec, pre)
    assert np.array_equal(H.to_bits(pre["out"]), H.to_bits(sep_p))
    assert np.array_equal(H.to_bits(dec["out"]), H.to_bits(sep_d))
    dsel = list(range(64))
    ref = H.OracleCase(w, case.data, dsel).attention(dsel)
    got = H.to_f64(dec["out"])
    print("mixed decode max err", np.max(np.abs(got - ref)), flush=True)
    assert H.excess(got, ref, "bf16") <= 0


@pytest.mark.parametrize("hq,hkv", [(16, 8), (32, 8), (8, 8), (16, 2), (40, 8), (64, 4)])
def test_mixed_small_groups(qil, hq, hkv):
    # decode requests (1 new token) and prefill requests in one workload
    ctx = [700, 33, 1, 260, 1500, 90, 64]
    new = [1, 1, 1, 200, 37, 90, 1]
    w = make_custom(ctx, new, hq=hq, hkv=hkv, page=16, seed=91)
    case = H.DeviceCase(w, DEV)
    dec_reqs, pre_reqs = [0, 1, 2, 6], [3, 4, 5]
    dec, pre = split_step(w, case, dec_reqs, pre_reqs)
    qil.paged_attention_mixed(case.kp, case.vp, float(w.scale), decode=dec, prefill=pre)
    torch.cuda.synchronize()
    ref = H.OracleCase(w, case.data, range(w.batch))
    got_d = H.to_f64(dec["out"])
    ref_d = ref.attention(dec_reqs)
    assert H.excess(got_d, ref_d, "bf16") <= 0
    got_p = H.to_f64(pre["out"])
    ref_p = ref.attention(pre_reqs)
    assert H.excess(got_p, ref_p, "bf16") <= 0


def test_mixed_one_side_only(qil):
    w = make_custom([300, 40, 1000], [1, 1, 120], page=16, seed=92)
    case = H.DeviceCase(w, DEV)
    dec, pre = split_step(w, case, [0, 1], [2])
    qil.paged_attention_mixed(case.kp, case.vp, float(w.scale), decode=dec)
    qil.paged_attention_mixed(case.kp, case.vp, float(w.scale), prefill=pre)
    sep_d, sep_p = separate(qil, w, case, dec, pre)
    assert np.array_equal(H.to_bits(pre["out"]), H.to_bits(sep_p))
    assert np.array_equal(H.to_bits(dec["out"]), H.to_bits(sep_d))
