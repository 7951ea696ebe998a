"""The fused Q/K RMSNorm + RoPE + scatter write and the mixed step of the
Qwen3-8B-shaped workload (32 query heads / 8 KV heads, 64 decode requests
and 4 prefill chunks of 512 per layer), against the oracle.

The fused rows are rounded to bf16 at the same three points on both sides,
but the GPU works in fp32 and the oracle in fp64, so a value that lands
within fp32 error of a bf16 tie can round the other way.  Before the
rotation that moves y by one bf16 ulp (at most 2^-7 relative), and the
weight product keeps that as at most 2^-7 |y w| and its own rounding can add
one more ulp, so the weighted row can differ by 2^-6 |y w|; the rotation
carries that into the output as at most 2^-6 (|y_a cos| + |y_b sin|) -- far
more than one output ulp where the two products cancel.  The bar: every
element within one output ulp plus that bound, and fewer than 1e-3 of the
elements not bit-exact.  The same bar pins the oracle against a literal
transcription of the page's code on the CPU
(tests/test_oracle_norm_rope_literal.py).  v and the placement are
bit-exact."""

import numpy as np
import pytest
import torch

from tests import harness as H
from oracle import norm_rope as o_nr
from oracle.bf16 import bf16_to_f64, round_bf16
from workloads import make_workload, sentinel_pool

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def rotation_bound(x_bits, w_bits, eps, cos, sin):
    """2^-6 (|y_a cos| + |y_b sin|) per output element, from the oracle's
    own rounded y (the row after RMSNorm and the weight product)."""
    y = round_bf16(round_bf16(o_nr.rms_normalize(bf16_to_f64(x_bits), eps)) * bf16_to_f64(w_bits))
    half = y.shape[-1] // 2
    y1, y2 = np.abs(y[..., :half]), np.abs(y[..., half:])
    c, s = np.abs(cos), np.abs(sin)
    return 2.0 ** -6 * np.concatenate([y1 * c + y2 * s, y2 * c + y1 * s], axis=-1)


def check_rotated(got_bits, ref_bits, x_bits, w_bits, eps, cos, sin, what):
    got, ref = bf16_to_f64(got_bits), bf16_to_f64(ref_bits)
    ulp = np.maximum(np.abs(ref), 2.0 ** -126) * 2.0 ** -7
    bound = ulp + rotation_bound(x_bits, w_bits, eps, cos, sin)
    inexact = np.mean(got_bits != ref_bits)
    worst = np.max(np.abs(got - ref) / bound)
    # distance in bf16 steps (bit patterns are ordered within one sign)
    gi = got_bits.astype(np.int64)
    ri = ref_bits.astype(np.int64)
    same_sign = (gi >> 15) == (ri >> 15)
    steps = np.where(same_sign, np.abs(gi - ri), np.abs(gi & 0x7FFF) + np.abs(ri & 0x7FFF))
    print(f"fused {what}: {got_bits.size} elements, non-exact fraction {inexact:.2e}, "
          f"worst distance {int(steps.max())} bf16 ulps, {int(np.sum(steps > 2))} elements past 2 ulps, "
          f"worst |diff|/bound {worst:.3f}", flush=True)
    assert inexact < 1e-3
    assert np.all(np.abs(got - ref) <= bound)


def test_rope_table_matches_oracle(qil):
    table = torch.empty(8192, 128, dtype=torch.float32, device=DEV)
    qil.rope_cos_sin(table, 1.0e6)
    torch.cuda.synchronize()
    mine = table.cpu().numpy()
    ref = o_nr.rope_table(8192, 128, 1.0e6)
    d = np.abs(mine.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    print("rope table: entries differing", int((d > 0).sum()), "max ulp", int(d.max()), flush=True)
    assert d.max() <= 1 and (d > 0).mean() < 1e-4


def fused_case(qil, w, table_dev, data):
    dev = DEV
    kp, vp = H.device_pools(w, dev)
    qil.kv_write(H.to_dev(data["k_cached"], "bf16", dev), H.to_dev(data["v_cached"], "bf16", dev),
                 kp, vp, H.i32(data["cached_slots"], dev))
    qw, kw = w.norm_weights()
    q = H.to_dev(data["q"], "bf16", dev)
    q_out = torch.empty_like(q)
    fuse = qil.QKNormRope(q, q_out, H.to_dev(qw, "bf16", dev), H.to_dev(kw, "bf16", dev),
                          H.i32(w.positions_new(), dev), table_dev, eps=w.eps)
    qil.kv_write(H.to_dev(data["k_new"], "bf16", dev), H.to_dev(data["v_new"], "bf16", dev),
                 kp, vp, H.i32(data["new_slots"], dev), fuse=fuse)
    return data, kp, vp, q_out


def test_fused_write_stage(qil):
    w = make_workload(5)
    print("cfg5 layer 0: tokens", int(w.new_lens.sum()), flush=True)
    data = w.gather()
    k_ref, q_ref, table = H.oracle_fused(w, data)
    table_dev = torch.from_numpy(table).to(DEV)        # same table on both sides
    data, kp, vp, q_out = fused_case(qil, w, table_dev, data)
    torch.cuda.synchronize()
    kb = H.to_bits(kp).reshape(w.num_pages, 8, 16, 128)
    vb = H.to_bits(vp).reshape(w.num_pages, 8, 16, 128)
    slots = data["new_slots"]
    pg, off = slots // 16, slots % 16
    assert np.array_equal(vb[pg, :, off], data["v_new"])
    qw, kw = w.norm_weights()
    tab = table.astype(np.float64)
    pos = w.positions_new()
    cos, sin = tab[pos, :64][:, None, :], tab[pos, 64:][:, None, :]
    check_rotated(H.to_bits(q_out), q_ref, data["q"], qw, w.eps, cos, sin, "q")
    check_rotated(kb[pg, :, off], k_ref, data["k_new"], kw, w.eps, cos, sin, "k")
    # every slot not written this step still holds what it held before
    mask = np.ones((w.num_pages, 16), bool)
    mask[pg, off] = False
    cached = data["cached_slots"]
    mask[cached // 16, cached % 16] = False
    assert np.all(kb.transpose(0, 2, 1, 3)[mask] == 0x7FC0)


@pytest.mark.parametrize("layer", range(36))
def test_mixed_step_chain(qil, layer):
    """One layer of the 36-layer step, every request: fused write -> decode
    (all 64 requests) -> prefill (all 4 chunks of 512, the unsplit path the
    step runs) with the library's own RoPE table, against the oracle's own
    chain on the same seeded inputs."""
    w = make_workload(5, layer)
    table_dev = torch.empty(w.max_position, 128, dtype=torch.float32, device=DEV)
    qil.rope_cos_sin(table_dev, w.theta)
    data, kp, vp, q_out = fused_case(qil, w, table_dev, w.gather())
    q_dec = q_out[:64].contiguous()                 # decode requests come first, one row each
    bt = H.i32(w.block_tables, DEV)
    ctx = H.i32(w.context_lens, DEV)
    out_dec = torch.empty_like(q_dec)
    qil.paged_decode(out_dec, q_dec, kp, vp, bt[:64].contiguous(), ctx[:64].contiguous(),
                     int(w.context_lens[:64].max()), float(w.scale))
    q_pre = q_out[64:].contiguous()
    out_pre = torch.empty_like(q_pre)
    pre = w.prefill_idx
    qil.paged_prefill(out_pre, q_pre, kp, vp, bt[64:].contiguous(), H.i32(w.cu_seqlens(pre), DEV),
                      ctx[64:].contiguous(), 512, int(w.context_lens[64:].max()), float(w.scale))
    torch.cuda.synchronize()
    got_dec, got_pre = H.to_f64(out_dec), H.to_f64(out_pre)
    del kp, vp, out_dec, out_pre, q_out
    torch.cuda.empty_cache()

    k_ref, q_ref, _ = H.oracle_fused(w, data)
    oc = H.OracleCase(w, data, range(68), k_new=k_ref, q=q_ref)
    ref_dec = oc.attention(range(64))
    ref_pre = oc.attention(pre)
    print(f"layer {layer}: decode (64 requests) max err {np.max(np.abs(got_dec - ref_dec)):.3e}, "
          f"excess {H.excess(got_dec, ref_dec, 'bf16'):.3e}; prefill (4 x 512) max err "
          f"{np.max(np.abs(got_pre - ref_pre)):.3e}, excess {H.excess(got_pre, ref_pre, 'bf16'):.3e}",
          flush=True)
    assert H.excess(got_dec, ref_dec, "bf16") <= 0
    assert H.excess(got_pre, ref_pre, "bf16") <= 0
