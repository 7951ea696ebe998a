"""The merged QKV projection with the fused norm + RoPE + scatter epilogue
(qil_qkv_proj_write) against the oracle, in two stages.

Projection.  Products of bf16 values are exact in fp32, so the GPU's fp32
sum differs from the exact sum by at most gamma_K * sum_k |x_k w_k| with
gamma_K = K u / (1 - K u), u = 2^-24, for any summation order.  After both
sides round to bf16 the difference is at most one bf16 ulp of the oracle's
value plus that bound.  Few elements sit that close to a rounding boundary:
fewer than 1 % may differ at all.

Epilogue.  It is checked on the GPU's own rounded projection (qkv_out), fed
to the oracle's fused write (stage isolation, as the fused-write tests
state): v rows and the placement are bit-exact, and q / k rows meet the
fused-write bar (one output ulp plus the rotation bound, under 1e-3 of the
elements not bit-exact)."""

import numpy as np
import pytest
import torch

from tests import harness as H
from tests.test_gpu_fused import check_rotated
from oracle import norm_rope as o_nr
from oracle import projection as o_proj
from oracle.bf16 import bf16_to_f64
from workloads import bf16_from_f32, make_custom, make_workload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def check_projection(got_bits, x_bits, w_bits):
    ref_bits = o_proj.qkv_projection(x_bits, w_bits)
    k = x_bits.shape[1]
    u = 2.0 ** -24
    gamma = k * u / (1 - k * u)
    mag = np.abs(bf16_to_f64(x_bits)) @ np.abs(bf16_to_f64(w_bits)).T
    ref, got = bf16_to_f64(ref_bits), bf16_to_f64(got_bits)
    ulp = np.maximum(np.abs(ref), 2.0 ** -126) * 2.0 ** -7
    bound = ulp + gamma * mag
    inexact = float(np.mean(got_bits != ref_bits))
    worst = float(np.max(np.abs(got - ref) / bound))
    print(f"projection: non-exact fraction {inexact:.2e}, worst |diff|/bound {worst:.3f}", flush=True)
    assert np.all(np.abs(got - ref) <= bound)
    assert inexact < 1e-2


def run_case(qil, x_bits, w_bits, hq, hkv, page, num_pages, slots, positions, qw, kw, eps, table,
             x_pad=0):
    t, hidden = x_bits.shape
    n = (hq + 2 * hkv) * 128
    # optional padding after each activation row: a token stride above hidden
    xfull = np.zeros((t, hidden + x_pad), dtype=np.uint16)
    xfull[:, :hidden] = x_bits
    x = H.to_dev(xfull, "bf16", DEV)[:, :hidden]
    wdev = H.to_dev(w_bits, "bf16", DEV)
    raw = torch.full((num_pages, hkv, page, 128), 0x7FC0, dtype=torch.int16, device=DEV)
    kp, vp = raw.view(torch.bfloat16), raw.clone().view(torch.bfloat16)
    q_out = torch.empty(t, hq, 128, dtype=torch.bfloat16, device=DEV)
    qkv = torch.empty(t, n, dtype=torch.bfloat16, device=DEV)
    qil.qkv_proj_write(x, wdev, kp, vp, H.i32(slots, DEV), q_out, hq,
                       H.to_dev(qw, "bf16", DEV), H.to_dev(kw, "bf16", DEV),
                       H.i32(positions, DEV), torch.from_numpy(table).to(DEV), eps=eps, qkv_out=qkv)
    torch.cuda.synchronize()
    return H.to_bits(qkv), H.to_bits(q_out), H.to_bits(kp), H.to_bits(vp)


def check_case(qil, x_bits, w_bits, hq, hkv, page, num_pages, slots, positions, qw, kw, eps,
               table, x_pad=0):
    qkv, q_out, kb, vb = run_case(qil, x_bits, w_bits, hq, hkv, page, num_pages, slots, positions,
                                  qw, kw, eps, table, x_pad)
    check_projection(qkv, x_bits, w_bits)
    # epilogue on the GPU's own projection
    q, k, v = o_proj.split_qkv(qkv, hq, hkv)
    tab = table.astype(np.float64)
    cos, sin = tab[positions, :64][:, None, :], tab[positions, 64:][:, None, :]
    q_ref = o_nr.qk_norm_rope(q, qw, eps, cos, sin)
    k_ref = o_nr.qk_norm_rope(k, kw, eps, cos, sin)
    check_rotated(q_out, q_ref, q, qw, eps, cos, sin, "q")
    kb = kb.reshape(num_pages, hkv, page, 128)
    vb = vb.reshape(num_pages, hkv, page, 128)
    live = slots >= 0
    pg, off = slots[live] // page, slots[live] % page
    assert np.array_equal(vb[pg, :, off], v[live])
    check_rotated(kb[pg, :, off], k_ref[live], k[live], kw, eps, cos[live], sin[live], "k")
    mask = np.ones((num_pages, page), bool)
    mask[pg, off] = False
    assert np.all(kb.transpose(0, 2, 1, 3)[mask] == 0x7FC0)
    assert np.all(vb.transpose(0, 2, 1, 3)[mask] == 0x7FC0)


def small_case(seed, hidden, hq, hkv, ntok, page=16, drop=()):
    """ntok new tokens of a few requests (a custom workload's slots and
    positions), seeded activations and weights, some slots set to -1."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(ntok // 3 + 1, 3 * ntok, size=3)
    new = np.array([ntok // 3, ntok // 3, ntok - 2 * (ntok // 3)])
    ctx = np.maximum(ctx, new)
    w = make_custom(ctx, new, hq=hq, hkv=hkv, page=page, seed=seed)
    x_bits, w_bits = w.projection_inputs(hidden)
    slots = w.slot_mapping_new().copy()
    for i in drop:
        slots[i] = -1
    positions = w.positions_new()
    qw = bf16_from_f32(rng.uniform(0.5, 1.5, 128).astype(np.float32))
    kw = bf16_from_f32(rng.uniform(0.5, 1.5, 128).astype(np.float32))
    table = o_nr.rope_table(int(positions.max()) + 1, 128, 1.0e6)
    return x_bits, w_bits, w.num_pages, slots, positions, qw, kw, table


@pytest.mark.parametrize("hidden,hq,hkv,ntok,x_pad", [
    (64, 16, 8, 77, 0),      # one stage, a ragged token tile
    (128, 16, 8, 130, 8),    # two stages, a token stride above hidden
    (192, 32, 8, 129, 0),    # three stages, 8B head counts
    (1024, 40, 8, 200, 0),   # 14B head counts (28 head pairs), 0.6B hidden size
    (1024, 16, 8, 1100, 0),  # one round of 128-token workgroups, ragged last tile
    (512, 32, 8, 1500, 0),   # 256-token workgroups (one round of 144), ragged last tile
    (4096, 32, 8, 64, 0),    # a decode step of the 8B shape: 10 splits of the hidden dimension
    (4096, 32, 8, 16, 0),    # 16 tokens, 10 splits
    (1088, 40, 8, 1, 64),    # one token: split path, 17 64-column slices
    (192, 32, 8, 33, 8),     # 33 tokens over 3 slices, a token stride
    (2048, 16, 8, 300, 8),   # 0.6B-like heads, 3 token tiles, split path with a token stride
])
def test_small_shapes(qil, hidden, hq, hkv, ntok, x_pad):
    print(f"qkv_proj hidden={hidden} hq={hq} hkv={hkv} tokens={ntok}", flush=True)
    drop = tuple(sorted({0, ntok - 1, ntok // 2}))[:ntok - 1]  # at least one token stays
    x_bits, w_bits, npg, slots, pos, qw, kw, table = small_case(
        hidden + hq + ntok, hidden, hq, hkv, ntok, drop=drop)
    check_case(qil, x_bits, w_bits, hq, hkv, 16, npg, slots, pos, qw, kw, 1e-6, table, x_pad)


def test_qwen3_8b_layer(qil):
    """The Qwen3-8B-shaped step's new tokens (64 decode + 4 x 512 chunk
    tokens of the mixed workload, layer 0): hidden 4096, 32 q / 8 KV heads."""
    w = make_workload(5)
    x_bits, w_bits = w.projection_inputs(4096)
    print(f"qkv_proj 8B layer: tokens {x_bits.shape[0]}, hidden 4096", flush=True)
    qw, kw = w.norm_weights()
    table = o_nr.rope_table(w.max_position, 128, w.theta)
    check_case(qil, x_bits, w_bits, w.num_q_heads, w.num_kv_heads, w.page_size, w.num_pages,
               w.slot_mapping_new(), w.positions_new(), qw, kw, w.eps, table)


def test_matches_project_then_fused_write(qil):
    """Projection alone (qkv_out) followed by qil_kv_write's fused path on it
    gives rows within the fused-write bar of the one-kernel epilogue (both
    are the same arithmetic on the same rounded rows; sums of squares may be
    added in another order)."""
    hq, hkv, hidden, ntok = 32, 8, 256, 150
    x_bits, w_bits, npg, slots, pos, qw, kw, table = small_case(5, hidden, hq, hkv, ntok)
    qkv, q_out, kb, vb = run_case(qil, x_bits, w_bits, hq, hkv, 16, npg, slots, pos, qw, kw, 1e-6,
                                  table)
    qkv_dev = H.to_dev(qkv, "bf16", DEV)
    q2 = qkv_dev[:, :hq * 128]
    k2 = qkv_dev[:, hq * 128:(hq + hkv) * 128]
    v2 = qkv_dev[:, (hq + hkv) * 128:]
    raw = torch.full((npg, hkv, 16, 128), 0x7FC0, dtype=torch.int16, device=DEV)
    kp, vp = raw.view(torch.bfloat16), raw.clone().view(torch.bfloat16)
    q_out2 = torch.empty(ntok, hq, 128, dtype=torch.bfloat16, device=DEV)
    fuse = qil.QKNormRope(q2, q_out2, H.to_dev(qw, "bf16", DEV), H.to_dev(kw, "bf16", DEV),
                          H.i32(pos, DEV), torch.from_numpy(table).to(DEV), eps=1e-6,
                          num_q_heads=hq)
    qil.kv_write(k2, v2, kp, vp, H.i32(slots, DEV), fuse=fuse)
    torch.cuda.synchronize()
    assert np.array_equal(H.to_bits(vp), vb)
    same_q = float(np.mean(H.to_bits(q_out2) == q_out))
    same_k = float(np.mean(H.to_bits(kp) == kb))
    print(f"fused-write path vs epilogue: identical q {same_q:.5f}, k {same_k:.5f}", flush=True)
    assert same_q > 0.999 and same_k > 0.999


def test_zero_tokens_is_a_no_op(qil):
    x = torch.empty(0, 128, dtype=torch.bfloat16, device=DEV)
    wt = torch.zeros(32 * 128, 128, dtype=torch.bfloat16, device=DEV)
    kp = torch.zeros(4, 8, 16, 128, dtype=torch.bfloat16, device=DEV)
    vp = torch.zeros_like(kp)
    q_out = torch.empty(0, 16, 128, dtype=torch.bfloat16, device=DEV)
    e = torch.empty(0, dtype=torch.int32, device=DEV)
    wn = torch.ones(128, dtype=torch.bfloat16, device=DEV)
    table = torch.zeros(16, 128, dtype=torch.float32, device=DEV)
    qil.qkv_proj_write(x, wt, kp, vp, e, q_out, 16, wn, wn, e, table)
    torch.cuda.synchronize()
    assert int(kp.abs().sum()) == 0


@pytest.mark.parametrize("case", range(8))
def test_drawn_shapes(qil, case):
    """Seeded draws of hidden size, head counts, token count, token stride and
    dropped slots; the split path and both one-pass tile shapes all occur."""
    rng = np.random.default_rng(9200 + case)
    hidden = 64 * int(rng.integers(1, 41))
    hkv = int(rng.choice([1, 2, 4, 8]))
    hq = hkv * int(rng.choice([1, 2, 4, 5, 8]))
    if hq % 2:
        hq += hkv
    ntok = int(rng.choice([1, 7, 64, 65, 128, 129, 255, 256, 257, int(rng.integers(1, 1500))]))
    x_pad = int(rng.choice([0, 8, 64]))
    ndrop = min(ntok - 1, int(rng.integers(0, 4)))
    drop = tuple(int(i) for i in rng.choice(ntok, size=ndrop, replace=False)) if ndrop else ()
    print(f"qkv_proj drawn {case}: hidden={hidden} hq={hq} hkv={hkv} tokens={ntok} "
          f"pad={x_pad} dropped={drop}", flush=True)
    x_bits, w_bits, npg, slots, pos, qw, kw, table = small_case(
        700 + case, hidden, hq, hkv, max(ntok, 3), drop=drop)
    x_bits, slots, pos = x_bits[:ntok], slots[:ntok], pos[:ntok]
    check_case(qil, x_bits, w_bits, hq, hkv, 16, npg, slots, pos, qw, kw, 1e-6, table, x_pad)
