"""qil_paged_decode on the GPU against the oracle: the three decode
workloads (fp32 at 1e-5, bf16 at 2e-2 abs/rel), split-count invariance,
run-twice determinism, the bit-exact block-table indexing probe, page
permutation invariance, single-key and GQA 32:8 cases."""

import numpy as np
import pytest
import torch

from tests import harness as H
from workloads import make_workload, make_custom, bf16_from_f32

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_cfg1_fp32(qil):
    w = make_workload(1)
    got, ref = H.run_decode_case(w, DEV)
    print("cfg1 max abs err", np.max(np.abs(got - ref)), flush=True)
    assert H.excess(got, ref, "f32") <= 0


def test_cfg2_bf16_all_requests(qil):
    w = make_workload(2)
    got, ref = H.run_decode_case(w, DEV)
    print("cfg2 max abs err", np.max(np.abs(got - ref)), flush=True)
    assert H.excess(got, ref, "bf16") <= 0


def test_cfg3_bf16_full_size_sampled(qil):
    w = make_workload(3)
    L = w.context_lens
    sample = sorted(set([int(np.argmin(L)), int(np.argmax(L))] +
                        np.random.default_rng(0).choice(w.batch, 22, replace=False).tolist()))
    got, ref = H.run_decode_case(w, DEV, requests=sample)
    print("cfg3 sampled", len(sample), "max abs err", np.max(np.abs(got - ref)), flush=True)
    assert H.excess(got, ref, "bf16") <= 0


@pytest.mark.parametrize("split", [64, 128, 512, 4096])
def test_split_invariance(qil, split):
    w = make_workload(2)
    case = H.DeviceCase(w, DEV)
    auto = H.to_f64(case.decode())
    forced = H.to_f64(case.decode(keys_per_split=split))
    torch.cuda.synchronize()
    assert np.max(np.abs(auto - forced)) < 1e-2
    ref = H.OracleCase(w, case.data, range(4)).attention(range(4))
    assert H.excess(forced[:4], ref, "bf16") <= 0


@pytest.mark.parametrize("split", [256, 4096])
def test_longest_first_order_is_invisible(qil, split):
    """The B = 256 workload's grid (2,048 workgroups and more) runs its
    requests longest first; each request's output equals, bit for bit, the
    same request decoded in a batch of 4, whose small grid runs in batch
    order (the split size is fixed, so both use the same splits)."""
    w = make_workload(3)
    case = H.DeviceCase(w, DEV)
    full = H.to_bits(case.decode(keys_per_split=split))
    rng = np.random.default_rng(4)
    L = w.context_lens
    groups = [[int(np.argmax(L)), int(np.argmin(L)), 7, 200]] + \
             [sorted(rng.choice(w.batch, 4, replace=False).tolist()) for _ in range(5)]
    for grp in groups:
        small = H.to_bits(case.decode(requests=grp, keys_per_split=split))
        assert np.array_equal(full[grp], small), grp
    print(f"split {split}: {len(groups)} groups of 4 match the full batch bit for bit", flush=True)


@pytest.mark.parametrize("dtype,batch,page", [("bf16", 3000, 16), ("bf16", 256, 16),
                                               ("bf16", 257, 16), ("f32", 200, 32)])
def test_ordered_large_batches(qil, dtype, batch, page):
    """Grids far past one round of the GPU run longest first: 3,000 bf16
    requests (the ordering kernel's strided loops), 256 bf16 requests (the
    most that the decode workgroups rank themselves) and 257 (the first batch
    that takes the ordering kernel), and 200 fp32 requests, contexts from 1 to
    a few hundred keys (many equal lengths).
    Every output row is written (the output starts as NaN), sampled requests
    match the oracle, and the same requests decoded 3 at a time match bit for
    bit."""
    rng = np.random.default_rng(batch)
    ctx = rng.integers(1, 400 if dtype == "bf16" else 300, size=batch)
    w = make_custom(ctx, np.ones(batch, np.int64), page=page, dtype=dtype, seed=batch % 97,
                    decode=True)
    print(f"{dtype} batch {batch}: {batch * 8} workgroups", flush=True)
    case = H.DeviceCase(w, DEV)
    sample = sorted(set([int(np.argmax(ctx)), int(np.argmin(ctx))] +
                        rng.choice(batch, 10, replace=False).tolist()))
    got, ref = H.run_decode_case(w, DEV, requests=sample, keys_per_split=256, case=case)
    assert H.excess(got, ref, dtype) <= 0
    out = torch.full_like(case.q_all, float("nan"))
    full_out = case.decode(keys_per_split=256, out=out)
    assert bool(torch.isfinite(full_out).all()), "a request of the batch was not decoded"
    full = H.to_bits(full_out)
    for i in range(0, len(sample), 3):
        grp = sample[i:i + 3]
        assert np.array_equal(full[grp], H.to_bits(case.decode(requests=grp, keys_per_split=256)))


def test_ranked_small_batch_many_splits(qil):
    """A batch of 3 whose grid still takes the longest-first order (3 requests
    x 8 KV heads x 24 splits of 256 keys = 576 workgroups), so every
    workgroup ranks the 3 requests itself, two of them with nearly equal
    lengths.  All rows are written, match the oracle, and match each request
    decoded alone (a 192-workgroup grid in batch order) bit for bit."""
    ctx = [6000, 100, 6001]
    w = make_custom(ctx, [1, 1, 1], page=16, seed=31, decode=True)
    case = H.DeviceCase(w, DEV)
    out = torch.full_like(case.q_all, float("nan"))
    full_out = case.decode(keys_per_split=256, out=out)
    assert bool(torch.isfinite(full_out).all())
    torch.cuda.synchronize()
    ref = H.OracleCase(w, case.data, range(3)).attention(range(3))
    assert H.excess(H.to_f64(full_out), ref, "bf16") <= 0
    full = H.to_bits(full_out)
    for r in range(3):
        assert np.array_equal(full[[r]], H.to_bits(case.decode(requests=[r], keys_per_split=256)))


def test_run_twice_bitwise(qil):
    w = make_workload(2)
    case = H.DeviceCase(w, DEV)
    a = H.to_bits(case.decode(keys_per_split=128))
    b = H.to_bits(case.decode(keys_per_split=128))
    assert np.array_equal(a, b)


def probe_workload(page, hq=16, hkv=8):
    lengths = [1, 15, 16, 17, 250, 513, 1000, 2048]
    w = make_custom(lengths, [1] * len(lengths), hq=hq, hkv=hkv, page=page, seed=page, decode=True)
    data = w.gather()
    # one-hot softmax: key j* of request r matches q in every dim, all other
    # keys oppose it; the score gap (~5800) underflows every other weight.
    targets = [(7 * r + 3) % L for r, L in enumerate(lengths)]
    ks, vs = [], []
    for r, L in enumerate(lengths):
        k = np.full((L, hkv, 128), -16.0, np.float32)
        k[targets[r]] = 16.0
        # V row (r, j, g) holds small exact integers
        j = np.arange(L)[:, None, None]
        g = np.arange(hkv)[None, :, None]
        d = np.arange(128)[None, None, :]
        v = ((j * 3 + g * 5 + d + r) % 200).astype(np.float32) - 100.0
        ks.append(bf16_from_f32(k))
        vs.append(bf16_from_f32(v))
    kc = np.concatenate([k[:-1] for k in ks]); vc = np.concatenate([v[:-1] for v in vs])
    kn = np.stack([k[-1] for k in ks]); vn = np.stack([v[-1] for v in vs])
    data.update(k_cached=kc, v_cached=vc, k_new=kn, v_new=vn,
                q=bf16_from_f32(np.full((len(lengths), hq, 128), 16.0, np.float32)))
    expect = np.stack([np.repeat(vs[r][targets[r]], hq // hkv, axis=0) for r in range(len(lengths))])
    return w, data, expect


@pytest.mark.parametrize("page", [16, 64, 256])
def test_indexing_probe_bit_exact(qil, page):
    w, data, expect = probe_workload(page)
    case = H.DeviceCase(w, DEV, data=data)
    for split in (0, 64, 256):
        out = H.to_bits(case.decode(keys_per_split=split))
        assert np.array_equal(out, expect), f"split {split}"


def test_page_permutation_invariance_bitwise(qil):
    w = make_workload(2)
    case = H.DeviceCase(w, DEV)
    base = H.to_bits(case.decode())
    perm = torch.from_numpy(np.random.default_rng(1).permutation(w.num_pages).astype(np.int64)).to(DEV)
    kp2 = torch.empty_like(case.kp); vp2 = torch.empty_like(case.vp)
    kp2[perm] = case.kp; vp2[perm] = case.vp
    bt = case.bt.long()
    case.bt = torch.where(bt >= 0, perm[bt.clamp(min=0)], bt).int()
    case.kp, case.vp = kp2, vp2
    moved = H.to_bits(case.decode())
    assert np.array_equal(base, moved)


def test_single_key_returns_v(qil):
    w = make_custom([1, 1, 1], [1, 1, 1], page=16, seed=4, decode=True)
    case = H.DeviceCase(w, DEV)
    out = H.to_bits(case.decode())
    v = case.data["v_new"]                               # [3][Hkv][D]
    assert np.array_equal(out, np.repeat(v, 2, axis=1))


@pytest.mark.parametrize("hq,hkv,page", [(32, 8, 16), (8, 8, 32), (64, 8, 128), (4, 1, 16),
                                         (40, 8, 16), (64, 4, 64)])
def test_gqa_shapes(qil, hq, hkv, page):
    w = make_custom([700, 33, 4096, 5, 129], [1] * 5, hq=hq, hkv=hkv, page=page, seed=hq + page,
                    decode=True)
    got, ref = H.run_decode_case(w, DEV)
    assert H.excess(got, ref, "bf16") <= 0


def test_fp32_ragged(qil):
    w = make_custom([1, 63, 64, 65, 300, 1024], [1] * 6, page=16, dtype="f32", seed=11, decode=True)
    for split in (0, 64):
        got, ref = H.run_decode_case(w, DEV, keys_per_split=split)
        assert H.excess(got, ref, "f32") <= 0


@pytest.mark.parametrize("split", [0, 64])
def test_max_jumps_across_groups_and_splits(qil, split):
    # Keys whose scores jump by ~10 in base 2 at several points of a long
    # context: every running maximum, the cross-row and cross-wave merges and
    # the split merge see large corrections.
    from oracle import bf16 as obf
    w = make_custom([1000, 300], [1, 1], hq=32, hkv=8, page=16, seed=41, decode=True)
    d = w.gather()
    kc = obf.bf16_to_f64(d["k_cached"]).astype(np.float32)
    q = obf.bf16_to_f64(d["q"]).astype(np.float32)
    for r0, n in ((0, 999), (999, 299)):   # cached rows of each request
        for frac, mag in ((0.1, 10.0), (0.35, 30.0), (0.6, 50.0), (0.9, 70.0)):
            kc[r0 + int(frac * n), :, 0] = mag
    q[:, :, 0] = 4.0
    d["k_cached"] = bf16_from_f32(kc)
    d["q"] = bf16_from_f32(q)
    case = H.DeviceCase(w, DEV, data=d)
    got, ref = H.run_decode_case(w, DEV, keys_per_split=split, case=case)
    print("spiked decode max abs err", np.max(np.abs(got - ref)), flush=True)
    assert H.excess(got, ref, "bf16") <= 0
