"""The seeded workloads: determinism, distributions within their stated
ranges, disjoint page placement, -1 padding and slot consistency."""

import hashlib

import numpy as np
import pytest

from workloads import make_workload


def digest(w, requests):
    h = hashlib.sha256(w.metadata_digest().encode())
    for r in requests:
        d = w.request(r)
        for a in (d.k_cached, d.v_cached, d.k_new, d.v_new, d.q):
            h.update(a.tobytes())
    return h.hexdigest()


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_deterministic(cfg):
    a, b = make_workload(cfg), make_workload(cfg)
    reqs = [0, a.batch - 1]
    assert digest(a, reqs) == digest(b, reqs)
    if cfg == 5:
        assert make_workload(5, 1).metadata_digest() != a.metadata_digest()


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_structure(cfg):
    w = make_workload(cfg)
    L = w.context_lens
    need = -(-L // w.page_size)
    bt = w.block_tables
    used = np.concatenate([bt[r, :need[r]] for r in range(w.batch)])
    assert len(np.unique(used)) == len(used)              # disjoint pages
    assert used.min() >= 0 and used.max() < w.num_pages
    for r in range(w.batch):
        assert np.all(bt[r, need[r]:] == -1)
    slots = np.concatenate([w.cached_slots(r) for r in range(w.batch)] + [w.slot_mapping_new()])
    assert len(np.unique(slots)) == len(slots)            # every slot written once
    if cfg == 1:
        assert L.tolist() == [64] and w.num_pages == 16 and need.tolist() == [4]
    if cfg == 2:
        assert w.batch == 32 and L.min() >= 128 and L.max() <= 2048 and w.num_pages == 8192
    if cfg == 3:
        assert w.batch == 256 and L.min() >= 16 and L.max() <= 2048
        assert w.num_pages == int(np.ceil(1.2 * need.sum()))
    if cfg == 4:
        assert np.all((w.new_lens >= 32) & (w.new_lens <= 2048)) and np.all(w.cached_lens <= 512)
    if cfg == 5:
        assert len(w.decode_idx) == 64 and len(w.prefill_idx) == 4
        assert np.all(w.new_lens[w.prefill_idx] == 512) and np.all(w.cached_lens[w.prefill_idx] <= 4096)
        assert np.all((L[w.decode_idx] >= 512) & (L[w.decode_idx] <= 8192))
        assert w.positions_new().max() < w.max_position
        qw, kw = w.norm_weights()
        assert qw.shape == (128,) and kw.dtype == np.uint16


def test_request_streams_are_independent():
    w = make_workload(3)
    a = w.request(5).q
    w.request(6)
    assert np.array_equal(a, w.request(5).q)
