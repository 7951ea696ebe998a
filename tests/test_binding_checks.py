"""Host-only checks of the Python binding's argument validation (CPU
tensors, no GPU): the binding rejects, before any library call, what the C
ABI cannot see on raw pointers -- a tensor whose dtype differs from the
pools', int64 or non-contiguous metadata, a non-contiguous q or out, shapes
that disagree -- and a call whose tensors are all valid but live on the host
fails because they are not GPU memory."""

import pytest
import torch

import paged_kv_attention_16_amd as qil

BF, F32, I32 = torch.bfloat16, torch.float32, torch.int32


def pools(dtype=BF, pages=8, hkv=2, page=16):
    return (torch.zeros(pages, hkv, page, 128, dtype=dtype),
            torch.zeros(pages, hkv, page, 128, dtype=dtype))


def decode_args(**kw):
    kp, vp = pools()
    a = dict(out=torch.zeros(3, 4, 128, dtype=BF), q=torch.zeros(3, 4, 128, dtype=BF), k_cache=kp,
             v_cache=vp, block_tables=torch.zeros(3, 4, dtype=I32),
             context_lens=torch.ones(3, dtype=I32), max_context_len=64, scale=0.088)
    a.update(kw)
    return a


def expect(fn, text):
    with pytest.raises(qil.QilError) as ei:
        fn()
    assert ei.value.code == 1 and text in str(ei.value), str(ei.value)


def test_decode_checks():
    run = lambda **kw: qil.paged_decode(**decode_args(**kw))
    expect(lambda: run(q=torch.zeros(3, 4, 128, dtype=F32)), "q has dtype torch.float32")
    expect(lambda: run(out=torch.zeros(3, 4, 128, dtype=F32)), "out has dtype")
    expect(lambda: run(out=torch.zeros(3, 2, 128, dtype=BF)), "out shape")
    expect(lambda: run(q=torch.zeros(3, 128, 4, dtype=BF).transpose(1, 2)), "q must be contiguous")
    expect(lambda: run(block_tables=torch.zeros(3, 4, dtype=torch.int64)), "block_tables has dtype")
    expect(lambda: run(block_tables=torch.zeros(4, 3, dtype=I32).t()), "block_tables must be contiguous")
    expect(lambda: run(context_lens=torch.ones(3, dtype=torch.int64)), "context_lens has dtype")
    expect(lambda: run(context_lens=torch.ones(2, dtype=I32)), "context_lens has 2 entries")
    kp, _ = pools(F32)
    expect(lambda: run(k_cache=kp), "v_cache has dtype")
    expect(lambda: run(), "must be GPU tensors")          # every check passes on the host


def test_decode_append_checks():
    a = decode_args()
    a["k_new"] = torch.zeros(3, 2, 128, dtype=BF)
    a["v_new"] = torch.zeros(3, 2, 128, dtype=BF)
    a["slot_mapping"] = torch.zeros(3, dtype=I32)

    def run(**kw):
        b = dict(a, **kw)
        qil.paged_decode_append(b["out"], b["q"], b["k_new"], b["v_new"], b["slot_mapping"],
                                b["k_cache"], b["v_cache"], b["block_tables"], b["context_lens"],
                                b["max_context_len"], b["scale"])
    expect(lambda: run(k_new=torch.zeros(3, 2, 128, dtype=F32)), "k_new has dtype")
    expect(lambda: run(slot_mapping=torch.zeros(3, dtype=torch.int64)), "slot_mapping has dtype")
    expect(lambda: run(v_new=torch.zeros(2, 2, 128, dtype=BF)), "one row per request")
    expect(lambda: run(), "must be GPU tensors")


def test_prefill_checks():
    kp, vp = pools()

    def run(**kw):
        a = dict(out=torch.zeros(10, 4, 128, dtype=BF), q=torch.zeros(10, 4, 128, dtype=BF),
                 block_tables=torch.zeros(2, 4, dtype=I32), cu=torch.tensor([0, 4, 10], dtype=I32),
                 ctx=torch.tensor([8, 6], dtype=I32))
        a.update(kw)
        qil.paged_prefill(a["out"], a["q"], kp, vp, a["block_tables"], a["cu"], a["ctx"], 6, 8, 0.088)
    expect(lambda: run(cu=torch.tensor([0, 4, 10], dtype=torch.int64)), "cu_seqlens_q has dtype")
    expect(lambda: run(cu=torch.tensor([0, 10], dtype=I32)), "cu_seqlens_q has 2 entries, expected 3")
    expect(lambda: run(q=torch.zeros(10, 4, 128, dtype=F32)), "q has dtype")
    expect(lambda: run(out=torch.zeros(9, 4, 128, dtype=BF)), "out shape")
    expect(lambda: run(ctx=torch.tensor([[8, 6]], dtype=I32)), "context_lens must have 1 dimensions")
    expect(lambda: run(), "must be GPU tensors")


def test_prefill_append_checks():
    kp, vp = pools()

    def run(**kw):
        a = dict(out=torch.zeros(10, 4, 128, dtype=BF), q=torch.zeros(10, 4, 128, dtype=BF),
                 k_new=torch.zeros(10, 2, 128, dtype=BF), v_new=torch.zeros(10, 2, 128, dtype=BF),
                 slots=torch.zeros(10, dtype=I32), block_tables=torch.zeros(2, 4, dtype=I32),
                 cu=torch.tensor([0, 4, 10], dtype=I32), ctx=torch.tensor([8, 6], dtype=I32))
        a.update(kw)
        qil.paged_prefill_append(a["out"], a["q"], a["k_new"], a["v_new"], a["slots"], kp, vp,
                                 a["block_tables"], a["cu"], a["ctx"], 6, 8, 0.088)
    expect(lambda: run(k_new=torch.zeros(10, 2, 128, dtype=F32)), "k_new has dtype")
    expect(lambda: run(v_new=torch.zeros(9, 2, 128, dtype=BF)), "one row per new token")
    expect(lambda: run(slots=torch.zeros(10, dtype=torch.int64)), "slot_mapping has dtype")
    expect(lambda: run(slots=torch.zeros(9, dtype=I32)), "slot_mapping has 9 entries")
    expect(lambda: run(cu=torch.tensor([0, 4, 10], dtype=torch.int64)), "cu_seqlens_q has dtype")
    expect(lambda: run(out=torch.zeros(10, 4, 128, dtype=F32)), "out has dtype")
    expect(lambda: run(), "must be GPU tensors")


def test_kv_write_checks():
    kp, vp = pools()
    k = torch.zeros(5, 2, 128, dtype=BF)
    slots = torch.zeros(5, dtype=I32)
    expect(lambda: qil.kv_write(k.float(), k, kp, vp, slots), "k has dtype")
    expect(lambda: qil.kv_write(k, k, kp, vp, slots.long()), "slot_mapping has dtype")
    expect(lambda: qil.kv_write(k, k, kp, vp, slots[:4]), "slot_mapping has 4 entries, expected 5")
    expect(lambda: qil.kv_write(k, k, kp, vp, torch.zeros(10, dtype=I32)[::2]), "slot_mapping must be contiguous")
    expect(lambda: qil.kv_write(k, k, kp, pools(pages=9)[1], slots), "shapes differ")
    # a strided row view (a slice of a fused QKV buffer) passes the binding's checks
    qkv = torch.zeros(5, 6, 128, dtype=BF)
    expect(lambda: qil.kv_write(qkv[:, 2:4], qkv[:, 4:6], kp, vp, slots), "must be GPU tensors")


def test_fused_write_checks():
    kp, vp = pools()
    k = torch.zeros(5, 2, 128, dtype=BF)
    slots = torch.zeros(5, dtype=I32)
    q = torch.zeros(5, 4, 128, dtype=BF)
    w = torch.ones(128, dtype=BF)
    table = torch.zeros(16, 128, dtype=F32)
    pos = torch.zeros(5, dtype=I32)
    fz = lambda **kw: qil.QKNormRope(**dict(dict(q=q, q_out=torch.empty_like(q), q_norm_weight=w,
                                                 k_norm_weight=w, positions=pos, cos_sin=table), **kw))
    expect(lambda: qil.kv_write(k, k, kp, vp, slots, fuse=fz(cos_sin=table.double())), "fuse.cos_sin has dtype")
    expect(lambda: qil.kv_write(k, k, kp, vp, slots, fuse=fz(positions=pos.long())), "fuse.positions has dtype")
    expect(lambda: qil.kv_write(k, k, kp, vp, slots, fuse=fz(q_norm_weight=w.float())), "fuse.q_norm_weight")
    expect(lambda: qil.kv_write(k, k, kp, vp, slots, fuse=fz(positions=pos[:3])), "fuse.positions must have one entry per token")
    expect(lambda: qil.kv_write(k, k, kp, vp, slots, fuse=fz()), "must be GPU tensors")


def test_mixed_checks():
    kp, vp = pools()
    a = decode_args()
    dec = dict(out=a["out"], q=a["q"], block_tables=a["block_tables"], context_lens=a["context_lens"],
               max_context_len=64)
    bad = dict(dec, context_lens=torch.ones(3, dtype=torch.int64))
    expect(lambda: qil.paged_attention_mixed(kp, vp, 0.088, decode=bad), "decode context_lens has dtype")
    expect(lambda: qil.paged_attention_mixed(kp, vp, 0.088), "give a decode batch")
    expect(lambda: qil.paged_attention_mixed(kp, vp, 0.088, decode=dec), "must be GPU tensors")
