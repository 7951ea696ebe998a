"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments with the documented codes before
any HIP call (so these calls never reach the device)."""

import ctypes
import os
import re

import pytest

import paged_kv_attention_16_amd as qil

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qil.h")

EINVAL, EUNSUP, EWS = 1, 2, 3
FAKE = 0x100000  # 16-byte aligned, never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    # QIL_ABI_LIB: another build of the library (the host-sanitized one)
    other = os.environ.get("QIL_ABI_LIB")
    if other:
        return qil.load(other)
    if not os.path.exists(qil.lib_path()):
        import __graft_entry__
        __graft_entry__.build()
    return qil.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(qil_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert {"qil_kv_write", "qil_paged_decode", "qil_paged_prefill"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.qil_version().decode().startswith("qil ")


def kvw(lib, **kw):
    a = dict(k=FAKE, v=FAKE, ks=1024, vs=1024, kc=FAKE, vc=FAKE, slots=FAKE, T=4, hkv=8, d=128,
             page=16, pages=10, dtype=1, fuse=None)
    a.update(kw)
    return lib.qil_kv_write(a["k"], a["v"], a["ks"], a["vs"], a["kc"], a["vc"], a["slots"], a["T"],
                            a["hkv"], a["d"], a["page"], a["pages"], a["dtype"], a["fuse"], None)


def test_kv_write_validation(lib):
    assert kvw(lib, T=0) == 0                      # no-op, no HIP call
    assert kvw(lib, T=-1) == EINVAL
    assert kvw(lib, k=None) == EINVAL
    assert kvw(lib, k=FAKE + 4) == EINVAL          # misaligned
    assert kvw(lib, ks=1000) == EINVAL             # stride below a row
    assert kvw(lib, ks=1028) == EINVAL             # stride not a multiple of 8
    assert kvw(lib, d=64) == EUNSUP
    assert kvw(lib, page=48) == EUNSUP
    assert kvw(lib, page=8) == EUNSUP
    assert kvw(lib, dtype=7) == EUNSUP
    assert kvw(lib, pages=0) == EINVAL
    assert kvw(lib, T=2**27, hkv=8, ks=2048, vs=2048) == EINVAL  # 2^30 rows + 2^30 V rows
    assert "page_size" in lib.qil_last_error().decode() or True
    f = qil._QKNormRopeC(FAKE, FAKE, 4096, 32, FAKE, FAKE, 1e-6, FAKE, FAKE, 8192)
    assert kvw(lib, fuse=ctypes.pointer(f), dtype=0) == EUNSUP   # fused is bf16 only
    f2 = qil._QKNormRopeC(FAKE, FAKE, 4096, 12, FAKE, FAKE, 1e-6, FAKE, FAKE, 8192)
    assert kvw(lib, fuse=ctypes.pointer(f2)) == EINVAL           # 12 % 8 != 0
    f3 = qil._QKNormRopeC(FAKE, FAKE, 8192, 32, FAKE, FAKE, 1e-6, FAKE, FAKE, 8192)
    assert kvw(lib, fuse=ctypes.pointer(f3)) == EINVAL           # in place needs contiguous q
    f4 = qil._QKNormRopeC(FAKE, FAKE + 4096 * 64, 4096, 32, None, FAKE, 1e-6, FAKE, FAKE, 8192)
    assert kvw(lib, fuse=ctypes.pointer(f4)) == EINVAL           # null weight


def qkvp(lib, **kw):
    a = dict(x=FAKE, xs=4096, w=FAKE, ws=4096, hidden=4096, q_out=FAKE, qkv=None, kc=FAKE, vc=FAKE,
             slots=FAKE, T=4, hq=32, hkv=8, d=128, page=16, pages=10, qw=FAKE, kw=FAKE, eps=1e-6,
             pos=FAKE, cs=FAKE, maxpos=8192, work=FAKE, workb=1 << 30, dtype=1)
    a.update(kw)
    return lib.qil_qkv_proj_write(a["x"], a["xs"], a["w"], a["ws"], a["hidden"], a["q_out"],
                                  a["qkv"], a["kc"], a["vc"], a["slots"], a["T"], a["hq"], a["hkv"],
                                  a["d"], a["page"], a["pages"], a["qw"], a["kw"], a["eps"],
                                  a["pos"], a["cs"], a["maxpos"], a["work"], a["workb"],
                                  a["dtype"], None)


def test_qkv_proj_validation(lib):
    assert qkvp(lib, T=0) == 0                     # no-op, no HIP call
    assert qkvp(lib, T=-1) == EINVAL
    assert qkvp(lib, dtype=0) == EUNSUP            # bf16 only
    assert qkvp(lib, hq=31) == EUNSUP              # 31 + 16 heads: odd
    assert qkvp(lib, hidden=4000, xs=4000, ws=4000) == EUNSUP   # not a multiple of 64
    assert qkvp(lib, xs=4088) == EINVAL            # stride below hidden
    assert qkvp(lib, ws=4100) == EINVAL            # stride not a multiple of 8
    assert qkvp(lib, d=64) == EUNSUP
    assert qkvp(lib, page=8) == EUNSUP
    assert qkvp(lib, pages=0) == EINVAL
    assert qkvp(lib, maxpos=0) == EINVAL
    assert qkvp(lib, eps=-1.0) == EINVAL
    assert qkvp(lib, x=None) == EINVAL
    assert qkvp(lib, kw=None) == EINVAL
    assert qkvp(lib, w=FAKE + 8) == EINVAL         # misaligned
    assert qkvp(lib, qkv=FAKE + 2) == EINVAL       # misaligned optional output
    # small batches split the hidden dimension and need the workspace
    need = lib.qil_qkv_proj_workspace_size(64, 32, 8, 4096)
    assert need == 10 * 64 * 48 * 128 * 4            # 10 splits (240 workgroups) of fp32 partials
    assert lib.qil_qkv_proj_workspace_size(2112, 32, 8, 4096) == 0
    assert lib.qil_qkv_proj_workspace_size(64, 32, 8, 4000) == 0
    assert qkvp(lib, T=64, work=None, workb=0) == EWS
    assert qkvp(lib, T=64, workb=need - 1) == EWS
    assert qkvp(lib, T=64, work=FAKE + 4) == EWS


def dec(lib, **kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, bts=128, ctx=FAKE, B=2, hq=16, hkv=8,
             d=128, page=16, pages=8192, maxL=2048, scale=0.088, dtype=1, S=0, ws=None, wsb=0)
    a.update(kw)
    return lib.qil_paged_decode(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["bts"], a["ctx"],
                                a["B"], a["hq"], a["hkv"], a["d"], a["page"], a["pages"], a["maxL"],
                                a["scale"], a["dtype"], a["S"], a["ws"], a["wsb"], None)


def test_decode_validation(lib):
    # 2 requests x 8 KV heads over up to 2048 keys: the plan splits (256 keys)
    need = lib.qil_paged_decode_workspace_size(2, 16, 8, 2048, 16, 0)
    assert need > 0
    assert lib.qil_paged_decode_workspace_size(1, 16, 8, 64, 16, 0) == 0   # one split: none
    assert lib.qil_paged_decode_workspace_size(32, 16, 8, 2048, 16, 0) == 0  # one split per request
    assert lib.qil_paged_decode_workspace_size(2, 16, 8, 2048, 16, 4096) == 0
    assert dec(lib, B=0) == 0
    assert dec(lib) == EWS                          # workspace missing
    assert dec(lib, ws=FAKE, wsb=need - 1) == EWS
    assert dec(lib, hq=12) == EINVAL
    assert dec(lib, hq=24) == EUNSUP                # G = 3
    assert dec(lib, hq=48) == EUNSUP                # G = 6
    assert dec(lib, hq=128, dtype=0) == EUNSUP      # fp32 is built up to G = 8
    assert dec(lib, d=256) == EUNSUP
    assert dec(lib, page=1) == EUNSUP
    assert dec(lib, S=100) == EINVAL                # not a multiple of 64
    assert dec(lib, maxL=128 * 16 + 1) == EINVAL    # beyond the block table
    assert dec(lib, maxL=0) == EINVAL
    assert dec(lib, q=None) == EINVAL
    assert dec(lib, scale=float("nan")) == EINVAL
    assert dec(lib, dtype=3) == EUNSUP
    assert len(lib.qil_last_error()) > 0


def pre(lib, **kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, bts=200, cu=FAKE, ctx=FAKE, B=8, T=8000,
             maxq=2048, maxL=2560, hq=16, hkv=8, d=128, page=16, pages=900, scale=0.088, dtype=1,
             kps=0, ws=None, wsb=0)
    a.update(kw)
    return lib.qil_paged_prefill(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["bts"], a["cu"],
                                 a["ctx"], a["B"], a["T"], a["maxq"], a["maxL"], a["hq"], a["hkv"],
                                 a["d"], a["page"], a["pages"], a["scale"], a["dtype"], a["kps"],
                                 a["ws"], a["wsb"], None)


def test_prefill_validation(lib):
    assert pre(lib, B=0) == 0
    assert pre(lib, T=0) == 0
    assert pre(lib, dtype=2) == EUNSUP              # no such dtype
    # fp32 runs on the fp32 decode kernel: contexts up to 4,096 keys, G <= 8,
    # at most 65,535 tokens
    assert pre(lib, dtype=0, maxL=5000, bts=400) == EUNSUP
    assert pre(lib, dtype=0, hq=32, hkv=2) == EUNSUP
    assert pre(lib, dtype=0, T=70000) == EUNSUP
    assert pre(lib, maxq=9000) == EINVAL            # above total_q
    assert pre(lib, maxL=100) == EINVAL             # below max_seqlen_q
    assert pre(lib, maxL=200 * 16 + 1) == EINVAL
    assert pre(lib, cu=None) == EINVAL
    assert pre(lib, hq=16, hkv=3) == EINVAL
    assert pre(lib, page=512) == EUNSUP
    assert pre(lib, B=-1) == EINVAL
    assert pre(lib, kps=100) == EINVAL              # not a multiple of 64
    assert pre(lib, kps=-64) == EINVAL
    assert pre(lib, kps=64 * 1024) == EINVAL        # above 65472


def pre_app(lib, **kw):
    a = dict(out=FAKE, q=FAKE, kn=FAKE, vn=FAKE, ks=1024, vs=1024, slots=FAKE, kc=FAKE, vc=FAKE,
             bt=FAKE, bts=200, cu=FAKE, ctx=FAKE, B=8, T=8000, maxq=2048, maxL=2560, hq=16,
             hkv=8, d=128, page=16, pages=900, scale=0.088, dtype=1, kps=0, ws=None, wsb=0)
    a.update(kw)
    return lib.qil_paged_prefill_append(
        a["out"], a["q"], a["kn"], a["vn"], a["ks"], a["vs"], a["slots"], a["kc"], a["vc"],
        a["bt"], a["bts"], a["cu"], a["ctx"], a["B"], a["T"], a["maxq"], a["maxL"], a["hq"],
        a["hkv"], a["d"], a["page"], a["pages"], a["scale"], a["dtype"], a["kps"], a["ws"],
        a["wsb"], None)


def test_prefill_append_validation(lib):
    assert pre_app(lib, B=0) == 0
    assert pre_app(lib, T=0) == 0
    # the prefill's own checks come first
    assert pre_app(lib, maxq=9000) == EINVAL
    assert pre_app(lib, cu=None) == EINVAL
    assert pre_app(lib, dtype=2) == EUNSUP
    assert pre_app(lib, kps=100) == EINVAL
    # then the new rows and their slots
    assert pre_app(lib, kn=None) == EINVAL
    assert pre_app(lib, slots=None) == EINVAL
    assert pre_app(lib, vn=FAKE + 8) == EINVAL       # misaligned
    assert pre_app(lib, ks=1000) == EINVAL           # stride below a row
    assert pre_app(lib, vs=1028) == EINVAL           # stride not a multiple of 8
    # a call split over keys needs its workspace, as qil_paged_prefill
    assert pre_app(lib, B=1, T=512, maxq=512, maxL=8192, hq=32, hkv=8, bts=512) == EWS
    assert len(lib.qil_last_error()) > 0


def test_prefill_split_workspace(lib):
    ws = lib.qil_paged_prefill_workspace_size
    # 8 chunks of up to 2,048 tokens: 568 query tiles x KV heads, never split automatically
    assert ws(8, 8000, 2048, 2560, 16, 8, 0) == 0
    # an explicit split of the same call needs a workspace; longer pieces need no more
    s1024 = ws(8, 8000, 2048, 2560, 16, 8, 1024)
    assert s1024 > 0 and ws(8, 8000, 2048, 2560, 16, 8, 2048) <= s1024
    assert ws(8, 8000, 2048, 2560, 16, 8, 4096) == 0    # every tile fits one piece
    # one 512-token chunk over an 8k context (Hq 32 / Hkv 8): 64 tiles, split automatically
    auto = ws(1, 512, 512, 8192, 32, 8, 0)
    assert auto > 0
    # at most 32 pieces per tile: a tiny keys_per_split is raised, so the size is bounded
    assert ws(1, 512, 512, 8192, 32, 8, 64) == ws(1, 512, 512, 8192, 32, 8, 256)
    # more than 4,096 query tiles in the plan: unsplit
    assert ws(5000, 5000, 1, 4096, 16, 8, 1024) == 0
    assert ws(1, 512, 512, 8192, 32, 8, 100) == 0       # invalid keys_per_split
    # calls that need a workspace reject a missing, short or misaligned one
    kw = dict(B=1, T=512, maxq=512, maxL=8192, hq=32, hkv=8, bts=512)
    assert pre(lib, **kw) == EWS
    assert pre(lib, ws=FAKE, wsb=auto - 1, **kw) == EWS
    assert pre(lib, ws=FAKE + 4, wsb=auto, **kw) == EWS
    assert pre(lib, kps=4096, **kw) == EWS             # two explicit 4k-key pieces
    assert ws(1, 512, 512, 8192, 32, 8, 8192) == 0       # one piece covers every tile


def app(lib, **kw):
    a = dict(out=FAKE, q=FAKE, kn=FAKE, vn=FAKE, ks=1024, vs=1024, slots=FAKE, kc=FAKE, vc=FAKE,
             bt=FAKE, bts=128, ctx=FAKE, B=4, hq=16, hkv=8, d=128, page=16, pages=100, maxL=2048,
             scale=0.088, dtype=1, S=0, ws=None, wsb=0)
    a.update(kw)
    return lib.qil_paged_decode_append(a["out"], a["q"], a["kn"], a["vn"], a["ks"], a["vs"],
                                       a["slots"], a["kc"], a["vc"], a["bt"], a["bts"], a["ctx"],
                                       a["B"], a["hq"], a["hkv"], a["d"], a["page"], a["pages"],
                                       a["maxL"], a["scale"], a["dtype"], a["S"], a["ws"], a["wsb"],
                                       None)


def test_decode_append_validation(lib):
    need = lib.qil_paged_decode_workspace_size(4, 16, 8, 2048, 16, 0)
    ok = dict(ws=FAKE, wsb=need)
    assert app(lib, B=0) == 0
    assert app(lib, kn=None, **ok) == EINVAL
    assert app(lib, slots=None, **ok) == EINVAL
    assert app(lib, vn=FAKE + 4, **ok) == EINVAL        # misaligned
    assert app(lib, ks=1000, **ok) == EINVAL            # below num_kv_heads*head_dim
    assert app(lib, vs=1028, **ok) == EINVAL            # not a multiple of 8
    assert app(lib, hq=24, **ok) == EUNSUP
    assert app(lib, dtype=3, **ok) == EUNSUP
    if need > 0:
        assert app(lib) == EWS                          # workspace missing


def test_rope_table_validation(lib):
    assert lib.qil_rope_cos_sin(None, 10, 128, 1e6, None) == EINVAL
    assert lib.qil_rope_cos_sin(FAKE, 0, 128, 1e6, None) == EINVAL
    assert lib.qil_rope_cos_sin(FAKE, 10, 64, 1e6, None) == EUNSUP
    assert lib.qil_rope_cos_sin(FAKE, 10, 128, 0.5, None) == EINVAL


def test_mixed_validation(lib):
    args = (FAKE, FAKE, 16, 8, 128, 16, 100, 0.088)
    assert lib.qil_paged_attention_mixed(None, None, *args, 1, None) == 0      # nothing to do
    assert lib.qil_paged_attention_mixed(None, None, *args, 0, None) == EUNSUP  # bf16 only
    d = qil._DecodeBatchC(FAKE, FAKE, FAKE, 128, FAKE, 2, 2048, 0, None, 0)
    assert lib.qil_paged_attention_mixed(ctypes.pointer(d), None, *args, 1, None) == EWS
    p = qil._PrefillBatchC(FAKE, FAKE, FAKE, 200, FAKE, FAKE, 8, 8000, 9000, 2560)
    assert lib.qil_paged_attention_mixed(None, ctypes.pointer(p), *args, 1, None) == EINVAL


def test_debug_switch(lib):
    was = lib.qil_debug_enabled()
    lib.qil_set_debug(1)
    assert lib.qil_debug_enabled() == 1
    lib.qil_set_debug(0)
    assert lib.qil_debug_enabled() == 0
    lib.qil_set_debug(was)


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(qil.QilError):
        qil.load(str(tmp_path / "missing.so"))


def test_decode_no_alloc_rejects_above_its_scratch(lib):
    """The fixed-scratch decode refuses, before any HIP call, a shape whose
    workspace would exceed the library's 32 MiB array."""
    def call(**kw):
        a = dict(B=2, hq=16, hkv=8, maxL=2048, S=0, bts=128)
        a.update(kw)
        return lib.qil_paged_decode_no_alloc(FAKE, FAKE, FAKE, FAKE, FAKE, a["bts"], FAKE, a["B"],
                                             a["hq"], a["hkv"], 128, 16, 8192, a["maxL"], 0.088, 1,
                                             a["S"], None)
    big = dict(B=4096, hq=64, hkv=8, maxL=16384, S=1024, bts=1024)
    need = lib.qil_paged_decode_workspace_size(4096, 64, 8, 16384, 16, 1024)
    assert need > 32 << 20
    assert call(**big) == EWS
    assert b"scratch" in lib.qil_last_error()
    assert call(hq=12) == EINVAL                    # the usual checks run too
    assert call(S=100) == EINVAL
