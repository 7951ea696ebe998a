"""The five seeded workloads (shapes and distributions of the engines on the
pages) and their per-request input streams.

Workloads (D = 128 everywhere; "U[a, b]" is an inclusive integer uniform):
  1 tiny-f32-decode  fp32, 1 request, Hq 16 / Hkv 8, page 16, context 64 in 4
                     pages drawn from a permutation of a 16-page pool.
  2 decode-b32       bf16, 32 requests, Hq 16 / Hkv 8 (Qwen3-0.6B attention),
                     context U[128, 2048], page 16, pool 8192 pages.
  3 decode-b256      bf16, 256 requests, context U[16,1024] + U[0,1024],
                     page 256, pool ceil(1.2 x pages needed).
  4 prefill-varlen   bf16, 8 requests, cached prefix U[0, 512] + new chunk
                     U[32, 2048], page 16, Hq 16 / Hkv 8.
  5 mixed-8b         bf16, Hq 32 / Hkv 8 (Qwen3-8B attention), per layer 64
                     decode requests with context U[512, 8192] plus 4 prefill
                     chunks of 512 over a cached prefix U[0, 4096]; page 16;
                     Q/K RMSNorm weights U(0.5, 1.5), eps 1e-6, RoPE theta 1e6;
                     36 layers with independent seeds.

A request's context length L counts every key after this step's write,
including its new tokens; its new tokens are its last positions.  Pages are
placed by one permutation of the pool, handed out to requests in order; each
block-table row lists a request's pages and is padded with -1.  The slot of
logical token j of request r is its page times page_size plus j mod
page_size -- the metadata an engine's host side builds (the "nano-vLLM
learning note" ``prepare_decode`` / ``prepare_prefill`` blocks).

Randomness: numpy PCG64 streams keyed by SeedSequence([1234, cfg, layer,
stream, ...]).  Stream 0 draws lengths then the page permutation; stream
(1, r) draws request r's cached k, cached v, new k, new v and q, in that
order, as float32 standard normals (rounded to bf16 with ties-to-even for
the bf16 workloads); stream 2 draws the norm weights.  Per-request streams
let a checker regenerate any subset of requests on its own.
"""

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import hashlib
import os

import numpy as np

BASE_SEED = 1234
HEAD_DIM = 128

CONFIGS = {
    1: dict(name="tiny-f32-decode", dtype="f32", hq=16, hkv=8, page=16),
    2: dict(name="decode-b32", dtype="bf16", hq=16, hkv=8, page=16),
    3: dict(name="decode-b256", dtype="bf16", hq=16, hkv=8, page=256),
    4: dict(name="prefill-varlen", dtype="bf16", hq=16, hkv=8, page=16),
    5: dict(name="mixed-8b", dtype="bf16", hq=32, hkv=8, page=16, layers=36,
            eps=1e-6, theta=1.0e6, max_position=8192),
}

BF16_NAN = np.uint16(0x7FC0)
F32_NAN = np.uint32(0x7FC00000)


def config_names():
    return {k: v["name"] for k, v in CONFIGS.items()}


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, *key])))


def bf16_from_f32(x):
    """float32 array -> uint16 bf16 bits, round-to-nearest-even (finite
    inputs; this only shapes synthetic data)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def element_bits_dtype(dtype):
    return np.uint16 if dtype == "bf16" else np.uint32


def sentinel_pool(num_pages, num_kv_heads, page_size, head_dim, dtype):
    """A pool whose every element holds the quiet-NaN pattern, so a read of
    an unwritten slot poisons the result."""
    fill = BF16_NAN if dtype == "bf16" else F32_NAN
    return np.full((num_pages, num_kv_heads, page_size, head_dim), fill,
                   dtype=element_bits_dtype(dtype))


@dataclass
class RequestData:
    """Raw element bits of one request's inputs."""
    k_cached: np.ndarray   # [cached][Hkv][D]
    v_cached: np.ndarray
    k_new: np.ndarray      # [new][Hkv][D]
    v_new: np.ndarray
    q: np.ndarray          # [new][Hq][D]


@dataclass
class Workload:
    cfg: int
    layer: int
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    cached_lens: np.ndarray          # int64 [B]
    new_lens: np.ndarray             # int64 [B]
    block_tables: np.ndarray         # int32 [B][stride], -1 padded
    decode_idx: np.ndarray           # requests served by the decode call
    prefill_idx: np.ndarray          # requests served by the prefill call
    fused: bool = False
    eps: float = 1e-6
    theta: float = 1.0e6
    max_position: int = 0
    scale: np.float32 = field(default_factory=lambda: np.float32(1.0 / np.sqrt(HEAD_DIM)))

    # ---- shape helpers -------------------------------------------------
    @property
    def batch(self):
        return len(self.cached_lens)

    @property
    def context_lens(self):
        return (self.cached_lens + self.new_lens).astype(np.int32)

    @property
    def elem_dtype(self):
        return element_bits_dtype(self.dtype)

    @property
    def elem_bytes(self):
        return 2 if self.dtype == "bf16" else 4

    def pages_needed(self, r):
        return -(-int(self.context_lens[r]) // self.page_size)

    # ---- metadata ------------------------------------------------------
    def slots(self, r, start, stop):
        """Slots of logical tokens start..stop-1 of request r."""
        j = np.arange(start, stop, dtype=np.int64)
        pages = self.block_tables[r][j // self.page_size].astype(np.int64)
        return (pages * self.page_size + j % self.page_size).astype(np.int32)

    def cached_slots(self, r):
        return self.slots(r, 0, int(self.cached_lens[r]))

    def new_slots(self, r):
        c = int(self.cached_lens[r])
        return self.slots(r, c, c + int(self.new_lens[r]))

    def new_positions(self, r):
        c = int(self.cached_lens[r])
        return np.arange(c, c + int(self.new_lens[r]), dtype=np.int32)

    def slot_mapping_new(self, requests=None):
        reqs = range(self.batch) if requests is None else requests
        return np.concatenate([self.new_slots(r) for r in reqs]).astype(np.int32)

    def positions_new(self, requests=None):
        reqs = range(self.batch) if requests is None else requests
        return np.concatenate([self.new_positions(r) for r in reqs]).astype(np.int32)

    def cu_seqlens(self, requests):
        n = [int(self.new_lens[r]) for r in requests]
        return np.concatenate([[0], np.cumsum(n)]).astype(np.int32)

    def new_token_offset(self, r):
        """Row of request r's first new token in the all-requests packing."""
        return int(np.sum(self.new_lens[:r]))

    # ---- data ----------------------------------------------------------
    def request(self, r):
        rng = _rng(self.cfg, self.layer, 1, r)
        c, n = int(self.cached_lens[r]), int(self.new_lens[r])
        hkv, hq, d = self.num_kv_heads, self.num_q_heads, self.head_dim

        def draw(*shape):
            x = rng.standard_normal(shape, dtype=np.float32)
            if self.dtype == "bf16":
                return bf16_from_f32(x)
            return x.view(np.uint32)

        kc = draw(c, hkv, d)
        vc = draw(c, hkv, d)
        kn = draw(n, hkv, d)
        vn = draw(n, hkv, d)
        q = draw(n, hq, d)
        return RequestData(kc, vc, kn, vn, q)

    def norm_weights(self):
        """(q_norm_weight, k_norm_weight) bf16 bits, U(0.5, 1.5)."""
        rng = _rng(self.cfg, self.layer, 2)
        w = rng.uniform(0.5, 1.5, size=(2, self.head_dim)).astype(np.float32)
        b = bf16_from_f32(w)
        return b[0].copy(), b[1].copy()

    def projection_inputs(self, hidden, tokens=None):
        """Inputs of the merged QKV projection ahead of the fused write, bf16
        bits: activations x [T][hidden] ~ N(0, 1) (the input RMSNorm leaves
        rows at unit scale) and the weight [(Hq + 2 Hkv) * D][hidden] ~
        N(0, 1/hidden), so the projected rows are near unit scale, like the q,
        k and v the other configs draw directly.  T defaults to every new
        token of the workload."""
        rng = _rng(self.cfg, self.layer, 3, hidden)
        t = int(self.new_lens.sum()) if tokens is None else int(tokens)
        n = (self.num_q_heads + 2 * self.num_kv_heads) * self.head_dim
        x = rng.standard_normal((t, hidden), dtype=np.float32)
        w = rng.standard_normal((n, hidden), dtype=np.float32) * np.float32(1.0 / np.sqrt(hidden))
        return bf16_from_f32(x), bf16_from_f32(w)

    def gather(self, requests=None):
        """All requests' data concatenated in request order:
        (k_cached, v_cached, cached_slots, k_new, v_new, q, new_slots)."""
        reqs = list(range(self.batch)) if requests is None else list(requests)
        workers = max(1, min(16, len(os.sched_getaffinity(0)), len(reqs)))
        with ThreadPoolExecutor(workers) as pool:   # numpy fills drop the GIL
            parts = list(pool.map(self.request, reqs))
        cat = lambda xs: np.concatenate(xs, axis=0)
        return dict(
            k_cached=cat([p.k_cached for p in parts]),
            v_cached=cat([p.v_cached for p in parts]),
            cached_slots=np.concatenate([self.cached_slots(r) for r in reqs]).astype(np.int32),
            k_new=cat([p.k_new for p in parts]),
            v_new=cat([p.v_new for p in parts]),
            q=cat([p.q for p in parts]),
            new_slots=np.concatenate([self.new_slots(r) for r in reqs]).astype(np.int32),
        )

    def metadata_digest(self):
        h = hashlib.sha256()
        for a in (self.cached_lens, self.new_lens, self.block_tables):
            h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()

    # ---- algorithmic work ---------------------------------------------
    def decode_kv_bytes(self):
        """K+V bytes the decode call must read (each key row once)."""
        L = self.context_lens[self.decode_idx].astype(np.int64)
        return int(L.sum()) * self.num_kv_heads * self.head_dim * self.elem_bytes * 2

    def decode_io_bytes(self):
        """q read + output written by the decode call."""
        return 2 * len(self.decode_idx) * self.num_q_heads * self.head_dim * self.elem_bytes

    def prefill_pairs(self):
        """Visible (query, key) pairs per query head in the prefill call."""
        total = 0
        for r in self.prefill_idx:
            c, n = int(self.cached_lens[r]), int(self.new_lens[r])
            # new token i at position c + i sees c + i + 1 keys
            total += n * (c + 1) + n * (n - 1) // 2
        return total

    def prefill_flops(self):
        """2 * D flops for q.k plus 2 * D for p.v per visible pair and head."""
        return self.prefill_pairs() * self.num_q_heads * 4 * self.head_dim


def _uniform(rng, lo, hi, n):
    return rng.integers(lo, hi + 1, size=n, dtype=np.int64)


def make_workload(cfg, layer=0):
    spec = CONFIGS[cfg]
    rng = _rng(cfg, layer, 0)
    if cfg == 1:
        context = np.array([64], dtype=np.int64)
        new = np.ones(1, np.int64)
    elif cfg == 2:
        context = _uniform(rng, 128, 2048, 32)
        new = np.ones(32, np.int64)
    elif cfg == 3:
        context = _uniform(rng, 16, 1024, 256) + _uniform(rng, 0, 1024, 256)
        new = np.ones(256, np.int64)
    elif cfg == 4:
        prefix = _uniform(rng, 0, 512, 8)
        new = _uniform(rng, 32, 2048, 8)
        context = prefix + new
    elif cfg == 5:
        dec = _uniform(rng, 512, 8192, 64)
        prefix = _uniform(rng, 0, 4096, 4)
        context = np.concatenate([dec, prefix + 512])
        new = np.concatenate([np.ones(64, np.int64), np.full(4, 512, np.int64)])
    else:
        raise ValueError(f"unknown config {cfg}")
    cached = context - new
    page = spec["page"]
    need = -(-context // page)
    if cfg == 1:
        num_pages = 16
    elif cfg == 2:
        num_pages = 8192
    else:
        num_pages = int(np.ceil(1.2 * int(need.sum())))
    perm = rng.permutation(num_pages).astype(np.int32)
    stride = int(need.max())
    tables = np.full((len(context), stride), -1, dtype=np.int32)
    at = 0
    for r, k in enumerate(need.tolist()):
        tables[r, :k] = perm[at:at + k]
        at += k
    batch = len(context)
    if cfg in (1, 2, 3):
        dec_idx, pre_idx = np.arange(batch), np.arange(0)
    elif cfg == 4:
        dec_idx, pre_idx = np.arange(0), np.arange(batch)
    else:
        dec_idx, pre_idx = np.arange(64), np.arange(64, 68)
    return Workload(
        cfg=cfg, layer=layer, name=spec["name"], dtype=spec["dtype"],
        num_q_heads=spec["hq"], num_kv_heads=spec["hkv"], head_dim=HEAD_DIM,
        page_size=page, num_pages=num_pages, cached_lens=cached, new_lens=new,
        block_tables=tables, decode_idx=dec_idx, prefill_idx=pre_idx,
        fused=(cfg == 5), eps=spec.get("eps", 1e-6), theta=spec.get("theta", 1e6),
        max_position=spec.get("max_position", 0),
    )


def make_custom(context, new, hq=16, hkv=8, page=16, dtype="bf16", seed=0, spare_pages=7,
                decode=False):
    """A small ad-hoc workload with the same structure as the five configs
    (edge cases of the tests): given context lengths and new-token counts
    per request, pages placed by a seeded permutation with spare pages."""
    context = np.asarray(context, dtype=np.int64)
    new = np.asarray(new, dtype=np.int64)
    rng = _rng(1000 + seed, 0, 0)
    need = -(-context // page)
    num_pages = int(need.sum()) + spare_pages
    perm = rng.permutation(num_pages).astype(np.int32)
    stride = max(1, int(need.max()))
    tables = np.full((len(context), stride), -1, dtype=np.int32)
    at = 0
    for r, k in enumerate(need.tolist()):
        tables[r, :k] = perm[at:at + k]
        at += k
    idx = np.arange(len(context))
    empty = np.arange(0)
    return Workload(
        cfg=1000 + seed, layer=0, name=f"custom-{seed}", dtype=dtype, num_q_heads=hq,
        num_kv_heads=hkv, head_dim=HEAD_DIM, page_size=page, num_pages=num_pages,
        cached_lens=context - new, new_lens=new, block_tables=tables,
        decode_idx=idx if decode else empty, prefill_idx=empty if decode else idx)
