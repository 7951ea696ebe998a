"""HIP-graph capture of the decode step at padded batch buckets.

A serving loop runs the same decode step every iteration: for each layer,
write the new tokens' K/V rows into the pool, then run paged decode.  Each
launch costs host time, and at small batches that host time, not the GPU,
sets the pace.  The "nano-vLLM learning note" (ModelRunner, its
capture_cudagraph block) records the model's decode step once per batch
size of a fixed list (1, 2, 4, 8, then steps of 16 up to 512) against static
input buffers and replays the graph of the smallest size that holds the
running batch; the "qwen-engine" README credits graph replay with most of
its decode throughput.

`DecodeStepGraph` does the same for the attention part of the step.  It owns
static buffers sized for one bucket, pads a smaller batch up to the bucket,
captures `layers x qil_paged_decode_append` (the write fused into the decode
kernel; `fused_write=False` captures `qil_kv_write, qil_paged_decode`
instead) into a HIP graph (torch.cuda.CUDAGraph, which is hipGraph on ROCm)
and replays it.  Every
kernel in the graph is a libqil kernel; the library calls contain no host
synchronisation, allocation or memset, so they capture as they are.

Padding rows (batch <= r < bucket) write nothing (slot -1) and decode one key
from `pad_page`, so they cost one page read each; their outputs are
meaningless and are not part of `out`'s first `batch` rows.
"""

import paged_kv_attention_16_amd as qil

__all__ = ["DEFAULT_BUCKETS", "bucket_for", "DecodeStepGraph"]

# 1, 2, 4, 8, then every multiple of 16 up to 512.
DEFAULT_BUCKETS = (1, 2, 4, 8) + tuple(range(16, 513, 16))


def bucket_for(batch, buckets=DEFAULT_BUCKETS):
    """The smallest bucket that holds `batch` requests."""
    for b in sorted(buckets):
        if b >= batch:
            return b
    raise ValueError(f"batch {batch} exceeds the largest bucket {max(buckets)}")


class DecodeStepGraph:
    """The decode step of `len(pools)` layers at one batch bucket.

    pools            list of (k_cache, v_cache) per layer, each
                     [num_pages, num_kv_heads, page_size, 128]
    bucket           batch size the graph is recorded at
    num_q_heads      query heads per token
    bt_stride        block-table columns (pages per request at most)
    max_context_len  host bound on every context length the graph will see:
                     it sizes the split grid, so it is fixed at capture
    scale            q.k scale
    pad_page         a valid page id that padding rows read (one key)

    Static buffers, filled by `update` before `replay`:
      q[l], k_new[l], v_new[l], out[l]  [bucket, H, 128] per layer
      slots [bucket], block_tables [bucket, bt_stride], context_lens [bucket]
    """

    def __init__(self, pools, bucket, num_q_heads, bt_stride, max_context_len, scale,
                 pad_page=0, keys_per_split=0, fused_write=True):
        import torch
        self.pools = list(pools)
        k0 = self.pools[0][0]
        self.device = k0.device
        self.dtype = k0.dtype
        _, hkv, page, d = (int(x) for x in k0.shape)
        self.bucket, self.hq, self.hkv, self.page = int(bucket), int(num_q_heads), hkv, page
        self.bt_stride = int(bt_stride)
        self.max_context_len = int(max_context_len)
        self.scale = float(scale)
        self.pad_page = int(pad_page)
        self.keys_per_split = int(keys_per_split)
        self.fused_write = bool(fused_write)
        B, dev = self.bucket, self.device
        if self.max_context_len > self.bt_stride * page:
            raise qil.QilError(1, "max_context_len exceeds bt_stride * page_size")
        self.q = [torch.zeros(B, self.hq, d, dtype=self.dtype, device=dev) for _ in self.pools]
        self.out = [torch.zeros(B, self.hq, d, dtype=self.dtype, device=dev) for _ in self.pools]
        self.k_new = [torch.zeros(B, hkv, d, dtype=self.dtype, device=dev) for _ in self.pools]
        self.v_new = [torch.zeros(B, hkv, d, dtype=self.dtype, device=dev) for _ in self.pools]
        self.slots = torch.full((B,), -1, dtype=torch.int32, device=dev)
        self.block_tables = torch.full((B, self.bt_stride), -1, dtype=torch.int32, device=dev)
        self.block_tables[:, 0] = self.pad_page
        self.context_lens = torch.ones(B, dtype=torch.int32, device=dev)
        need = qil.paged_decode_workspace_size(B, self.hq, hkv, self.max_context_len, page,
                                               self.keys_per_split)
        self.workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        self.batch = 0
        self.graph = None

    # ---- the step, as issued eagerly or under capture ----------------------
    def run_eager(self):
        """Issue the step's launches on the current stream."""
        for l, (kc, vc) in enumerate(self.pools):
            if self.fused_write:
                qil.paged_decode_append(self.out[l], self.q[l], self.k_new[l], self.v_new[l],
                                        self.slots, kc, vc, self.block_tables, self.context_lens,
                                        self.max_context_len, self.scale,
                                        keys_per_split=self.keys_per_split,
                                        workspace=self.workspace)
                continue
            qil.kv_write(self.k_new[l], self.v_new[l], kc, vc, self.slots)
            qil.paged_decode(self.out[l], self.q[l], kc, vc, self.block_tables, self.context_lens,
                             self.max_context_len, self.scale, keys_per_split=self.keys_per_split,
                             workspace=self.workspace)

    def capture(self):
        """Record the step into a HIP graph (after one eager warm-up on a side
        stream, as torch's capture requires)."""
        import torch
        side = torch.cuda.Stream(device=self.device)
        side.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(side):
            self.run_eager()
        torch.cuda.current_stream(self.device).wait_stream(side)
        torch.cuda.synchronize(self.device)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.run_eager()
        torch.cuda.synchronize(self.device)
        return self

    def replay(self):
        if self.graph is None:
            raise RuntimeError("capture() first")
        self.graph.replay()

    # ---- inputs ------------------------------------------------------------
    def update(self, slots, block_tables, context_lens, q=None, k_new=None, v_new=None):
        """Copy a batch of `batch <= bucket` requests into the static buffers
        (device-to-device copies on the current stream) and pad the rest.
        q / k_new / v_new: per-layer lists of [batch, H, 128] tensors, or None
        to keep the buffers' contents."""
        batch = int(context_lens.shape[0])
        if batch > self.bucket:
            raise qil.QilError(1, f"batch {batch} exceeds the bucket {self.bucket}")
        if int(block_tables.shape[1]) > self.bt_stride:
            raise qil.QilError(1, "block table wider than the captured stride")
        w = int(block_tables.shape[1])
        self.slots[:batch].copy_(slots)
        self.slots[batch:].fill_(-1)
        self.block_tables[:batch, :w].copy_(block_tables)
        self.block_tables[:batch, w:].fill_(-1)
        self.block_tables[batch:].fill_(-1)
        self.block_tables[batch:, 0] = self.pad_page
        self.context_lens[:batch].copy_(context_lens)
        self.context_lens[batch:].fill_(1)
        for name, src in (("q", q), ("k_new", k_new), ("v_new", v_new)):
            if src is None:
                continue
            for dst, s in zip(getattr(self, name), src):
                dst[:batch].copy_(s)
        self.batch = batch
        return self
