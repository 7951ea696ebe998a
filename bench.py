"""Benchmark of the paged KV attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-flush]
                    [--keys-per-split S] [--cpu-seconds T]

Headline workload (decode-b256): 256 requests, 16 query / 8 KV heads,
head_dim 128, page_size 256, contexts U[16,1024] + U[0,1024], bf16.  One step
is the hot path over one batch: the scatter write of the 256 new tokens,
then paged decode.  ``value`` is the step's algorithmic HBM bytes (every K/V
row of every context read once, q read, output and new rows written) per
second.  A second leg times the varlen prefill workload (8 requests, cached
prefix U[0,512] + chunk U[32,2048], page 16): its step is the chunk write
then prefill, reported as causal TFLOP/s.

Inputs are seeded synthetic data put in HBM before timing.  Before every
timed step a 512 MiB buffer is written so the 256 MB Infinity Cache holds
nothing of the inputs.  Each step is bracketed by HIP events on the stream
the kernels run on; the roofline figure divides the decode call's
algorithmic bytes by its own event-timed duration.  The CPU baseline runs the
fp64 oracle (as is) on a bounded sample of the same workload on the host.
"""

import argparse
import hashlib
import json
import os
import resource
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
METRIC = "paged-decode attn GB/s (% of HBM peak) @B=256; prefill attn TFLOP/s (% MFMA)"
FLUSH_BYTES = 512 << 20
CUS, CLOCK_HZ = 256, 2.4e9     # MI355X compute units and peak engine clock


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--keys-per-split", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--skip-prefill", action="store_true")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--mixed-layers", type=int, default=36,
                    help="layers of the Qwen3-8B-shaped mixed step to time (36 in the full model)")
    ap.add_argument("--graph-layers", type=int, default=28,
                    help="layers of the decode step captured into a HIP graph per batch bucket "
                         "(28 in Qwen3-0.6B; 0 skips the leg)")
    ap.add_argument("--skip-shared", action="store_true",
                    help="skip the shared-prefix leg (prefill and decode over a common prefix)")
    ap.add_argument("--skip-qkv-proj", action="store_true",
                    help="skip the QKV-projection leg (projection GEMM with the fused write as "
                         "its epilogue, vs a library GEMM followed by the fused write)")
    ap.add_argument("--ingest-counters", metavar="DIR",
                    help="read rocprofv3 --pmc CSVs under DIR/{fetch,write,cfetch,cwrite} "
                         "(FETCH_SIZE / WRITE_SIZE of a bench run and of --calibrate), write "
                         "profiles/traffic.json and print its table, then exit (no GPU)")
    ap.add_argument("--calibrate", action="store_true",
                    help="time torch's copy and sum over 1 GiB (reference ceilings and the "
                         "plain copy kernel used to scale HBM byte counters), then exit")
    return ap.parse_args()


def calibrate(steps):
    """Plain library kernels of known size: a 1 GiB device-to-device copy
    (reads 1 GiB, writes 1 GiB) and a 1 GiB bf16 sum (reads 1 GiB)."""
    import torch
    dev = torch.device("cuda:0")
    n = (1 << 30) // 2
    src = torch.ones(n, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    out = {}
    for name, fn, nbytes in (("copy_1GiB", lambda: dst.copy_(src), 2 << 30),
                             ("sum_1GiB", lambda: src.sum(dtype=torch.float32), 1 << 30)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            a.record(); fn(); b.record()
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
        out[name] = dict(us=round(ms * 1e3, 1), gbs=round(nbytes / (ms * 1e-3) / 1e9, 1))
    print(json.dumps({"calibration": out}), flush=True)


# ---- device inputs (workload bits -> tensors, written through the library) ---
def _to_dev(bits, dev):
    import torch
    arr = np.ascontiguousarray(bits)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(arr.view(np.int32)).to(dev).view(torch.float32)


def _i32(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def _pools(w, dev):
    import torch
    shape = (w.num_pages, w.num_kv_heads, w.page_size, w.head_dim)
    raw = torch.full(shape, 0x7FC0, dtype=torch.int16, device=dev)
    return raw.view(torch.bfloat16), raw.clone().view(torch.bfloat16)


class DeviceFilledInputs:
    """A workload's inputs for timing only, drawn on the device: the same
    metadata (lengths, block tables, slots, positions) as the workload, pools
    and new rows N(0, 1) bf16 from a seeded device generator.  The 36 layers
    of the mixed step (51 GB of pools) are filled in seconds this way; parity
    runs use the host-drawn inputs."""

    def __init__(self, w, dev, seed):
        import torch
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        shape = (w.num_pages, w.num_kv_heads, w.page_size, w.head_dim)
        self.kp = torch.randn(shape, generator=g, device=dev, dtype=torch.bfloat16)
        self.vp = torch.randn(shape, generator=g, device=dev, dtype=torch.bfloat16)
        t = int(w.new_lens.sum())
        self.k_new = torch.randn((t, w.num_kv_heads, w.head_dim), generator=g, device=dev,
                                 dtype=torch.bfloat16)
        self.v_new = torch.randn((t, w.num_kv_heads, w.head_dim), generator=g, device=dev,
                                 dtype=torch.bfloat16)
        self.q = torch.randn((t, w.num_q_heads, w.head_dim), generator=g, device=dev,
                             dtype=torch.bfloat16)
        self.slots = _i32(w.slot_mapping_new(), dev)
        self.bt = _i32(w.block_tables, dev)
        self.ctx = _i32(w.context_lens, dev)
        self.out = self.q.new_empty(self.q.shape)


class Inputs:
    """A workload's inputs in HBM: pools (NaN sentinels) with the cached rows
    written through the library, the new rows, q and the metadata."""

    def __init__(self, w, dev):
        import paged_kv_attention_16_amd as qil
        d = w.gather()
        self.kp, self.vp = _pools(w, dev)
        qil.kv_write(_to_dev(d["k_cached"], dev), _to_dev(d["v_cached"], dev), self.kp, self.vp,
                     _i32(d["cached_slots"], dev))
        self.k_new = _to_dev(d["k_new"], dev)
        self.v_new = _to_dev(d["v_new"], dev)
        self.q = _to_dev(d["q"], dev)
        self.slots = _i32(d["new_slots"], dev)
        self.bt = _i32(w.block_tables, dev)
        self.ctx = _i32(w.context_lens, dev)
        self.out = self.q.new_empty(self.q.shape)
        del d


def timed_steps(segments, steps, warmup, flush, stream):
    """Warm up, then two timed passes of `steps` steps; a step calls each
    segment in order, and before each step the flush buffer (if any) is
    rewritten.
      Pass 1 brackets every segment with HIP events on `stream`: the
      per-segment breakdown.  An event marker between two kernels delays the
      dispatch of the second by a few microseconds, and that gap lands in the
      second segment's bracket.
      Pass 2 brackets only the whole step, so its kernels run back to back as
      in a real step: its mean is the step time.
    `last_ms` = pass-2 step time minus the pass-1 times of all segments but
    the last: the last segment's kernel time without a marker in front of it
    (each pass has the same single marker before the first kernel)."""
    import torch
    for _ in range(warmup):
        for f in segments:
            f()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(segments) + 1)]
          for _ in range(steps)]
    for i in range(steps):
        if flush is not None:
            flush.fill_(float(i))
        ev[i][0].record(stream)
        for j, f in enumerate(segments):
            f()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    seg = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(len(segments))] for e in ev])
    ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        if flush is not None:
            flush.fill_(float(i))
        ev2[i][0].record(stream)
        for f in segments:
            f()
        ev2[i][1].record(stream)
    torch.cuda.synchronize()
    step = np.array([e[0].elapsed_time(e[1]) for e in ev2])
    mean = seg.mean(axis=0)
    return dict(mean=mean, median=np.median(seg, axis=0),
                p10=np.percentile(seg, 10, axis=0), p90=np.percentile(seg, 90, axis=0),
                step_mean=float(step.mean()), step_median=float(np.median(step)),
                step_p10=float(np.percentile(step, 10)), step_p90=float(np.percentile(step, 90)),
                last_ms=float(step.mean() - mean[:-1].sum()))


def flushed_kernel_ms(fn, args, flush, stream):
    """Mean time of `fn` right after the cache flush, with no event marker in
    front of it: time of (flush, fn) minus time of (flush)."""
    if flush is None:
        return timed_steps([fn], args.steps, args.warmup, None, stream)["step_mean"]
    return timed_steps([lambda: flush.fill_(1.0), fn], args.steps, args.warmup, None,
                       stream)["last_ms"]


def write_bytes(w, tokens):
    """Algorithmic bytes of a scatter write: read and write both rows."""
    return tokens * w.num_kv_heads * w.head_dim * w.elem_bytes * 2 * 2 + 4 * tokens


def decode_leg(w, args, dev, stream, flush, label):
    """One decode workload: the step (write the batch's new tokens, then paged
    decode over every context) as one qil_paged_decode_append call, the same
    without the cache flush, and as two calls (qil_kv_write, then
    qil_paged_decode).  The decode call's launch time is (flush, write,
    decode) minus (flush, write): both steps start with the same single event
    marker and have none between their kernels."""
    import torch
    import paged_kv_attention_16_amd as qil
    t0 = time.time()
    x = Inputs(w, dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    max_l = int(w.context_lens.max())
    need = qil.paged_decode_workspace_size(w.batch, w.num_q_heads, w.num_kv_heads, max_l,
                                           w.page_size, args.keys_per_split)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def write():
        qil.kv_write(x.k_new, x.v_new, x.kp, x.vp, x.slots, stream=stream)

    def decode():
        qil.paged_decode(x.out, x.q, x.kp, x.vp, x.bt, x.ctx, max_l, float(w.scale),
                         keys_per_split=args.keys_per_split, workspace=ws, stream=stream)

    def append():
        # the same step as one call: the decode kernel stores the new rows
        qil.paged_decode_append(x.out, x.q, x.k_new, x.v_new, x.slots, x.kp, x.vp, x.bt, x.ctx,
                                max_l, float(w.scale), keys_per_split=args.keys_per_split,
                                workspace=ws, stream=stream)

    kv_bytes = w.decode_kv_bytes()
    step_bytes = kv_bytes + w.decode_io_bytes() + write_bytes(w, w.batch)
    dec_bytes = kv_bytes + w.decode_io_bytes()
    wall0 = time.perf_counter()
    # the step as one qil_paged_decode_append call (the headline step) ...
    tf = timed_steps([append], args.steps, args.warmup, flush, stream)
    # ... the same with warm caches (no flush): a labelled secondary number ...
    th = timed_steps([append], args.steps, args.warmup, None, stream)
    # ... and as two calls (qil_kv_write, then qil_paged_decode): the decode
    # call alone is the roofline kernel (run last, so counter runs that keep
    # the last launches of the largest decode grid see this call)
    tw = timed_steps([write], args.steps, args.warmup, flush, stream)
    t = timed_steps([write, decode], args.steps, args.warmup, flush, stream)
    wall = time.perf_counter() - wall0
    dec_ms = t["step_mean"] - tw["step_mean"]
    out = dict(
        workload=w, step_ms=tf["step_mean"], step_ms_median=tf["step_median"],
        step_ms_p10=tf["step_p10"], step_ms_p90=tf["step_p90"],
        step_bracket_ms=float(tf["mean"][0]), step_bracket_ms_median=float(tf["median"][0]),
        hot_step_ms=th["step_mean"],
        two_call_step_ms=t["step_mean"], dec_ms=dec_ms, dec_bracket_ms=float(t["mean"][1]),
        write_ms=tw["step_mean"],
        step_bytes=step_bytes, dec_bytes=dec_bytes,
        kv_bytes=kv_bytes, wall_s=wall, setup_s=setup_s, workspace=need)
    print(f"[bench] {label}: one-call step {tf['step_mean']*1e3:.1f} us "
          f"({step_bytes / (tf['step_mean'] * 1e-3) / 1e9:.0f} GB/s); two calls {t['step_mean']*1e3:.1f} us, "
          f"write alone {tw['step_mean']*1e3:.1f} us, decode {dec_ms*1e3:.1f} us "
          f"({dec_bytes / (dec_ms * 1e-3) / 1e9:.0f} GB/s), setup {setup_s:.1f}s", flush=True)
    del x, ws
    torch.cuda.empty_cache()
    return out


def gpu_legs(args):
    import torch
    import paged_kv_attention_16_amd as qil
    from workloads import make_workload

    if not os.path.exists(qil.lib_path()):
        import __graft_entry__
        __graft_entry__.build()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    flush = None if args.no_flush else torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    res = {}

    res["ceilings"] = measured_ceilings(dev, stream)

    # ---- decode legs: decode-b256 (headline), then decode-b32 -------------
    res["decode"] = decode_leg(make_workload(3), args, dev, stream, flush, "decode-b256")
    res["decode_b32"] = decode_leg(make_workload(2), args, dev, stream, flush, "decode-b32")

    # ---- prefill leg ---------------------------------------------------------
    if not args.skip_prefill:
        w4 = make_workload(4)
        x = Inputs(w4, dev)
        cu = _i32(w4.cu_seqlens(np.arange(w4.batch)), dev)
        maxq, maxk = int(w4.new_lens.max()), int(w4.context_lens.max())

        def write4():
            qil.kv_write(x.k_new, x.v_new, x.kp, x.vp, x.slots, stream=stream)

        def prefill():
            qil.paged_prefill(x.out, x.q, x.kp, x.vp, x.bt, cu, x.ctx, maxq, maxk,
                              float(w4.scale), stream=stream)

        t = timed_steps([write4, prefill], args.steps, args.warmup, flush, stream)
        # the chunk write alone, right after the flush writes (no event marker
        # in front of it): time of (flush, write) minus time of the flush
        write_ms = flushed_kernel_ms(write4, args, flush, stream)

        def append4():
            # the same step as one call: the prefill kernel stores the new rows
            qil.paged_prefill_append(x.out, x.q, x.k_new, x.v_new, x.slots, x.kp, x.vp, x.bt, cu,
                                     x.ctx, maxq, maxk, float(w4.scale), stream=stream)
        ta = timed_steps([append4], args.steps, args.warmup, flush, stream)
        flops = w4.prefill_flops()
        ntok = int(w4.new_lens.sum())
        res["prefill"] = dict(workload=w4, pre_ms=t["last_ms"], pre_bracket_ms=float(t["mean"][1]),
                              pre_bracket_ms_median=float(t["median"][1]), step_ms=t["step_mean"],
                              append_step_ms=ta["step_mean"], flops=flops, write_ms=write_ms,
                              write_bytes=write_bytes(w4, ntok), write_tokens=ntok)
        print(f"[bench] prefill-varlen: prefill {t['last_ms']*1e3:.1f} us "
              f"({flops / (t['last_ms'] * 1e-3) / 1e12:.1f} TFLOP/s; event bracket "
              f"{t['mean'][1]*1e3:.1f} us); chunk write {ntok} tokens "
              f"{write_ms*1e3:.1f} us ({write_bytes(w4, ntok) / (write_ms * 1e-3) / 1e9:.0f} GB/s); "
              f"step as two calls {t['step_mean']*1e3:.1f} us, as one qil_paged_prefill_append "
              f"call {ta['step_mean']*1e3:.1f} us", flush=True)
        del x
        torch.cuda.empty_cache()

    # ---- mixed step (fused write + decode + prefill per layer) -----------
    if args.mixed_layers > 0:
        layers = []
        t0 = time.time()
        for layer in range(args.mixed_layers):
            w5 = make_workload(5, layer)
            x = DeviceFilledInputs(w5, dev, seed=5000 + layer)
            qw, kw = w5.norm_weights()
            x.table = torch.empty(w5.max_position, w5.head_dim, dtype=torch.float32, device=dev)
            qil.rope_cos_sin(x.table, w5.theta, stream=stream)
            x.q_out = torch.empty_like(x.q)
            x.fuse = qil.QKNormRope(x.q, x.q_out, _to_dev(qw, dev), _to_dev(kw, dev),
                                    _i32(w5.positions_new(), dev), x.table, eps=w5.eps)
            x.q_dec = x.q_out[:64]
            x.q_pre = x.q_out[64:]
            x.out_dec = torch.empty_like(x.q_dec)
            x.out_pre = torch.empty_like(x.q_pre)
            x.bt_dec, x.bt_pre = x.bt[:64].contiguous(), x.bt[64:].contiguous()
            x.ctx_dec, x.ctx_pre = x.ctx[:64].contiguous(), x.ctx[64:].contiguous()
            x.cu_pre = _i32(w5.cu_seqlens(w5.prefill_idx), dev)
            x.maxl_dec = int(w5.context_lens[:64].max())
            x.maxl_pre = int(w5.context_lens[64:].max())
            need = qil.paged_decode_workspace_size(64, w5.num_q_heads, w5.num_kv_heads, x.maxl_dec,
                                                   w5.page_size, 0)
            x.ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
            x.pre_need = qil.paged_prefill_workspace_size(len(w5.prefill_idx), int(x.q_pre.shape[0]),
                                                          512, x.maxl_pre, w5.num_q_heads,
                                                          w5.num_kv_heads, 0)
            layers.append((w5, x))
        # one prefill workspace serves every layer: the calls run in order on one stream
        pre_ws = torch.empty(max(max(x.pre_need for _, x in layers), 1), dtype=torch.uint8,
                             device=dev)
        torch.cuda.synchronize()
        mixed_setup = time.time() - t0
        segs = []
        for w5, x in layers:
            def fused(x=x):
                qil.kv_write(x.k_new, x.v_new, x.kp, x.vp, x.slots, fuse=x.fuse, stream=stream)

            def dec(x=x, w5=w5):
                qil.paged_decode(x.out_dec, x.q_dec, x.kp, x.vp, x.bt_dec, x.ctx_dec, x.maxl_dec,
                                 float(w5.scale), workspace=x.ws, stream=stream)

            def pre(x=x, w5=w5):
                qil.paged_prefill(x.out_pre, x.q_pre, x.kp, x.vp, x.bt_pre, x.cu_pre, x.ctx_pre,
                                  512, x.maxl_pre, float(w5.scale), workspace=pre_ws, stream=stream)
            segs += [fused, dec, pre]
        t = timed_steps(segs, args.steps, args.warmup, flush, stream)
        nl = len(layers)
        m = t["mean"].reshape(nl, 3)

        # the same layers with decode and prefill in one launch per layer
        segs1 = []
        for i, (w5, x) in enumerate(layers):
            x.dec_batch = dict(out=x.out_dec, q=x.q_dec, block_tables=x.bt_dec,
                               context_lens=x.ctx_dec, max_context_len=x.maxl_dec, workspace=x.ws)
            x.pre_batch = dict(out=x.out_pre, q=x.q_pre, block_tables=x.bt_pre,
                               cu_seqlens_q=x.cu_pre, context_lens=x.ctx_pre, max_seqlen_q=512,
                               max_context_len=x.maxl_pre)

            def both(x=x, w5=w5):
                qil.paged_attention_mixed(x.kp, x.vp, float(w5.scale), decode=x.dec_batch,
                                          prefill=x.pre_batch, stream=stream)
            segs1 += [segs[3 * i], both]   # the layer's fused write, then both batches
        t1 = timed_steps(segs1, args.steps, args.warmup, flush, stream)
        fused_bytes = sum(int(w5.new_lens.sum()) * (w5.num_q_heads + 2 * w5.num_kv_heads) * 256 * 2
                          for w5, _ in layers) / nl
        dec_bytes5 = sum(w5.decode_kv_bytes() + w5.decode_io_bytes() for w5, _ in layers) / nl
        pre_flops5 = sum(w5.prefill_flops() for w5, _ in layers) / nl
        layer_ms = t["step_mean"] / nl
        res["mixed"] = dict(layers=nl, layer_ms=layer_ms, single_launch_layer_ms=t1["step_mean"] / nl,
                            step_ms=t["step_mean"], step_ms_median=t["step_median"],
                            step_ms_p10=t["step_p10"], step_ms_p90=t["step_p90"],
                            single_launch_ms=float(t1["mean"].reshape(nl, 2)[:, 1].mean()),
                            fused_ms=float(m[:, 0].mean()),
                            dec_ms=float(m[:, 1].mean()), pre_ms=float(m[:, 2].mean()),

                            fused_bytes=fused_bytes, dec_bytes=dec_bytes5, pre_flops=pre_flops5,
                            setup_s=mixed_setup)
        print(f"[bench] mixed-8b x{nl} layers: step {t['step_mean']*1e3:.1f} us (median "
              f"{t['step_median']*1e3:.1f}, p10 {t['step_p10']*1e3:.1f}, p90 {t['step_p90']*1e3:.1f}), "
              f"{layer_ms*1e3:.1f} us/layer "
              f"(fused write {m[:,0].mean()*1e3:.1f} us, decode {m[:,1].mean()*1e3:.1f} us, "
              f"prefill {m[:,2].mean()*1e3:.1f} us); decode + prefill in one launch: "
              f"{t1['step_mean'] / nl * 1e3:.1f} us/layer; setup {mixed_setup:.1f}s", flush=True)
        del layers
        torch.cuda.empty_cache()
    if args.graph_layers > 0:
        res["graph"] = graph_leg(args, dev, stream, flush)
    if not args.skip_shared:
        res["shared"] = shared_prefix_leg(args, dev, stream, flush)
    res["shard"] = shard_leg(args, dev, stream, flush)
    if not args.skip_prefill:
        res["long_prefix"] = long_prefix_leg(args, dev, stream, flush)
    if not args.skip_qkv_proj:
        res["qkv_proj"] = qkv_proj_leg(args, dev, stream, flush)
    return res


def shared_prefix_leg(args, dev, stream, flush):
    """Requests over one common 4096-token prompt prefix held in 256 shared
    read-only pages (prefix caching), against the same requests with private
    copies of the prefix.  Qwen3-8B attention (Hq 32 / Hkv 8), page 16.
      prefill: 8 requests, each a 512-token chunk after the prefix
      decode:  64 requests, each one token after the prefix plus a private
               tail of U[0, 1024] tokens
    Timing only (N(0,1) bf16 pool values); parity is a GPU test."""
    import torch
    import paged_kv_attention_16_amd as qil
    rng = np.random.default_rng(11)
    hq, hkv, page, D, pre_pages = 32, 8, 16, 128, 256
    scale = 0.08838834764831845

    def tables(tails, shared):
        B = len(tails)
        tail_pages = -(-np.asarray(tails) // page)
        n_pages = (pre_pages if shared else B * pre_pages) + int(tail_pages.sum())
        perm = rng.permutation(n_pages).astype(np.int32)
        bt = np.full((B, pre_pages + int(tail_pages.max())), -1, np.int32)
        at = 0
        if shared:
            common = perm[:pre_pages]
            at = pre_pages
        for r in range(B):
            if shared:
                bt[r, :pre_pages] = common
            else:
                bt[r, :pre_pages] = perm[at:at + pre_pages]
                at += pre_pages
            bt[r, pre_pages:pre_pages + tail_pages[r]] = perm[at:at + tail_pages[r]]
            at += tail_pages[r]
        kp = torch.empty(n_pages, hkv, page, D, dtype=torch.bfloat16, device=dev).normal_()
        return kp, torch.empty_like(kp).normal_(), torch.from_numpy(bt).to(dev)

    out = {}
    # prefill: 8 chunks of 512 after the shared prefix
    tails = np.full(8, 512)
    ctx = torch.from_numpy((pre_pages * page + tails).astype(np.int32)).to(dev)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(tails)]).astype(np.int32)).to(dev)
    q = torch.randn(int(tails.sum()), hq, D, device=dev).to(torch.bfloat16)
    o = torch.empty_like(q)
    maxk = int(pre_pages * page + tails.max())
    pairs = sum(sum(pre_pages * page + i + 1 for i in range(n)) for n in tails.tolist())
    flops = pairs * hq * 512
    for shared in (True, False):
        kp, vp, bt = tables(tails, shared)
        t = timed_steps([lambda: qil.paged_prefill(o, q, kp, vp, bt, cu, ctx, 512, maxk, scale,
                                                   stream=stream)], args.steps, args.warmup, flush, stream)
        key = "prefill_shared" if shared else "prefill_private"
        out[key] = dict(us=round(t["step_mean"] * 1e3, 2),
                        TFLOP_per_s=round(flops / (t["step_mean"] * 1e-3) / 1e12, 1))
        del kp, vp, bt
    # decode: 64 requests, prefix + private tail, one query token each
    tails = rng.integers(1, 1025, 64)
    ctx_np = (pre_pages * page + tails).astype(np.int32)
    ctx = torch.from_numpy(ctx_np).to(dev)
    q = torch.randn(64, hq, D, device=dev).to(torch.bfloat16)
    o = torch.empty_like(q)
    maxl = int(ctx_np.max())
    need = qil.paged_decode_workspace_size(64, hq, hkv, maxl, page, 0)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    algo = int(ctx_np.sum()) * hkv * D * 2 * 2
    unique = (pre_pages * page + int(tails.sum())) * hkv * D * 2 * 2
    for shared in (True, False):
        kp, vp, bt = tables(tails, shared)
        t = timed_steps([lambda: qil.paged_decode(o, q, kp, vp, bt, ctx, maxl, scale, workspace=ws,
                                                  stream=stream)], args.steps, args.warmup, flush, stream)
        key = "decode_shared" if shared else "decode_private"
        out[key] = dict(us=round(t["step_mean"] * 1e3, 2),
                        context_GB_per_s=round(algo / (t["step_mean"] * 1e-3) / 1e9, 1))
        if shared:
            out[key]["unique_GB_per_s"] = round(unique / (t["step_mean"] * 1e-3) / 1e9, 1)
        del kp, vp, bt
    torch.cuda.empty_cache()
    print(f"[bench] shared-prefix: prefill {out['prefill_shared']['TFLOP_per_s']} vs "
          f"{out['prefill_private']['TFLOP_per_s']} TFLOP/s (shared vs private), decode "
          f"{out['decode_shared']['us']} vs {out['decode_private']['us']} us", flush=True)
    return out


GRAPH_BUCKETS = (1, 2, 4, 8, 16, 32, 64, 128, 256)


def long_prefix_leg(args, dev, stream, flush):
    """Chunked prefill of a long prompt: one 512-token chunk after a cached
    prefix of 7,680 / 15,872 / 32,256 tokens (contexts 8k / 16k / 32k),
    Qwen3-8B attention (Hq 32 / Hkv 8), page 16.  Only 64 query tiles x KV
    heads, so whole tiles leave most CUs idle; the automatic plan splits each
    tile over its keys.  Timing only (N(0,1) bf16 pools, random placement);
    parity is a GPU test."""
    import torch
    import paged_kv_attention_16_amd as qil
    rng = np.random.default_rng(17)
    hq, hkv, page, D, n = 32, 8, 16, 128, 512
    scale = 0.08838834764831845
    out = []
    for L in (8192, 16384, 32768):
        pages = L // page
        num_pages = int(pages * 1.2)
        bt = torch.from_numpy(rng.permutation(num_pages)[:pages].astype(np.int32)[None]).to(dev)
        kp = torch.empty(num_pages, hkv, page, D, dtype=torch.bfloat16, device=dev).normal_()
        vp = torch.empty_like(kp).normal_()
        q = torch.randn(n, hq, D, device=dev).to(torch.bfloat16)
        o = torch.empty_like(q)
        cu = torch.tensor([0, n], dtype=torch.int32, device=dev)
        ctx = torch.tensor([L], dtype=torch.int32, device=dev)
        need = qil.paged_prefill_workspace_size(1, n, n, L, hq, hkv, 0)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        flops = sum(L - n + i + 1 for i in range(n)) * hq * 512
        row = dict(workload=f"one {n}-token chunk over a {L - n}-token prefix", context=L)
        for label, kps in (("split", 0), ("unsplit", L)):
            ms = flushed_kernel_ms(lambda: qil.paged_prefill(o, q, kp, vp, bt, cu, ctx, n, L, scale,
                                                             keys_per_split=kps, workspace=ws,
                                                             stream=stream), args, flush, stream)
            tf = flops / (ms * 1e-3) / 1e12
            row[label] = dict(us=round(ms * 1e3, 2), TFLOP_per_s=round(tf, 1),
                              frac=round(tf / BF16_PEAK_TFLOPS, 4))
        out.append(row)
        print(f"[bench] long prefix L={L}: split {row['split']['us']} us "
              f"({row['split']['TFLOP_per_s']} TFLOP/s), unsplit {row['unsplit']['us']} us", flush=True)
        del kp, vp
    torch.cuda.empty_cache()
    return out


def shard_leg(args, dev, stream, flush):
    """Decode at one GPU's share of an 8-way tensor-parallel split by KV head
    (each GPU holds Hkv/8 = 1 KV head and its G query heads; no exchange is
    needed inside attention).  Fewer workgroups per call, so the split plan
    carries the parallelism.  Synthetic N(0,1) bf16 pools, random placement."""
    import torch
    import paged_kv_attention_16_amd as qil
    rng = np.random.default_rng(13)
    cases = [
        ("0.6B TP8: B 256, Hq 2 / Hkv 1, page 256, context U[16,1024]+U[0,1024]", 256, 2, 256,
         rng.integers(16, 1025, 256) + rng.integers(0, 1025, 256)),
        ("8B TP8: B 64, Hq 4 / Hkv 1, page 16, context U[512,8192]", 64, 4, 16,
         rng.integers(512, 8193, 64)),
    ]
    out = []
    for label, B, hq, page, ctx in cases:
        ctx = ctx.astype(np.int32)
        need = -(-ctx // page)
        num_pages = int(np.ceil(need.sum() * 1.2))
        perm = rng.permutation(num_pages).astype(np.int32)
        bt = np.full((B, int(need.max())), -1, np.int32)
        at = 0
        for r, k in enumerate(need.tolist()):
            bt[r, :k] = perm[at:at + k]
            at += k
        kp = torch.empty(num_pages, 1, page, 128, dtype=torch.bfloat16, device=dev).normal_()
        vp = torch.empty_like(kp).normal_()
        q = torch.randn(B, hq, 128, device=dev).to(torch.bfloat16)
        o = torch.empty_like(q)
        bt_d, ctx_d = torch.from_numpy(bt).to(dev), torch.from_numpy(ctx).to(dev)
        maxl = int(ctx.max())
        wsz = qil.paged_decode_workspace_size(B, hq, 1, maxl, page, 0)
        ws = torch.empty(max(wsz, 1), dtype=torch.uint8, device=dev)
        ms = flushed_kernel_ms(lambda: qil.paged_decode(o, q, kp, vp, bt_d, ctx_d, maxl,
                                                        0.08838834764831845, workspace=ws,
                                                        stream=stream), args, flush, stream)
        nbytes = int(ctx.astype(np.int64).sum()) * 512 + 2 * B * hq * 256
        gbs = nbytes / (ms * 1e-3) / 1e9
        out.append(dict(workload=label, us=round(ms * 1e3, 2), GB_per_s=round(gbs, 1),
                        frac=round(gbs / HBM_PEAK_GBS, 4)))
        print(f"[bench] shard {label}: {ms*1e3:.1f} us, {gbs:.0f} GB/s", flush=True)
        del kp, vp
    torch.cuda.empty_cache()
    return out


def qkv_proj_leg(args, dev, stream, flush):
    """The merged QKV projection of the Qwen3-8B-shaped step (2112 new tokens:
    64 decode + 4 x 512 chunk, hidden 4096, 32 q / 8 KV heads, page 16) with
    the Q/K RMSNorm + RoPE + scatter write as its epilogue, in one kernel;
    next to it, the same work as a library GEMM (torch.matmul) followed by
    the fused qil_kv_write.  Synthetic activations N(0,1) and weights
    N(0, 1/hidden), bf16."""
    import torch
    import paged_kv_attention_16_amd as qil
    from workloads import make_workload
    w5 = make_workload(5)
    hidden = 4096
    x_bits, w_bits = w5.projection_inputs(hidden)
    t, n = x_bits.shape[0], w_bits.shape[0]
    hq, hkv = w5.num_q_heads, w5.num_kv_heads
    x = torch.from_numpy(x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    wt = torch.from_numpy(w_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    kp = torch.zeros(w5.num_pages, hkv, w5.page_size, 128, dtype=torch.bfloat16, device=dev)
    vp = torch.zeros_like(kp)
    qw, kw = (torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
              for a in w5.norm_weights())
    table = torch.empty(w5.max_position, 128, dtype=torch.float32, device=dev)
    qil.rope_cos_sin(table, w5.theta, stream=stream)
    slots = _i32(w5.slot_mapping_new(), dev)
    pos = _i32(w5.positions_new(), dev)
    q_out = torch.empty(t, hq, 128, dtype=torch.bfloat16, device=dev)
    qkv = torch.empty(t, n, dtype=torch.bfloat16, device=dev)

    def fused():
        qil.qkv_proj_write(x, wt, kp, vp, slots, q_out, hq, qw, kw, pos, table, eps=w5.eps,
                           stream=stream)

    def gemm():
        torch.matmul(x, wt.t(), out=qkv)

    fuse = qil.QKNormRope(qkv[:, :hq * 128], q_out, qw, kw, pos, table, eps=w5.eps, num_q_heads=hq)

    def write():
        qil.kv_write(qkv[:, hq * 128:(hq + hkv) * 128], qkv[:, (hq + hkv) * 128:], kp, vp, slots,
                     fuse=fuse, stream=stream)

    with torch.cuda.stream(stream):
        fused_ms = flushed_kernel_ms(fused, args, flush, stream)
        gemm_ms = flushed_kernel_ms(gemm, args, flush, stream)
        write_ms = flushed_kernel_ms(write, args, flush, stream)
        # the decode-only step of the same model: its 64 tokens (split path)
        d = 64
        xd, qd, qkvd = x[:d], q_out[:d], qkv[:d]
        sd, pd = slots[:d], pos[:d]
        wsd = torch.empty(max(qil.qkv_proj_workspace_size(d, hq, hkv, hidden), 1),
                          dtype=torch.uint8, device=dev)
        fused_d = lambda: qil.qkv_proj_write(xd, wt, kp, vp, sd, qd, hq, qw, kw, pd, table,
                                             eps=w5.eps, workspace=wsd, stream=stream)
        gemm_d = lambda: torch.matmul(xd, wt.t(), out=qkvd)
        fuse_d = qil.QKNormRope(qkvd[:, :hq * 128], qd, qw, kw, pd, table, eps=w5.eps, num_q_heads=hq)
        write_d = lambda: qil.kv_write(qkvd[:, hq * 128:(hq + hkv) * 128], qkvd[:, (hq + hkv) * 128:],
                                       kp, vp, sd, fuse=fuse_d, stream=stream)
        fused_d_ms = flushed_kernel_ms(fused_d, args, flush, stream)
        lib_d_ms = flushed_kernel_ms(gemm_d, args, flush, stream) + \
            flushed_kernel_ms(write_d, args, flush, stream)
    flops = 2 * t * n * hidden
    tf = flops / (fused_ms * 1e-3) / 1e12
    print(f"[bench] qkv-proj-8b: one kernel {fused_ms*1e3:.1f} us ({tf:.0f} TFLOP/s); "
          f"library GEMM {gemm_ms*1e3:.1f} us + fused write {write_ms*1e3:.1f} us; "
          f"64-token decode step: {fused_d_ms*1e3:.1f} us vs {lib_d_ms*1e3:.1f} us", flush=True)
    del kp, vp
    torch.cuda.empty_cache()
    return dict(tokens=t, flops=flops, fused_ms=fused_ms, gemm_ms=gemm_ms, write_ms=write_ms,
                decode_step_ms=fused_d_ms, decode_step_library_ms=lib_d_ms)


def measured_ceilings(dev, stream):
    """What plain kernels reach on this GPU: a non-temporal streaming read of
    2 GiB (best of 1024 / 2048 / 4096 workgroups) and a loop of independent
    bf16 32x32x16 MFMAs on every SIMD.  The secondary roofline denominators."""
    import ctypes
    import torch
    from paged_kv_attention_16_amd import build as qbuild
    lib = ctypes.CDLL(qbuild.CEILING_LIB)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    lib.qil_ceiling_stream_read.argtypes = [vp, sz, vp, i32, vp]
    lib.qil_ceiling_mfma_bf16.argtypes = [vp, i32, i32, vp]
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(256, dtype=torch.float32, device=dev)
    s = ctypes.c_void_p(stream.cuda_stream)
    best = 0.0
    for blocks in (1024, 2048, 4096):
        def rd():
            rc = lib.qil_ceiling_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                             ctypes.c_void_p(sink.data_ptr()), blocks, s)
            assert rc == 0, rc
        t = timed_steps([rd], 5, 2, None, stream)
        best = max(best, nbytes / (t["step_mean"] * 1e-3) / 1e9)
    del buf
    blocks, iters = 1024, 20000

    def mm():
        rc = lib.qil_ceiling_mfma_bf16(ctypes.c_void_p(sink.data_ptr()), blocks, iters, s)
        assert rc == 0, rc
    t = timed_steps([mm], 3, 1, None, stream)
    flops = blocks * 4 * 4 * iters * 32768
    tf = flops / (t["step_mean"] * 1e-3) / 1e12
    # LDS operand reads: bytes per clock per CU at the 2.4 GHz peak clock
    lds = {}
    lib.qil_ceiling_lds_read.argtypes = [i32, vp, i32, i32, vp]
    for tr, name, per_lane in ((0, "ds_read_b128", 16), (1, "ds_read_b64_tr_b16", 8)):
        lb, li = 1024, 2000

        def lr():
            rc = lib.qil_ceiling_lds_read(tr, ctypes.c_void_p(sink.data_ptr()), lb, li, s)
            assert rc == 0, rc
        t = timed_steps([lr], 3, 1, None, stream)
        nb = lb * 512 * li * 16 * per_lane
        lds[name] = round(nb / (t["step_mean"] * 1e-3) / CUS / CLOCK_HZ, 1)
    torch.cuda.empty_cache()
    print(f"[bench] measured ceilings: stream read {best:.0f} GB/s, bf16 MFMA {tf:.0f} TFLOP/s, "
          f"LDS reads {lds['ds_read_b128']:.0f} B/clk/CU (b128), {lds['ds_read_b64_tr_b16']:.0f} "
          f"(b64_tr_b16)", flush=True)
    return dict(stream_read_GB_s=round(best, 1), mfma_bf16_TFLOP_s=round(tf, 1),
                lds_read_B_per_clk_per_CU=lds)


def graph_leg(args, dev, stream, flush):
    """Decode step of `graph_layers` layers (per layer one
    qil_paged_decode_append call: the new token's K/V write fused into paged
    decode) at batch buckets 1 .. 256, issued eagerly from Python and
    replayed as a HIP graph; at buckets up to 8 also the graph of the
    two-call step (qil_kv_write, then qil_paged_decode).  Contexts U[16,1024] + U[0,1024],
    Hq 16 / Hkv 8, page 256, independent pools per layer with random page
    placement; values are N(0,1) in bf16 (timing only: parity of the graph
    path is a GPU test)."""
    import torch
    from paged_kv_attention_16_amd.graph import DecodeStepGraph
    rng = np.random.default_rng(7)
    B, hq, hkv, page, D = max(GRAPH_BUCKETS), 16, 8, 256, 128
    ctx = (rng.integers(16, 1025, B) + rng.integers(0, 1025, B)).astype(np.int32)
    need = -(-ctx // page)
    num_pages = int(need.sum()) + 1
    stride = int(need.max())
    max_l = 2048
    t0 = time.time()
    # one page placement, shared by every layer's pools as in a real model
    perm = rng.permutation(num_pages - 1).astype(np.int32) + 1   # page 0 is the pad page
    bt = np.full((B, stride), -1, np.int32)
    at = 0
    for r, k in enumerate(need.tolist()):
        bt[r, :k] = perm[at:at + k]
        at += k
    slots = (bt[np.arange(B), (ctx - 1) // page] * page + (ctx - 1) % page).astype(np.int32)
    pools = []
    for _ in range(args.graph_layers):
        kp = torch.empty(num_pages, hkv, page, D, dtype=torch.bfloat16, device=dev).normal_()
        pools.append((kp, torch.empty_like(kp).normal_()))
    torch.cuda.synchronize()
    setup = time.time() - t0
    out = []
    for bucket in GRAPH_BUCKETS:
        g = DecodeStepGraph(pools, bucket, hq, stride, max_l, 0.08838834764831845, pad_page=0)
        g.update(torch.from_numpy(slots[:bucket]).to(dev), torch.from_numpy(bt[:bucket]).to(dev),
                 torch.from_numpy(ctx[:bucket]).to(dev),
                 q=[torch.randn(bucket, hq, D, device=dev).to(torch.bfloat16) for _ in pools],
                 k_new=[torch.randn(bucket, hkv, D, device=dev).to(torch.bfloat16) for _ in pools],
                 v_new=[torch.randn(bucket, hkv, D, device=dev).to(torch.bfloat16) for _ in pools])
        g.capture()
        te = timed_steps([g.run_eager], args.steps, args.warmup, flush, stream)
        tg = timed_steps([g.replay], args.steps, args.warmup, flush, stream)
        eager_us, graph_us = te["step_mean"] * 1e3, tg["step_mean"] * 1e3
        kv = int(ctx[:bucket].sum()) * hkv * D * 2 * 2 * len(pools)
        row = dict(batch=bucket, eager_us=round(eager_us, 1), graph_us=round(graph_us, 1),
                   launch_overhead_share=round(1 - graph_us / eager_us, 4),
                   graph_GB_per_s=round(kv / (graph_us * 1e-6) / 1e9, 1))
        del g
        if bucket <= 8:
            g2 = DecodeStepGraph(pools, bucket, hq, stride, max_l, 0.08838834764831845, pad_page=0,
                                 fused_write=False)
            g2.update(torch.from_numpy(slots[:bucket]).to(dev), torch.from_numpy(bt[:bucket]).to(dev),
                      torch.from_numpy(ctx[:bucket]).to(dev))
            g2.capture()
            t2 = timed_steps([g2.replay], args.steps, args.warmup, flush, stream)
            row["two_call_graph_us"] = round(t2["step_mean"] * 1e3, 1)
            del g2
        out.append(row)
        print(f"[bench] decode-graph B={bucket:3d}: eager {eager_us:8.1f} us, graph {graph_us:8.1f} us "
              f"({100 * (1 - graph_us / eager_us):.1f}% launch overhead)"
              + (f", two-call graph {row['two_call_graph_us']:.1f} us" if bucket <= 8 else ""),
              flush=True)
    del pools
    torch.cuda.empty_cache()
    return dict(layers=args.graph_layers, setup_s=setup, buckets=out)


# ---- CPU baseline: the oracle, unchanged, on a bounded sample -------------
def cpu_baseline(seconds):
    """The fp64 oracle on the host: the decode-b256 step (scatter write +
    decode, every request; the whole workload fits in a few seconds) and, for
    context, the prefill of as many prefill-varlen requests as fit in the
    remaining time budget."""
    from oracle import attention as o_attn
    from oracle import paged as o_paged
    from workloads import make_workload, sentinel_pool

    w = make_workload(3)
    kp = sentinel_pool(w.num_pages, w.num_kv_heads, w.page_size, w.head_dim, w.dtype)
    vp = sentinel_pool(w.num_pages, w.num_kv_heads, w.page_size, w.head_dim, w.dtype)
    nbytes, busy = 0, 0.0
    ru0 = resource.getrusage(resource.RUSAGE_SELF)
    for r in range(w.batch):
        d = w.request(r)
        t0 = time.perf_counter()
        o_paged.kv_write(kp, vp, d.k_cached, d.v_cached, w.cached_slots(r), w.page_size)
        o_paged.kv_write(kp, vp, d.k_new, d.v_new, w.new_slots(r), w.page_size)
        o_attn.paged_decode(d.q, kp, vp, w.block_tables[r:r + 1], w.context_lens[r:r + 1],
                            w.scale, w.page_size, w.dtype)
        busy += time.perf_counter() - t0
        nbytes += int(w.context_lens[r]) * w.num_kv_heads * w.head_dim * 2 * 2
    ru1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (ru1.ru_utime - ru0.ru_utime) + (ru1.ru_stime - ru0.ru_stime)
    cores = round(cpu / max(busy, 1e-9), 1)      # CPU time / wall time: cores busy on average
    del kp, vp

    w4 = make_workload(4)
    kp = sentinel_pool(w4.num_pages, w4.num_kv_heads, w4.page_size, w4.head_dim, w4.dtype)
    vp = sentinel_pool(w4.num_pages, w4.num_kv_heads, w4.page_size, w4.head_dim, w4.dtype)
    pflops, pbusy, pdone = 0, 0.0, 0
    for r in np.argsort(w4.new_lens).tolist():      # shortest chunks first
        if pbusy >= max(1.0, seconds - busy):
            break
        d = w4.request(r)
        t0 = time.perf_counter()
        o_paged.kv_write(kp, vp, d.k_cached, d.v_cached, w4.cached_slots(r), w4.page_size)
        o_paged.kv_write(kp, vp, d.k_new, d.v_new, w4.new_slots(r), w4.page_size)
        o_attn.paged_attention(d.q, kp, vp, w4.block_tables[r:r + 1],
                               np.array([0, int(w4.new_lens[r])]), w4.context_lens[r:r + 1],
                               w4.scale, w4.page_size, w4.dtype)
        pbusy += time.perf_counter() - t0
        c, n = int(w4.cached_lens[r]), int(w4.new_lens[r])
        pflops += (n * (c + 1) + n * (n - 1) // 2) * w4.num_q_heads * 4 * w4.head_dim
        pdone += 1
    # the QKV projection + fused write of the first 256 tokens of the
    # Qwen3-8B-shaped step (fp64 matmul of the bf16 inputs, then the fused
    # write), as GFLOP/s of the projection
    from oracle import norm_rope as o_nr
    from oracle import projection as o_proj
    w5 = make_workload(5)
    ntok = 256
    xb, wb = w5.projection_inputs(4096)
    xb = xb[:ntok]
    qw, kw = w5.norm_weights()
    table = o_nr.rope_table(w5.max_position, w5.head_dim, w5.theta)
    kp5 = sentinel_pool(w5.num_pages, w5.num_kv_heads, w5.page_size, w5.head_dim, w5.dtype)
    vp5 = sentinel_pool(w5.num_pages, w5.num_kv_heads, w5.page_size, w5.head_dim, w5.dtype)
    t0 = time.perf_counter()
    o_proj.qkv_proj_write(kp5, vp5, xb, wb, w5.num_q_heads, w5.num_kv_heads,
                          w5.slot_mapping_new()[:ntok], w5.positions_new()[:ntok], qw, kw, w5.eps,
                          table, w5.page_size)
    qbusy = time.perf_counter() - t0
    qflops = 2 * ntok * wb.shape[0] * 4096
    del kp5, vp5
    try:
        from threadpoolctl import threadpool_info
        blas = max((int(i.get("num_threads", 1)) for i in threadpool_info()
                    if i.get("user_api") == "blas"), default=1)
    except Exception:  # the count is informational
        blas = None
    return dict(value=nbytes / busy / 1e9, unit="GB/s", cores=len(os.sched_getaffinity(0)),
                busy_cores_estimate=cores, kind="oracle", blas_threads=blas,
                sample=f"decode-b256 step, all {w.batch} requests (scatter write + fp64 decode over "
                       f"{nbytes / 1e6:.0f} MB of K/V), {busy:.1f} s on the host; "
                       f"{len(os.sched_getaffinity(0))} usable cores",
                prefill={"value": pflops / max(pbusy, 1e-9) / 1e9, "unit": "GFLOP/s",
                         "sample": f"{pdone} of {w4.batch} prefill-varlen requests (shortest chunks "
                                   f"first), {pflops / 1e9:.1f} causal GFLOP in {pbusy:.1f} s"},
                qkv_proj={"value": qflops / max(qbusy, 1e-9) / 1e9, "unit": "GFLOP/s",
                          "sample": f"{ntok} of {int(w5.new_lens.sum())} qkv-proj-8b tokens "
                                    f"(fp64 projection + fused write), {qflops / 1e9:.1f} GFLOP "
                                    f"in {qbusy:.2f} s"})


# every source file a kernel is compiled from (its launcher, its body and the
# shared headers): traffic figures are used only while all are unchanged
KERNEL_SOURCES = {
    "decode-b256": ("decode.hip", "decode_body.h", "device_common.h", "qil_internal.h"),
    "prefill-varlen": ("prefill.hip", "prefill_body.h", "device_common.h", "qil_internal.h"),
    "qkv-proj-8b": ("qkv_proj.hip", "device_common.h", "qil_internal.h"),
    "kv-write-chunk": ("kv_write.hip", "device_common.h", "qil_internal.h"),
    "fused-write-8b": ("kv_write.hip", "device_common.h", "qil_internal.h"),
}


def sources_sha256(files):
    """SHA-256 over the kernel's source files, in order, and the compiler
    flags of its translation unit (the first file): a flag change alone
    also retires the traffic figures."""
    from paged_kv_attention_16_amd import build as qbuild
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "paged_kv_attention_16_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    flags = [a for a in qbuild.common_flags() if not a.startswith(os.sep) and a != "-I"]
    h.update(" ".join(flags + qbuild.EXTRA_FLAGS.get(files[0], [])).encode())
    return h.hexdigest()


# kernel each traffic figure is for: name prefix in the counter CSVs
# (kernel, which of its grids): "largest" for the legs whose grid is the
# kernel's biggest in the run; "frequent" for the write kernels, whose biggest
# grid is the bench's one-off pool fill.
TRAFFIC_KERNELS = {
    "decode-b256": ("decode_mfma_kernel<2>", "largest"),
    "prefill-varlen": ("prefill_kernel<2, 4, false>", "largest"),   # 128-row workgroups (short contexts)
    "qkv-proj-8b": ("qkv_proj_kernel<4, false>", "largest"),
    "kv-write-chunk": ("kv_write_kernel<16>", "frequent"),     # the 8,946-token chunk write
    "fused-write-8b": ("kv_write_fused_kernel", "frequent"),   # 2,112 tokens of qkv-proj-8b
}


def _counter_rows(folder, counter):
    """(kernel name, grid size, value) per dispatch from rocprofv3 --pmc CSVs."""
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(folder, "**", "*counter_collection.csv"),
                                 recursive=True)):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                rows.append((int(r.get("Dispatch_Id", 0)), r["Kernel_Name"], int(r["Grid_Size"]),
                             float(r["Counter_Value"])))
    rows.sort()
    return [(n, g, v) for _, n, g, v in rows]


def _kernel_kib(rows, name, which="largest"):
    """Mean counter value (KiB) of the last 3 dispatches of one of `name`'s
    grids: the largest, or the most frequent (the largest on a tie)."""
    import collections

    def short(n):
        return n.replace("qil::(anonymous namespace)::", "").replace("void ", "").replace(" ", "")
    mine = [(g, v) for n, g, v in rows if short(n).startswith(name.replace(" ", ""))]
    if not mine:
        return None
    if which == "frequent":
        counts = collections.Counter(g for g, _ in mine)
        grid = max(counts, key=lambda g: (counts[g], g))
    else:
        grid = max(g for g, _ in mine)
    vals = [v for g, v in mine if g == grid][-3:]
    return sum(vals) / len(vals)


def ingest_counters(root):
    """HBM bytes per launch of each leg's kernel from FETCH_SIZE / WRITE_SIZE,
    scaled by what the same counters read for a 1 GiB device copy."""
    fetch = _counter_rows(os.path.join(root, "fetch"), "FETCH_SIZE")
    write = _counter_rows(os.path.join(root, "write"), "WRITE_SIZE")
    cfetch = _counter_rows(os.path.join(root, "cfetch"), "FETCH_SIZE")
    cwrite = _counter_rows(os.path.join(root, "cwrite"), "WRITE_SIZE")
    copy_f = _kernel_kib(cfetch, "__amd_rocclr_copyBuffer")
    copy_w = _kernel_kib(cwrite, "__amd_rocclr_copyBuffer")
    if not copy_f or not copy_w:
        sys.exit("no calibration copy in the counter CSVs")
    gib_kib = float(1 << 20)
    fs, ws = gib_kib / copy_f, gib_kib / copy_w
    table = {"calibration": {"kernel": "torch copy_ of 1 GiB (__amd_rocclr_copyBuffer): reads 1 GiB, "
                                       "writes 1 GiB",
                             "FETCH_SIZE_KiB": round(copy_f, 1), "WRITE_SIZE_KiB": round(copy_w, 1),
                             "fetch_scale": round(fs, 4), "write_scale": round(ws, 4)}}
    print("| kernel | HBM read MB/launch | HBM write MB/launch |")
    print("|---|---|---|")
    for key, (kname, which) in TRAFFIC_KERNELS.items():
        f, w = _kernel_kib(fetch, kname, which), _kernel_kib(write, kname, which)
        if f is None or w is None:
            print(f"| {kname} ({key}) | missing | missing |")
            continue
        fb, wb = int(f * 1024 * fs), int(w * 1024 * ws)
        table[key] = {"kernel": kname, "source_sha256": sources_sha256(KERNEL_SOURCES[key]),
                      "sources": list(KERNEL_SOURCES[key]), "fetch_bytes_per_launch": fb,
                      "write_bytes_per_launch": wb, "hbm_bytes_per_launch": fb + wb}
        print(f"| {kname} ({key}) | {fb / 1e6:.1f} | {wb / 1e6:.2f} |")
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(table, f, indent=1)
        f.write("\n")
    print(f"calibration: FETCH_SIZE x 1024 x {fs:.4f} + WRITE_SIZE x 1024 x {ws:.4f}")


def traffic_for(launches_bytes_key):
    """HBM bytes per launch from committed counter runs, only while the
    kernel's sources are unchanged since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)
    entry = table.get(launches_bytes_key)
    if not entry:
        return None
    if entry.get("source_sha256") != sources_sha256(KERNEL_SOURCES[launches_bytes_key]):
        return None
    return entry.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); this build has no "
              f"multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if args.ingest_counters:
        ingest_counters(args.ingest_counters)
        return
    if args.calibrate:
        calibrate(args.steps)
        return
    res = gpu_legs(args)
    dec = res["decode"]
    w = dec["workload"]
    value = dec["step_bytes"] / (dec["step_ms"] * 1e-3) / 1e9
    achieved = dec["dec_bytes"] / (dec["dec_ms"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "decode-b256: 256 requests, Hq 16 / Hkv 8, head_dim 128, page 256, "
                        "context U[16,1024]+U[0,1024], step = write 256 new tokens + paged decode "
                        "(one qil_paged_decode_append call)",
            "batch": int(w.batch),
            "total_context_tokens": int(w.context_lens.sum()),
            "max_context": int(w.context_lens.max()),
            "page_size": int(w.page_size),
            "mall_flush": not args.no_flush,
            "inputs": {"rng": "numpy PCG64, SeedSequence([1234, 3, 0, ...])",
                       "metadata_sha256": w.metadata_digest()},
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "qil_paged_decode (the decode call of the two-call step): one launch of "
                      "decode_mfma_kernel<2>, one split per request, each workgroup ranking the "
                      "batch longest first itself; no ordering or merge launch",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_for("decode-b256"),
            "algorithmic_bytes_per_launch": int(dec["dec_bytes"]),
            "launch_us_mean": round(dec["dec_ms"] * 1e3, 2),
            "launch_timing": "mean time of (flush, write, decode) minus mean time of (flush, write): "
                             "one event marker before the first kernel of each, none between kernels",
            "event_bracket_us_mean": round(dec["dec_bracket_ms"] * 1e3, 2),
            "measured_ceiling": res["ceilings"]["stream_read_GB_s"],
            "frac_of_measured": round(achieved / res["ceilings"]["stream_read_GB_s"], 4),
        },
        "fused_step": {
            "call": "qil_paged_decode_append: the 256 new tokens' K/V write fused into the decode "
                    "kernel (value and ms_per_step)",
            "GB_per_s": round(value, 1),
            "frac": round(value / HBM_PEAK_GBS, 4),
            "event_bracket_us_mean": round(dec["step_bracket_ms"] * 1e3, 2),
            "event_bracket_us_median": round(dec["step_bracket_ms_median"] * 1e3, 2),
            "hot_no_flush_GB_s": round(dec["step_bytes"] / (dec["hot_step_ms"] * 1e-3) / 1e9, 1),
        },
        "two_call_step": {
            "calls": "qil_kv_write (256 tokens) then qil_paged_decode",
            "step_us": round(dec["two_call_step_ms"] * 1e3, 2),
            "GB_per_s": round(dec["step_bytes"] / (dec["two_call_step_ms"] * 1e-3) / 1e9, 1),
            "write_alone_us": round(dec["write_ms"] * 1e3, 2),
        },
        "step_us": {"mean": round(dec["step_ms"] * 1e3, 2), "median": round(dec["step_ms_median"] * 1e3, 2),
                    "p10": round(dec["step_ms_p10"] * 1e3, 2), "p90": round(dec["step_ms_p90"] * 1e3, 2)},
        "decode_tokens_per_s": round(w.batch / (dec["step_ms"] * 1e-3), 1),
    }
    d2 = res["decode_b32"]
    a2 = d2["dec_bytes"] / (d2["dec_ms"] * 1e-3) / 1e9
    v2 = d2["step_bytes"] / (d2["step_ms"] * 1e-3) / 1e9
    line["decode_b32"] = {
        "workload": "decode-b32: 32 requests, Hq 16 / Hkv 8 (Qwen3-0.6B attention), page 16, "
                    "context U[128,2048], pool 8192 pages; step = write 32 new tokens + paged decode",
        "bound": "hbm", "achieved": round(a2, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(a2 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_launch": int(d2["dec_bytes"]),
        "launch_us_mean": round(d2["dec_ms"] * 1e3, 2),
        "launch_timing": "(flush, write, decode) minus (flush, write), as for the roofline kernel",
        "fused_step": {"us": round(d2["step_ms"] * 1e3, 2), "GB_per_s": round(v2, 1),
                       "frac": round(v2 / HBM_PEAK_GBS, 4)},
        "two_call_step_us": round(d2["two_call_step_ms"] * 1e3, 2),
        "decode_tokens_per_s": round(d2["workload"].batch / (d2["step_ms"] * 1e-3), 1),
    }
    if "prefill" in res:
        p = res["prefill"]
        tf = p["flops"] / (p["pre_ms"] * 1e-3) / 1e12
        line["prefill"] = {
            "workload": "prefill-varlen: 8 requests, cached prefix U[0,512] + chunk U[32,2048], "
                        "Hq 16 / Hkv 8, page 16",
            "bound": "mfma",
            "achieved": round(tf, 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "causal_flops": int(p["flops"]),
            "launch_us_mean": round(p["pre_ms"] * 1e3, 2),
            "event_bracket_us_mean": round(p["pre_bracket_ms"] * 1e3, 2),
            "event_bracket_us_median": round(p["pre_bracket_ms_median"] * 1e3, 2),
            "step_us_mean": round(p["step_ms"] * 1e3, 2),
            "append_step_us_mean": round(p["append_step_ms"] * 1e3, 2),
            "step_timing": "step_us_mean: the chunk's qil_kv_write then qil_paged_prefill; "
                           "append_step_us_mean: the same step as one qil_paged_prefill_append "
                           "call (event bracket around each step)",
            "traffic": traffic_for("prefill-varlen"),
            "measured_ceiling": res["ceilings"]["mfma_bf16_TFLOP_s"],
            "frac_of_measured": round(tf / res["ceilings"]["mfma_bf16_TFLOP_s"], 4),
            # each wavefront reads a 64-key tile's K (16 x ds_read_b128) and V
            # (32 x ds_read_b64_tr_b16) from LDS for its 32 query rows
            "lds_reads_per_wave_tile": {"ds_read_b128": 16, "ds_read_b64_tr_b16": 32},
            "lds_read_ceiling_B_per_clk_per_CU": res["ceilings"]["lds_read_B_per_clk_per_CU"],
        }
    if "prefill" in res:
        p = res["prefill"]
        line["kv_write"] = {
            "workload": f"prefill-varlen chunk write, {p['write_tokens']} tokens x 8 KV heads, plain copy",
            "bound": "hbm", "achieved": round(p["write_bytes"] / (p["write_ms"] * 1e-3) / 1e9, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(p["write_bytes"] / (p["write_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "launch_us_mean": round(p["write_ms"] * 1e3, 2), "algorithmic_bytes": int(p["write_bytes"]),
            "traffic": traffic_for("kv-write-chunk")}
    if "mixed" in res:
        m = res["mixed"]
        line["mixed_step"] = {
            "workload": "mixed-8b: Hq 32 / Hkv 8, per layer fused Q/K RMSNorm+RoPE write of 2112 "
                        "tokens, decode of 64 requests (context U[512,8192]), prefill of 4 x 512 "
                        "over prefixes U[0,4096]; page 16",
            "inputs": "per layer the workload's own lengths, block tables, slots and positions; "
                      "pools and new rows N(0,1) bf16 from a seeded device generator (timing only)",
            "layers_timed": m["layers"], "us_per_layer": round(m["layer_ms"] * 1e3, 1),
            "step_us": {"mean": round(m["step_ms"] * 1e3, 1), "median": round(m["step_ms_median"] * 1e3, 1),
                        "p10": round(m["step_ms_p10"] * 1e3, 1), "p90": round(m["step_ms_p90"] * 1e3, 1)},
            "us_per_layer_single_launch": round(m["single_launch_layer_ms"] * 1e3, 1),
            "single_launch_us": round(m["single_launch_ms"] * 1e3, 2),
            "us_per_36_layer_step": round(m["layer_ms"] * 1e3 * 36, 1),
            "tokens_per_s_36_layers": round((64 + 2048) / (m["layer_ms"] * 36 * 1e-3), 1),
            "tokens_per_s_36_layers_single_launch":
                round((64 + 2048) / (m["single_launch_layer_ms"] * 36 * 1e-3), 1),
            "per_call_timing": "event brackets around each call (pass 1 of timed_steps); a bracket "
                               "includes the dispatch gap a marker puts in front of its kernel",
            "fused_write": {"us": round(m["fused_ms"] * 1e3, 2),
                            "GB_per_s": round(m["fused_bytes"] / (m["fused_ms"] * 1e-3) / 1e9, 1),
                            "bound": "hbm", "peak": HBM_PEAK_GBS,
                            "frac": round(m["fused_bytes"] / (m["fused_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "algorithmic_bytes": int(m["fused_bytes"]),
                            "traffic": traffic_for("fused-write-8b")},
            "decode": {"us": round(m["dec_ms"] * 1e3, 2),
                       "GB_per_s": round(m["dec_bytes"] / (m["dec_ms"] * 1e-3) / 1e9, 1),
                       "bound": "hbm", "peak": HBM_PEAK_GBS,
                       "frac": round(m["dec_bytes"] / (m["dec_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "prefill": {"us": round(m["pre_ms"] * 1e3, 2),
                        "TFLOP_per_s": round(m["pre_flops"] / (m["pre_ms"] * 1e-3) / 1e12, 1),
                        "bound": "mfma", "peak": BF16_PEAK_TFLOPS,
                        "frac": round(m["pre_flops"] / (m["pre_ms"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}}
    if "graph" in res:
        gr = res["graph"]
        line["decode_graph"] = {
            "workload": f"decode step of {gr['layers']} layers (write 1 new token + paged decode per "
                        "layer as one qil_paged_decode_append call), Hq 16 / Hkv 8, page 256, context "
                        "U[16,1024]+U[0,1024], eager Python launches vs HIP-graph replay per batch "
                        "bucket; two_call_graph_us: the graph of qil_kv_write + qil_paged_decode",
            "buckets": gr["buckets"]}
    if "shared" in res:
        line["shared_prefix"] = {
            "workload": "Hq 32 / Hkv 8, page 16, a 4096-token prefix in 256 shared pages vs "
                        "private copies; prefill: 8 chunks of 512 after it; decode: 64 requests "
                        "with private tails U[1,1024]",
            **res["shared"]}
    if "qkv_proj" in res:
        qp = res["qkv_proj"]
        tf = qp["flops"] / (qp["fused_ms"] * 1e-3) / 1e12
        line["qkv_proj"] = {
            "workload": f"qkv-proj-8b: {qp['tokens']} tokens x hidden 4096 -> 32 q + 2 x 8 KV heads "
                        "(N 6144), Q/K RMSNorm + RoPE + scatter into page-16 pools as the epilogue",
            "bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "flops": int(qp["flops"]), "launch_us": round(qp["fused_ms"] * 1e3, 2),
            "traffic": traffic_for("qkv-proj-8b"),
            "library_gemm_then_fused_write_us": {
                "gemm": round(qp["gemm_ms"] * 1e3, 2), "fused_write": round(qp["write_ms"] * 1e3, 2),
                "total": round((qp["gemm_ms"] + qp["write_ms"]) * 1e3, 2)},
            "decode_step_64_tokens_us": {
                "one_kernel_split": round(qp["decode_step_ms"] * 1e3, 2),
                "library_gemm_then_fused_write": round(qp["decode_step_library_ms"] * 1e3, 2)}}
    if "shard" in res:
        line["tp8_shard_decode"] = res["shard"]
    if "long_prefix" in res:
        line["prefill_long_prefix"] = {
            "workload": "chunked prefill of a long prompt: Hq 32 / Hkv 8, page 16, one 512-token "
                        "chunk after a cached prefix; query tiles split over keys (automatic plan) "
                        "vs run whole",
            "cases": res["long_prefix"]}
    if not args.skip_cpu:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
