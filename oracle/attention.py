"""GQA causal softmax attention read through block tables (oracle; test
infrastructure).

What the pages fix:
  * "qwen-inference-lab" README, feature list: GQA, causal attention, paged
    KV storage that never reads unwritten positions.
  * "qvllm" README, Scope: causal masking only (no dropout, alibi, sliding
    window or non-causal masks).
  * "nano-vLLM learning note": ``Qwen3Attention.forward`` (q has num_heads
    heads, k/v have num_kv_heads heads), ``Attention.forward`` (store k/v
    into the cache first, then attend over the cache: varlen for prefill,
    with-kvcache for decode), ``Context`` (cu_seqlens, context_lens,
    block_tables), ``prepare_decode`` (context length includes the token
    being decoded; its position is len - 1) and ``prepare_prefill``
    (positions run from num_cached_tokens).
  * "qwen-engine" README: flat varlen prefill packs requests by cu_seqlens.

Readings where the pages are silent:
  * Query head h reads KV head h // G with G = Hq / Hkv (contiguous groups).
  * The context length L_r counts every key of request r after this step's
    write; the n_r new tokens are its last n_r positions, so new token i
    sits at position L_r - n_r + i and sees keys 0 .. that position
    (bottom-right aligned causal mask).  Decode is n_r = 1.
  * ``scale`` multiplies q.k before the softmax.

The computation is the plain definition, in fp64: scores, max-subtracted
exponentials, normalised weighted sum of V.  A matmul is the only library
step.
"""

import numpy as np

from .bf16 import to_f64
from .paged import gather_request


def attend(q, keys, values, scale, num_kv_heads):
    """Causal GQA attention of one request's new tokens over its context.

    q      : float64 [n][Hq][D]   (the request's n new tokens)
    keys   : float64 [L][Hkv][D]  (its whole context, n <= L)
    values : float64 [L][Hkv][D]
    returns float64 [n][Hq][D]
    """
    n, hq, _ = q.shape
    length = keys.shape[0]
    group = hq // num_kv_heads
    out = np.zeros_like(q)
    pos = length - n + np.arange(n)                   # absolute positions
    visible = np.arange(length)[None, :] <= pos[:, None]
    for h in range(hq):
        g = h // group
        s = (q[:, h, :] @ keys[:, g, :].T) * float(scale)
        s = np.where(visible, s, -np.inf)
        m = np.max(s, axis=1, keepdims=True)
        w = np.exp(s - m)
        out[:, h, :] = (w @ values[:, g, :]) / np.sum(w, axis=1, keepdims=True)
    return out


def paged_attention(q_bits, k_pool, v_pool, block_tables, cu_seqlens,
                    context_lens, scale, page_size, dtype, requests=None):
    """Attention for a packed batch of new tokens over paged K/V.

    q_bits       : raw bits [T][Hq][D], requests packed by cu_seqlens
    k_pool/v_pool: raw bits [num_pages][Hkv][P][D]
    block_tables : int [B][stride]; context_lens [B]; cu_seqlens [B+1]
    requests     : optional iterable of request indices to evaluate
    returns float64 [T][Hq][D]; rows of requests not evaluated are NaN.
    """
    q = to_f64(q_bits, dtype)
    out = np.full(q.shape, np.nan)
    num_kv_heads = k_pool.shape[1]
    batch = len(context_lens)
    todo = range(batch) if requests is None else requests
    for r in todo:
        lo, hi = int(cu_seqlens[r]), int(cu_seqlens[r + 1])
        if hi == lo:
            continue
        length = int(context_lens[r])
        keys = to_f64(gather_request(k_pool, block_tables[r], length, page_size), dtype)
        vals = to_f64(gather_request(v_pool, block_tables[r], length, page_size), dtype)
        out[lo:hi] = attend(q[lo:hi], keys, vals, scale, num_kv_heads)
    return out


def paged_decode(q_bits, k_pool, v_pool, block_tables, context_lens, scale,
                 page_size, dtype, requests=None):
    """Decode: one new token per request (q_bits [B][Hq][D])."""
    batch = len(context_lens)
    cu = np.arange(batch + 1)
    return paged_attention(q_bits, k_pool, v_pool, block_tables, cu,
                           context_lens, scale, page_size, dtype, requests)
