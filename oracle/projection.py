"""The merged QKV projection ahead of the fused norm + RoPE + scatter write
(oracle; test infrastructure).

What the pages fix ("nano-vLLM learning note"):
  * ``QKVParallelLinear`` block: one linear layer produces q, k and v
    together; its output has (num_heads + 2 * num_kv_heads) * head_size
    columns laid out as [Q | K | V] (all q heads, then all k heads, then all
    v heads, head_size columns each).
  * ``Qwen3Attention.forward`` block: ``qkv = qkv_proj(hidden_states)``,
    split into q, k, v along the last axis, viewed per head, then q_norm /
    k_norm, rotary_emb, and attention (whose first step stores k and v).
  * The layer is an ``nn.Linear`` (weight [out_features][in_features], no
    bias for Qwen3's attention projection since ``qkv_bias`` is false), so
    the output is hidden_states @ weight^T in the activation dtype.

Readings where the pages leave a step open:
  * bf16 activations and weights; the product is exact in fp64 here and is
    rounded to bf16 once, as the bf16 linear layer's output.  The norm,
    RoPE and write then follow ``norm_rope.fused_kv_write`` on those bf16
    rows.
"""

import numpy as np

from .bf16 import bf16_to_f64, f64_to_bf16
from .norm_rope import fused_kv_write


def qkv_projection(x_bits, w_bits):
    """bf16 [T][hidden] activations times a bf16 [N][hidden] weight
    (nn.Linear layout): returns the bf16 bits of x @ w^T, [T][N].  The
    matrix product is numpy's fp64 matmul of the exactly decoded inputs."""
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_bits)
    return f64_to_bf16(x @ w.T)


def split_qkv(qkv_bits, num_q_heads, num_kv_heads, head_dim=128):
    """[T][(Hq + 2 Hkv) * D] -> q [T][Hq][D], k [T][Hkv][D], v [T][Hkv][D]
    (the [Q | K | V] column order of the merged layer)."""
    t = qkv_bits.shape[0]
    nq, nk = num_q_heads * head_dim, num_kv_heads * head_dim
    q = qkv_bits[:, :nq].reshape(t, num_q_heads, head_dim)
    k = qkv_bits[:, nq:nq + nk].reshape(t, num_kv_heads, head_dim)
    v = qkv_bits[:, nq + nk:nq + 2 * nk].reshape(t, num_kv_heads, head_dim)
    return q, k, v


def qkv_proj_write(k_pool, v_pool, x_bits, w_bits, num_q_heads, num_kv_heads, slot_mapping,
                   positions, q_norm_w, k_norm_w, eps, cos_sin, page_size):
    """Project, split, then the fused Q/K norm + RoPE + scatter write (in
    place on the pools).  Returns (q_out bits [T][Hq][D], qkv bits [T][N])."""
    qkv = qkv_projection(x_bits, w_bits)
    q, k, v = split_qkv(qkv, num_q_heads, num_kv_heads)
    q_out = fused_kv_write(k_pool, v_pool, q, k, v, slot_mapping, positions, q_norm_w, k_norm_w,
                           eps, cos_sin, page_size)
    return q_out, qkv
