"""Per-head Q/K RMSNorm, RoPE and the fused norm + RoPE + scatter write
(oracle; test infrastructure).

What the pages fix ("nano-vLLM learning note"):
  * ``Qwen3Attention.forward`` block: q is viewed as [tokens][num_heads][D],
    k as [tokens][num_kv_heads][D]; ``q_norm`` / ``k_norm`` act per head
    (over D), then ``rotary_emb(positions, q, k)``, then attention, whose
    first step stores k and v into the cache.
  * ``RMSNorm.rms_forward`` block: x is widened to float, var = mean(x^2)
    over the last axis, x *= rsqrt(var + eps), then x is cast back to the
    original dtype and multiplied by the weight (in that dtype).
  * ``apply_rotary_emb`` block: split x (as float) into halves x1, x2;
    y1 = x1*cos - x2*sin, y2 = x2*cos + x1*sin; concatenate; cast back.
  * ``RotaryEmbedding`` block: inv_freq = 1 / base^(arange(0, rd, 2) / rd);
    the cache concatenates cos and sin along the last axis.
The "qwen-inference-lab" README lists Q/K RMSNorm and absolute-position RoPE
among the Qwen3 forward features.

Readings where the pages leave a step open:
  * rotary_dim = head_dim (the whole head rotates, rotate-half pairing of
    d and d + D/2).
  * The cos/sin table is an fp32 input [max_position][D]: columns 0..D/2-1
    hold cos(pos * inv_freq[j]), columns D/2..D-1 hold sin(pos * inv_freq[j]).
    ``rope_table`` builds it in fp64 and rounds each entry to fp32 once.
  * All arithmetic is fp64; results are rounded to bf16 exactly where the
    page casts back: after the normalisation, after the weight product, and
    after the rotation.
"""

import numpy as np

from .bf16 import bf16_to_f64, f64_to_bf16, round_bf16


def rope_inv_freq(head_dim, theta):
    """inv_freq[j] = theta ** (-(2j) / head_dim), j = 0 .. head_dim/2 - 1."""
    j = np.arange(0, head_dim, 2, dtype=np.float64)
    return 1.0 / np.power(float(theta), j / head_dim)


def rope_table(max_position, head_dim, theta):
    """fp32 [max_position][head_dim]: cos block then sin block, angle
    pos * inv_freq[j] evaluated in fp64."""
    pos = np.arange(max_position, dtype=np.float64)[:, None]
    ang = pos * rope_inv_freq(head_dim, theta)[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def rms_normalize(x, eps):
    """x / sqrt(mean(x^2) + eps) along the last axis, fp64, unrounded."""
    x = np.asarray(x, dtype=np.float64)
    var = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(var + float(eps))


def rope_rotate(y, cos, sin):
    """Rotate-half RoPE in fp64, unrounded.  y [..., D]; cos, sin [..., D/2]."""
    half = y.shape[-1] // 2
    y1, y2 = y[..., :half], y[..., half:]
    return np.concatenate([y1 * cos - y2 * sin, y2 * cos + y1 * sin], axis=-1)


def qk_norm_rope(x_bits, w_bits, eps, cos, sin):
    """One or more bf16 head rows -> bf16 bits after RMSNorm then RoPE.

    x_bits : uint16 [..., D]   (bf16 input rows)
    w_bits : uint16 [D]        (bf16 norm weight)
    cos, sin : float64 [..., D/2] broadcastable to the rows (from the fp32
               table, widened exactly)
    Rounding points follow the page: bf16 after normalising, bf16 after the
    weight product, bf16 after the rotation.
    """
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_bits)
    y = round_bf16(rms_normalize(x, eps))
    y = round_bf16(y * w)
    return f64_to_bf16(rope_rotate(y, cos, sin))


def fused_kv_write(k_pool, v_pool, q_bits, k_bits, v_bits, slot_mapping,
                   positions, q_norm_w, k_norm_w, eps, cos_sin, page_size):
    """Fused Q/K RMSNorm + RoPE + scatter write (in place on the pools).

    q_bits [T][Hq][D], k_bits / v_bits [T][Hkv][D] (uint16 bf16 bits);
    positions [T] absolute token positions; cos_sin fp32 [max_pos][D].
    Returns q_out bits [T][Hq][D].  k goes to the pool normalised and
    rotated, v goes raw; tokens whose slot is -1 are not stored, but their
    q is still produced.
    """
    from .paged import kv_write

    half = q_bits.shape[-1] // 2
    table = np.asarray(cos_sin, dtype=np.float32).astype(np.float64)
    pos = np.asarray(positions, dtype=np.int64)
    cos = table[pos, :half][:, None, :]
    sin = table[pos, half:][:, None, :]
    q_out = qk_norm_rope(q_bits, q_norm_w, eps, cos, sin)
    k_out = qk_norm_rope(k_bits, k_norm_w, eps, cos, sin)
    kv_write(k_pool, v_pool, k_out, v_bits, slot_mapping, page_size)
    return q_out
