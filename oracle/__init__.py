"""CPU oracle for paged KV attention — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct fp64 (numpy) restatement of what the paged
KV attention hot path computes.  It exists to check the HIP library, never to
serve it: only the test-suite, the package smoke check and the CPU-baseline
leg of the benchmark may import it.  It shares no code, table or constant
generator with the HIP path (``paged_kv_attention_16_amd``), and the HIP path
never imports it.

Sources (web pages; cited by page title and the code block or section):
  * "nano-vLLM learning note" (floratopia): the ``store_kvcache_kernel``,
    ``RMSNorm.rms_forward``, ``apply_rotary_emb``, ``RotaryEmbedding``,
    ``QKVParallelLinear``, ``Qwen3Attention.forward``,
    ``ModelRunner.prepare_prefill`` / ``prepare_decode``, ``Context`` and
    ``allocate_kv_cache`` code blocks.
  * "qwen-inference-lab" README (qil): feature list (GQA, Q/K RMSNorm,
    absolute-position RoPE, causal attention, paged KV that never reads
    unwritten positions) and its validation section (full prefill,
    token-by-token and irregular-chunk logits agree).
  * "qwen-engine" README: paged KV cache / flat varlen prefill feature table
    and the prefill-vs-decode design note.

Modules:
  bf16       -- exact bf16 <-> fp64 conversion (round-to-nearest-even).
  paged      -- pool layout accessor and the plain ``kv_write`` scatter.
  norm_rope  -- per-head RMSNorm, RoPE table and the fused Q/K norm + RoPE
                + scatter write, with the pages' rounding points.
  attention  -- GQA causal softmax attention read through block tables
                (decode is the one-query-token case of prefill).
  projection -- the merged QKV linear layer ahead of the fused write
                ([Q | K | V] columns, bf16 output).

Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, library routines (torch float64 SDPA / rms_norm, numpy complex
arithmetic) and invariants the pages fix.
"""

from . import bf16, paged, norm_rope, attention, projection  # noqa: F401
