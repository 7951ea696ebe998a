/*
 * qil.h -- C ABI of libqil: attention over a paged KV cache on MI355X (gfx950).
 *
 * The operations follow the problem statement of the compact Qwen3 engines
 * described on these pages:
 *   - "nano-vLLM learning note" (floratopia): the store_kvcache_kernel block
 *     (scatter of new K/V rows through a slot mapping, -1 = skip), the
 *     Attention.forward block (store first, then varlen prefill or decode over
 *     the cache), the Context block (cu_seqlens, max_seqlen, slot_mapping,
 *     context_lens, block_tables), the ModelRunner.prepare_decode /
 *     prepare_prefill blocks (positions, context length, slot formula),
 *     RMSNorm.rms_forward, apply_rotary_emb and RotaryEmbedding.
 *   - "qwen-inference-lab" README: GQA, Q/K RMSNorm, absolute-position RoPE,
 *     causal attention, paged KV that never reads unwritten positions.
 *   - "qwen-engine" README: token-slot KV pool with per-request page tables,
 *     flat varlen prefill packed by cu_seqlens, prefill and decode as separate
 *     kernels (prefill compute-bound, decode memory-bound).
 *
 * Conventions common to every call
 * --------------------------------
 *  - Every tensor pointer is DEVICE memory owned by the caller.  The library
 *    never allocates, frees or synchronises; work is enqueued on `stream`
 *    (a hipStream_t passed as void*; NULL = the null stream).  Calls contain
 *    no host synchronisation, so they may be captured into a HIP graph.
 *  - Return value: QIL_OK (0) or an error code.  On error nothing has been
 *    enqueued and qil_last_error() (thread-local) describes the problem.
 *    All argument checks happen before any HIP call, so they run on a host
 *    without a GPU.  No exception crosses the ABI and nothing aborts.
 *  - head_dim must be 128.  page_size must be 16, 32, 64, 128 or 256.
 *    num_q_heads must be num_kv_heads * G with G in {1, 2, 4, 5, 8, 16}
 *    (G <= 8 for fp32 decode).
 *  - dtype: QIL_F32 (IEEE binary32) or QIL_BF16 (bfloat16).  Outputs have the
 *    input dtype; accumulation is fp32.  Pointers must be 16-byte aligned.
 *  - Device-resident metadata (slots, page ids, lengths) is a precondition,
 *    not checked by default.  The kernels still never dereference an
 *    out-of-range page id or slot and never read a block-table row past
 *    max_context_len: a write to such a slot is skipped, and the attention
 *    output of a request whose table holds such a page is unspecified (but
 *    finite memory is all that is touched).
 *  - Debug mode (environment variable QIL_DEBUG set to anything but "0" when
 *    the library first looks, or qil_set_debug(1)) checks that metadata on
 *    the device before each launch and returns QIL_EINVAL, with the first
 *    violation in qil_last_error(), instead of launching: slots that are
 *    neither -1 nor in the pool, duplicate slots within one kv_write call,
 *    positions outside [0, max_position), context lengths outside
 *    [1, min(max_context_len, block_table_stride*page_size)], block-table
 *    entries that a request reads and that are not pages of the pool, and
 *    cu_seqlens that do not run 0 <= ... <= total_q or give a request more
 *    new tokens than its context or max_seqlen_q.  The checks synchronize
 *    the stream, so debug-mode calls cannot be captured into a graph (they
 *    return QIL_EINVAL under capture).
 *
 * KV pool layout (the "paged KV cache")
 * -------------------------------------
 *  K and V live in two pools of identical shape
 *      [num_pages][num_kv_heads][page_size][head_dim]
 *  i.e. element (slot s, KV head g, dim d) is at flat index
 *      ((s / page_size * num_kv_heads + g) * page_size + s % page_size) * head_dim + d.
 *  A slot names (physical page, offset): s = page * page_size + offset.
 *  One (page, head) slab is contiguous (page_size rows of 256 bytes in bf16),
 *  and every 128-element row is 256-byte aligned when the pool is.
 *
 * Block tables
 *  int32 [batch][block_table_stride]: entry i of row r is the physical page
 *  holding logical tokens [i*page_size, (i+1)*page_size) of request r.  Only
 *  the first ceil(context_lens[r] / page_size) entries of a row are read.
 *
 * Context length
 *  context_lens[r] counts every key of request r after this step's write,
 *  including its new tokens; the new tokens are its last positions.  A new
 *  token at position p attends to keys 0..p (causal, bottom-right aligned).
 *  Query head h reads KV head h / G.
 */
#ifndef QIL_H
#define QIL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum qil_status {
  QIL_OK = 0,
  QIL_EINVAL = 1,        /* null/misaligned pointer, bad count or stride      */
  QIL_EUNSUPPORTED = 2,  /* head_dim, page_size, GQA ratio or dtype not built */
  QIL_EWORKSPACE = 3,    /* workspace missing or too small                    */
  QIL_EHIP = 4           /* the HIP runtime rejected a launch                 */
};

enum qil_dtype { QIL_F32 = 0, QIL_BF16 = 1 };

/* Library version string, e.g. "qil 0.1.0 gfx950". */
const char* qil_version(void);

/* Description of the last error on the calling thread ("" if none). */
const char* qil_last_error(void);

/* Debug mode (see above): on (non-zero) or off for every later call in the
 * process, overriding QIL_DEBUG.  qil_debug_enabled() reports the setting. */
void qil_set_debug(int enabled);
int qil_debug_enabled(void);

/*
 * Fused per-head Q/K RMSNorm + RoPE applied by qil_kv_write before the
 * scatter ("nano-vLLM learning note": Qwen3Attention.forward applies q_norm
 * and k_norm per head, then rotary_emb, then stores k and v; RMSNorm.rms_forward
 * and apply_rotary_emb give the arithmetic).  bf16 only.
 *
 * Per head row x (head_dim values, fp32 arithmetic):
 *     y = bf16(x * rsqrt(mean(x^2) + eps));   y = bf16(y * weight)
 *     out[j]        = bf16(y[j] * cos[j] - y[j + D/2] * sin[j])
 *     out[j + D/2]  = bf16(y[j + D/2] * cos[j] + y[j] * sin[j])     j < D/2
 * where cos[j] = cos_sin[pos][j] and sin[j] = cos_sin[pos][D/2 + j].
 * The rotated k rows go to the pool, v rows go raw, and the rotated q rows go
 * to q_out (written for every token, including tokens whose slot is -1).
 */
typedef struct qil_qknorm_rope {
  const void* q;             /* bf16 rows, token t head h at q + t*q_token_stride + h*head_dim */
  void* q_out;               /* bf16 [num_tokens][num_q_heads][head_dim] contiguous; may equal q
                                only when q_token_stride == num_q_heads*head_dim                */
  int64_t q_token_stride;    /* elements between consecutive tokens of q (>= num_q_heads*head_dim) */
  int32_t num_q_heads;
  const void* q_norm_weight; /* bf16 [head_dim] */
  const void* k_norm_weight; /* bf16 [head_dim] */
  float eps;
  const int32_t* positions;  /* [num_tokens] absolute positions, each in [0, max_position)   */
  const float* cos_sin;      /* fp32 [max_position][head_dim]: cos block then sin block        */
  int32_t max_position;
} qil_qknorm_rope;

/*
 * qil_kv_write -- scatter new K/V rows into the pools through slot_mapping
 * ("nano-vLLM learning note", store_kvcache_kernel block: one row of
 * num_kv_heads*head_dim elements per token, stored at its slot; slot -1 means
 * skip).
 *
 *   k, v            token t's row starts at k + t*k_token_stride (elements);
 *                   heads are contiguous within the row (stride head_dim).
 *                   Strides may exceed num_kv_heads*head_dim (a view into a
 *                   fused QKV buffer) and must be multiples of 8.
 *   k_cache/v_cache pools (layout above) of num_pages pages.
 *   slot_mapping    int32 [num_tokens]; -1 = skip; slots must be distinct
 *                   within one call (duplicates leave either row).
 *   fuse            NULL for a plain bit-exact copy, else the Q/K norm + RoPE
 *                   parameters above (dtype must be QIL_BF16).
 * num_tokens == 0 is a no-op.
 */
int qil_kv_write(const void* k, const void* v, int64_t k_token_stride, int64_t v_token_stride,
                 void* k_cache, void* v_cache, const int32_t* slot_mapping,
                 int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                 int32_t page_size, int32_t num_pages, int32_t dtype,
                 const qil_qknorm_rope* fuse, void* stream);

/*
 * qil_rope_cos_sin -- build the fp32 RoPE table used by the fused write
 * ("nano-vLLM learning note", RotaryEmbedding block: inv_freq[j] =
 * theta^(-2j/D), cache = cat(cos, sin)).  Entry [p][j] = cos(p * inv_freq[j])
 * and [p][D/2 + j] = sin(p * inv_freq[j]) for j < D/2, evaluated in fp64 and
 * rounded once to fp32.  cos_sin: device fp32 [max_position][head_dim].
 */
int qil_rope_cos_sin(float* cos_sin, int32_t max_position, int32_t head_dim, double theta,
                     void* stream);

/*
 * qil_qkv_proj_write -- the merged QKV projection with the fused write as its
 * epilogue ("nano-vLLM learning note": QKVParallelLinear gives one linear
 * layer whose output columns are all q heads, then all k heads, then all v
 * heads; Qwen3Attention.forward projects, splits per head, applies q_norm /
 * k_norm and rotary_emb, and its attention step stores k and v).  bf16 only;
 * one kernel, matrix cores with fp32 accumulation.
 *
 * For every token t and output column n of N = (Hq + 2 Hkv) * head_dim:
 *     qkv[t][n] = bf16( sum_k x[t][k] * weight[n][k] )      (no bias)
 * then columns [0, Hq*D) are the q heads, [Hq*D, (Hq+Hkv)*D) the k heads and
 * the rest the v heads, and each head row goes through exactly what
 * qil_kv_write does with a qil_qknorm_rope: q and k rows are normalised,
 * weighted and rotated (the formula above that struct), rotated k rows and
 * the projected v rows are stored at slot_mapping[t] (-1 = skip), and the
 * rotated q rows go to q_out.
 *
 *   x               bf16, token t's `hidden` values at x + t*x_token_stride
 *   weight          bf16 nn.Linear layout: row n (N rows) at weight + n*weight_row_stride,
 *                   `hidden` values each
 *   hidden          multiple of 64; strides are multiples of 8 elements and >= hidden
 *   q_out           bf16 [num_tokens][num_q_heads][head_dim]
 *   qkv_out         NULL, or bf16 [num_tokens][N]: also store the rounded projection
 *   k_cache/v_cache, slot_mapping, page_size, num_pages: as for qil_kv_write
 *   q_norm_weight, k_norm_weight, eps, positions, cos_sin, max_position:
 *                   as in qil_qknorm_rope
 *   workspace       device scratch of at least qil_qkv_proj_workspace_size(...)
 *                   bytes, 16-byte aligned (may be NULL when that size is 0).
 *                   Small batches (below 1024 tokens, when the grid of whole
 *                   heads would be small) split the hidden dimension: fp32
 *                   partial sums go here and a second kernel adds them in a
 *                   fixed order before the epilogue.  Contents on entry do not
 *                   matter.
 * Hq + 2 Hkv must be even (workgroups own pairs of heads).  Outputs must not
 * overlap the inputs.  num_tokens == 0 is a no-op.
 */
size_t qil_qkv_proj_workspace_size(int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t hidden);

int qil_qkv_proj_write(const void* x, int64_t x_token_stride, const void* weight,
                       int64_t weight_row_stride, int32_t hidden, void* q_out, void* qkv_out,
                       void* k_cache, void* v_cache, const int32_t* slot_mapping,
                       int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t page_size, int32_t num_pages,
                       const void* q_norm_weight, const void* k_norm_weight, float eps,
                       const int32_t* positions, const float* cos_sin, int32_t max_position,
                       void* workspace, size_t workspace_bytes, int32_t dtype, void* stream);

/*
 * qil_paged_decode -- one query token per request over its paged context
 * ("nano-vLLM learning note", Attention.forward decode branch and
 * prepare_decode: the token's position is context_len - 1; "qwen-engine"
 * README: decode is memory-bound).
 *
 *   out            [batch][num_q_heads][head_dim], dtype
 *   q              [batch][num_q_heads][head_dim], dtype
 *   block_tables   int32 [batch][block_table_stride]
 *   context_lens   int32 [batch], each in [1, block_table_stride*page_size]
 *   max_context_len host int >= every context_lens[r] (sizes the split grid)
 *   scale          multiplies q.k before the softmax (fp32)
 *   keys_per_split 0 = automatic, else a multiple of 64 up to 4096: the context of each
 *                  request is cut into splits of this many keys, each split
 *                  reduced by its own workgroup, then merged by a second
 *                  kernel through the log-sum-exp rule.
 *   workspace      device scratch of at least
 *                  qil_paged_decode_workspace_size(...) bytes (may be NULL when
 *                  that size is 0); its contents on entry do not matter.  It
 *                  holds the split partials when a request spans several
 *                  splits, and, when the grid has at least 512 workgroups
 *                  (batch * num_kv_heads * splits), room for the order in
 *                  which the requests are run, longest context first: bf16
 *                  batches of up to 256 requests are ranked by the decode
 *                  workgroups themselves, larger ones and fp32 by a first
 *                  small kernel that writes the order there.  Results do not
 *                  depend on that order.
 * batch == 0 is a no-op.
 */
size_t qil_paged_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t max_context_len, int32_t page_size,
                                       int32_t keys_per_split);

int qil_paged_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int32_t block_table_stride,
                     const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                     int32_t num_pages, int32_t max_context_len, float scale, int32_t dtype,
                     int32_t keys_per_split, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * qil_paged_decode_no_alloc -- qil_paged_decode for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments and
 * results as qil_paged_decode without workspace / workspace_bytes: the split
 * partials and the request order go to a fixed scratch array inside the
 * library, 32 MiB per GPU, held from the first call on that GPU until the
 * process ends.  A call that would need more (qil_paged_decode_workspace_size
 * above 33,554,432 bytes) returns QIL_EWORKSPACE before anything is enqueued.
 * The call allocates nothing.  All calls on one GPU share its array and its
 * contents need not start at zero: calls that overlap on one GPU (several
 * streams or threads at once) race; calls in order on one stream do not.
 */
int qil_paged_decode_no_alloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, int32_t block_table_stride,
                              const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                              int32_t num_pages, int32_t max_context_len, float scale,
                              int32_t dtype, int32_t keys_per_split, void* stream);

/*
 * qil_paged_decode_append -- the decode step's write and decode in one call:
 * the same result as qil_kv_write(k_new, v_new, slot_mapping) followed by
 * qil_paged_decode(...), for a batch whose new token of request r sits at
 * position context_lens[r] - 1 ("nano-vLLM learning note", prepare_decode:
 * the new token's slot is the block-table slot of the last position, and
 * Attention.forward stores k/v before attending).
 *
 *   k_new, v_new   [batch] rows of num_kv_heads*head_dim, dtype, token strides
 *                  in elements (>= num_kv_heads*head_dim, multiples of 8)
 *   slot_mapping   int32 [batch]: slot_mapping[r] must be the slot of position
 *                  context_lens[r] - 1 (block_tables[r][(L-1)/page_size] *
 *                  page_size + (L-1) % page_size), or -1 for a padding row
 *                  (nothing is stored; that row's output is unspecified);
 *                  QIL_DEBUG checks it
 *   other arguments as qil_paged_decode (workspace sized by
 *   qil_paged_decode_workspace_size).
 * bf16 runs one kernel (plus, when they apply, the ordering pass for more
 * than 256 requests and the split merge): the split that holds each
 * request's last key reads that key's rows
 * from k_new / v_new instead of the pool and stores them at their slot, so
 * the pool row is written and used in the same launch.  fp32 runs the write
 * and the decode as two kernels.  batch == 0 is a no-op.
 */
int qil_paged_decode_append(void* out, const void* q, const void* k_new, const void* v_new,
                            int64_t k_token_stride, int64_t v_token_stride,
                            const int32_t* slot_mapping, void* k_cache, void* v_cache,
                            const int32_t* block_tables, int32_t block_table_stride,
                            const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                            int32_t num_pages, int32_t max_context_len, float scale, int32_t dtype,
                            int32_t keys_per_split, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * qil_paged_prefill -- chunked varlen causal prefill over the paged cache
 * ("nano-vLLM learning note", Attention.forward prefill branch with cached
 * prefix and prepare_prefill: positions start at num_cached_tokens;
 * "qwen-engine" README: flat varlen prefill packed by cu_seqlens, compute-bound).
 * bf16 (QIL_BF16): QK^T and PV run on bf16 matrix cores with fp32
 * accumulation, the softmax weights are rounded to bf16 for the PV product.
 * fp32 (QIL_F32, a tight-tolerance path): each new token runs as one row of the
 * fp32 decode kernel over its own visible keys, on the vector ALUs; contexts up
 * to 4,096 keys, GQA groups up to 8, at most 65,535 tokens (else
 * QIL_EUNSUPPORTED); keys_per_split and the workspace are not used.
 *
 *   out, q         [total_q][num_q_heads][head_dim] (dtype), packed by cu_seqlens_q
 *   cu_seqlens_q   int32 [batch+1], cu[0] = 0, non-decreasing, cu[batch] = total_q;
 *                  request r owns rows cu[r] .. cu[r+1]-1 (n_r = cu[r+1]-cu[r] new tokens)
 *   context_lens   int32 [batch]: keys of request r including its n_r new tokens
 *                  (n_r <= context_lens[r]); new token i sits at position
 *                  context_lens[r] - n_r + i
 *   max_seqlen_q   host int >= every n_r;  max_context_len host int >= every context_lens[r]
 *   keys_per_split 0 = automatic, else a multiple of 64 up to 65472: a query
 *                  tile (256/G new tokens x the G query heads of one KV head)
 *                  whose visible keys span more than this many is cut into
 *                  pieces of near-equal length (at most 32 pieces: a smaller
 *                  value is raised to fit), each run by its own workgroup, and
 *                  the pieces are merged by the log-sum-exp rule.  Automatic
 *                  splitting applies when the call has at most 128 query
 *                  tiles x KV heads and max_context_len is at least 2,048, e.g.
 *                  a chunk of a long prompt.  Splitting needs
 *                  batch * ceil(max_seqlen_q / (256/G)) <= 4096; larger calls
 *                  run unsplit whatever keys_per_split says.
 *   workspace      device scratch of at least qil_paged_prefill_workspace_size(...)
 *                  bytes (may be NULL when that size is 0); its contents on
 *                  entry do not matter.  It holds the list of pieces, ordered
 *                  longest first by a small planning kernel, and the pieces'
 *                  partial rows.  Results do not depend on that order.
 * The K/V rows of the new tokens must already be in the pools (qil_kv_write
 * first).  Requests with n_r == 0 and batch == 0 are no-ops.
 */
size_t qil_paged_prefill_workspace_size(int32_t batch, int32_t total_q, int32_t max_seqlen_q,
                                        int32_t max_context_len, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t keys_per_split);

int qil_paged_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int32_t block_table_stride,
                      const int32_t* cu_seqlens_q, const int32_t* context_lens, int32_t batch,
                      int32_t total_q, int32_t max_seqlen_q, int32_t max_context_len,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t page_size, int32_t num_pages, float scale, int32_t dtype,
                      int32_t keys_per_split, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * qil_paged_prefill_append -- a prefill step's write and attention in one
 * call: the same result as qil_kv_write(k_new, v_new, slot_mapping) over the
 * call's total_q new tokens followed by qil_paged_prefill(...)
 * ("nano-vLLM learning note", prepare_prefill: each new token's slot is the
 * block-table slot of its position; Attention.forward stores k/v before
 * attending).
 *
 *   k_new, v_new   [total_q] rows of num_kv_heads*head_dim, packed like q by
 *                  cu_seqlens_q, dtype, token strides in elements
 *                  (>= num_kv_heads*head_dim, multiples of 8)
 *   slot_mapping   int32 [total_q]: the slot of each new token's position
 *                  (block_tables[r][p / page_size] * page_size + p % page_size
 *                  for position p = context_lens[r] - n_r + i); -1 stores
 *                  nothing.  The attention reads every new token's K/V from
 *                  k_new / v_new, so the result equals the two calls whenever
 *                  the slots follow the block tables (QIL_DEBUG checks the
 *                  slots' range).
 *   other arguments as qil_paged_prefill (workspace sized by
 *   qil_paged_prefill_workspace_size).
 * bf16 calls of whole query tiles (no split over keys) run one kernel: keys
 * at a request's new positions are loaded from k_new / v_new, and extra
 * workgroups at the end of the grid store the new rows into the pools, which
 * no other workgroup of the launch reads.  fp32 and calls split over keys run
 * qil_kv_write, then qil_paged_prefill.  batch == 0 or total_q == 0 is a
 * no-op.
 */
int qil_paged_prefill_append(void* out, const void* q, const void* k_new, const void* v_new,
                             int64_t k_token_stride, int64_t v_token_stride,
                             const int32_t* slot_mapping, void* k_cache, void* v_cache,
                             const int32_t* block_tables, int32_t block_table_stride,
                             const int32_t* cu_seqlens_q, const int32_t* context_lens,
                             int32_t batch, int32_t total_q, int32_t max_seqlen_q,
                             int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t page_size, int32_t num_pages, float scale,
                             int32_t dtype, int32_t keys_per_split, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * qil_paged_attention_mixed -- the decode batch and the prefill batch of one
 * step in a single launch over the same KV pool (plus the decode split merge
 * when the decode part has several splits).  The "qwen-engine" README keeps
 * prefill (compute-bound) and decode (memory-bound) in separate batches; here
 * they stay separate argument sets, with the meaning of qil_paged_decode and
 * qil_paged_prefill above, but their workgroups share the GPU: prefill query
 * tiles and decode splits are interleaved in one grid, so MFMA-bound and
 * HBM-bound work run side by side and the step has one tail.  bf16 only.
 *
 *   decode   NULL or a decode batch; its workspace is sized by
 *            qil_paged_decode_workspace_size (same split plan)
 *   prefill  NULL or a prefill batch (its K/V rows already written)
 * Both batches use k_cache / v_cache, the head counts, page size, scale and
 * dtype given here.  The prefill part runs whole query tiles (unsplit).  Each batch's arguments are checked as in its own call
 * (a NULL or empty batch is allowed); outputs must not overlap.
 */
typedef struct qil_decode_batch {
  void* out;                       /* [batch][num_q_heads][head_dim] */
  const void* q;                   /* [batch][num_q_heads][head_dim] */
  const int32_t* block_tables;     /* [batch][block_table_stride]    */
  int32_t block_table_stride;
  const int32_t* context_lens;     /* [batch]                        */
  int32_t batch;
  int32_t max_context_len;
  int32_t keys_per_split;          /* 0 = automatic                  */
  void* workspace;
  size_t workspace_bytes;
} qil_decode_batch;

typedef struct qil_prefill_batch {
  void* out;                       /* [total_q][num_q_heads][head_dim] */
  const void* q;                   /* [total_q][num_q_heads][head_dim] */
  const int32_t* block_tables;     /* [batch][block_table_stride]      */
  int32_t block_table_stride;
  const int32_t* cu_seqlens_q;     /* [batch + 1]                      */
  const int32_t* context_lens;     /* [batch]                          */
  int32_t batch;
  int32_t total_q;
  int32_t max_seqlen_q;
  int32_t max_context_len;
} qil_prefill_batch;

int qil_paged_attention_mixed(const qil_decode_batch* decode, const qil_prefill_batch* prefill,
                              const void* k_cache, const void* v_cache, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                              int32_t num_pages, float scale, int32_t dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QIL_H */
