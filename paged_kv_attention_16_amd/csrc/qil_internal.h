// Internal declarations shared by the libqil translation units (not part of
// the public ABI; the public header is include/qil.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qil {

constexpr int kHeadDim = 128;

// ---- kv_write --------------------------------------------------------------
struct KvWriteArgs {
  const void* k;
  const void* v;
  int64_t k_stride;  // elements between tokens
  int64_t v_stride;
  void* k_cache;
  void* v_cache;
  const int32_t* slots;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t log2_page;
  int32_t num_pages;
  int32_t elem_bytes;  // 2 (bf16) or 4 (fp32)
};

struct FusedArgs {
  const void* q;
  void* q_out;
  int64_t q_stride;
  int32_t num_q_heads;
  const void* q_w;
  const void* k_w;
  float eps;
  const int32_t* positions;
  const float* cos_sin;
  int32_t max_position;
};

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t s);
hipError_t launch_kv_write_fused(const KvWriteArgs& a, const FusedArgs& f, hipStream_t s);
hipError_t launch_rope_table(float* table, int32_t max_position, int32_t head_dim, double theta,
                             hipStream_t s);

// ---- merged QKV projection + fused norm / RoPE / scatter (bf16) -----------
struct QkvProjArgs {
  const void* x;          // [num_tokens] rows of `hidden` values, stride x_stride
  int64_t x_stride;       // elements
  const void* weight;     // [(Hq + 2 Hkv) * 128] rows of `hidden` values, stride weight_stride
  int64_t weight_stride;  // elements
  int32_t hidden;         // multiple of 64
  int32_t num_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  void* q_out;            // [num_tokens][Hq][128]
  void* qkv_out;          // [num_tokens][(Hq + 2 Hkv) * 128] or null
  void* k_cache;
  void* v_cache;
  const int32_t* slots;
  int32_t log2_page;
  int32_t num_pages;
  const void* q_w;
  const void* k_w;
  float eps;
  const int32_t* positions;
  const float* cos_sin;
  int32_t max_position;
  int32_t num_splits;     // 1: one pass; > 1: split over hidden, partial sums in `partials`
  float* partials;        // [num_splits][num_tokens][(Hq + 2 Hkv) * 128] fp32 (num_splits > 1)
};

hipError_t launch_qkv_proj(const QkvProjArgs& a, hipStream_t s);

// ---- decode ----------------------------------------------------------------
struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int32_t bt_stride;
  const int32_t* context_lens;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t log2_page;
  int32_t num_pages;
  int32_t max_context_len;  // contexts are clamped to it (block-table reads stay in the row)
  float scale;
  int32_t keys_per_split;  // resolved (> 0)
  int32_t num_splits;      // resolved (>= 1)
  float* ws_o;             // [batch][Hq][num_splits][128]   (num_splits > 1)
  float* ws_m;             // [batch][Hq][num_splits]
  float* ws_l;             // [batch][Hq][num_splits]
  int32_t* order;          // [batch] requests by decreasing context length, or null
                           // (then request r is grid row r)
  bool rank_inline;        // the bf16 decode workgroups derive the longest-first
                           // order themselves (set by the launcher, batch <= 256)
  bool bf16;
  // Append (bf16 matrix-core kernel only; null = plain decode): request r's
  // new token at position context_lens[r] - 1 has K/V rows k_new/v_new
  // [r][Hkv][128] (token strides in elements).  The split that holds that
  // key takes the rows from these inputs instead of the pool and stores them
  // at new_slots[r].
  const void* k_new;
  const void* v_new;
  int64_t k_new_stride;
  int64_t v_new_stride;
  const int32_t* new_slots;
  // fp32 prefill on the fp32 decode kernel (null = decode): grid row z is new
  // token z of the packed batch (q and out rows z), its request r is found in
  // cu_seqlens [prefill_requests + 1], and it attends to keys 0 .. its
  // position context_lens[r] - n_r + (z - cu_seqlens[r]) through r's block
  // table row.
  const int32_t* cu_seqlens;
  int32_t prefill_requests;
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
// the request-order pass alone (when a.order is set), for launches that read it
hipError_t launch_decode_order(const DecodeArgs& a, hipStream_t s);
// the split merge alone (num_splits > 1), for launches that ran the splits
hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t s);

// ---- prefill ---------------------------------------------------------------
struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int32_t bt_stride;
  const int32_t* cu_seqlens;
  const int32_t* context_lens;
  int32_t batch;
  int32_t total_q;
  int32_t max_seqlen_q;
  int32_t max_context_len;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t log2_page;
  int32_t num_pages;
  float scale;
  // Append (bf16 whole query tiles only; null = plain prefill): the new
  // tokens' K/V rows k_new/v_new [total_q][Hkv][128] (token strides in
  // elements).  Keys at a request's new positions are read from these rows
  // instead of the pool, and the workgroup that owns a query tile stores its
  // tokens' rows of its KV head at new_slots (-1 or out of range: skipped).
  const void* k_new;
  const void* v_new;
  int64_t k_new_stride;
  int64_t v_new_stride;
  const int32_t* new_slots;
};

// Split plan of a prefill call.  A query tile whose key range spans more
// than tiles_per_piece 64-key tiles is cut into pieces of near-equal length,
// each run by its own workgroup; a planning kernel orders all pieces longest
// first, and a merge kernel combines the pieces of each split tile.  The
// pointers lie in the caller's workspace.
struct PrefillSplit {
  int32_t tiles_per_piece;  // S >= 1 (<= kMaxPieceTiles)
  int32_t max_pieces;       // pieces of the longest possible tile, <= kMaxPieces
  int32_t n_qtiles;         // query tiles of the longest request
  int32_t max_entries;      // bound on query tiles with rows (split entries too)
  int32_t max_items;        // bound on pieces: max_entries * max_pieces
  int32_t* header;          // [0] pieces planned, [1] split tiles
  int32_t* items;           // [max_items][8]: r, tile, kt_begin, kt_end, piece, pieces, split slot, 0
  int32_t* splits;          // [max_entries][4]: r, tile, pieces, 0
  float* part_o;            // [max_entries][max_pieces][Hkv][256 rows][128] fp32, unnormalized
  float* part_ml;           // [max_entries][Hkv][256 rows][max_pieces][2]: integer reference
                            // max (log2 domain), weight sum
};

constexpr int kMaxPieceTiles = 1023;   // planner bins: piece lengths 1 .. 1023 tiles
constexpr int kMaxPieces = 32;         // pieces per query tile
constexpr int kMaxPlanEntries = 4096;  // batch * n_qtiles of a split call

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);
// whole query tiles with the append fields set (a.k_new non-null)
hipError_t launch_prefill_append(const PrefillArgs& a, hipStream_t s);
// plan, pieces and merge of a split call
hipError_t launch_prefill_split(const PrefillArgs& a, const PrefillSplit& sp, hipStream_t s);

// ---- single-launch mixed batch (bf16): prefill tiles and decode splits ----
// in one grid, then the decode merge when the decode part has several splits
hipError_t launch_mixed(const PrefillArgs& pa, const DecodeArgs& da, hipStream_t s);

}  // namespace qil

// ---- debug checks of device-resident metadata --------------------------------
namespace qil {

// First violation found by a check kernel (code 0 = none).
struct DebugReport {
  int32_t code;
  int32_t i, j, value;
};

enum DebugCode : int32_t {
  kBadSlot = 1,       // i = token, value = slot
  kDuplicateSlot = 2, // i < j tokens, value = slot
  kBadPosition = 3,   // i = token, value = position
  kBadContext = 4,    // i = request, value = context length
  kBadPage = 5,       // i = request, j = block-table column, value = page id
  kBadCuSeqlens = 6,  // i = index into cu_seqlens, value = entry
  kChunkTooLong = 7,  // i = request, j = new tokens, value = context length
  kChunkAboveMax = 8, // i = request, j = new tokens, value = max_seqlen_q
  kAppendSlot = 9,    // i = request, j = expected slot, value = slot_mapping entry
};

// Device address of this device's report (resolved once per device).
hipError_t debug_report_ptr(DebugReport** ptr);
hipError_t launch_debug_clear(DebugReport* rep, hipStream_t s);
hipError_t launch_check_slots(const int32_t* slots, int32_t n, int64_t num_slots,
                              DebugReport* rep, hipStream_t s);
hipError_t launch_check_positions(const int32_t* pos, int32_t n, int32_t max_position,
                                  DebugReport* rep, hipStream_t s);
hipError_t launch_check_tables(const int32_t* block_tables, int32_t bt_stride,
                               const int32_t* context_lens, int32_t batch, int32_t log2_page,
                               int32_t num_pages, int32_t max_context_len, DebugReport* rep,
                               hipStream_t s);
hipError_t launch_check_cu(const int32_t* cu, const int32_t* context_lens, int32_t batch,
                           int32_t total_q, int32_t max_seqlen_q, DebugReport* rep, hipStream_t s);
// slot_mapping[r] is the slot of position context_lens[r] - 1 (decode with append)
hipError_t launch_check_append(const int32_t* slots, const int32_t* block_tables, int32_t bt_stride,
                               const int32_t* context_lens, int32_t batch, int32_t log2_page,
                               int32_t num_pages, int32_t max_context_len, DebugReport* rep,
                               hipStream_t s);

}  // namespace qil
