// libqil C ABI: argument validation, split planning and launches.
//
// Every check runs before the first HIP call, so a caller on a host without a
// GPU still gets the documented error codes.  The operations and their
// argument lists follow the "nano-vLLM learning note" Context block
// (cu_seqlens, max_seqlen, slot_mapping, context_lens, block_tables) and
// store_kvcache_kernel block (key/value rows with a token stride, the two
// cache pools and the slot mapping).
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#include "qil.h"
#include "qil_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return QIL_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---- debug mode: check the device-resident metadata before each launch ----
std::atomic<int> g_debug{-1};  // -1: not yet read from QIL_DEBUG

bool debug_on() {
  int d = g_debug.load(std::memory_order_relaxed);
  if (d < 0) {
    const char* env = getenv("QIL_DEBUG");
    d = (env && env[0] && !(env[0] == '0' && env[1] == '\0')) ? 1 : 0;
    int expected = -1;
    g_debug.compare_exchange_strong(expected, d);
    d = g_debug.load();
  }
  return d > 0;
}

int describe(const qil::DebugReport& r) {
  switch (r.code) {
    case qil::kBadSlot:
      return fail(QIL_EINVAL, "QIL_DEBUG: slot_mapping[%d] = %d is neither -1 nor a slot of the pool",
                  r.i, r.value);
    case qil::kDuplicateSlot:
      return fail(QIL_EINVAL, "QIL_DEBUG: slot_mapping[%d] and slot_mapping[%d] are both %d", r.i,
                  r.j, r.value);
    case qil::kBadPosition:
      return fail(QIL_EINVAL, "QIL_DEBUG: positions[%d] = %d is outside [0, max_position)", r.i,
                  r.value);
    case qil::kBadContext:
      return fail(QIL_EINVAL,
                  "QIL_DEBUG: context_lens[%d] = %d is outside [1, min(max_context_len, "
                  "block_table_stride*page_size)]",
                  r.i, r.value);
    case qil::kBadPage:
      return fail(QIL_EINVAL, "QIL_DEBUG: block_tables[%d][%d] = %d is not a page of the pool", r.i,
                  r.j, r.value);
    case qil::kBadCuSeqlens:
      return fail(QIL_EINVAL,
                  "QIL_DEBUG: cu_seqlens_q[%d] = %d breaks 0 = cu[0] <= ... <= cu[batch] = total_q",
                  r.i, r.value);
    case qil::kChunkTooLong:
      return fail(QIL_EINVAL, "QIL_DEBUG: request %d has %d new tokens but context_len %d", r.i,
                  r.j, r.value);
    case qil::kAppendSlot:
      return fail(QIL_EINVAL,
                  "QIL_DEBUG: slot_mapping[%d] = %d is not the slot %d of the request's last "
                  "position",
                  r.i, r.value, r.j);
    case qil::kChunkAboveMax:
      return fail(QIL_EINVAL, "QIL_DEBUG: request %d has %d new tokens, above max_seqlen_q %d",
                  r.i, r.j, r.value);
    default:
      return fail(QIL_EINVAL, "QIL_DEBUG: metadata check failed (code %d)", r.code);
  }
}

// Run the check kernels `enqueue` adds, wait for them, and turn the first
// violation into QIL_EINVAL.  This synchronizes `s`, so it refuses to run
// while the stream is being captured into a graph.
template <class F>
int run_checks(hipStream_t s, F enqueue) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(s, &cap);
  if (e != hipSuccess) return fail(QIL_EHIP, "QIL_DEBUG: %s", hipGetErrorString(e));
  if (cap != hipStreamCaptureStatusNone)
    return fail(QIL_EINVAL, "QIL_DEBUG checks synchronize the stream; they cannot run under capture");
  qil::DebugReport* rep = nullptr;
  e = qil::debug_report_ptr(&rep);
  if (e == hipSuccess) e = qil::launch_debug_clear(rep, s);
  if (e == hipSuccess) e = enqueue(rep);
  qil::DebugReport host{};
  if (e == hipSuccess) e = hipMemcpyAsync(&host, rep, sizeof(host), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(QIL_EHIP, "QIL_DEBUG: %s", hipGetErrorString(e));
  return host.code ? describe(host) : QIL_OK;
}

int log2_page_size(int32_t page_size) {
  switch (page_size) {
    case 16: return 4;
    case 32: return 5;
    case 64: return 6;
    case 128: return 7;
    case 256: return 8;
    default: return -1;
  }
}

bool supported_group(int32_t hq, int32_t hkv) {
  if (hkv <= 0 || hq <= 0 || hq % hkv != 0) return false;
  const int g = hq / hkv;
  // 1 (MHA), 2 (Qwen3-0.6B / 1.7B), 4 (4B, 8B, 30B-A3B), 5 (14B), 8 (32B), 16 (235B-A22B)
  return g == 1 || g == 2 || g == 4 || g == 5 || g == 8 || g == 16;
}

int check_common(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                 int32_t num_pages) {
  if (num_kv_heads <= 0 || num_q_heads <= 0)
    return fail(QIL_EINVAL, "head counts must be positive (q %d, kv %d)", num_q_heads, num_kv_heads);
  if (num_q_heads % num_kv_heads != 0)
    return fail(QIL_EINVAL, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                num_kv_heads);
  if (!supported_group(num_q_heads, num_kv_heads))
    return fail(QIL_EUNSUPPORTED, "GQA group size %d not built (1, 2, 4, 5, 8, 16)",
                num_q_heads / num_kv_heads);
  if (head_dim != qil::kHeadDim)
    return fail(QIL_EUNSUPPORTED, "head_dim %d not built (128)", head_dim);
  if (log2_page_size(page_size) < 0)
    return fail(QIL_EUNSUPPORTED, "page_size %d not built (16, 32, 64, 128, 256)", page_size);
  if (num_pages <= 0) return fail(QIL_EINVAL, "num_pages must be positive (%d)", num_pages);
  return QIL_OK;
}

// Split plan of the decode call, a pure function of host integers.
struct SplitPlan {
  int32_t keys_per_split;
  int32_t num_splits;
};

constexpr int32_t kMaxSplits = 65535;
constexpr int32_t kMaxKeysPerSplit = 4096;  // 64 steps of 64 keys: one page id per lane

SplitPlan plan_splits(int32_t batch, int32_t num_kv_heads, int32_t max_context_len,
                      int32_t keys_per_split) {
  SplitPlan p;
  int32_t S = keys_per_split;
  if (S <= 0) {
    // Long streams per workgroup read HBM fastest and a single split skips
    // the merge pass, so split only as far as needed for ~128 non-empty
    // workgroups (contexts assumed to average half the maximum), with
    // 256 .. 4096 keys per split.  Measured on the bf16 kernel: 4096-key
    // splits at B = 64, contexts up to 8192, beat the 2048-key plan of a
    // 1024-workgroup target by 6 %, and one split per request at B = 32,
    // contexts up to 2048, beats eight by 27 %.
    const int64_t pairs = (int64_t)batch * num_kv_heads;
    int64_t s = (pairs * (int64_t)max_context_len) / (2 * 128);
    s = (s + 63) / 64 * 64;
    if (s < 256) s = 256;
    if (s >= kMaxKeysPerSplit) {
      // Long contexts over few (request, head) pairs: aim at four times as
      // many workgroups, but keep splits of at least 2048 keys (shorter ones
      // lose to their merge and start-up).  8 requests of 16k-32k keys:
      // 2048-key splits take 141.6 us, 4096-key splits 154.4 us.
      s = (pairs * (int64_t)max_context_len) / (2 * 512);
      s = (s + 63) / 64 * 64;
      if (s < 2048) s = 2048;
      if (s > kMaxKeysPerSplit) s = kMaxKeysPerSplit;
      // With 256 to 512 pairs, equal splits of about 2,800 keys measured best
      // (the longest split sets the pace; shorter ones add merge work):
      // contexts up to 8,192 over 256 / 512 pairs: 121 -> 102 us / 208 -> 191 us
      // against the plan above; up to 16,384 over 512 pairs: 478 -> 432 us;
      // 1,024 pairs of up to 4,096 keys keep one split (188 us; 232 us split).
      if (pairs >= 256 && pairs <= 512) {
        const int64_t n = ((int64_t)max_context_len + 2815) / 2816;
        s = ((max_context_len + n - 1) / n + 63) / 64 * 64;
      }
    }
    S = (int32_t)s;
  }
  const int64_t n = ((int64_t)max_context_len + S - 1) / S;
  p.keys_per_split = S;
  p.num_splits = (int32_t)(n < 1 ? 1 : n);
  return p;
}

// Decode grids of at least this many workgroups (two rounds of 256 CUs at
// two workgroups per CU, and more) run their requests longest first, through
// an order array in the workspace.  Measured at B = 256 (2,048 workgroups):
// 171 -> 158 us with the batch sorted by decreasing context length.
constexpr int64_t kOrderMinBlocks = 512;

bool decode_ordered(int32_t batch, int32_t num_kv_heads, const SplitPlan& p) {
  return (int64_t)batch * num_kv_heads * p.num_splits >= kOrderMinBlocks;
}

size_t split_bytes_for(int32_t batch, int32_t num_q_heads, const SplitPlan& p) {
  if (p.num_splits <= 1) return 0;
  const size_t parts = (size_t)batch * num_q_heads * p.num_splits;
  // o[128] then m, l per part; each array rounded up to 256 bytes.
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  return up(parts * qil::kHeadDim * 4) + 2 * up(parts * 4);
}

// Workspace: the split partials (when there are several splits), then the
// request order (when the grid is large enough to run longest first).
size_t workspace_bytes_for(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                           const SplitPlan& p) {
  const size_t order = decode_ordered(batch, num_kv_heads, p) ? ((size_t)batch * 4 + 255) / 256 * 256 : 0;
  return split_bytes_for(batch, num_q_heads, p) + order;
}

hipError_t check_decode_metadata(const qil::DecodeArgs& a, qil::DebugReport* rep, hipStream_t s) {
  return qil::launch_check_tables(a.block_tables, a.bt_stride, a.context_lens, a.batch, a.log2_page,
                                  a.num_pages, a.max_context_len, rep, s);
}

hipError_t check_prefill_metadata(const qil::PrefillArgs& a, qil::DebugReport* rep, hipStream_t s) {
  hipError_t e = qil::launch_check_cu(a.cu_seqlens, a.context_lens, a.batch, a.total_q,
                                      a.max_seqlen_q, rep, s);
  if (e == hipSuccess)
    e = qil::launch_check_tables(a.block_tables, a.bt_stride, a.context_lens, a.batch, a.log2_page,
                                 a.num_pages, a.max_context_len, rep, s);
  return e;
}

// ---- fixed scratch of qil_paged_decode_no_alloc ----------------------------
// The decode workspace (split partials and the request order) for callers
// that cannot allocate: one array per GPU, held until the process ends.  In
// host code `scratch` names a host-side stand-in; kernels get the device
// address resolved once per device by hipGetSymbolAddress.  Every call on one
// GPU shares the array, and nothing in it has to start at zero (the decode
// kernels write every entry they later read), so calls that overlap on one
// GPU race.
constexpr size_t kScratchBytes = (size_t)32 << 20;
__device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

hipError_t device_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// Validate a decode call and fill its launch arguments.  *empty is set when
// the call has nothing to do (batch == 0).
int prep_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, int32_t block_table_stride,
                const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t num_pages,
                int32_t max_context_len, float scale, int32_t dtype, int32_t keys_per_split,
                void* workspace, size_t workspace_bytes, qil::DecodeArgs& a, bool* empty) {
  *empty = false;
  if (batch < 0) return fail(QIL_EINVAL, "batch %d < 0", batch);
  if (dtype != QIL_F32 && dtype != QIL_BF16) return fail(QIL_EUNSUPPORTED, "dtype %d", dtype);
  int rc = check_common(num_q_heads, num_kv_heads, head_dim, page_size, num_pages);
  if (rc) return rc;
  if (keys_per_split < 0 || keys_per_split % 64 || keys_per_split > kMaxKeysPerSplit)
    return fail(QIL_EINVAL, "keys_per_split %d must be 0 or a multiple of 64 up to %d",
                keys_per_split, kMaxKeysPerSplit);
  if (dtype == QIL_F32 && num_q_heads / num_kv_heads > 8)
    return fail(QIL_EUNSUPPORTED, "fp32 decode is built for GQA group sizes up to 8");
  if (batch == 0) {
    *empty = true;
    return ok();
  }
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(QIL_EINVAL, "null pointer argument");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(QIL_EINVAL, "out, q and the pools must be 16-byte aligned");
  if (block_table_stride <= 0) return fail(QIL_EINVAL, "block_table_stride must be positive");
  if (max_context_len <= 0) return fail(QIL_EINVAL, "max_context_len must be positive");
  if ((int64_t)max_context_len > (int64_t)block_table_stride * page_size)
    return fail(QIL_EINVAL, "max_context_len %d exceeds block_table_stride*page_size", max_context_len);
  if (!(scale == scale)) return fail(QIL_EINVAL, "scale is NaN");
  const SplitPlan p = plan_splits(batch, num_kv_heads, max_context_len, keys_per_split);
  if (p.num_splits > kMaxSplits)
    return fail(QIL_EINVAL, "max_context_len %d needs %d splits (at most %d)", max_context_len,
                p.num_splits, kMaxSplits);
  const size_t need = workspace_bytes_for(batch, num_q_heads, num_kv_heads, p);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(QIL_EWORKSPACE, "workspace of %zu bytes (16-byte aligned) needed, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (num_kv_heads > 65535 || batch > 65535)
    return fail(QIL_EINVAL, "batch and num_kv_heads are limited to 65535");

  a = qil::DecodeArgs{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.bt_stride = block_table_stride;
  a.context_lens = context_lens;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.log2_page = log2_page_size(page_size);
  a.num_pages = num_pages;
  a.max_context_len = max_context_len;
  a.scale = scale;
  a.keys_per_split = p.keys_per_split;
  a.num_splits = p.num_splits;
  a.bf16 = dtype == QIL_BF16;
  if (p.num_splits > 1) {
    const size_t parts = (size_t)batch * num_q_heads * p.num_splits;
    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    char* base = static_cast<char*>(workspace);
    a.ws_o = reinterpret_cast<float*>(base);
    a.ws_m = reinterpret_cast<float*>(base + up(parts * qil::kHeadDim * 4));
    a.ws_l = reinterpret_cast<float*>(base + up(parts * qil::kHeadDim * 4) + up(parts * 4));
  }
  if (decode_ordered(batch, num_kv_heads, p))
    a.order = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                         split_bytes_for(batch, num_q_heads, p));
  return QIL_OK;
}

// Split plan of a prefill call (host integers only), counted in query tiles
// of 256 rows (8 waves, one workgroup per CU at a time; an unsplit call over
// short contexts runs its whole tiles as 128-row workgroups, two per CU).
// When the grid holds at most 128 tiles with rows, one round of long tiles sets
// the time while half the CUs or more idle.  Such calls cut every query tile
// into n = 256 / tiles pieces (rounded down: all pieces still fit one round),
// that is at most S = ceil(kt_max / n) 64-key tiles each, and at least 16.
// Each piece loads its queries and writes a partial row block, and the split
// adds a planning and a merge launch, so shorter pieces or busier grids cost
// more than they balance (measured on one chunk over a long prefix, and on
// the 8B mixed step's 256 tiles, where whole tiles stay faster).
struct PrefillPlan {
  int32_t S = 0;            // 0: unsplit
  int32_t pieces = 1;       // pieces of the longest possible tile
  int32_t n_qtiles = 0;
  int32_t entries = 0;      // bound on query tiles with rows
  int64_t items = 0;        // bound on pieces
};

constexpr int32_t kMaxPrefillKeysPerSplit = 64 * 1023;
constexpr int32_t kAutoSplitTiles = 128;   // auto-split up to this many query tiles x KV heads
constexpr int32_t kMinPieceTiles = 16;

PrefillPlan plan_prefill(int32_t batch, int32_t total_q, int32_t max_seqlen_q,
                         int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t keys_per_split) {
  PrefillPlan p;
  if (batch <= 0 || total_q <= 0 || max_seqlen_q <= 0 || max_context_len <= 0 ||
      num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads)
    return p;
  const int32_t tq = 256 / (num_q_heads / num_kv_heads);
  if (tq <= 0) return p;
  const int64_t n_qtiles = (max_seqlen_q + tq - 1) / tq;
  const int64_t all = (int64_t)batch * n_qtiles;
  if (all > qil::kMaxPlanEntries) return p;
  const int64_t entries = std::min<int64_t>(all, (total_q + tq - 1) / tq + batch);
  const int64_t kt_max = (max_context_len + 63) / 64;
  int64_t S;
  if (keys_per_split > 0) {
    S = keys_per_split / 64;
  } else {
    const int64_t tiles = entries * num_kv_heads;
    if (tiles > kAutoSplitTiles || kt_max < 2 * kMinPieceTiles) return p;
    const int64_t n = 256 / tiles;  // >= 2
    S = std::max<int64_t>(kMinPieceTiles, (kt_max + n - 1) / n);
  }
  S = std::min<int64_t>(S, qil::kMaxPieceTiles);
  if ((kt_max + S - 1) / S > qil::kMaxPieces) S = (kt_max + qil::kMaxPieces - 1) / qil::kMaxPieces;
  const int64_t pieces = (kt_max + S - 1) / S;
  if (pieces <= 1 || entries * pieces * num_kv_heads > INT32_MAX) return p;
  p.S = (int32_t)S;
  p.pieces = (int32_t)pieces;
  p.n_qtiles = (int32_t)n_qtiles;
  p.entries = (int32_t)entries;
  p.items = entries * pieces;
  return p;
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace of a split prefill: header, piece list, split list, then the
// partial rows (fp32 sums) and their (max, sum) pairs.
size_t prefill_workspace_bytes(const PrefillPlan& p, int32_t num_kv_heads) {
  if (p.S == 0) return 0;
  const size_t slabs = (size_t)p.entries * p.pieces * num_kv_heads;
  return 256 + round256((size_t)p.items * 32) + round256((size_t)p.entries * 16) +
         round256(slabs * 256 * 128 * 4) + slabs * 256 * 2 * 4;
}

qil::PrefillSplit prefill_split_args(const PrefillPlan& p, int32_t num_kv_heads, void* ws) {
  char* b = static_cast<char*>(ws);
  const size_t slabs = (size_t)p.entries * p.pieces * num_kv_heads;
  qil::PrefillSplit sp;
  sp.tiles_per_piece = p.S;
  sp.max_pieces = p.pieces;
  sp.n_qtiles = p.n_qtiles;
  sp.max_entries = p.entries;
  sp.max_items = (int32_t)p.items;
  sp.header = reinterpret_cast<int32_t*>(b);
  b += 256;
  sp.items = reinterpret_cast<int32_t*>(b);
  b += round256((size_t)p.items * 32);
  sp.splits = reinterpret_cast<int32_t*>(b);
  b += round256((size_t)p.entries * 16);
  sp.part_o = reinterpret_cast<float*>(b);
  b += round256(slabs * 256 * 128 * 4);
  sp.part_ml = reinterpret_cast<float*>(b);
  return sp;
}

// Validate a prefill call and fill its launch arguments.  *empty is set when
// the call has nothing to do.
int prep_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, int32_t block_table_stride,
                 const int32_t* cu_seqlens_q, const int32_t* context_lens, int32_t batch,
                 int32_t total_q, int32_t max_seqlen_q, int32_t max_context_len,
                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                 int32_t num_pages, float scale, int32_t dtype, qil::PrefillArgs& a, bool* empty) {
  *empty = false;
  if (batch < 0 || total_q < 0 || max_seqlen_q < 0)
    return fail(QIL_EINVAL, "negative batch / total_q / max_seqlen_q");
  if (dtype != QIL_BF16 && dtype != QIL_F32) return fail(QIL_EUNSUPPORTED, "dtype %d", dtype);
  int rc = check_common(num_q_heads, num_kv_heads, head_dim, page_size, num_pages);
  if (rc) return rc;
  if (dtype == QIL_F32) {
    // the fp32 path runs one query token per workgroup row on the fp32
    // decode kernel, one split per token
    if (num_q_heads / num_kv_heads > 8)
      return fail(QIL_EUNSUPPORTED, "fp32 prefill is built for GQA group sizes up to 8");
    if (max_context_len > kMaxKeysPerSplit)
      return fail(QIL_EUNSUPPORTED, "fp32 prefill is built for contexts up to %d keys",
                  kMaxKeysPerSplit);
    if (total_q > 65535) return fail(QIL_EUNSUPPORTED, "fp32 prefill takes at most 65535 tokens");
  }
  if (batch == 0 || total_q == 0 || max_seqlen_q == 0) {
    *empty = true;
    return ok();
  }
  if (!out || !q || !k_cache || !v_cache || !block_tables || !cu_seqlens_q || !context_lens)
    return fail(QIL_EINVAL, "null pointer argument");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(QIL_EINVAL, "out, q and the pools must be 16-byte aligned");
  if (block_table_stride <= 0) return fail(QIL_EINVAL, "block_table_stride must be positive");
  if (max_seqlen_q > total_q) return fail(QIL_EINVAL, "max_seqlen_q exceeds total_q");
  if (max_context_len < max_seqlen_q)
    return fail(QIL_EINVAL, "max_context_len %d below max_seqlen_q %d", max_context_len,
                max_seqlen_q);
  if ((int64_t)max_context_len > (int64_t)block_table_stride * page_size)
    return fail(QIL_EINVAL, "max_context_len %d exceeds block_table_stride*page_size", max_context_len);
  if (!(scale == scale)) return fail(QIL_EINVAL, "scale is NaN");
  if (num_kv_heads > 65535 || batch > 65535)
    return fail(QIL_EINVAL, "batch and num_kv_heads are limited to 65535");

  a = qil::PrefillArgs{out, q, k_cache, v_cache, block_tables, block_table_stride, cu_seqlens_q,
                       context_lens, batch, total_q, max_seqlen_q, max_context_len, num_q_heads,
                       num_kv_heads, log2_page_size(page_size), num_pages, scale};
  return QIL_OK;
}

}  // namespace

extern "C" {

const char* qil_version(void) { return "qil 0.1.0 gfx950"; }

const char* qil_last_error(void) { return g_err; }

void qil_set_debug(int enabled) { g_debug.store(enabled ? 1 : 0); }

int qil_debug_enabled(void) { return debug_on() ? 1 : 0; }

int qil_kv_write(const void* k, const void* v, int64_t k_token_stride, int64_t v_token_stride,
                 void* k_cache, void* v_cache, const int32_t* slot_mapping, int32_t num_tokens,
                 int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t num_pages,
                 int32_t dtype, const qil_qknorm_rope* fuse, void* stream) {
  if (num_tokens < 0) return fail(QIL_EINVAL, "num_tokens %d < 0", num_tokens);
  if (dtype != QIL_F32 && dtype != QIL_BF16) return fail(QIL_EUNSUPPORTED, "dtype %d", dtype);
  const int32_t hq_check = fuse ? fuse->num_q_heads : num_kv_heads;
  int rc = check_common(hq_check, num_kv_heads, head_dim, page_size, num_pages);
  if (rc) return rc;
  if (num_tokens == 0) return ok();
  if (!k || !v || !k_cache || !v_cache || !slot_mapping)
    return fail(QIL_EINVAL, "null pointer argument");
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(QIL_EINVAL, "k, v and the pools must be 16-byte aligned");
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (k_token_stride < row || v_token_stride < row)
    return fail(QIL_EINVAL, "token stride (%lld, %lld) below num_kv_heads*head_dim %lld",
                (long long)k_token_stride, (long long)v_token_stride, (long long)row);
  if (k_token_stride % 8 || v_token_stride % 8)
    return fail(QIL_EINVAL, "token strides must be multiples of 8 elements");
  if ((int64_t)num_pages * page_size > INT32_MAX)
    return fail(QIL_EINVAL, "num_pages*page_size exceeds the int32 slot range");
  if ((int64_t)num_tokens * (hq_check + 2 * num_kv_heads) > (int64_t)1 << 30)
    return fail(QIL_EINVAL, "num_tokens*heads exceeds 2^30 head rows per call");

  qil::KvWriteArgs a{k, v, k_token_stride, v_token_stride, k_cache, v_cache, slot_mapping,
                     num_tokens, num_kv_heads, log2_page_size(page_size), num_pages,
                     dtype == QIL_BF16 ? 2 : 4};
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t num_slots = (int64_t)num_pages * page_size;
  if (!fuse) {
    if (debug_on()) {
      rc = run_checks(s, [&](qil::DebugReport* rep) {
        return qil::launch_check_slots(slot_mapping, num_tokens, num_slots, rep, s);
      });
      if (rc) return rc;
    }
    hipError_t e = qil::launch_kv_write(a, s);
    if (e != hipSuccess) return fail(QIL_EHIP, "kv_write launch: %s", hipGetErrorString(e));
    return ok();
  }
  if (dtype != QIL_BF16) return fail(QIL_EUNSUPPORTED, "fused norm/RoPE write is bf16 only");
  if (!fuse->q || !fuse->q_out || !fuse->q_norm_weight || !fuse->k_norm_weight ||
      !fuse->positions || !fuse->cos_sin)
    return fail(QIL_EINVAL, "null pointer in the fused parameters");
  if (!aligned16(fuse->q) || !aligned16(fuse->q_out) || !aligned16(fuse->q_norm_weight) ||
      !aligned16(fuse->k_norm_weight) || !aligned16(fuse->cos_sin))
    return fail(QIL_EINVAL, "fused tensors must be 16-byte aligned");
  const int64_t qrow = (int64_t)fuse->num_q_heads * head_dim;
  if (fuse->q_token_stride < qrow || fuse->q_token_stride % 8)
    return fail(QIL_EINVAL, "q_token_stride %lld invalid (>= %lld, multiple of 8)",
                (long long)fuse->q_token_stride, (long long)qrow);
  if (fuse->q_out == fuse->q && fuse->q_token_stride != qrow)
    return fail(QIL_EINVAL, "q_out may alias q only when q is contiguous");
  if (fuse->max_position <= 0) return fail(QIL_EINVAL, "max_position must be positive");
  if (!(fuse->eps >= 0.f)) return fail(QIL_EINVAL, "eps must be >= 0");
  qil::FusedArgs f{fuse->q, fuse->q_out, fuse->q_token_stride, fuse->num_q_heads,
                   fuse->q_norm_weight, fuse->k_norm_weight, fuse->eps, fuse->positions,
                   fuse->cos_sin, fuse->max_position};
  if (debug_on()) {
    rc = run_checks(s, [&](qil::DebugReport* rep) {
      hipError_t e = qil::launch_check_slots(slot_mapping, num_tokens, num_slots, rep, s);
      if (e == hipSuccess) e = qil::launch_check_positions(fuse->positions, num_tokens,
                                                            fuse->max_position, rep, s);
      return e;
    });
    if (rc) return rc;
  }
  hipError_t e = qil::launch_kv_write_fused(a, f, s);
  if (e != hipSuccess) return fail(QIL_EHIP, "fused kv_write launch: %s", hipGetErrorString(e));
  return ok();
}

namespace {
// Split plan of the QKV projection (host integers only).  A workgroup holds
// whole heads, so small batches give a grid of a few dozen workgroups, each
// streaming a large slice of the weight; such batches split the hidden
// dimension instead, into as many splits as fit one round of 256 workgroups
// (one per CU: a split workgroup takes 144 KB of LDS; one workgroup more
// would double the time), with at least four 64-column slices per split and
// at most 16 splits.
int32_t qkv_proj_splits(int32_t num_tokens, int32_t heads, int32_t hidden) {
  if (num_tokens <= 0 || num_tokens >= 1024) return 1;
  const int64_t blocks = (int64_t)(heads / 2) * ((num_tokens + 127) / 128);
  if (blocks >= 128) return 1;
  int64_t s = 256 / blocks;
  const int64_t smax = (int64_t)(hidden / 64) / 4;
  if (s > smax) s = smax;
  if (s > 16) s = 16;
  return s < 2 ? 1 : (int32_t)s;
}

size_t qkv_proj_workspace_bytes(int32_t num_tokens, int32_t heads, int32_t hidden) {
  const int32_t s = qkv_proj_splits(num_tokens, heads, hidden);
  return s > 1 ? (size_t)s * num_tokens * heads * qil::kHeadDim * 4 : 0;
}
}  // namespace

size_t qil_qkv_proj_workspace_size(int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t hidden) {
  if (num_tokens <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || hidden <= 0 || hidden % 64)
    return 0;
  return qkv_proj_workspace_bytes(num_tokens, num_q_heads + 2 * num_kv_heads, hidden);
}

int qil_qkv_proj_write(const void* x, int64_t x_token_stride, const void* weight,
                       int64_t weight_row_stride, int32_t hidden, void* q_out, void* qkv_out,
                       void* k_cache, void* v_cache, const int32_t* slot_mapping,
                       int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t page_size, int32_t num_pages,
                       const void* q_norm_weight, const void* k_norm_weight, float eps,
                       const int32_t* positions, const float* cos_sin, int32_t max_position,
                       void* workspace, size_t workspace_bytes, int32_t dtype, void* stream) {
  if (num_tokens < 0) return fail(QIL_EINVAL, "num_tokens %d < 0", num_tokens);
  if (dtype != QIL_BF16) return fail(QIL_EUNSUPPORTED, "the QKV projection is bf16 only");
  if (num_kv_heads <= 0 || num_q_heads <= 0)
    return fail(QIL_EINVAL, "head counts must be positive (q %d, kv %d)", num_q_heads, num_kv_heads);
  if ((num_q_heads + 2 * num_kv_heads) % 2)
    return fail(QIL_EUNSUPPORTED, "num_q_heads + 2*num_kv_heads = %d is odd",
                num_q_heads + 2 * num_kv_heads);
  if (head_dim != qil::kHeadDim) return fail(QIL_EUNSUPPORTED, "head_dim %d not built (128)", head_dim);
  if (log2_page_size(page_size) < 0)
    return fail(QIL_EUNSUPPORTED, "page_size %d not built (16, 32, 64, 128, 256)", page_size);
  if (num_pages <= 0) return fail(QIL_EINVAL, "num_pages must be positive (%d)", num_pages);
  if (hidden <= 0 || hidden % 64)
    return fail(QIL_EUNSUPPORTED, "hidden %d is not a positive multiple of 64", hidden);
  if (x_token_stride < hidden || weight_row_stride < hidden || x_token_stride % 8 ||
      weight_row_stride % 8)
    return fail(QIL_EINVAL, "strides (%lld, %lld) must be >= hidden %d and multiples of 8",
                (long long)x_token_stride, (long long)weight_row_stride, hidden);
  if (max_position <= 0) return fail(QIL_EINVAL, "max_position must be positive");
  if (!(eps >= 0.f)) return fail(QIL_EINVAL, "eps must be >= 0");
  if ((int64_t)num_pages * page_size > INT32_MAX)
    return fail(QIL_EINVAL, "num_pages*page_size exceeds the int32 slot range");
  if (num_tokens == 0) return ok();
  if (!x || !weight || !q_out || !k_cache || !v_cache || !slot_mapping || !q_norm_weight ||
      !k_norm_weight || !positions || !cos_sin)
    return fail(QIL_EINVAL, "null pointer argument");
  if (!aligned16(x) || !aligned16(weight) || !aligned16(q_out) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(q_norm_weight) || !aligned16(k_norm_weight) ||
      !aligned16(cos_sin) || (qkv_out && !aligned16(qkv_out)))
    return fail(QIL_EINVAL, "tensors must be 16-byte aligned");
  const int32_t heads = num_q_heads + 2 * num_kv_heads;
  if ((int64_t)num_tokens * heads > (int64_t)1 << 31)
    return fail(QIL_EINVAL, "num_tokens*heads exceeds 2^31 head rows per call");
  const size_t need = qkv_proj_workspace_bytes(num_tokens, heads, hidden);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(QIL_EWORKSPACE, "workspace of %zu bytes (16-byte aligned) needed, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);

  qil::QkvProjArgs a{x, x_token_stride, weight, weight_row_stride, hidden, num_tokens,
                     num_q_heads, num_kv_heads, q_out, qkv_out, k_cache, v_cache, slot_mapping,
                     log2_page_size(page_size), num_pages, q_norm_weight, k_norm_weight, eps,
                     positions, cos_sin, max_position,
                     qkv_proj_splits(num_tokens, heads, hidden),
                     need > 0 ? static_cast<float*>(workspace) : nullptr};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_on()) {
    const int64_t num_slots = (int64_t)num_pages * page_size;
    int rc = run_checks(s, [&](qil::DebugReport* rep) {
      hipError_t e = qil::launch_check_slots(slot_mapping, num_tokens, num_slots, rep, s);
      if (e == hipSuccess) e = qil::launch_check_positions(positions, num_tokens, max_position, rep, s);
      return e;
    });
    if (rc) return rc;
  }
  hipError_t e = qil::launch_qkv_proj(a, s);
  if (e != hipSuccess) return fail(QIL_EHIP, "qkv projection launch: %s", hipGetErrorString(e));
  return ok();
}

int qil_rope_cos_sin(float* cos_sin, int32_t max_position, int32_t head_dim, double theta,
                     void* stream) {
  if (!cos_sin) return fail(QIL_EINVAL, "null table");
  if (max_position <= 0) return fail(QIL_EINVAL, "max_position must be positive");
  if (head_dim != qil::kHeadDim) return fail(QIL_EUNSUPPORTED, "head_dim %d not built", head_dim);
  if (!(theta > 1.0)) return fail(QIL_EINVAL, "theta must exceed 1");
  hipError_t e = qil::launch_rope_table(cos_sin, max_position, head_dim, theta,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(QIL_EHIP, "rope table launch: %s", hipGetErrorString(e));
  return ok();
}

size_t qil_paged_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t max_context_len, int32_t page_size,
                                       int32_t keys_per_split) {
  (void)page_size;
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len <= 0) return 0;
  if (keys_per_split < 0 || keys_per_split % 64 || keys_per_split > kMaxKeysPerSplit) return 0;
  const SplitPlan p = plan_splits(batch, num_kv_heads, max_context_len, keys_per_split);
  if (p.num_splits > kMaxSplits) return 0;
  return workspace_bytes_for(batch, num_q_heads, num_kv_heads, p);
}

int qil_paged_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int32_t block_table_stride,
                     const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t num_pages,
                     int32_t max_context_len, float scale, int32_t dtype, int32_t keys_per_split,
                     void* workspace, size_t workspace_bytes, void* stream) {
  qil::DecodeArgs a;
  bool empty = false;
  int rc = prep_decode(out, q, k_cache, v_cache, block_tables, block_table_stride, context_lens,
                       batch, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                       max_context_len, scale, dtype, keys_per_split, workspace, workspace_bytes,
                       a, &empty);
  if (rc || empty) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_on()) {
    rc = run_checks(s, [&](qil::DebugReport* rep) { return check_decode_metadata(a, rep, s); });
    if (rc) return rc;
  }
  hipError_t e = qil::launch_decode(a, s);
  if (e != hipSuccess) return fail(QIL_EHIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

int qil_paged_decode_no_alloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, int32_t block_table_stride,
                              const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                              int32_t num_pages, int32_t max_context_len, float scale,
                              int32_t dtype, int32_t keys_per_split, void* stream) {
  // Every check first, on the host: the arguments (with a stand-in workspace
  // of the scratch array's size), then the scratch the call needs.
  qil::DecodeArgs a;
  bool empty = false;
  int rc = prep_decode(out, q, k_cache, v_cache, block_tables, block_table_stride, context_lens,
                       batch, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                       max_context_len, scale, dtype, keys_per_split,
                       reinterpret_cast<void*>(kScratchBytes), kScratchBytes, a, &empty);
  if (rc == QIL_EWORKSPACE) {
    const SplitPlan p = plan_splits(batch, num_kv_heads, max_context_len, keys_per_split);
    return fail(QIL_EWORKSPACE, "this decode needs %zu bytes of scratch; the library's fixed scratch "
                "array holds %zu", workspace_bytes_for(batch, num_q_heads, num_kv_heads, p),
                kScratchBytes);
  }
  if (rc || empty) return rc;
  void* scratch_ptr = nullptr;
  hipError_t e = device_scratch(&scratch_ptr);
  if (e != hipSuccess) return fail(QIL_EHIP, "scratch address: %s", hipGetErrorString(e));
  rc = prep_decode(out, q, k_cache, v_cache, block_tables, block_table_stride, context_lens, batch,
                   num_q_heads, num_kv_heads, head_dim, page_size, num_pages, max_context_len,
                   scale, dtype, keys_per_split, scratch_ptr, kScratchBytes, a, &empty);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_on()) {
    rc = run_checks(s, [&](qil::DebugReport* rep) { return check_decode_metadata(a, rep, s); });
    if (rc) return rc;
  }
  e = qil::launch_decode(a, s);
  if (e != hipSuccess) return fail(QIL_EHIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

int qil_paged_decode_append(void* out, const void* q, const void* k_new, const void* v_new,
                            int64_t k_token_stride, int64_t v_token_stride,
                            const int32_t* slot_mapping, void* k_cache, void* v_cache,
                            const int32_t* block_tables, int32_t block_table_stride,
                            const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                            int32_t num_pages, int32_t max_context_len, float scale, int32_t dtype,
                            int32_t keys_per_split, void* workspace, size_t workspace_bytes,
                            void* stream) {
  qil::DecodeArgs a;
  bool empty = false;
  int rc = prep_decode(out, q, k_cache, v_cache, block_tables, block_table_stride, context_lens,
                       batch, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                       max_context_len, scale, dtype, keys_per_split, workspace, workspace_bytes,
                       a, &empty);
  if (rc || empty) return rc;
  if (!k_new || !v_new || !slot_mapping) return fail(QIL_EINVAL, "null pointer argument");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(QIL_EINVAL, "k_new and v_new must be 16-byte aligned");
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (k_token_stride < row || v_token_stride < row || k_token_stride % 8 || v_token_stride % 8)
    return fail(QIL_EINVAL, "token strides (%lld, %lld) must be >= num_kv_heads*head_dim %lld and "
                "multiples of 8", (long long)k_token_stride, (long long)v_token_stride,
                (long long)row);
  if ((int64_t)num_pages * page_size > INT32_MAX)
    return fail(QIL_EINVAL, "num_pages*page_size exceeds the int32 slot range");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_on()) {
    const int64_t num_slots = (int64_t)num_pages * page_size;
    rc = run_checks(s, [&](qil::DebugReport* rep) {
      hipError_t e = check_decode_metadata(a, rep, s);
      if (e == hipSuccess) e = qil::launch_check_slots(slot_mapping, batch, num_slots, rep, s);
      if (e == hipSuccess)
        e = qil::launch_check_append(slot_mapping, block_tables, block_table_stride, context_lens,
                                     batch, a.log2_page, num_pages, max_context_len, rep, s);
      return e;
    });
    if (rc) return rc;
  }
  hipError_t e;
  if (a.bf16) {
    // one kernel: the split holding each request's last key takes the new
    // rows from k_new / v_new and stores them
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_new_stride = k_token_stride;
    a.v_new_stride = v_token_stride;
    a.new_slots = slot_mapping;
    e = qil::launch_decode(a, s);
  } else {
    // fp32: the plain write, then the decode
    qil::KvWriteArgs w{k_new, v_new, k_token_stride, v_token_stride, k_cache, v_cache,
                       slot_mapping, batch, num_kv_heads, a.log2_page, num_pages, 4};
    e = qil::launch_kv_write(w, s);
    if (e == hipSuccess) e = qil::launch_decode(a, s);
  }
  if (e != hipSuccess) return fail(QIL_EHIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

size_t qil_paged_prefill_workspace_size(int32_t batch, int32_t total_q, int32_t max_seqlen_q,
                                        int32_t max_context_len, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t keys_per_split) {
  if (keys_per_split < 0 || keys_per_split % 64 || keys_per_split > kMaxPrefillKeysPerSplit)
    return 0;
  return prefill_workspace_bytes(plan_prefill(batch, total_q, max_seqlen_q, max_context_len,
                                              num_q_heads, num_kv_heads, keys_per_split),
                                 num_kv_heads);
}

int qil_paged_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int32_t block_table_stride,
                      const int32_t* cu_seqlens_q, const int32_t* context_lens, int32_t batch,
                      int32_t total_q, int32_t max_seqlen_q, int32_t max_context_len,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t page_size, int32_t num_pages, float scale, int32_t dtype,
                      int32_t keys_per_split, void* workspace, size_t workspace_bytes,
                      void* stream) {
  qil::PrefillArgs a;
  bool empty = false;
  if (keys_per_split < 0 || keys_per_split % 64 || keys_per_split > kMaxPrefillKeysPerSplit)
    return fail(QIL_EINVAL, "keys_per_split %d must be 0 or a multiple of 64 up to %d",
                keys_per_split, kMaxPrefillKeysPerSplit);
  int rc = prep_prefill(out, q, k_cache, v_cache, block_tables, block_table_stride, cu_seqlens_q,
                        context_lens, batch, total_q, max_seqlen_q, max_context_len, num_q_heads,
                        num_kv_heads, head_dim, page_size, num_pages, scale, dtype, a, &empty);
  if (rc || empty) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == QIL_F32) {
    if (debug_on()) {
      rc = run_checks(s, [&](qil::DebugReport* rep) { return check_prefill_metadata(a, rep, s); });
      if (rc) return rc;
    }
    // each new token is a decode row over its own visible keys: no split,
    // no workspace
    qil::DecodeArgs d{};
    d.out = out;
    d.q = q;
    d.k_cache = k_cache;
    d.v_cache = v_cache;
    d.block_tables = block_tables;
    d.bt_stride = block_table_stride;
    d.context_lens = context_lens;
    d.batch = total_q;
    d.num_q_heads = num_q_heads;
    d.num_kv_heads = num_kv_heads;
    d.log2_page = a.log2_page;
    d.num_pages = num_pages;
    d.max_context_len = max_context_len;
    d.scale = scale;
    d.keys_per_split = (max_context_len + 63) / 64 * 64;
    d.num_splits = 1;
    d.bf16 = false;
    d.cu_seqlens = cu_seqlens_q;
    d.prefill_requests = batch;
    hipError_t e = qil::launch_decode(d, s);
    if (e != hipSuccess) return fail(QIL_EHIP, "prefill launch: %s", hipGetErrorString(e));
    return ok();
  }
  const PrefillPlan plan = plan_prefill(batch, total_q, max_seqlen_q, max_context_len,
                                        num_q_heads, num_kv_heads, keys_per_split);
  const size_t need = prefill_workspace_bytes(plan, num_kv_heads);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(QIL_EWORKSPACE, "workspace of %zu bytes (16-byte aligned) needed, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (debug_on()) {
    rc = run_checks(s, [&](qil::DebugReport* rep) { return check_prefill_metadata(a, rep, s); });
    if (rc) return rc;
  }
  hipError_t e = need > 0 ? qil::launch_prefill_split(a, prefill_split_args(plan, num_kv_heads, workspace), s)
                          : qil::launch_prefill(a, s);
  if (e != hipSuccess) return fail(QIL_EHIP, "prefill launch: %s", hipGetErrorString(e));
  return ok();
}

int qil_paged_prefill_append(void* out, const void* q, const void* k_new, const void* v_new,
                             int64_t k_token_stride, int64_t v_token_stride,
                             const int32_t* slot_mapping, void* k_cache, void* v_cache,
                             const int32_t* block_tables, int32_t block_table_stride,
                             const int32_t* cu_seqlens_q, const int32_t* context_lens,
                             int32_t batch, int32_t total_q, int32_t max_seqlen_q,
                             int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t page_size, int32_t num_pages, float scale,
                             int32_t dtype, int32_t keys_per_split, void* workspace,
                             size_t workspace_bytes, void* stream) {
  qil::PrefillArgs a;
  bool empty = false;
  if (keys_per_split < 0 || keys_per_split % 64 || keys_per_split > kMaxPrefillKeysPerSplit)
    return fail(QIL_EINVAL, "keys_per_split %d must be 0 or a multiple of 64 up to %d",
                keys_per_split, kMaxPrefillKeysPerSplit);
  int rc = prep_prefill(out, q, k_cache, v_cache, block_tables, block_table_stride, cu_seqlens_q,
                        context_lens, batch, total_q, max_seqlen_q, max_context_len, num_q_heads,
                        num_kv_heads, head_dim, page_size, num_pages, scale, dtype, a, &empty);
  if (rc || empty) return rc;
  if (!k_new || !v_new || !slot_mapping) return fail(QIL_EINVAL, "null pointer argument");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(QIL_EINVAL, "k_new and v_new must be 16-byte aligned");
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (k_token_stride < row || v_token_stride < row || k_token_stride % 8 || v_token_stride % 8)
    return fail(QIL_EINVAL, "token strides (%lld, %lld) must be >= num_kv_heads*head_dim %lld and "
                "multiples of 8", (long long)k_token_stride, (long long)v_token_stride,
                (long long)row);
  if ((int64_t)num_pages * page_size > INT32_MAX)
    return fail(QIL_EINVAL, "num_pages*page_size exceeds the int32 slot range");
  const PrefillPlan plan = plan_prefill(batch, total_q, max_seqlen_q, max_context_len,
                                        num_q_heads, num_kv_heads, keys_per_split);
  const size_t need = dtype == QIL_F32 ? 0 : prefill_workspace_bytes(plan, num_kv_heads);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(QIL_EWORKSPACE, "workspace of %zu bytes (16-byte aligned) needed, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_on()) {
    const int64_t num_slots = (int64_t)num_pages * page_size;
    rc = run_checks(s, [&](qil::DebugReport* rep) {
      hipError_t e = check_prefill_metadata(a, rep, s);
      if (e == hipSuccess) e = qil::launch_check_slots(slot_mapping, total_q, num_slots, rep, s);
      return e;
    });
    if (rc) return rc;
  }
  if (dtype == QIL_BF16 && need == 0) {
    // one kernel: keys at new positions come from k_new / v_new, and each
    // query tile's workgroup stores its tokens' rows
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_new_stride = k_token_stride;
    a.v_new_stride = v_token_stride;
    a.new_slots = slot_mapping;
    hipError_t e = qil::launch_prefill_append(a, s);
    if (e != hipSuccess) return fail(QIL_EHIP, "prefill launch: %s", hipGetErrorString(e));
    return ok();
  }
  // fp32, or a call split over keys: the plain write, then the prefill
  qil::KvWriteArgs w{k_new, v_new, k_token_stride, v_token_stride, k_cache, v_cache,
                     slot_mapping, total_q, num_kv_heads, a.log2_page, num_pages,
                     dtype == QIL_BF16 ? 2 : 4};
  hipError_t e = qil::launch_kv_write(w, s);
  if (e != hipSuccess) return fail(QIL_EHIP, "kv_write launch: %s", hipGetErrorString(e));
  return qil_paged_prefill(out, q, k_cache, v_cache, block_tables, block_table_stride,
                           cu_seqlens_q, context_lens, batch, total_q, max_seqlen_q,
                           max_context_len, num_q_heads, num_kv_heads, head_dim, page_size,
                           num_pages, scale, dtype, keys_per_split, workspace, workspace_bytes,
                           stream);
}

int qil_paged_attention_mixed(const qil_decode_batch* decode, const qil_prefill_batch* prefill,
                              const void* k_cache, const void* v_cache, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                              int32_t num_pages, float scale, int32_t dtype, void* stream) {
  if (dtype != QIL_BF16) return fail(QIL_EUNSUPPORTED, "the mixed launch is built for bf16 only");
  qil::DecodeArgs da{};
  qil::PrefillArgs pa{};
  bool dec_empty = true, pre_empty = true;
  int rc;
  if (decode) {
    rc = prep_decode(decode->out, decode->q, k_cache, v_cache, decode->block_tables,
                     decode->block_table_stride, decode->context_lens, decode->batch, num_q_heads,
                     num_kv_heads, head_dim, page_size, num_pages, decode->max_context_len, scale,
                     dtype, decode->keys_per_split, decode->workspace, decode->workspace_bytes, da,
                     &dec_empty);
    if (rc) return rc;
  }
  if (prefill) {
    rc = prep_prefill(prefill->out, prefill->q, k_cache, v_cache, prefill->block_tables,
                      prefill->block_table_stride, prefill->cu_seqlens_q, prefill->context_lens,
                      prefill->batch, prefill->total_q, prefill->max_seqlen_q,
                      prefill->max_context_len, num_q_heads, num_kv_heads, head_dim, page_size,
                      num_pages, scale, dtype, pa, &pre_empty);
    if (rc) return rc;
  }
  if (dec_empty && pre_empty) return ok();
  if (dec_empty) {
    da = qil::DecodeArgs{};
    da.num_kv_heads = num_kv_heads;
    da.num_q_heads = num_q_heads;
    da.num_splits = 1;
  }
  if (pre_empty) {
    pa = qil::PrefillArgs{};
    pa.num_kv_heads = num_kv_heads;
    pa.num_q_heads = num_q_heads;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_on()) {
    rc = run_checks(s, [&](qil::DebugReport* rep) {
      hipError_t e = dec_empty ? hipSuccess : check_decode_metadata(da, rep, s);
      if (e == hipSuccess && !pre_empty) e = check_prefill_metadata(pa, rep, s);
      return e;
    });
    if (rc) return rc;
  }
  hipError_t e = qil::launch_mixed(pa, da, s);
  if (e != hipSuccess) return fail(QIL_EHIP, "mixed launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
