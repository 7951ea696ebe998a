// Debug-mode checks of the device-resident metadata that the kernels take as
// a precondition: slots, positions, block tables, context lengths and
// cu_seqlens.  Each kernel records the first violation it sees in a small
// report (one per device, in a __device__ variable of this library) with a
// compare-and-swap on its code; the host reads the report after the checks.
// The conditions restate the preconditions of include/qil.h, which follow the
// "nano-vLLM learning note" Context, prepare_prefill / prepare_decode and
// store_kvcache_kernel blocks (slot -1 = skip, block tables padded past a
// request's pages, cu_seqlens packing the new tokens).
#include <mutex>

#include "qil_internal.h"

namespace qil {
namespace {

__device__ DebugReport g_report;

__device__ void report(DebugReport* rep, int32_t code, int32_t i, int32_t j, int32_t value) {
  if (atomicCAS(&rep->code, 0, code) == 0) {
    rep->i = i;
    rep->j = j;
    rep->value = value;
  }
}

__global__ void clear_kernel(DebugReport* rep) {
  if (threadIdx.x == 0) {
    rep->code = 0;
    rep->i = rep->j = rep->value = 0;
  }
}

// Range of every slot, and duplicates among the non-negative slots (each
// thread compares its token with all later ones).
__global__ void slots_kernel(const int32_t* slots, int32_t n, int64_t num_slots, DebugReport* rep) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  const int32_t s = slots[t];
  if (s < -1 || (int64_t)s >= num_slots) {
    report(rep, kBadSlot, t, 0, s);
    return;
  }
  if (s < 0) return;
  for (int u = t + 1; u < n; ++u)
    if (slots[u] == s) {
      report(rep, kDuplicateSlot, t, u, s);
      return;
    }
}

__global__ void positions_kernel(const int32_t* pos, int32_t n, int32_t max_position,
                                 DebugReport* rep) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  const int32_t p = pos[t];
  if (p < 0 || p >= max_position) report(rep, kBadPosition, t, 0, p);
}

// One workgroup per request: its context length, then every block-table
// entry the kernels read for it.
__global__ void tables_kernel(const int32_t* bt, int32_t stride, const int32_t* ctx,
                              int32_t log2_page, int32_t num_pages, int32_t max_context_len,
                              DebugReport* rep) {
  const int r = blockIdx.x;
  const int32_t L = ctx[r];
  const int64_t cap = min((int64_t)max_context_len, (int64_t)stride << log2_page);
  if (L < 1 || (int64_t)L > cap) {
    if (threadIdx.x == 0) report(rep, kBadContext, r, 0, L);
    return;
  }
  const int npages = (L + (1 << log2_page) - 1) >> log2_page;
  for (int j = threadIdx.x; j < npages; j += blockDim.x) {
    const int32_t page = bt[(int64_t)r * stride + j];
    if (page < 0 || page >= num_pages) report(rep, kBadPage, r, j, page);
  }
}

// Decode with append: request r's new token goes to the slot of its last
// position, or nowhere (-1).  tables_kernel runs first on the same stream
// but does not stop this kernel, so a context length outside
// [1, min(max_context_len, stride * page_size)] (already reported there) is
// skipped here before any block-table read, and so is a table entry that is
// not a page of the pool (also reported there).
__global__ void append_kernel(const int32_t* slots, const int32_t* bt, int32_t stride,
                              const int32_t* ctx, int32_t batch, int32_t log2_page,
                              int32_t num_pages, int32_t max_context_len, DebugReport* rep) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= batch) return;
  const int32_t L = ctx[r];
  const int64_t cap = min((int64_t)max_context_len, (int64_t)stride << log2_page);
  if (L < 1 || (int64_t)L > cap || slots[r] == -1) return;  // -1: no pool write for this request
  const int32_t pos = L - 1;
  const int32_t page = bt[(int64_t)r * stride + (pos >> log2_page)];
  if (page < 0 || page >= num_pages) return;
  const int32_t want = (page << log2_page) + (pos & ((1 << log2_page) - 1));
  if (slots[r] != want) report(rep, kAppendSlot, r, want, slots[r]);
}

// cu_seqlens: starts at 0, non-decreasing, ends at total_q; each request's
// new tokens fit its context and max_seqlen_q.
__global__ void cu_kernel(const int32_t* cu, const int32_t* ctx, int32_t batch, int32_t total_q,
                          int32_t max_seqlen_q, DebugReport* rep) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r > batch) return;
  if (r == 0) {
    if (cu[0] != 0) report(rep, kBadCuSeqlens, 0, 0, cu[0]);
    return;
  }
  const int32_t a = cu[r - 1], b = cu[r];
  if (b < a || (r == batch && b != total_q) || b > total_q) {
    report(rep, kBadCuSeqlens, r, 0, b);
    return;
  }
  const int32_t n = b - a;
  if (n > ctx[r - 1]) report(rep, kChunkTooLong, r - 1, n, ctx[r - 1]);
  else if (n > max_seqlen_q) report(rep, kChunkAboveMax, r - 1, n, max_seqlen_q);
}

std::mutex g_ptr_mu;
DebugReport* g_ptr[64] = {};

}  // namespace

hipError_t debug_report_ptr(DebugReport** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_ptr_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_report));
    if (e != hipSuccess) return e;
    g_ptr[dev] = static_cast<DebugReport*>(p);
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

hipError_t launch_debug_clear(DebugReport* rep, hipStream_t s) {
  hipLaunchKernelGGL(clear_kernel, dim3(1), dim3(64), 0, s, rep);
  return hipGetLastError();
}

hipError_t launch_check_slots(const int32_t* slots, int32_t n, int64_t num_slots,
                              DebugReport* rep, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(slots_kernel, dim3((n + 255) / 256), dim3(256), 0, s, slots, n, num_slots, rep);
  return hipGetLastError();
}

hipError_t launch_check_positions(const int32_t* pos, int32_t n, int32_t max_position,
                                  DebugReport* rep, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(positions_kernel, dim3((n + 255) / 256), dim3(256), 0, s, pos, n,
                     max_position, rep);
  return hipGetLastError();
}

hipError_t launch_check_tables(const int32_t* block_tables, int32_t bt_stride,
                               const int32_t* context_lens, int32_t batch, int32_t log2_page,
                               int32_t num_pages, int32_t max_context_len, DebugReport* rep,
                               hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(tables_kernel, dim3(batch), dim3(256), 0, s, block_tables, bt_stride,
                     context_lens, log2_page, num_pages, max_context_len, rep);
  return hipGetLastError();
}

hipError_t launch_check_append(const int32_t* slots, const int32_t* block_tables, int32_t bt_stride,
                               const int32_t* context_lens, int32_t batch, int32_t log2_page,
                               int32_t num_pages, int32_t max_context_len, DebugReport* rep,
                               hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3((batch + 255) / 256), dim3(256), 0, s, slots,
                     block_tables, bt_stride, context_lens, batch, log2_page, num_pages,
                     max_context_len, rep);
  return hipGetLastError();
}

hipError_t launch_check_cu(const int32_t* cu, const int32_t* context_lens, int32_t batch,
                           int32_t total_q, int32_t max_seqlen_q, DebugReport* rep, hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(cu_kernel, dim3((batch + 1 + 255) / 256), dim3(256), 0, s, cu, context_lens,
                     batch, total_q, max_seqlen_q, rep);
  return hipGetLastError();
}

}  // namespace qil
