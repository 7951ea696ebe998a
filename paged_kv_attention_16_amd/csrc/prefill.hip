// qil_paged_prefill's launch: one workgroup per (KV head, request, query
// tile); the kernel itself is in prefill_body.h.
#include "prefill_body.h"

namespace qil {
namespace {

template <int G>
hipError_t launch_g(const PrefillArgs& a, hipStream_t s) {
  constexpr int TQ = kRowsWG / G;
  const int n_qtiles = (a.max_seqlen_q + TQ - 1) / TQ;
  if (n_qtiles == 0 || a.batch == 0) return hipSuccess;
  dim3 grid(a.num_kv_heads, a.batch, n_qtiles);
  hipLaunchKernelGGL((prefill_kernel<G>), grid, dim3(kThreads), 0, s, a, n_qtiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_g<1>(a, s);
    case 2: return launch_g<2>(a, s);
    case 4: return launch_g<4>(a, s);
    case 5: return launch_g<5>(a, s);
    case 8: return launch_g<8>(a, s);
    case 16: return launch_g<16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qil
