// Single-launch mixed batch: one grid holds the query tiles of a varlen
// prefill and the splits of a paged decode over the same KV pool, so the
// MFMA-bound prefill tiles and the HBM-bound decode splits run side by side
// on different CUs instead of one kernel after the other, and the step pays
// one launch and one tail instead of two.
//
// The "qwen-engine" README keeps prefill and decode in separate batches
// (prefill compute-bound, decode memory-bound); this launch keeps them
// separate calls' worth of work but co-schedules them.  Each block runs
// either prefill_tile (prefill_body.h, 8 wavefronts) or decode_mfma_split
// (decode_body.h, here with 8 wavefronts per split).  Blocks are dealt in
// chunks of 8 of one kind, alternating while both kinds remain: workgroups
// go to the 8 XCDs round robin, so each prefill block keeps its KV head's
// XCD (KV head = block index mod 8 when num_kv_heads = 8), as in the
// prefill-only launch.  On large decode grids the decode blocks take their
// requests longest first, in the order qil_paged_decode uses (ranked by each
// block for batches up to 256, else written by the ordering kernel).
#include "decode_body.h"
#include "prefill_body.h"

namespace qil {
namespace {

constexpr int kMixedWaves = kThreads / 64;  // 8: the prefill workgroup shape
constexpr size_t kMixedLds =
    sizeof(PrefillLds) > kMixedWaves * sizeof(DecodeRing) ? sizeof(PrefillLds)
                                                          : kMixedWaves * sizeof(DecodeRing);

template <int G>
__global__ __launch_bounds__(kThreads) void mixed_kernel(PrefillArgs pa, int n_qtiles, int n_pre,
                                                         DecodeArgs da, int n_dec) {
  __shared__ __attribute__((aligned(1024))) char lds[kMixedLds];
  const int c = blockIdx.x >> 3, o = blockIdx.x & 7;
  const int pc = (n_pre + 7) >> 3, dc = (n_dec + 7) >> 3;  // chunks of 8 of each kind
  const int m = min(pc, dc);
  bool prefill;
  int idx;
  if (c < 2 * m) {
    prefill = (c & 1) == 0;
    idx = ((c >> 1) << 3) + o;
  } else {
    prefill = pc > dc;
    idx = ((c - m) << 3) + o;
  }
  if (idx >= (prefill ? n_pre : n_dec)) return;  // padding of a partial chunk (uniform)
  if (prefill) {
    // the prefill-only grid is (KV head, request, tile from the last), KV head fastest
    const int g = idx % pa.num_kv_heads;
    const int rest = idx / pa.num_kv_heads;
    prefill_tile<G>(pa, n_qtiles, g, rest % pa.batch, rest / pa.batch,
                    *reinterpret_cast<PrefillLds*>(lds));
  } else {
    // the decode-only grid is (split, KV head, request), split fastest;
    // requests longest first when the order pass ran
    const int split = idx % da.num_splits;
    const int rest = idx / da.num_splits;
    int r = rest / da.num_kv_heads;
    if (da.rank_inline)
      r = decode_rank_request<kMixedWaves>(da.context_lens, da.batch, da.max_context_len, r);
    else if (da.order != nullptr)
      r = da.order[r];
    decode_mfma_split<G, kMixedWaves>(da, split, rest % da.num_kv_heads, r,
                                      reinterpret_cast<DecodeRing*>(lds));
  }
}

template <int G>
hipError_t launch_g(const PrefillArgs& pa, const DecodeArgs& da, hipStream_t s) {
  constexpr int TQ = kRowsWG / G;
  const int n_qtiles = pa.batch > 0 ? (pa.max_seqlen_q + TQ - 1) / TQ : 0;
  const int64_t n_pre = (int64_t)pa.num_kv_heads * pa.batch * n_qtiles;
  const int64_t n_dec = da.batch > 0 ? (int64_t)da.num_splits * da.num_kv_heads * da.batch : 0;
  const int64_t blocks = 8 * ((n_pre + 7) / 8 + (n_dec + 7) / 8);
  if (blocks == 0) return hipSuccess;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  DecodeArgs di = da;
  if (n_dec > 0) {
    if (da.order != nullptr && da.batch <= kRankMaxBatch) {
      di.rank_inline = true;  // the decode blocks rank the batch themselves
    } else {
      hipError_t e = launch_decode_order(da, s);
      if (e != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL((mixed_kernel<G>), dim3((unsigned)blocks), dim3(kThreads), 0, s, pa, n_qtiles,
                     (int)n_pre, di, (int)n_dec);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || da.batch == 0 || da.num_splits == 1) return e;
  return launch_decode_merge(da, s);
}

}  // namespace

hipError_t launch_mixed(const PrefillArgs& pa, const DecodeArgs& da, hipStream_t s) {
  switch (pa.num_q_heads / pa.num_kv_heads) {
    case 1: return launch_g<1>(pa, da, s);
    case 2: return launch_g<2>(pa, da, s);
    case 4: return launch_g<4>(pa, da, s);
    case 5: return launch_g<5>(pa, da, s);
    case 8: return launch_g<8>(pa, da, s);
    case 16: return launch_g<16>(pa, da, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qil
