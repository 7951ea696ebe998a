// Single-launch mixed batch: one grid holds the query tiles of a varlen
// prefill and the splits of a paged decode over the same KV pool, so the
// MFMA-bound prefill tiles and the HBM-bound decode splits run side by side
// (two blocks per CU, so also on the same CU) instead of one kernel after
// the other, and the step pays one launch and one tail instead of two.
//
// The "qwen-engine" README keeps prefill and decode in separate batches
// (prefill compute-bound, decode memory-bound); this launch keeps them
// separate calls' worth of work but co-schedules them.  Each block runs
// either prefill_tile (prefill_body.h, a 128-row query tile of 4 wavefronts)
// or decode_mfma_split (decode_body.h, 4 wavefronts per split, as in
// qil_paged_decode), so both kinds give the same bits as the separate calls
// with the same tiles and splits.  Blocks are dealt in
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

// Blocks of 4 wavefronts with 66 KB of LDS: two per CU, so a memory-bound
// decode split and a matrix-bound prefill tile can share a CU.  Measured on
// the 8B step (12 layers, side by side): 299.8-300.0 us per layer against
// 325.9-326.2 us with blocks of 8 wavefronts (128 KB, one per CU), and
// against 311.5-311.6 us for the decode and prefill as separate launches.
constexpr int kMixedWaves = 4;

template <int W>
constexpr size_t mixed_lds() {
  return sizeof(PrefillLds) > W * sizeof(DecodeRing) ? sizeof(PrefillLds) : W * sizeof(DecodeRing);
}

template <int G, int W>
__global__ __launch_bounds__(64 * W, 2) void mixed_kernel(PrefillArgs pa, int n_qtiles, int n_pre,
                                                          DecodeArgs da, int n_dec) {
  __shared__ __attribute__((aligned(1024))) char lds[mixed_lds<W>()];
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
    prefill_tile<G, W>(pa, n_qtiles, g, rest % pa.batch, rest / pa.batch,
                       *reinterpret_cast<PrefillLds*>(lds));
  } else {
    // the decode-only grid is (split, KV head, request), split fastest;
    // requests longest first when the order pass ran
    const int split = idx % da.num_splits;
    const int rest = idx / da.num_splits;
    int r = rest / da.num_kv_heads;
    if (da.rank_inline)
      r = decode_rank_request<W>(da.context_lens, da.batch, da.max_context_len, r);
    else if (da.order != nullptr)
      r = da.order[r];
    decode_mfma_split<G, W>(da, split, rest % da.num_kv_heads, r,
                            reinterpret_cast<DecodeRing*>(lds));
  }
}

template <int G>
hipError_t launch_g(const PrefillArgs& pa, const DecodeArgs& da, hipStream_t s) {
  constexpr int W = kMixedWaves;
  constexpr int TQ = 32 * W / G;
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
  hipLaunchKernelGGL((mixed_kernel<G, W>), dim3((unsigned)blocks), dim3(64 * W), 0, s, pa, n_qtiles,
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
