// qil_paged_prefill's launches; the tile kernel itself is in prefill_body.h.
//
// Unsplit: one workgroup per (KV head, request, query tile).
//
// Split (long key ranges over few query tiles, e.g. a chunk of a long
// prompt): three kernels on the caller's stream.
//   1. prefill_plan_kernel (one workgroup) lists the pieces: a query tile of
//      n key tiles becomes ceil(n / S) pieces of near-equal length.  The list
//      (a counting sort) runs piece 0 of every split tile, then piece 1, ...,
//      so pieces over the same keys share L2, then the unsplit tiles longest
//      first.
//   2. prefill_piece_kernel<G> runs one piece per workgroup: whole tiles
//      write the output, pieces of split tiles write their unnormalized fp32
//      rows and (integer max, sum) to the workspace.
//   3. prefill_merge_kernel combines the pieces of each split tile by the
//      log-sum-exp rule: out = sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) l_p.
// The order of pieces within one place is arbitrary, but every piece and
// every merge computes the same values whatever the order, so results are
// deterministic.
#include <climits>

#include "prefill_body.h"

namespace qil {
namespace {

// Whole query tiles run as workgroups of 128 query rows (two per CU) when
// no context exceeds this many keys, and of 256 rows (one per CU) beyond.
// Few keys per tile leave the per-workgroup start-up and the uneven tail as
// the larger costs, and the second workgroup of a CU covers them; with many,
// each K/V tile serving 256 rows halves its fetches per row.  Measured side
// by side (bit-identical): 128 rows are 4-12 % faster up to 2,153-key
// contexts (the 8-request varlen workload, 16 x 1,000, 32 x 512,
// 2 x 2,048 tokens), and 256 rows 3-11 % faster from 3,000 keys (8 x 3,000
// tokens, 2,048-token chunks over 1,024 and 2,048 cached keys, the 8B
// step's chunks, one 4,096- or 8,192-token prompt).
constexpr int kNarrowMaxContext = 2560;

template <int G, int W, bool APPEND>
hipError_t launch_gw(const PrefillArgs& a, hipStream_t s) {
  constexpr int TQ = 32 * W / G;
  const int n_qtiles = (a.max_seqlen_q + TQ - 1) / TQ;
  if (n_qtiles == 0 || a.batch == 0) return hipSuccess;
  int zc = 0;  // copy slices: about two passes of 4 chunks per thread each
  if (APPEND && a.total_q > 0) {
    const int64_t chunks = (int64_t)a.total_q * a.num_kv_heads * 32;
    const int64_t blocks = (chunks + 8 * 64 * W - 1) / (8 * 64 * W);
    const int64_t slice = (int64_t)a.num_kv_heads * a.batch;
    zc = (int)std::min<int64_t>((blocks + slice - 1) / slice, 1024);
  }
  dim3 grid(a.num_kv_heads, a.batch, n_qtiles + zc);
  hipLaunchKernelGGL((prefill_kernel<G, W, APPEND>), grid, dim3(64 * W), 0, s, a, n_qtiles);
  return hipGetLastError();
}

template <int G, bool APPEND = false>
hipError_t launch_g(const PrefillArgs& a, hipStream_t s) {
  return a.max_context_len <= kNarrowMaxContext ? launch_gw<G, 4, APPEND>(a, s)
                                                : launch_gw<G, 8, APPEND>(a, s);
}

// Key tiles of query tile `tile` of request r (0 when the tile has no rows),
// with the same clamping as the tile kernel.
__device__ __forceinline__ int entry_key_tiles(const PrefillArgs& a, int r, int tile, int TQ) {
  const int q0 = a.cu_seqlens[r];
  const int n = min(a.cu_seqlens[r + 1], a.total_q) - max(q0, 0);
  const int t0 = tile * TQ;
  if (q0 < 0 || t0 >= n) return 0;
  const int L = min(a.context_lens[r], a.max_context_len);
  const int kmax = L - n + t0 + min(TQ, n - t0);
  return kmax > 0 ? (kmax + kBN - 1) / kBN : 0;
}

constexpr int kPlanThreads = 1024;
constexpr int kOrderBins = kPlanThreads;             // one scan bin per thread
constexpr int kUnsplitBins = kOrderBins - kMaxPieces;

// Place in the launch order: split tiles' pieces first, piece 0 of every
// split tile, then piece 1, ..., so the pieces that read the same key range
// of a request run side by side (each K/V tile is fetched from HBM once and
// served from L2 to the others); then the whole tiles, longest first.
__device__ __forceinline__ int order_bin(int p, int pcs, int len) {
  return pcs > 1 ? p : kMaxPieces + (kUnsplitBins - min(len, kUnsplitBins));
}

__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(PrefillArgs a, PrefillSplit sp,
                                                                     int TQ) {
  __shared__ int hist[kOrderBins];
  __shared__ int start[kOrderBins];
  __shared__ int cursor[kOrderBins];
  __shared__ int slot_of[kMaxPlanEntries];
  __shared__ int ntiles_of[kMaxPlanEntries];
  __shared__ int wave_sum[kPlanThreads / 64];
  __shared__ int nsplit, total;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int S = sp.tiles_per_piece;
  const int E = a.batch * sp.n_qtiles;
  hist[tid] = cursor[tid] = 0;
  if (tid == 0) nsplit = 0;
  __syncthreads();

  // Count the pieces per place; split tiles get a slot for their partials.
  for (int e = tid; e < E; e += kPlanThreads) {
    const int r = e / sp.n_qtiles, tile = e % sp.n_qtiles;
    const int nt = entry_key_tiles(a, r, tile, TQ);
    slot_of[e] = -1;
    ntiles_of[e] = nt;
    if (nt == 0) continue;
    int pcs = (nt + S - 1) / S;
    if (pcs > 1) {
      const int j = atomicAdd(&nsplit, 1);
      if (j < sp.max_entries) {
        slot_of[e] = j;
        *reinterpret_cast<int4*>(sp.splits + 4 * j) = make_int4(r, tile, pcs, 0);
      } else {
        pcs = 1;  // only with metadata outside its preconditions
      }
    }
    for (int p = 0; p < pcs; ++p) atomicAdd(&hist[order_bin(p, pcs, nt)], 1);
  }
  __syncthreads();

  // start[b] = pieces in the bins before b (exclusive scan).
  {
    static_assert(kOrderBins == kPlanThreads, "one scan bin per thread");
    int v = hist[tid];
    const int own = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(v, o);
      if (lane >= o) v += t;
    }
    if (lane == 63) wave_sum[wv] = v;
    __syncthreads();
    int before = 0;
    for (int i = 0; i < wv; ++i) before += wave_sum[i];
    start[tid] = before + v - own;
    if (tid == kPlanThreads - 1) total = before + v;  // every piece
  }
  __syncthreads();

  for (int e = tid; e < E; e += kPlanThreads) {
    const int r = e / sp.n_qtiles, tile = e % sp.n_qtiles;
    const int nt = ntiles_of[e];
    if (nt == 0) continue;
    const int j = slot_of[e];
    const int pcs = j >= 0 ? (nt + S - 1) / S : 1;
    const int base = nt / pcs, rem = nt % pcs;
    int kb = 0;
    for (int p = 0; p < pcs; ++p) {
      const int len = base + (p < rem ? 1 : 0);
      const int bin = order_bin(p, pcs, nt);
      const int pos = start[bin] + atomicAdd(&cursor[bin], 1);
      if (pos < sp.max_items) {
        int4* it = reinterpret_cast<int4*>(sp.items + 8 * pos);
        it[0] = make_int4(r, tile, kb, kb + len);
        it[1] = make_int4(p, pcs, j, 0);
      }
      kb += len;
    }
  }
  if (tid == 0) {
    sp.header[0] = min(total, sp.max_items);
    sp.header[1] = min(nsplit, sp.max_entries);
  }
}

// Workgroup i runs piece i / Hkv of the plan for KV head i % Hkv, so the
// KV heads of one piece land on different XCDs as in the unsplit grid.
template <int G>
__global__ __launch_bounds__(kThreads) void prefill_piece_kernel(PrefillArgs a, PrefillSplit sp) {
  __shared__ __attribute__((aligned(1024))) PrefillLds smem;
  const int g = blockIdx.x % a.num_kv_heads;
  const int idx = blockIdx.x / a.num_kv_heads;
  if (idx >= sp.header[0]) return;
  const int4 i0 = *reinterpret_cast<const int4*>(sp.items + 8 * idx);
  const int4 i1 = *reinterpret_cast<const int4*>(sp.items + 8 * idx + 4);
  const int r = wave_uniform(i0.x), tile = wave_uniform(i0.y);
  const int kb = wave_uniform(i0.z), ke = wave_uniform(i0.w);
  const int p = wave_uniform(i1.x), j = wave_uniform(i1.z);
  float* po = nullptr;
  float* pml = nullptr;
  if (j >= 0) {
    const int64_t slab = ((int64_t)j * sp.max_pieces + p) * a.num_kv_heads + g;
    po = sp.part_o + slab * kRowsWG * kHeadDim;
    pml = sp.part_ml + (((int64_t)j * a.num_kv_heads + g) * kRowsWG * sp.max_pieces + p) * 2;
  }
  prefill_range<G>(a, g, r, tile, kb, ke, po, pml, sp.max_pieces, smem);
}

// One workgroup per (KV head, split tile, 8-row block); each wavefront
// merges two rows, a 32-lane half per row.  Lane p of the half holds piece
// p's (m, l) (at most 32 pieces), and every lane sums 4 dims of the pieces'
// fp32 rows.  The loads of the first eight pieces are issued together with
// the (m, l) load, before the half reduces the maximum M and the weights
// 2^(m_p - M) with lane shuffles.  The references m_p are integers, so each
// weight is an exact power of two:
//     out = sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) l_p
// is the whole row's O / l up to the order of the fp32 additions.
constexpr int kMergeThreads = 256;
constexpr int kMergeRows = 8;

__device__ __forceinline__ float pow2_weight(float m, float M) {
  // m <= M; pieces that saw no visible key keep the -1e30 start value
  return ldexpf(1.0f, (int)fmaxf(m - M, -200.0f));
}

__global__ __launch_bounds__(kMergeThreads) void prefill_merge_kernel(PrefillArgs a, PrefillSplit sp,
                                                                      int G) {
  static_assert(kMaxPieces <= 32, "one lane of a half wavefront per piece");
  const int g = blockIdx.x;
  const int j = blockIdx.y;
  if (j >= sp.header[1]) return;
  const int4 e = *reinterpret_cast<const int4*>(sp.splits + 4 * j);
  const int r = e.x, tile = e.y, pcs = e.z;
  const int TQ = kRowsWG / G;
  const int q0 = a.cu_seqlens[r];
  const int n = min(a.cu_seqlens[r + 1], a.total_q) - max(q0, 0);
  const int t0 = tile * TQ;
  const int tvalid = min(TQ, n - t0);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int hl = lane & 31, hbase = lane & 32;
  const int row = kMergeRows * blockIdx.z + 2 * wv + (lane >> 5);
  const int tok = row / G, hh = row % G;
  const bool live = tok < tvalid;  // rows past the tile's tokens hold nothing
  const int64_t ostride = (int64_t)a.num_kv_heads * kRowsWG * kHeadDim;  // between pieces
  const float* orow = sp.part_o +
                      ((int64_t)j * sp.max_pieces * a.num_kv_heads + g) * kRowsWG * kHeadDim +
                      (int64_t)row * kHeadDim + 4 * hl;
  const float* mlrow = sp.part_ml +
                       (((int64_t)j * a.num_kv_heads + g) * kRowsWG + row) * sp.max_pieces * 2;
  float2 ml = make_float2(-1.0e30f, 0.f);
  if (hl < pcs && live) ml = *reinterpret_cast<const float2*>(mlrow + 2 * hl);
  float4 o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    o[k] = k < pcs && live ? *reinterpret_cast<const float4*>(orow + k * ostride)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
  // both halves run the shuffles (whole-wavefront instructions)
  float M = ml.x;
#pragma unroll
  for (int d = 16; d >= 1; d >>= 1) M = fmaxf(M, __shfl_xor(M, d));
  const float w = hl < pcs && live ? pow2_weight(ml.x, M) : 0.f;
  float lsum = w * ml.y;
#pragma unroll
  for (int d = 16; d >= 1; d >>= 1) lsum += __shfl_xor(lsum, d);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0;;) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float wp = __shfl(w, hbase + ((p0 + k) & 31));
      acc[0] = fmaf(wp, o[k].x, acc[0]);
      acc[1] = fmaf(wp, o[k].y, acc[1]);
      acc[2] = fmaf(wp, o[k].z, acc[2]);
      acc[3] = fmaf(wp, o[k].w, acc[3]);
    }
    p0 += 8;
    if (p0 >= pcs) break;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      o[k] = p0 + k < pcs && live ? *reinterpret_cast<const float4*>(orow + (int64_t)(p0 + k) * ostride)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (!live) return;
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  uint2 st;
  st.x = cvt_pk_bf16(acc[0] * inv, acc[1] * inv);
  st.y = cvt_pk_bf16(acc[2] * inv, acc[3] * inv);
  uint16_t* out = static_cast<uint16_t*>(a.out) +
                  ((int64_t)(q0 + t0 + tok) * a.num_q_heads + g * G + hh) * kHeadDim;
  *reinterpret_cast<uint2*>(out + 4 * hl) = st;
}

template <int G>
hipError_t launch_split_g(const PrefillArgs& a, const PrefillSplit& sp, hipStream_t s) {
  constexpr int TQ = kRowsWG / G;
  if (sp.n_qtiles == 0 || a.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a, sp, TQ);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prefill_piece_kernel<G>), dim3((unsigned)sp.max_items * a.num_kv_heads),
                     dim3(kThreads), 0, s, a, sp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prefill_merge_kernel, dim3(a.num_kv_heads, sp.max_entries, kRowsWG / kMergeRows),
                     dim3(kMergeThreads), 0, s, a, sp, G);
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

hipError_t launch_prefill_append(const PrefillArgs& a, hipStream_t s) {
  if (a.k_new == nullptr || a.v_new == nullptr || a.new_slots == nullptr) return hipErrorInvalidValue;
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_g<1, true>(a, s);
    case 2: return launch_g<2, true>(a, s);
    case 4: return launch_g<4, true>(a, s);
    case 5: return launch_g<5, true>(a, s);
    case 8: return launch_g<8, true>(a, s);
    case 16: return launch_g<16, true>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_split(const PrefillArgs& a, const PrefillSplit& sp, hipStream_t s) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_split_g<1>(a, sp, s);
    case 2: return launch_split_g<2>(a, sp, s);
    case 4: return launch_split_g<4>(a, sp, s);
    case 5: return launch_split_g<5>(a, sp, s);
    case 8: return launch_split_g<8>(a, sp, s);
    case 16: return launch_split_g<16>(a, sp, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qil
