// Chunked varlen causal prefill over the paged cache, on bf16 matrix cores.
//
// What is computed follows the "nano-vLLM learning note" Attention.forward
// prefill branch (with a cached prefix the keys come from the cache through
// the block tables) and prepare_prefill block (the new tokens of a request
// sit at positions num_cached .. num_cached + n - 1), and the "qwen-engine"
// README's flat varlen prefill (requests packed by cu_seqlens) and its note
// that prefill is compute-bound.
//
// One workgroup (4 wavefronts) owns 256 query rows of one request and one KV
// head: 256/G consecutive new tokens times the G query heads that share the
// KV head (GQA packing), so each K/V tile fetched from HBM/L2 serves 256 rows.
// Each wavefront owns 64 rows as two 32-row MFMA blocks, so every operand it
// reads from LDS feeds two MFMAs.  The workgroup walks key tiles of 64 keys
// up to its last visible key.  Per tile:
//   * K (64 x 128) is gathered through the block table into LDS row-major
//     with an XOR swizzle of the 16-byte chunks; V is written transposed
//     (128 x 64) so that the PV product can read it as an MFMA operand.  LDS
//     is double-buffered: the next tile's global loads are in flight while
//     the current tile is computed, then land in the other buffer (one
//     barrier per tile).  Block-table entries are fetched a tile earlier.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys on the M side, query
//     rows on the N side), so that every lane owns one query row per block
//     and the row statistics of the online softmax stay per lane.
//   * Causal mask only on tiles that reach past the first token's position.
//   * Online softmax in base 2 with a lazy reference maximum: the output is
//     rescaled only when some row's maximum grows by more than 2^8, so the
//     weights exp2(s - m_ref) stay below 256 and most tiles skip the rescale.
//     P is rounded to bf16 and used directly from registers as the B operand
//     of O^T = V^T P^T; the row sum adds the same rounded weights.
// Block ids are laid out KV-head fastest, so with 8 KV heads all tiles of one
// KV head land on one XCD (workgroups are dealt to the 8 XCDs round robin)
// and its K/V stay in that XCD's L2.  Query tiles are issued last-first: the
// tiles with the most keys start earliest.
#include <stdlib.h>

#include <type_traits>

#include "device_common.h"
#include "qil_internal.h"

namespace qil {
namespace {

constexpr int kBN = 64;        // keys per tile
constexpr int kRowsWG = 256;   // query rows per workgroup (4 wavefronts x 64)
constexpr float kLazyRescale = 8.0f;  // log2 of the largest weight allowed before rescaling

// Row (M index) of accumulator register v held by lanes of half hf, for the
// 32x32 MFMA output: rows 8*(v/4) + 4*hf + v%4, column = lane % 32.
__device__ __forceinline__ int acc_row(int v, int hf) { return 8 * (v >> 2) + 4 * hf + (v & 3); }

// Position of key o (0..15 inside a 16-key group) in a V^T row: bits 2 and 3
// swapped, so that the 8 keys a half-wavefront feeds to one PV k-step are
// contiguous.
__device__ __forceinline__ int swap23(int o) { return (o & 3) | ((o & 4) << 1) | ((o & 8) >> 1); }

// Byte offset of (row d, position p) in the V^T tile: 128-byte rows; rows are
// swapped within pairs when bit 3 of d is set and the 16-byte chunks are XOR
// swizzled, which keeps both the transposing writes and the operand reads
// spread over the LDS banks.
__device__ __forceinline__ int vt_offset(int d, int p) {
  const int prow = d ^ ((d >> 3) & 1);
  const int chunk = (p >> 3) ^ (((d >> 1) ^ (d >> 4)) & 7);
  return prow * 128 + chunk * 16 + (p & 7) * 2;
}

// Byte offset of (key row kk, 16-byte chunk c) in the K tile.
__device__ __forceinline__ int k_offset(int kk, int c) { return kk * 256 + ((c ^ (kk & 15)) << 4); }

__device__ __forceinline__ uint32_t lo16(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t hi16(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

// QB = 32-row MFMA blocks per wavefront; the workgroup has 8/QB wavefronts
// (256 query rows either way).  QB = 2 shares every LDS operand between two
// MFMAs; QB = 1 halves the registers of a wavefront so two fit on a SIMD.
template <int G, int QB>
__global__ __launch_bounds__(512 / QB) void prefill_kernel(PrefillArgs a, int n_qtiles) {
  constexpr int NT = 512 / QB;     // threads per workgroup
  constexpr int TQ = kRowsWG / G;  // tokens per workgroup
  const int g = blockIdx.x;
  const int r = blockIdx.y;
  const int tile = n_qtiles - 1 - (int)blockIdx.z;
  const int q0 = a.cu_seqlens[r];
  // rows of this request, kept inside [0, total_q)
  const int n = min(a.cu_seqlens[r + 1], a.total_q) - max(q0, 0);
  const int t0 = tile * TQ;
  if (q0 < 0 || t0 >= n) return;
  const int L = min(a.context_lens[r], a.max_context_len);
  const int prefix = L - n;
  const int tvalid = min(TQ, n - t0);
  const int kmax = prefix + t0 + tvalid;  // keys [0, kmax) are visible to some row
  const int ntiles = kmax > 0 ? (kmax + kBN - 1) / kBN : 0;
  const int pos_min = prefix + t0;

  const int tid = threadIdx.x;
  const int w = wave_uniform(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int hf = lane >> 5;
  const int Hq = a.num_q_heads;

  // This lane's query row in each of the wavefront's 32-row blocks.
  int tok[QB], hh[QB], my_pos[QB];
  bool row_valid[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int rho = 32 * (QB * w + qb) + lq;
    tok[qb] = rho / G;
    hh[qb] = rho % G;
    row_valid[qb] = tok[qb] < tvalid;
    my_pos[qb] = prefix + t0 + min(tok[qb], tvalid - 1);
  }

  bf16x8_t qreg[QB][8];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           ((int64_t)(q0 + t0 + tok[qb]) * Hq + g * G + hh[qb]) * kHeadDim;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint4 x = row_valid[qb] ? *reinterpret_cast<const uint4*>(qrow + 16 * t + 8 * hf)
                              : make_uint4(0, 0, 0, 0);
      qreg[qb][t] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  __shared__ __attribute__((aligned(16))) char sK[2][kBN * 256];
  __shared__ __attribute__((aligned(16))) char sVt[2][kHeadDim * kBN * 2];

  // Loader role: a thread moves 16-byte chunk lc of keys 4lk .. 4lk+3 of a
  // tile (four consecutive keys always share a page).  With 256 threads each
  // thread moves K and V; with 512, the first half moves K, the second V.
  const int lt = tid & 255;
  const int lc = lt & 15;
  const int lk = lt >> 4;
  const bool do_k = NT == 256 || tid < 256;
  const bool do_v = NT == 256 || tid >= 256;
  const int32_t* bt_row = a.block_tables + (int64_t)r * a.bt_stride;
  const char* kpool = static_cast<const char*>(a.k_cache);
  const char* vpool = static_cast<const char*>(a.v_cache);
  const int P = 1 << a.log2_page;

  auto page_of = [&](int kt) __attribute__((always_inline)) -> int {
    const int key0 = kt * kBN + 4 * lk;
    return key0 < L ? bt_row[key0 >> a.log2_page] : -1;
  };

  // Staging registers: with 256 threads a thread carries both its K and V
  // chunks; with 512 it carries one of them (xreg[1] is then unused).
  constexpr int NREG = NT == 256 ? 2 : 1;
  uint4 xreg[NREG][4];
  auto gload = [&](int kt, int page) __attribute__((always_inline)) {
    const int key0 = kt * kBN + 4 * lk;
#pragma unroll
    for (int x = 0; x < NREG; ++x)
#pragma unroll
      for (int i = 0; i < 4; ++i) xreg[x][i] = make_uint4(0, 0, 0, 0);
    if ((unsigned)page < (unsigned)a.num_pages) {
      const int64_t row0 = (((int64_t)page * a.num_kv_heads + g) << a.log2_page) + (key0 & (P - 1));
      const int nvalid = kt * kBN + kBN <= L ? 4 : min(4, L - key0);
      const char* p0 = (NT == 256 || do_k ? kpool : vpool) + row0 * 256 + lc * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < nvalid) xreg[0][i] = *reinterpret_cast<const uint4*>(p0 + i * 256);
      if (NT == 256) {
        const char* p1 = vpool + row0 * 256 + lc * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i < nvalid) xreg[NREG - 1][i] = *reinterpret_cast<const uint4*>(p1 + i * 256);
      }
    }
  };

  auto swrite = [&](int buf) __attribute__((always_inline)) {
    if (do_k) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(sK[buf] + k_offset(4 * lk + i, lc)) = xreg[0][i];
    }
    if (do_v) {
      // V^T: this thread holds keys 4lk .. 4lk+3 at dims 8lc .. 8lc+7.
      const uint4* vreg = xreg[NREG - 1];
      const int key0 = 4 * lk;
      const int p0 = (key0 & ~15) | swap23(key0 & 15);
      const uint32_t v0[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
      const uint32_t v1[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
      const uint32_t v2[4] = {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w};
      const uint32_t v3[4] = {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dw = e >> 1;
        uint2 pk;
        if (e & 1) {
          pk.x = hi16(v0[dw], v1[dw]);
          pk.y = hi16(v2[dw], v3[dw]);
        } else {
          pk.x = lo16(v0[dw], v1[dw]);
          pk.y = lo16(v2[dw], v3[dw]);
        }
        *reinterpret_cast<uint2*>(sVt[buf] + vt_offset(8 * lc + e, p0)) = pk;
      }
    }
  };

  f32x16_t oacc[QB][4];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[qb][i][v] = 0.f;
  float mref[QB], lrun[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mref[qb] = -1.0e30f;  // base-2 domain
    lrun[qb] = 0.f;
  }
  const float qs = a.scale * kLog2e;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  const f32x16_t zero16 = {};

  // Softmax of one 32-key half-tile for row block qb: sacc holds S^T for the
  // 32 keys (this lane: 16 of them, for its query row).  Produces the bf16
  // weights as the B operands of two PV k-steps.
  auto softmax_half = [&](auto mask_tag, int qb, f32x16_t& sacc, int kbase,
                          bf16x8_t (&pb)[2]) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      if (MASK && kbase + acc_row(v, hf) > my_pos[qb]) sacc[v] = -INFINITY;
      mx = fmaxf(mx, sacc[v]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * qs;
    if (__ballot(mx > mref[qb] + kLazyRescale) != 0) {  // uniform: rescale the output
      const float mnew = fmaxf(mref[qb], mx);
      const float corr = fast_exp2(mref[qb] - mnew);
      mref[qb] = mnew;
      lrun[qb] *= corr;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[qb][i][v] *= corr;
    }
    const float neg = -mref[qb];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      uint32_t pk[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = fast_exp2(fmaf(sacc[8 * s2 + 2 * i], qs, neg));
        const float p1 = fast_exp2(fmaf(sacc[8 * s2 + 2 * i + 1], qs, neg));
        pk[i] = cvt_pk_bf16(p0, p1);
        lrun[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[i]), ones,
                                                   lrun[qb], false);
      }
      const uint4 u = {pk[0], pk[1], pk[2], pk[3]};
      pb[s2] = __builtin_bit_cast(bf16x8_t, u);
    }
  };

  // One tile, as two 32-key halves: S^T for the row blocks (every K operand
  // feeds QB MFMAs), softmax, then O^T += V^T P^T (every V^T operand feeds QB
  // MFMAs).  MASK: the tile reaches past the first token's position.
  auto compute = [&](auto mask_tag, int buf, int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      f32x16_t sacc[QB];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int kk = 32 * b + lq;
        const bf16x8_t kop = *reinterpret_cast<const bf16x8_t*>(sK[buf] + k_offset(kk, 2 * t + hf));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[qb][t],
                                                             t == 0 ? zero16 : sacc[qb], 0, 0, 0);
      }
      const int kbase = kt * kBN + 32 * b;
      bf16x8_t pb[QB][2];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) softmax_half(mask_tag, qb, sacc[qb], kbase, pb[qb]);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = 32 * db + lq;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const bf16x8_t vop = *reinterpret_cast<const bf16x8_t*>(
              sVt[buf] + vt_offset(d, 16 * (2 * b + s2) + 8 * hf));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            oacc[qb][db] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[qb][s2], oacc[qb][db], 0, 0, 0);
        }
      }
    }
  };

  // Tiles [0, nfree) lie wholly at or before the first token's position and
  // need no mask; the rest (the diagonal band) are masked.  Each tile: issue
  // the next tile's loads, fetch the block-table entry two tiles ahead,
  // compute from LDS, stage the next tile into the other buffer, barrier.
  const int nfree = min(ntiles, (pos_min + 1) / kBN);
  int pg = -1;
  auto tile_step = [&](auto mask_tag, int kt) __attribute__((always_inline)) {
    const int buf = kt & 1;
    if (kt + 1 < ntiles) gload(kt + 1, pg);
    if (kt + 2 < ntiles) pg = page_of(kt + 2);
    compute(mask_tag, buf, kt);
    if (kt + 1 < ntiles) swrite(buf ^ 1);
    __syncthreads();
  };
  if (ntiles > 0) {
    pg = page_of(0);
    gload(0, pg);
    swrite(0);
    if (ntiles > 1) pg = page_of(1);
    __syncthreads();
    for (int kt = 0; kt < nfree; ++kt) tile_step(std::false_type{}, kt);
    for (int kt = nfree; kt < ntiles; ++kt) tile_step(std::true_type{}, kt);
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float ltot = lrun[qb] + __shfl_xor(lrun[qb], 32);
    if (!row_valid[qb]) continue;
    const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
    uint16_t* orow = static_cast<uint16_t*>(a.out) +
                     ((int64_t)(q0 + t0 + tok[qb]) * Hq + g * G + hh[qb]) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * db + 8 * q4 + 4 * hf;
        uint2 st;
        st.x = pack_bf16x2(oacc[qb][db][4 * q4] * inv, oacc[qb][db][4 * q4 + 1] * inv);
        st.y = pack_bf16x2(oacc[qb][db][4 * q4 + 2] * inv, oacc[qb][db][4 * q4 + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d0) = st;
      }
    }
  }
}

template <int G, int QB>
hipError_t launch_g(const PrefillArgs& a, hipStream_t s) {
  constexpr int TQ = kRowsWG / G;
  const int n_qtiles = (a.max_seqlen_q + TQ - 1) / TQ;
  if (n_qtiles == 0 || a.batch == 0) return hipSuccess;
  dim3 grid(a.num_kv_heads, a.batch, n_qtiles);
  hipLaunchKernelGGL((prefill_kernel<G, QB>), grid, dim3(512 / QB), 0, s, a, n_qtiles);
  return hipGetLastError();
}

template <int QB>
hipError_t launch_qb(const PrefillArgs& a, hipStream_t s) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_g<1, QB>(a, s);
    case 2: return launch_g<2, QB>(a, s);
    case 4: return launch_g<4, QB>(a, s);
    case 8: return launch_g<8, QB>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  // QIL_PREFILL_QB selects the wavefront shape (1 or 2 row blocks) for tuning.
  static const int qb = [] {
    const char* e = getenv("QIL_PREFILL_QB");
    return (e && e[0] == '2') ? 2 : 1;
  }();
  return qb == 2 ? launch_qb<2>(a, s) : launch_qb<1>(a, s);
}

}  // namespace qil
