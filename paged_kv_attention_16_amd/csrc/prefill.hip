// Chunked varlen causal prefill over the paged cache, on bf16 matrix cores.
//
// What is computed follows the "nano-vLLM learning note" Attention.forward
// prefill branch (with a cached prefix the keys come from the cache through
// the block tables) and prepare_prefill block (the new tokens of a request
// sit at positions num_cached .. num_cached + n - 1), and the "qwen-engine"
// README's flat varlen prefill (requests packed by cu_seqlens) and its note
// that prefill is compute-bound.
//
// One workgroup (4 wavefronts) owns 128 query rows of one request and one KV
// head: 128/G consecutive new tokens times the G query heads that share the
// KV head (GQA packing), so each K/V tile fetched from HBM/L2 serves 128 rows.
// The workgroup walks key tiles of 64 keys up to its last visible key.  Per
// tile:
//   * K (64 x 128) is gathered through the block table into LDS row-major
//     with an XOR swizzle of the 16-byte chunks; V is written transposed
//     (128 x 64) so that the PV product can read it as an MFMA operand.
//     The next tile's global loads are issued before the current tile is
//     computed.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys on the M side, the
//     wavefront's 32 query rows on the N side), so that every lane owns one
//     query row and the row statistics of the online softmax stay per lane.
//   * Causal mask only on tiles that reach past the first token's position.
//   * Online softmax in base 2; P is rounded to bf16 and used directly from
//     the accumulator registers as the B operand of O^T = V^T P^T, whose
//     accumulator again keeps one query row per lane, so the rescale by the
//     running-max correction is a per-lane multiply.
// Block ids are laid out KV-head fastest, so with 8 KV heads all tiles of one
// KV head land on one XCD (workgroups are dealt to the 8 XCDs round robin)
// and its K/V stay in that XCD's L2.  Query tiles are issued last-first: the
// tiles with the most keys start earliest.
#include "device_common.h"
#include "qil_internal.h"

namespace qil {
namespace {

constexpr int kBN = 64;     // keys per tile
constexpr int kRowsWG = 128;  // query rows per workgroup (4 wavefronts x 32)

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

__device__ __forceinline__ uint4 load_kv_chunk(const char* pool, const int32_t* bt_row, int key,
                                               int L, int log2P, int num_pages, int Hkv, int g,
                                               int chunk) {
  if (key >= L) return make_uint4(0, 0, 0, 0);
  const int page = bt_row[key >> log2P];
  if ((unsigned)page >= (unsigned)num_pages) return make_uint4(0, 0, 0, 0);
  const int64_t row = (((int64_t)page * Hkv + g) << log2P) + (key & ((1 << log2P) - 1));
  return *reinterpret_cast<const uint4*>(pool + row * 256 + chunk * 16);
}

__device__ __forceinline__ uint32_t lo16(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t hi16(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

template <int G>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a, int n_qtiles) {
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
  const int ntiles = (kmax + kBN - 1) / kBN;
  const int pos_min = prefix + t0;

  const int tid = threadIdx.x;
  const int w = wave_uniform(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int hf = lane >> 5;

  // This lane's query row (column of S^T and O^T).
  const int rho = 32 * w + lq;
  const int tq = rho / G;
  const int hh = rho % G;
  const bool row_valid = tq < tvalid;
  const int my_pos = prefix + t0 + min(tq, tvalid - 1);
  const int Hq = a.num_q_heads;

  bf16x8_t qreg[8];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           ((int64_t)(q0 + t0 + tq) * Hq + g * G + hh) * kHeadDim;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint4 x = row_valid ? *reinterpret_cast<const uint4*>(qrow + 16 * t + 8 * hf)
                          : make_uint4(0, 0, 0, 0);
      qreg[t] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  __shared__ __attribute__((aligned(16))) char sK[kBN * 256];
  __shared__ __attribute__((aligned(16))) char sVt[kHeadDim * kBN * 2];

  const int lc = tid & 15;  // 16-byte chunk of a 256-byte row this thread moves
  const int lk = tid >> 4;  // 0..15
  const int32_t* bt_row = a.block_tables + (int64_t)r * a.bt_stride;
  const char* kpool = static_cast<const char*>(a.k_cache);
  const char* vpool = static_cast<const char*>(a.v_cache);

  uint4 kreg[4], vreg[4];
  auto gload = [&](int kt) {
    const int kb = kt * kBN;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      kreg[i] = load_kv_chunk(kpool, bt_row, kb + lk + 16 * i, L, a.log2_page, a.num_pages,
                              a.num_kv_heads, g, lc);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vreg[i] = load_kv_chunk(vpool, bt_row, kb + 4 * lk + i, L, a.log2_page, a.num_pages,
                              a.num_kv_heads, g, lc);
  };
  auto swrite = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(sK + k_offset(lk + 16 * i, lc)) = kreg[i];
    // V^T: thread holds keys 4lk .. 4lk+3 at dims 8lc .. 8lc+7.
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
      *reinterpret_cast<uint2*>(sVt + vt_offset(8 * lc + e, p0)) = pk;
    }
  };

  f32x16_t oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[i][v] = 0.f;
  float mrun = -1.0e30f, lrun = 0.f;
  const float qs = a.scale * kLog2e;

  gload(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();  // previous tile fully consumed
    swrite();
    __syncthreads();
    if (kt + 1 < ntiles) gload(kt + 1);

    // S^T = K Q^T  (two 32-key blocks)
    f32x16_t sacc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[b][v] = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int kk = 32 * b + lq;
        const bf16x8_t kop = *reinterpret_cast<const bf16x8_t*>(sK + k_offset(kk, 2 * t + hf));
        sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[t], sacc[b], 0, 0, 0);
      }
    }

    const int kbase = kt * kBN;
    const bool need_mask = kbase + kBN - 1 > pos_min;  // uniform
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = sacc[b][v] * qs;
        if (need_mask && kbase + 32 * b + acc_row(v, hf) > my_pos) x = -INFINITY;
        sacc[b][v] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(mrun, mx);
    const float corr = fast_exp2(mrun - mnew);
    mrun = mnew;
    float psum = 0.f;
    bf16x8_t pb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t pk[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = fast_exp2(sacc[s >> 1][8 * (s & 1) + 2 * i] - mnew);
        const float p1 = fast_exp2(sacc[s >> 1][8 * (s & 1) + 2 * i + 1] - mnew);
        psum += p0 + p1;
        pk[i] = cvt_pk_bf16(p0, p1);
      }
      const uint4 u = {pk[0], pk[1], pk[2], pk[3]};
      pb[s] = __builtin_bit_cast(bf16x8_t, u);
    }
    lrun = lrun * corr + psum;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[i][v] *= corr;

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = 32 * db + lq;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8_t vop =
            *reinterpret_cast<const bf16x8_t*>(sVt + vt_offset(d, 16 * s + 8 * hf));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[s], oacc[db], 0, 0, 0);
      }
    }
  }

  const float ltot = lrun + __shfl_xor(lrun, 32);
  if (!row_valid) return;
  const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
  uint16_t* orow = static_cast<uint16_t*>(a.out) +
                   ((int64_t)(q0 + t0 + tq) * Hq + g * G + hh) * kHeadDim;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * db + 8 * q4 + 4 * hf;
      uint2 st;
      st.x = pack_bf16x2(oacc[db][4 * q4] * inv, oacc[db][4 * q4 + 1] * inv);
      st.y = pack_bf16x2(oacc[db][4 * q4 + 2] * inv, oacc[db][4 * q4 + 3] * inv);
      *reinterpret_cast<uint2*>(orow + d0) = st;
    }
  }
}

template <int G>
hipError_t launch_g(const PrefillArgs& a, hipStream_t s) {
  constexpr int TQ = kRowsWG / G;
  const int n_qtiles = (a.max_seqlen_q + TQ - 1) / TQ;
  if (n_qtiles == 0 || a.batch == 0) return hipSuccess;
  dim3 grid(a.num_kv_heads, a.batch, n_qtiles);
  hipLaunchKernelGGL((prefill_kernel<G>), grid, dim3(256), 0, s, a, n_qtiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_g<1>(a, s);
    case 2: return launch_g<2>(a, s);
    case 4: return launch_g<4>(a, s);
    case 8: return launch_g<8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qil
