// bf16 paged decode on matrix cores: the device code of one split, included
// by decode.hip and mixed.hip.  What is computed follows the "nano-vLLM
// learning note" Attention.forward decode branch and prepare_decode block.
#pragma once

#include "device_common.h"
#include "qil_internal.h"

namespace qil {
namespace {

constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima

// ---------------------------------------------------------------------------
// bf16 split kernel on matrix cores with LDS-staged K/V tiles.
//
// Same grid and split walk as decode_f32_kernel, but each wavefront streams
// its 16-key groups through a private ring of kMD LDS slots (global_load_lds,
// 16 bytes per lane, no staging registers; no workgroup barrier inside the
// loop, since no other wavefront reads a wavefront's slots) and computes on
// 16x16 MFMAs with the G query heads of the KV head as the N side (padded to
// 16 with copies of real heads):
//   S^T (16 keys x 16 heads) = K Q^T      4 x v_mfma_f32_16x16x32_bf16
//   O^T (128 dims x 16 heads) += V^T P^T  8 x v_mfma_f32_16x16x16bf16_1k
// Lane l holds head (l % 16) in both accumulators, so the softmax state of a
// head is per lane; its 16 keys of a group sit in the four lanes l, l^16,
// l^32, l^48 (permlane swaps).  V^T operands come from ds_read_b64_tr_b16.
// The weights are rounded to bf16 for the PV product and the row sum adds
// the same rounded weights; the output is rescaled lazily (when a head's
// maximum grows by more than 2^8), so a weight never exceeds 256.
constexpr int kMW = 4;               // wavefronts per workgroup of decode_mfma_kernel
constexpr int kMD = 2;               // LDS slots per wavefront (16-key K and V tiles)
constexpr int kTile = 16 * 256;      // bytes of one 16-key bf16 tile
constexpr float kLazy = 8.0f;

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Physical 16-byte chunk of logical chunk c in tile row `row`.  K: XOR with
// row mod 16 (the 16 rows of an A-operand read hit 16 different chunks).
// V: XOR with 2 * (row mod 8) (the 32-byte pieces of the 8 rows of a
// transposing read fall into 8 different bank windows).
__device__ __forceinline__ int mk_chunk(int row, int c) { return c ^ (row & 15); }
__device__ __forceinline__ int mv_chunk(int row, int c) { return c ^ ((row & 7) << 1); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ float swap_max16(float x) {
  const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float swap_max32(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float swap_sum16(float x) {
  const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}
__device__ __forceinline__ float swap_sum32(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// LDS ring of one wavefront: [slot][K | V][16 rows x 256 bytes].
typedef char DecodeRing[kMD][2][kTile];

// One split of one (KV head g, request r), computed by the W wavefronts of the
// calling workgroup; `smem` holds one ring per wavefront.
template <int G, int W>
__device__ __forceinline__ void decode_mfma_split(const DecodeArgs& a, int split, int g, int r,
                                                  DecodeRing* smem) {
  const int L = min(a.context_lens[r], a.max_context_len);
  const int kbeg = split * a.keys_per_split;
  if (kbeg >= L) return;  // this split lies past the context (uniform per block)
  const int kend = min(L, kbeg + a.keys_per_split);

  const int tid = threadIdx.x;
  const int w = wave_uniform(tid >> 6);
  const int lane = tid & 63;
  const int q4 = lane >> 4;   // 16-lane group
  const int c16 = lane & 15;  // M/N index of the 16x16 MFMAs
  const int P = 1 << a.log2_page;

  // B operand of S^T: head c16 (padding heads repeat real ones), dims 32t + 8 q4 .. +7.
  bf16x8_t qop[4];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           ((int64_t)r * a.num_q_heads + g * G + (c16 % G)) * kHeadDim;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      qop[t] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qrow + 32 * t + 8 * q4));
  }

  char* ring = &smem[w][0][0][0];

  // Append: the new token's key L - 1 lies in this split.  The wavefront
  // whose group holds it takes its K and V rows from the inputs (lanes 0-15
  // one 16-byte chunk of K each, lanes 16-31 of V), writes them over that
  // row of its LDS tile once the tile has landed, so the pool is never read
  // for that row, and stores them at the token's slot after its last group.
  // The row load is issued behind the first group's tile loads, so the
  // count waits of the ring cover it without delaying the stream.
  const int app_rel = a.k_new != nullptr && L - 1 >= kbeg && L - 1 < kend ? L - 1 - kbeg : -1;
  const int app_w = app_rel >= 0 ? (app_rel >> 4) % W : -1;
  const int app_i = app_rel >= 0 ? app_rel / (16 * W) : -1;
  const int app_row = app_rel & 15;
  const bool app_lane = w == app_w && lane < 32;
  const int app_c = lane & 15;
  const bool app_is_v = lane >= 16;
  uint4 app_val = make_uint4(0u, 0u, 0u, 0u);

  const int32_t* bt_row = a.block_tables + (int64_t)r * a.bt_stride;
  const char* kpool = static_cast<const char*>(a.k_cache);
  const char* vpool = static_cast<const char*>(a.v_cache);
  // Group i of this wavefront: keys first + 16 W i .. +15 (inside one page).
  const int first = kbeg + 16 * w;
  const int ngroups = first < kend ? (kend - first + 16 * W - 1) / (16 * W) : 0;
  int page_of_lane = -1;
  if (lane < ngroups) page_of_lane = bt_row[(first + 16 * W * lane) >> a.log2_page];

  // Issue the 8 tile loads of group i into slot i % kMD.  Every lane always
  // loads (rows past the context re-read the group's first row, and a page
  // id out of range reads page 0), so each group is exactly 8 vector-memory
  // instructions and the ring can be waited on by count.
  const int lrow = lane >> 4;  // row within a 4-row load
  const int lpc = lane & 15;   // physical chunk this lane fills
  auto issue = [&](int i) __attribute__((always_inline)) {
    const int key0 = first + 16 * W * i;
    int page = __builtin_amdgcn_readlane(page_of_lane, i);
    page = (unsigned)page < (unsigned)a.num_pages ? page : 0;
    const int64_t row0 = ((int64_t)page * a.num_kv_heads + g) * P + (key0 & (P - 1));
    lds_char* kdst = (lds_char*)(ring + (i % kMD) * 2 * kTile);
    lds_char* vdst = kdst + kTile;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int row = 4 * m + lrow;
      const int srow = key0 + row < kend ? row : 0;
      const char* kp = kpool + (row0 + srow) * 256 + 16 * mk_chunk(row, lpc);
      const char* vp = vpool + (row0 + srow) * 256 + 16 * mv_chunk(row, lpc);
      __builtin_amdgcn_global_load_lds(kp, kdst + m * 1024, 16, 0, 2);
      __builtin_amdgcn_global_load_lds(vp, vdst + m * 1024, 16, 0, 2);
    }
  };

  // Transposing-read offsets: source lane (j + 4k) of a 16-lane group points
  // at V row 4 q4 + k, dims 16 db + 4j .. +3; lane o of the group receives
  // the four keys 4 q4 .. 4 q4 + 3 at dim 16 db + o.
  int vofs[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const int j = lane & 3, k = (lane >> 2) & 3;
    const int row = 4 * q4 + k;
    const int c = 2 * db + (j >> 1);
    vofs[db] = row * 256 + 16 * mv_chunk(row, c) + 8 * (j & 1);
  }

  const float qs = a.scale * kLog2e;
  f32x4_t oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mref = kNegBig;
  float lsum = 0.f;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  auto compute = [&](int i) __attribute__((always_inline)) {
    const char* kt = ring + (i % kMD) * 2 * kTile;
    const lds_char* vt = (const lds_char*)(kt + kTile);
    f32x4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x8_t kop =
          *reinterpret_cast<const bf16x8_t*>(kt + c16 * 256 + 16 * mk_chunk(c16, 4 * t + q4));
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[t], st, 0, 0, 0);
    }
    // st[e]: key 4 q4 + e of the group, head c16.  Mask keys past the split.
    const int kb = first + 16 * W * i + 4 * q4;
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (kb + e >= kend) st[e] = -INFINITY;
      mx = fmaxf(mx, st[e]);
    }
    mx = swap_max32(swap_max16(mx)) * qs;
    if (__ballot(mx > mref + kLazy) != 0) {
      asm volatile("" ::: "memory");  // keep the rare rescale a real branch
      const float mnew = fmaxf(mref, mx);
      const float corr = fast_exp2(mref - mnew);
      mref = mnew;
      lsum *= corr;
#pragma unroll
      for (int db = 0; db < 8; ++db) oacc[db] *= corr;
    }
    const float p0 = fast_exp2(fmaf(st[0], qs, -mref));
    const float p1 = fast_exp2(fmaf(st[1], qs, -mref));
    const float p2 = fast_exp2(fmaf(st[2], qs, -mref));
    const float p3 = fast_exp2(fmaf(st[3], qs, -mref));
    const uint32_t pk0 = cvt_pk_bf16(p0, p1);
    const uint32_t pk1 = cvt_pk_bf16(p2, p3);
    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk0), ones, lsum, false);
    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk1), ones, lsum, false);
    const uint2 pu = {pk0, pk1};
    const i16x4_t pb = __builtin_bit_cast(i16x4_t, pu);
    // The transposing reads are written as inline assembly: the compiler
    // cannot tell which ring slot an LDS-DMA load writes, and in front of the
    // intrinsic it waits for every load in flight, which would drain the ring
    // each group.  The explicit count wait above already covers this group's
    // loads; the operands pass through the lgkmcnt wait below, so no MFMA can
    // be scheduled before the data is in registers.
    i16x4_t vop[8];
    const uint32_t vaddr = (uint32_t)(uintptr_t)vt;
#pragma unroll
    for (int db = 0; db < 8; ++db)
      asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(vop[db]) : "v"(vaddr + vofs[db]) : "memory");
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(vop[0]), "+v"(vop[1]), "+v"(vop[2]), "+v"(vop[3]), "+v"(vop[4]),
                   "+v"(vop[5]), "+v"(vop[6]), "+v"(vop[7])
                 :
                 : "memory");
#pragma unroll
    for (int db = 0; db < 8; ++db)
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop[db], pb, oacc[db], 0, 0, 0);
  };

  // The ring: kMD - 1 groups in flight ahead of the one being computed.
#pragma unroll
  for (int i = 0; i < kMD - 1; ++i)
    if (i < ngroups) issue(i);
  if (app_lane) {
    const uint16_t* src = static_cast<const uint16_t*>(app_is_v ? a.v_new : a.k_new) +
                          (int64_t)r * (app_is_v ? a.v_new_stride : a.k_new_stride) + g * kHeadDim;
    app_val = *reinterpret_cast<const uint4*>(src + 8 * app_c);
  }
  for (int i = 0; i < ngroups; ++i) {
    // refill the slot computed at i - 1 (its LDS reads are complete), then
    // wait until group i has landed: the groups issued after it may still fly
    if (i + kMD - 1 < ngroups) issue(i + kMD - 1);
    const int ahead = min(ngroups - 1 - i, kMD - 1);
    if (kMD > 3 && ahead >= 3) wait_vmcnt<24>();
    else if (kMD > 2 && ahead == 2) wait_vmcnt<16>();
    else if (ahead == 1) wait_vmcnt<8>();
    else wait_vmcnt<0>();
    if (w == app_w && i == app_i) {
      // The tile has landed (the count wait above): overwrite the new
      // token's row.  When it is the group's first row, the rows past the
      // context were loaded as copies of it (stale pool contents): they get
      // the new row too, since their weights are 0 but must multiply finite
      // values.  This wavefront's LDS reads below come after the writes.
      char* kt = ring + (i % kMD) * 2 * kTile;
      const int last = app_row == 0 ? 15 : app_row;
      for (int row = app_row; row <= last; ++row) {
        if (lane < 16)
          *reinterpret_cast<uint4*>(kt + row * 256 + 16 * mk_chunk(row, lane)) = app_val;
        else if (lane < 32)
          *reinterpret_cast<uint4*>(kt + kTile + row * 256 + 16 * mv_chunk(row, lane - 16)) = app_val;
      }
    }
    compute(i);
  }
  static_assert(kMD >= 2 && kMD <= 4, "the wait ladder above covers 1 to 3 groups in flight");
  if (app_lane) {
    const int32_t slot = a.new_slots[r];
    const int64_t page = slot >> a.log2_page;
    if (slot >= 0 && page < a.num_pages) {
      const int64_t prow = ((page * a.num_kv_heads + g) << a.log2_page) + (slot & (P - 1));
      // the append entry point hands over writable pools
      char* pool = const_cast<char*>(static_cast<const char*>(app_is_v ? a.v_cache : a.k_cache));
      *reinterpret_cast<uint4*>(pool + prow * 256 + 16 * app_c) = app_val;
    }
  }

  // Row sums over the four lanes of each head.
  lsum = swap_sum32(swap_sum16(lsum));

  // Merge the W wavefronts through LDS (the ring is free now).
  __syncthreads();
  float* sh_o = reinterpret_cast<float*>(&smem[0][0][0][0]);   // [W][G][128]
  float* sh_m = sh_o + W * G * kHeadDim;                      // [W][G]
  float* sh_l = sh_m + W * G;                                 // [W][G]
  if (c16 < G) {
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sh_o[(w * G + c16) * kHeadDim + 16 * db + 4 * q4 + e] = oacc[db][e];
    if (q4 == 0) {
      sh_m[w * G + c16] = mref;
      sh_l[w * G + c16] = lsum;
    }
  }
  __syncthreads();

  const bool single = a.num_splits == 1;
  for (int idx = tid; idx < G * kHeadDim; idx += 64 * W) {
    const int h = idx / kHeadDim;
    const int d = idx % kHeadDim;
    float mx = sh_m[h];
#pragma unroll
    for (int ww = 1; ww < W; ++ww) mx = fmaxf(mx, sh_m[ww * G + h]);
    float acc = 0.f, ls = 0.f;
#pragma unroll
    for (int ww = 0; ww < W; ++ww) {
      const float f = fast_exp2(sh_m[ww * G + h] - mx);
      acc = fmaf(f, sh_o[(ww * G + h) * kHeadDim + d], acc);
      ls = fmaf(f, sh_l[ww * G + h], ls);
    }
    const int qh = g * G + h;
    if (single) {
      const float val = ls > 0.f ? acc / ls : 0.f;
      static_cast<uint16_t*>(a.out)[((int64_t)r * a.num_q_heads + qh) * kHeadDim + d] =
          (uint16_t)f32_to_bf16_bits(val);
    } else {
      const int64_t pi = ((int64_t)r * a.num_q_heads + qh) * a.num_splits + split;
      a.ws_o[pi * kHeadDim + d] = acc;
      if (d == 0) {
        a.ws_m[pi] = mx;
        a.ws_l[pi] = ls;
      }
    }
  }
}

// Longest-first order inside the workgroup, for batches of at most
// kRankMaxBatch requests: every workgroup (of 64 W >= 256 threads) sorts the
// batch the same way and keeps the request at its own grid row z.  The sort
// is a stable counting sort over 256 buckets of decreasing context length
// (bucket 0 holds the longest), ties in request order, so every workgroup
// derives the same permutation: the bucket that holds position z comes from
// the histogram's prefix sum, and the request inside it from one ballot per
// wavefront over the bucket's members.  Threads 0..255 hold one request and
// one bucket each.  No global writes; it replaces a separate ordering launch
// and the dependent read of its result.  Larger batches measured slower this
// way (each workgroup reads every length) and keep the ordering launch.
constexpr int kRankMaxBatch = 256;

template <int W>
__device__ __forceinline__ int decode_rank_request(const int32_t* context_lens, int batch,
                                                   int max_len, int z) {
  static_assert(64 * W >= kRankMaxBatch, "a thread per bucket and per request");
  constexpr int kRankWaves = kRankMaxBatch / 64;
  __shared__ int hist[kRankMaxBatch];
  __shared__ int wave_sum[kRankWaves];
  __shared__ unsigned long long members[kRankWaves];
  __shared__ int pick[3];  // bucket of position z, its offset in the bucket, the request
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const bool holder = tid < kRankMaxBatch;  // whole wavefronts
  if (holder) hist[tid] = 0;
  if (tid == 0) {
    pick[0] = -1;
    pick[2] = z;  // stays in range even if no bucket claims z
  }
  int b = -1;  // bucket of request tid
  if (tid < batch) {
    int L = context_lens[tid];
    L = L < 0 ? 0 : (L > max_len ? max_len : L);
    b = (int)((int64_t)(max_len - L) * kRankMaxBatch / ((int64_t)max_len + 1));
  }
  __syncthreads();
  if (b >= 0) atomicAdd(&hist[b], 1);
  __syncthreads();
  // exclusive prefix sum over the buckets, thread t holding bucket t
  int own = 0, v = 0;
  if (holder) {
    own = v = hist[tid];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(v, o);
      if (lane >= o) v += t;
    }
    if (lane == 63) wave_sum[wv] = v;
  }
  __syncthreads();
  if (holder) {
    int start = v - own;
    for (int i = 0; i < wv; ++i) start += wave_sum[i];
    if (z >= start && z < start + own) {
      pick[0] = tid;
      pick[1] = z - start;
    }
  }
  __syncthreads();
  const int pb = pick[0];
  unsigned long long m = 0;
  if (holder) {
    m = __ballot(b == pb);
    if (lane == 0) members[wv] = m;
  }
  __syncthreads();
  if (b >= 0 && b == pb) {
    // members before request tid: those of lower wavefronts and lower lanes
    int rank = __popcll(m & ((1ull << lane) - 1));
    for (int i = 0; i < wv; ++i) rank += __popcll(members[i]);
    if (rank == pick[1]) pick[2] = tid;
  }
  __syncthreads();
  return pick[2];
}

template <int G>
__global__ __launch_bounds__(64 * kMW) void decode_mfma_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) DecodeRing smem[kMW];
  int r = blockIdx.z;
  if (a.rank_inline)
    r = decode_rank_request<kMW>(a.context_lens, a.batch, a.max_context_len, r);
  else if (a.order != nullptr)
    r = a.order[r];
  decode_mfma_split<G, kMW>(a, blockIdx.x, blockIdx.y, r, smem);
}

}  // namespace
}  // namespace qil
