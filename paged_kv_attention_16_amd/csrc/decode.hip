// Paged decode attention: one query token per request, GQA, split-K over the
// context with a log-sum-exp merge.
//
// What is computed follows the "nano-vLLM learning note" Attention.forward
// decode branch and prepare_decode block (the query is the last token, at
// position context_len - 1, so it sees the whole context) and the
// "qwen-engine" README's note that decode is memory-bound: every key and
// value row of a request is read exactly once, and the kernels are sized so
// the HBM stream never stalls.
//
// Kernel 1 (split): one workgroup per (split, KV head, request).  A split is
// a run of keys_per_split consecutive keys; each of the four wavefronts of
// the workgroup takes every fourth 16-key group of the split (a group lies
// inside one page, page_size >= 16), and the wavefronts' partial softmax
// states are merged through LDS at the end.  With one split the result is
// final; otherwise (m, l, o) go to the workspace.
//   bf16: decode_mfma_kernel -- K/V tiles staged in LDS, QK^T and PV on
//         16x16 matrix cores with the G query heads of the KV head as the
//         N side.
//   fp32: decode_f32_kernel -- K/V rows streamed into registers, dot products
//         and PV on the vector ALUs.
//
// Kernel 2 (merge): one workgroup per (query head, request) combines the
// splits: m* = max m_s, l = sum 2^(m_s - m*) l_s, o = sum 2^(m_s - m*) o_s / l.
#include <type_traits>

#include "device_common.h"
#include "qil_internal.h"

namespace qil {
namespace {

constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// fp32 split kernel on the vector ALUs.
//
// Sixteen lanes own one key row: lane j holds elements 4j .. 4j+3 and
// 64+4j .. 64+4j+3 (two 16-byte loads, each instruction covering whole
// contiguous half rows), so one pair of load instructions moves four 512-byte
// rows.  The G query heads are dotted against each row, the partial dot
// products are summed across the 16 lanes by DPP, and each 16-lane row keeps
// its own online-softmax state (running max m, sum l, and its slice of o) in
// base 2; the four rows of a wavefront are merged with shuffles at the end.
constexpr int kFW = 4;             // wavefronts per workgroup
constexpr int kFKeysPerStep = 64;  // 4 wavefronts x 16 keys

__device__ __forceinline__ int f32_elem(int j, int e) {
  return e < 4 ? 4 * j + e : 64 + 4 * j + (e - 4);
}

struct RowF32 {
  uint4 a, b;
};

// Row data is streamed once per call: non-temporal loads, so it does not
// displace reusable lines from the caches.
__device__ __forceinline__ uint4 load_stream16(const char* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ RowF32 load_row_f32(const char* row, int j) {
  return RowF32{load_stream16(row + 16 * j), load_stream16(row + 256 + 16 * j)};
}

__device__ __forceinline__ void unpack_f32(const RowF32& c, float x[8]) {
  x[0] = __uint_as_float(c.a.x); x[1] = __uint_as_float(c.a.y);
  x[2] = __uint_as_float(c.a.z); x[3] = __uint_as_float(c.a.w);
  x[4] = __uint_as_float(c.b.x); x[5] = __uint_as_float(c.b.y);
  x[6] = __uint_as_float(c.b.z); x[7] = __uint_as_float(c.b.w);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Sum over the 16 lanes of a row with DPP: swap neighbours, swap pairs,
// mirror within 8, mirror within 16.  Every lane ends with the same sum.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);  // row_half_mirror
  x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}

template <int G>
__global__ __launch_bounds__(64 * kFW) void decode_f32_kernel(DecodeArgs a) {
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int r = blockIdx.z;
  const int L = min(a.context_lens[r], a.max_context_len);
  const int kbeg = split * a.keys_per_split;
  if (kbeg >= L) return;  // this split lies past the context (uniform per block)
  const int kend = min(L, kbeg + a.keys_per_split);

  const int tid = threadIdx.x;
  const int w = wave_uniform(tid >> 6);
  const int lane = tid & 63;
  const int row = lane >> 4;  // which of the 4 key rows of a load
  const int j = lane & 15;
  const int P = 1 << a.log2_page;
  constexpr int64_t row_bytes = kHeadDim * 4;

  // q of the G heads of this KV head, pre-scaled into the base-2 domain.
  const float qs = a.scale * kLog2e;
  float qf[G][8];
  {
    const char* qbase = static_cast<const char*>(a.q) +
                        ((int64_t)r * a.num_q_heads + (int64_t)g * G) * row_bytes;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const char* qr = qbase + h * row_bytes;
      const RowF32 c{*reinterpret_cast<const uint4*>(qr + 16 * j),
                     *reinterpret_cast<const uint4*>(qr + 256 + 16 * j)};
      unpack_f32(c, qf[h]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[h][e] *= qs;
    }
  }

  float m[G], l[G], o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  }

  const int32_t* bt_row = a.block_tables + (int64_t)r * a.bt_stride;
  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);

  // Group i of this wavefront covers keys kbeg + 64 i + 16 w .. +15, inside
  // one page.  Lane i holds the page id of group i (a split has at most 64
  // groups per wavefront), read into a scalar register when the group's loads
  // are issued, so no load waits on the block table inside the loop.
  const int first = kbeg + 16 * w;
  const int ngroups = first < kend ? (kend - first + kFKeysPerStep - 1) / kFKeysPerStep : 0;
  const int nfull = first + 16 <= kend ? (kend - first - 16) / kFKeysPerStep + 1 : 0;
  int page_of_lane = -1;
  if (lane < ngroups) page_of_lane = bt_row[(first + kFKeysPerStep * lane) >> a.log2_page];

  struct Group {
    RowF32 k[4], v[4];
    bool ok;
  };

  auto load_group = [&](auto full_tag, int i, Group& gr) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int key0 = first + kFKeysPerStep * i;
    const int page = __builtin_amdgcn_readlane(page_of_lane, i);
    gr.ok = (unsigned)page < (unsigned)a.num_pages;
    const int64_t row0 = ((int64_t)page * a.num_kv_heads + g) * P + (key0 & (P - 1));
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t off = (row0 + 4 * u + row) * row_bytes;
      const bool valid = gr.ok && (FULL || key0 + 4 * u + row < kend);
      if (FULL ? gr.ok : valid) {
        gr.k[u] = load_row_f32(kbase + off, j);
        gr.v[u] = load_row_f32(vbase + off, j);
      } else {
        gr.k[u].a = gr.k[u].b = gr.v[u].a = gr.v[u].b = make_uint4(0, 0, 0, 0);
      }
    }
  };

  auto compute_group = [&](auto full_tag, int i, const Group& gr) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int key0 = first + kFKeysPerStep * i;
    float s[4][G];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool valid = gr.ok && (FULL || key0 + 4 * u + row < kend);
      float kx[8];
      unpack_f32(gr.k[u], kx);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(qf[h][e], kx[e], acc);
        acc = row_sum16(acc);
        s[u][h] = valid ? acc : -INFINITY;
      }
    }
    float vx[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) unpack_f32(gr.v[u], vx[u]);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mt = fmaxf(fmaxf(m[h], fmaxf(s[0][h], s[1][h])), fmaxf(s[2][h], s[3][h]));
      const float corr = fast_exp2(m[h] - mt);
      m[h] = mt;
      float p[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) p[u] = fast_exp2(s[u][h] - mt);
      l[h] = fmaf(l[h], corr, (p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float acc = o[h][e] * corr;
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = fmaf(p[u], vx[u][e], acc);
        o[h][e] = acc;
      }
    }
  };

  // Full groups, two in flight: the next group's loads are issued before the
  // current group is computed.
  Group ga, gb;
  if (nfull > 0) load_group(std::true_type{}, 0, ga);
  for (int i = 0; i < nfull; i += 2) {
    if (i + 1 < nfull) load_group(std::true_type{}, i + 1, gb);
    compute_group(std::true_type{}, i, ga);
    if (i + 1 < nfull) {
      if (i + 2 < nfull) load_group(std::true_type{}, i + 2, ga);
      compute_group(std::true_type{}, i + 1, gb);
    }
  }
  if (ngroups > nfull) {  // the context ends inside this wavefront's last group
    load_group(std::false_type{}, nfull, ga);
    compute_group(std::false_type{}, nfull, ga);
  }

  // Merge the 4 rows of this wavefront (lanes 16 and 32 apart).
#pragma unroll
  for (int step = 16; step <= 32; step <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], step);
      const float lo = __shfl_xor(l[h], step);
      const float mn = fmaxf(m[h], mo);
      const float fa = fast_exp2(m[h] - mn);
      const float fb = fast_exp2(mo - mn);
      l[h] = l[h] * fa + lo * fb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float oo = __shfl_xor(o[h][e], step);
        o[h][e] = o[h][e] * fa + oo * fb;
      }
      m[h] = mn;
    }
  }

  // Merge the 4 wavefronts through LDS.
  __shared__ float sh_o[kFW][G][kHeadDim];
  __shared__ float sh_m[kFW][G];
  __shared__ float sh_l[kFW][G];
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sh_o[w][h][f32_elem(j, e)] = o[h][e];
      if (j == 0) {
        sh_m[w][h] = m[h];
        sh_l[w][h] = l[h];
      }
    }
  }
  __syncthreads();

  const bool single = a.num_splits == 1;
  for (int idx = tid; idx < G * kHeadDim; idx += 64 * kFW) {
    const int h = idx / kHeadDim;
    const int d = idx % kHeadDim;
    float mx = sh_m[0][h];
#pragma unroll
    for (int ww = 1; ww < kFW; ++ww) mx = fmaxf(mx, sh_m[ww][h]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int ww = 0; ww < kFW; ++ww) {
      const float f = fast_exp2(sh_m[ww][h] - mx);
      acc = fmaf(f, sh_o[ww][h][d], acc);
      lsum = fmaf(f, sh_l[ww][h], lsum);
    }
    const int qh = g * G + h;
    if (single) {
      const float val = lsum > 0.f ? acc / lsum : 0.f;
      static_cast<float*>(a.out)[((int64_t)r * a.num_q_heads + qh) * kHeadDim + d] = val;
    } else {
      const int64_t pi = ((int64_t)r * a.num_q_heads + qh) * a.num_splits + split;
      a.ws_o[pi * kHeadDim + d] = acc;
      if (d == 0) {
        a.ws_m[pi] = mx;
        a.ws_l[pi] = lsum;
      }
    }
  }
}

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
constexpr int kMW = 4;               // wavefronts per workgroup
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

template <int G>
__global__ __launch_bounds__(64 * kMW) void decode_mfma_kernel(DecodeArgs a) {
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int r = blockIdx.z;
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

  // Each wavefront's ring: [slot][K | V][16 rows x 256 bytes].
  __shared__ __attribute__((aligned(1024))) char smem[kMW][kMD][2][kTile];
  char* ring = &smem[w][0][0][0];

  const int32_t* bt_row = a.block_tables + (int64_t)r * a.bt_stride;
  const char* kpool = static_cast<const char*>(a.k_cache);
  const char* vpool = static_cast<const char*>(a.v_cache);
  // Group i of this wavefront: keys first + 16 kMW i .. +15 (inside one page).
  const int first = kbeg + 16 * w;
  const int ngroups = first < kend ? (kend - first + 16 * kMW - 1) / (16 * kMW) : 0;
  int page_of_lane = -1;
  if (lane < ngroups) page_of_lane = bt_row[(first + 16 * kMW * lane) >> a.log2_page];

  // Issue the 8 tile loads of group i into slot i % kMD.  Every lane always
  // loads (rows past the context re-read the group's first row, and a page
  // id out of range reads page 0), so each group is exactly 8 vector-memory
  // instructions and the ring can be waited on by count.
  const int lrow = lane >> 4;  // row within a 4-row load
  const int lpc = lane & 15;   // physical chunk this lane fills
  auto issue = [&](int i) __attribute__((always_inline)) {
    const int key0 = first + 16 * kMW * i;
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
    const int kb = first + 16 * kMW * i + 4 * q4;
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
  for (int i = 0; i < ngroups; ++i) {
    // refill the slot computed at i - 1 (its LDS reads are complete), then
    // wait until group i has landed: the groups issued after it may still fly
    if (i + kMD - 1 < ngroups) issue(i + kMD - 1);
    const int ahead = min(ngroups - 1 - i, kMD - 1);
    if (kMD > 3 && ahead >= 3) wait_vmcnt<24>();
    else if (kMD > 2 && ahead == 2) wait_vmcnt<16>();
    else if (ahead == 1) wait_vmcnt<8>();
    else wait_vmcnt<0>();
    compute(i);
  }
  static_assert(kMD >= 2 && kMD <= 4, "the wait ladder above covers 1 to 3 groups in flight");

  // Row sums over the four lanes of each head.
  lsum = swap_sum32(swap_sum16(lsum));

  // Merge the kMW wavefronts through LDS (the ring is free now).
  __syncthreads();
  float* sh_o = reinterpret_cast<float*>(&smem[0][0][0][0]);   // [kMW][G][128]
  float* sh_m = sh_o + kMW * G * kHeadDim;                      // [kMW][G]
  float* sh_l = sh_m + kMW * G;                                 // [kMW][G]
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
  for (int idx = tid; idx < G * kHeadDim; idx += 64 * kMW) {
    const int h = idx / kHeadDim;
    const int d = idx % kHeadDim;
    float mx = sh_m[h];
#pragma unroll
    for (int ww = 1; ww < kMW; ++ww) mx = fmaxf(mx, sh_m[ww * G + h]);
    float acc = 0.f, ls = 0.f;
#pragma unroll
    for (int ww = 0; ww < kMW; ++ww) {
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

template <bool BF16>
__global__ __launch_bounds__(128) void decode_merge_kernel(DecodeArgs a) {
  const int qh = blockIdx.x;
  const int r = blockIdx.y;
  const int d = threadIdx.x;
  const int L = min(a.context_lens[r], a.max_context_len);
  int n = (L + a.keys_per_split - 1) / a.keys_per_split;
  n = n < 0 ? 0 : (n > a.num_splits ? a.num_splits : n);
  const int64_t base = ((int64_t)r * a.num_q_heads + qh) * a.num_splits;
  float mx = kNegBig;
  for (int s = 0; s < n; ++s) mx = fmaxf(mx, a.ws_m[base + s]);
  float acc = 0.f, lsum = 0.f;
  for (int s = 0; s < n; ++s) {
    const float f = fast_exp2(a.ws_m[base + s] - mx);
    lsum = fmaf(f, a.ws_l[base + s], lsum);
    acc = fmaf(f, a.ws_o[(base + s) * kHeadDim + d], acc);
  }
  const float val = lsum > 0.f ? acc / lsum : 0.f;
  const int64_t oi = ((int64_t)r * a.num_q_heads + qh) * kHeadDim + d;
  if (BF16)
    static_cast<uint16_t*>(a.out)[oi] = (uint16_t)f32_to_bf16_bits(val);
  else
    static_cast<float*>(a.out)[oi] = val;
}

template <int G, bool BF16>
hipError_t launch_g(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.num_splits, a.num_kv_heads, a.batch);
  if constexpr (BF16)
    hipLaunchKernelGGL((decode_mfma_kernel<G>), grid, dim3(64 * kMW), 0, s, a);
  else
    hipLaunchKernelGGL((decode_f32_kernel<G>), grid, dim3(64 * kFW), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_splits == 1) return e;
  hipLaunchKernelGGL((decode_merge_kernel<BF16>), dim3(a.num_q_heads, a.batch), dim3(128), 0, s, a);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dtype(const DecodeArgs& a, hipStream_t s) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_g<1, BF16>(a, s);
    case 2: return launch_g<2, BF16>(a, s);
    case 4: return launch_g<4, BF16>(a, s);
    case 8: return launch_g<8, BF16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  return a.bf16 ? launch_dtype<true>(a, s) : launch_dtype<false>(a, s);
}

}  // namespace qil
