// Paged decode attention: one query token per request, GQA, split-K over the
// context with a log-sum-exp merge.
//
// What is computed follows the "nano-vLLM learning note" Attention.forward
// decode branch and prepare_decode block (the query is the last token, at
// position context_len - 1, so it sees the whole context) and the
// "qwen-engine" README's note that decode is memory-bound: every key and
// value row of a request is read exactly once, and the kernel is sized so the
// HBM stream never stalls.
//
// Kernel 1 (split): one workgroup per (split, KV head, request).  A split is
// a run of keys_per_split consecutive keys.  The four wavefronts of the
// workgroup stream 64 keys per step: wavefront w takes keys [16w, 16w+16) of
// the step, all inside one page (page_size >= 16), so its page id is one
// scalar load.  Sixteen lanes own one key row (16 bytes each, so one load
// instruction moves four whole 256-byte bf16 rows), the G query heads of the
// KV head are dotted against it and the partial dot products are summed
// across the 16 lanes.  Each 16-lane row keeps its own online-softmax state
// (running max m, sum l, and its slice of o) in base 2; the four rows of a
// wavefront are merged with cross-lane shuffles at the end and the four
// wavefronts through LDS.  With one split the result is final; otherwise
// (m, l, o) go to the workspace.
//
// Kernel 2 (merge): one workgroup per (query head, request) combines the
// splits: m* = max m_s, l = sum 2^(m_s - m*) l_s, o = sum 2^(m_s - m*) o_s / l.
#include <type_traits>

#include "device_common.h"
#include "qil_internal.h"

namespace qil {
namespace {

constexpr int kWaves = 4;
constexpr int kKeysPerStep = 64;  // 4 wavefronts x 16 keys
constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima

// Element of the 128-wide row held in slot e (0..7) of lane j (0..15).
// bf16: one 16-byte load per lane -> elements 8j .. 8j+7.
// fp32: two 16-byte loads per lane, each instruction covering one contiguous
//       half row -> elements 4j .. 4j+3 and 64+4j .. 64+4j+3.
template <bool BF16>
__device__ __forceinline__ int elem_of(int j, int e) {
  if (BF16) return 8 * j + e;
  return e < 4 ? 4 * j + e : 64 + 4 * j + (e - 4);
}

template <bool BF16>
struct RowChunk {
  uint4 a, b;  // b unused for bf16
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load; K/V rows are streamed once per call, so they are loaded
// non-temporally (they should not displace reusable lines from the caches).
template <bool NT>
__device__ __forceinline__ uint4 load16(const char* p) {
  if (NT) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  }
  return *reinterpret_cast<const uint4*>(p);
}

template <bool BF16, bool NT = false>
__device__ __forceinline__ RowChunk<BF16> load_chunk(const char* row, int j) {
  RowChunk<BF16> c;
  if (BF16) {
    c.a = load16<NT>(row + 16 * j);
    c.b = make_uint4(0, 0, 0, 0);
  } else {
    c.a = load16<NT>(row + 16 * j);
    c.b = load16<NT>(row + 256 + 16 * j);
  }
  return c;
}

template <bool BF16>
__device__ __forceinline__ void unpack(const RowChunk<BF16>& c, float x[8]) {
  if (BF16) {
    const uint32_t w[4] = {c.a.x, c.a.y, c.a.z, c.a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(w[i]);
      x[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    x[0] = __uint_as_float(c.a.x); x[1] = __uint_as_float(c.a.y);
    x[2] = __uint_as_float(c.a.z); x[3] = __uint_as_float(c.a.w);
    x[4] = __uint_as_float(c.b.x); x[5] = __uint_as_float(c.b.y);
    x[6] = __uint_as_float(c.b.z); x[7] = __uint_as_float(c.b.w);
  }
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

// Partial dot product of this lane's 8 elements of q and k.
template <bool BF16>
__device__ __forceinline__ float dot8(const uint32_t qraw[4], const float qf[8],
                                      const RowChunk<BF16>& k) {
  if (BF16) {
    const uint32_t kw[4] = {k.a.x, k.a.y, k.a.z, k.a.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qraw[i]),
                                            __builtin_bit_cast(bf16x2_t, kw[i]), acc, false);
    return acc;
  } else {
    float kx[8];
    unpack<BF16>(k, kx);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(qf[e], kx[e], acc);
    return acc;
  }
}

template <int G, bool BF16>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
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
  const int eb = BF16 ? 2 : 4;
  const int64_t row_bytes = (int64_t)kHeadDim * eb;

  // q of the G heads of this KV head.  bf16: raw pairs for v_dot2 and the
  // scale (into the base-2 domain) applied to the score; fp32: pre-scaled.
  const float qs = a.scale * kLog2e;
  uint32_t qraw[G][4];
  float qf[G][8];
  {
    const char* qbase = static_cast<const char*>(a.q) +
                        ((int64_t)r * a.num_q_heads + (int64_t)g * G) * row_bytes;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      RowChunk<BF16> c = load_chunk<BF16>(qbase + h * row_bytes, j);
      qraw[h][0] = c.a.x; qraw[h][1] = c.a.y; qraw[h][2] = c.a.z; qraw[h][3] = c.a.w;
      unpack<BF16>(c, qf[h]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[h][e] *= qs;
    }
  }
  const float score_scale = BF16 ? qs : 1.0f;

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
  const int ngroups = first < kend ? (kend - first + kKeysPerStep - 1) / kKeysPerStep : 0;
  const int nfull = first + 16 <= kend ? (kend - first - 16) / kKeysPerStep + 1 : 0;
  int page_of_lane = -1;
  if (lane < ngroups) page_of_lane = bt_row[(first + kKeysPerStep * lane) >> a.log2_page];

  struct Group {
    RowChunk<BF16> k[4], v[4];
    bool ok;
  };

  auto load_group = [&](auto full_tag, int i, Group& gr) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int key0 = first + kKeysPerStep * i;
    const int page = __builtin_amdgcn_readlane(page_of_lane, i);
    gr.ok = (unsigned)page < (unsigned)a.num_pages;
    const int64_t row0 = ((int64_t)page * a.num_kv_heads + g) * P + (key0 & (P - 1));
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t off = (row0 + 4 * u + row) * row_bytes;
      const bool valid = gr.ok && (FULL || key0 + 4 * u + row < kend);
      if (FULL ? gr.ok : valid) {
        gr.k[u] = load_chunk<BF16, true>(kbase + off, j);
        gr.v[u] = load_chunk<BF16, true>(vbase + off, j);
      } else {
        gr.k[u].a = gr.k[u].b = gr.v[u].a = gr.v[u].b = make_uint4(0, 0, 0, 0);
      }
    }
  };

  auto compute_group = [&](auto full_tag, int i, const Group& gr) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int key0 = first + kKeysPerStep * i;
    float s[4][G];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool valid = gr.ok && (FULL || key0 + 4 * u + row < kend);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float acc = row_sum16(dot8<BF16>(qraw[h], qf[h], gr.k[u])) * score_scale;
        s[u][h] = valid ? acc : -INFINITY;
      }
    }
    float vx[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) unpack<BF16>(gr.v[u], vx[u]);
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
  __shared__ float sh_o[kWaves][G][kHeadDim];
  __shared__ float sh_m[kWaves][G];
  __shared__ float sh_l[kWaves][G];
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sh_o[w][h][elem_of<BF16>(j, e)] = o[h][e];
      if (j == 0) {
        sh_m[w][h] = m[h];
        sh_l[w][h] = l[h];
      }
    }
  }
  __syncthreads();

  const bool single = a.num_splits == 1;
  for (int idx = tid; idx < G * kHeadDim; idx += 256) {
    const int h = idx / kHeadDim;
    const int d = idx % kHeadDim;
    float mx = sh_m[0][h];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) mx = fmaxf(mx, sh_m[ww][h]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = fast_exp2(sh_m[ww][h] - mx);
      acc = fmaf(f, sh_o[ww][h][d], acc);
      lsum = fmaf(f, sh_l[ww][h], lsum);
    }
    const int qh = g * G + h;
    if (single) {
      const float val = lsum > 0.f ? acc / lsum : 0.f;
      const int64_t oi = ((int64_t)r * a.num_q_heads + qh) * kHeadDim + d;
      if (BF16)
        static_cast<uint16_t*>(a.out)[oi] = (uint16_t)f32_to_bf16_bits(val);
      else
        static_cast<float*>(a.out)[oi] = val;
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
  hipLaunchKernelGGL((decode_split_kernel<G, BF16>), grid, dim3(256), 0, s, a);
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
