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

#include "decode_body.h"

namespace qil {
namespace {
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

template <int G>
__global__ __launch_bounds__(64 * kFW) void decode_f32_kernel(DecodeArgs a) {
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  // z: the q / out row; r: the request whose block table and context it reads
  const int z = a.order != nullptr ? a.order[blockIdx.z] : (int)blockIdx.z;
  int r = z, L;
  if (a.cu_seqlens != nullptr) {
    // fp32 prefill: the last request whose rows start at or before z owns it
    // (cu_seqlens is non-decreasing, so empty requests are passed over)
    int lo = 0, hi = a.prefill_requests;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.cu_seqlens[mid] <= z) lo = mid;
      else hi = mid;
    }
    r = lo;
    const int n = a.cu_seqlens[r + 1] - a.cu_seqlens[r];
    L = min(min(a.context_lens[r], a.max_context_len) - n + (z - a.cu_seqlens[r]) + 1,
            a.max_context_len);
  } else {
    L = min(a.context_lens[r], a.max_context_len);
  }
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
                        ((int64_t)z * a.num_q_heads + (int64_t)g * G) * row_bytes;
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
      static_cast<float*>(a.out)[((int64_t)z * a.num_q_heads + qh) * kHeadDim + d] = val;
    } else {
      const int64_t pi = ((int64_t)z * a.num_q_heads + qh) * a.num_splits + split;
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

// Longest requests first.  Workgroups are dispatched in grid order, and when
// the grid takes several rounds of the GPU, a long context started last
// leaves the GPU idle around it while it finishes.  One workgroup sorts the
// requests into 256 buckets of decreasing context length (counting sort with
// LDS atomics; the order inside a bucket does not matter, since every
// request's result is independent of which workgroup computes it) and
// writes the permutation that the decode grid reads its request ids through.
// The bf16 kernel ranks batches of up to 256 requests itself
// (decode_rank_request) and skips this launch.
constexpr int kOrderBuckets = 256;
constexpr int kOrderThreads = 1024;

__global__ __launch_bounds__(kOrderThreads) void decode_order_kernel(const int32_t* context_lens,
                                                                     int batch, int max_len,
                                                                     int32_t* order) {
  static_assert(kOrderBuckets == 4 * 64, "four wavefronts scan the buckets");
  constexpr int kHeld = 4;  // requests per thread whose bucket stays in a register
  __shared__ int hist[kOrderBuckets];
  __shared__ int wave_sum[kOrderBuckets / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  auto bucket = [&](int r) {
    int L = context_lens[r];
    L = L < 0 ? 0 : (L > max_len ? max_len : L);
    return (int)((int64_t)(max_len - L) * kOrderBuckets / ((int64_t)max_len + 1));  // 0 = longest
  };
  if (tid < kOrderBuckets) hist[tid] = 0;
  // the first kHeld requests of each thread: one round of loads, kept
  int held[kHeld];
#pragma unroll
  for (int k = 0; k < kHeld; ++k) {
    const int r = tid + k * kOrderThreads;
    held[k] = r < batch ? bucket(r) : 0;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kHeld; ++k)
    if (tid + k * kOrderThreads < batch) atomicAdd(&hist[held[k]], 1);
  for (int r = tid + kHeld * kOrderThreads; r < batch; r += kOrderThreads)
    atomicAdd(&hist[bucket(r)], 1);
  __syncthreads();
  // first free position of each bucket: exclusive scan, a wavefront per 64 buckets
  int own = 0, v = 0;
  if (tid < kOrderBuckets) {
    own = v = hist[tid];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(v, o);
      if (lane >= o) v += t;
    }
    if (lane == 63) wave_sum[wv] = v;
  }
  __syncthreads();
  if (tid < kOrderBuckets) {
    int before = 0;
    for (int i = 0; i < wv; ++i) before += wave_sum[i];
    hist[tid] = before + v - own;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kHeld; ++k) {
    const int r = tid + k * kOrderThreads;
    if (r < batch) order[atomicAdd(&hist[held[k]], 1)] = r;
  }
  for (int r = tid + kHeld * kOrderThreads; r < batch; r += kOrderThreads)
    order[atomicAdd(&hist[bucket(r)], 1)] = r;
}

template <int G, bool BF16>
hipError_t launch_g(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.num_splits, a.num_kv_heads, a.batch);
  if constexpr (BF16) {
    if (a.order != nullptr && a.batch <= kRankMaxBatch) {
      // the workgroups rank the batch themselves: no ordering launch
      DecodeArgs ai = a;
      ai.rank_inline = true;
      hipLaunchKernelGGL((decode_mfma_kernel<G>), grid, dim3(64 * kMW), 0, s, ai);
    } else {
      hipError_t e = launch_decode_order(a, s);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((decode_mfma_kernel<G>), grid, dim3(64 * kMW), 0, s, a);
    }
  } else {
    hipError_t e = launch_decode_order(a, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_f32_kernel<G>), grid, dim3(64 * kFW), 0, s, a);
  }
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
    case 5: return launch_g<5, BF16>(a, s);
    case 8: return launch_g<8, BF16>(a, s);
    case 16:
      if constexpr (BF16) return launch_g<16, true>(a, s);
      return hipErrorInvalidValue;  // fp32 is built up to G = 8 (validated before)
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_order(const DecodeArgs& a, hipStream_t s) {
  if (a.order == nullptr || a.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_order_kernel, dim3(1), dim3(kOrderThreads), 0, s, a.context_lens,
                     a.batch, a.max_context_len, a.order);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  return a.bf16 ? launch_dtype<true>(a, s) : launch_dtype<false>(a, s);
}

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t s) {
  if (a.num_splits <= 1) return hipSuccess;
  if (a.bf16)
    hipLaunchKernelGGL((decode_merge_kernel<true>), dim3(a.num_q_heads, a.batch), dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL((decode_merge_kernel<false>), dim3(a.num_q_heads, a.batch), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace qil
