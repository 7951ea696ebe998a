// Merged QKV projection with the per-head Q/K RMSNorm, RoPE and KV scatter
// as its epilogue, on bf16 matrix cores.
//
// What is computed follows the "nano-vLLM learning note": the
// QKVParallelLinear block (one linear layer whose output columns are all q
// heads, then all k heads, then all v heads, head_size each) and the
// Qwen3Attention.forward block (project, split per head, q_norm / k_norm,
// rotary_emb, then the attention step that stores k and v).  The projection
// is an nn.Linear without bias: qkv[t][n] = sum_k x[t][k] w[n][k], rounded to
// bf16 as the layer's output; the epilogue then applies the same arithmetic
// as the fused qil_kv_write to those rounded rows.
//
// Work split: one workgroup (4 wavefronts) owns 128 tokens x 2 output heads
// (256 weight rows).  Each wavefront owns one head (128 columns) x 64 tokens
// and computes the transposed block C^T = W X^T on v_mfma_f32_32x32x16_bf16
// with the head's columns on the M side and tokens on the N side.  That
// puts one token per lane and, for each lane, 64 of the head's 128 values
// (the other 64 sit in lane l ^ 32): the RMSNorm sum of squares closes with
// one cross-half swap, and a value's RoPE partner (column + 64) sits in the
// same lane, two 32-row blocks further on.
//
//   * Both operands are K-contiguous (x rows and nn.Linear weight rows), so
//     64-value slices of rows go from memory straight into LDS with
//     global_load_lds (16 bytes per lane), 16-byte chunks XOR-swizzled per
//     row so that 16 lanes reading one chunk column hit 16 distinct bank
//     groups.  A three-stage ring keeps two slices in flight while one is
//     multiplied; one barrier per slice.
//   * Workgroups are numbered head pair fastest.  They are dealt to the 8
//     XCDs round robin, so with a multiple of 8 head pairs each XCD always
//     serves the same head pairs and streams their weight rows through its
//     own L2, while every XCD reads all activations.
#include "device_common.h"
#include "qil_internal.h"

namespace qil {
namespace {

constexpr int kPK = 64;                    // hidden values per stage
constexpr int kPRowBytes = kPK * 2;        // 128-byte LDS rows
constexpr int kPTok = 128;                 // tokens per workgroup
constexpr int kPCols = 2 * kHeadDim;       // weight rows (output columns) per workgroup
constexpr int kPThreads = 256;
constexpr int kPStages = 3;
constexpr int kPWInstr = kPCols * kPRowBytes / 1024 / 4;  // 1-KB weight loads per wave per stage
constexpr int kPXInstr = kPTok * kPRowBytes / 1024 / 4;   // 1-KB activation loads per wave per stage

struct ProjLds {
  char w[kPStages][kPCols * kPRowBytes];
  char x[kPStages][kPTok * kPRowBytes];
};

typedef __attribute__((address_space(3))) char lds_char;

// Physical 16-byte chunk of logical chunk c in an LDS row: XOR with bits
// 1..3 of the row, so rows r .. r+15 put one logical chunk in 16 distinct
// 16-byte bank groups (two rows per 256 bytes, eight chunk positions).
__device__ __forceinline__ int pswz(int row, int c) { return c ^ ((row >> 1) & 7); }

template <int N>
__device__ __forceinline__ void proj_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ float sum_halves32(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

__global__ __launch_bounds__(kPThreads) void qkv_proj_kernel(QkvProjArgs a) {
  __shared__ __attribute__((aligned(1024))) ProjLds lds;

  const int tid = threadIdx.x;
  const int w = wave_uniform(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int hf = lane >> 5;
  const int pair = blockIdx.x;
  const int t0 = blockIdx.y * kPTok;
  const int n0 = pair * kPCols;  // first weight row of the workgroup
  const int T = a.num_tokens;
  const int nst = a.hidden / kPK;

  const char* xg = static_cast<const char*>(a.x);
  const char* wg = static_cast<const char*>(a.weight);

  // Loader role: 1-KB blocks of 8 LDS rows; lane l lands at byte 16 l of
  // the block, i.e. row 8 b + l/8, physical chunk l%8, so it fetches the
  // logical chunk that the swizzle puts there.
  const int lrow = lane >> 3;
  const int lpc = lane & 7;
  auto issue = [&](int st) __attribute__((always_inline)) {
    const int buf = st % kPStages;
    const int64_t kofs = (int64_t)st * kPRowBytes;
#pragma unroll
    for (int i = 0; i < kPWInstr; ++i) {
      const int blk = kPWInstr * w + i;
      const int row = 8 * blk + lrow;
      const char* src = wg + (int64_t)(n0 + row) * a.weight_stride * 2 + kofs + 16 * pswz(row, lpc);
      __builtin_amdgcn_global_load_lds(src, (lds_char*)&lds.w[buf][blk * 1024], 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kPXInstr; ++i) {
      const int blk = kPXInstr * w + i;
      const int row = 8 * blk + lrow;
      const int tok = min(t0 + row, T - 1);  // rows past the last token repeat it (never stored)
      const char* src = xg + (int64_t)tok * a.x_stride * 2 + kofs + 16 * pswz(row, lpc);
      __builtin_amdgcn_global_load_lds(src, (lds_char*)&lds.x[buf][blk * 1024], 16, 0, 0);
    }
  };

  f32x16_t acc[2][4];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[nb][mb][v] = 0.f;

  // Operand rows of this wavefront: weight rows 128 (w & 1) + 32 mb + lq
  // (its head), activation rows 64 (w >> 1) + 32 nb + lq (its tokens).  The
  // bases are multiples of 16, so every row's swizzle term is (lq >> 1) & 7.
  const int wrow0 = kHeadDim * (w & 1);
  const int xrow0 = 64 * (w >> 1);
  const int sw = (lq >> 1) & 7;
  auto compute = [&](int st) __attribute__((always_inline)) {
    const int buf = st % kPStages;
    const char* wb = &lds.w[buf][0] + (wrow0 + lq) * kPRowBytes;
    const char* xb = &lds.x[buf][0] + (xrow0 + lq) * kPRowBytes;
#pragma unroll
    for (int kk = 0; kk < kPK / 16; ++kk) {
      // lanes 0-31 take k 16kk .. +7, lanes 32-63 k 16kk+8 .. +15
      const int pc = 16 * ((2 * kk + hf) ^ sw);
      bf16x8_t av[4], bv[2];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        av[mb] = *reinterpret_cast<const bf16x8_t*>(wb + 32 * mb * kPRowBytes + pc);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        bv[nb] = *reinterpret_cast<const bf16x8_t*>(xb + 32 * nb * kPRowBytes + pc);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mb], bv[nb], acc[nb][mb], 0, 0, 0);
    }
  };

  // Ring: stage s sits in buffer s % 3.  At the top of iteration s the
  // wavefront's own loads of stage s are waited for (stage s+1 may stay in
  // flight), the barrier publishes everyone's, and also marks that every
  // wavefront has finished reading buffer (s-1) % 3, which stage s+2 refills.
  constexpr int kPer = kPWInstr + kPXInstr;
  issue(0);
  if (nst > 1) issue(1);
  for (int s = 0; s < nst; ++s) {
    if (s + 1 < nst) proj_wait_vmcnt<kPer>();
    else proj_wait_vmcnt<0>();
    // a bare barrier: __syncthreads() would also drain the stage still in flight
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (s + 2 < nst) issue(s + 2);
    compute(s);
  }

  // ---- epilogue ---------------------------------------------------------
  // acc[nb][mb][v] is column 32 mb + 8 (v/4) + 4 hf + v%4 of this wave's head
  // for token t0 + 64 (w >> 1) + 32 nb + lq.
  const int head = 2 * pair + (w & 1);
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int kind = head < Hq ? 0 : (head < Hq + Hkv ? 1 : 2);  // q, k, v
  const int hidx = kind == 0 ? head : (kind == 1 ? head - Hq : head - Hq - Hkv);
  const int ncols = (Hq + 2 * Hkv) * kHeadDim;
  const int P = 1 << a.log2_page;

#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int t = t0 + xrow0 + 32 * nb + lq;
    const bool tv = t < T;
    // the projection rounded to bf16, two columns per word
    uint32_t px[4][8];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 8; ++i) px[mb][i] = cvt_pk_bf16(acc[nb][mb][2 * i], acc[nb][mb][2 * i + 1]);

    if (a.qkv_out != nullptr && tv) {
      uint16_t* orow = static_cast<uint16_t*>(a.qkv_out) + (int64_t)t * ncols + head * kHeadDim;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<uint2*>(orow + 32 * mb + 8 * j + 4 * hf) =
              make_uint2(px[mb][2 * j], px[mb][2 * j + 1]);
    }

    int32_t slot = -1;
    if (tv && kind != 0) slot = a.slots[t];
    const int64_t page = slot >> a.log2_page;
    const bool store_kv = slot >= 0 && page < a.num_pages;
    const int64_t dst_row = ((page * Hkv + hidx) << a.log2_page) + (slot & (P - 1));

    if (kind == 2) {  // v: the rounded projection as it is
      if (store_kv) {
        uint16_t* vrow = static_cast<uint16_t*>(a.v_cache) + dst_row * kHeadDim;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *reinterpret_cast<uint2*>(vrow + 32 * mb + 8 * j + 4 * hf) =
                make_uint2(px[mb][2 * j], px[mb][2 * j + 1]);
      }
      continue;
    }

    // q / k: RMSNorm over the head's 128 values, then RoPE
    float ss = 0.f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float lo = bf16_lo(px[mb][i]), hi = bf16_hi(px[mb][i]);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
      }
    ss = sum_halves32(ss);
    const float inv_rms = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + a.eps);

    const uint16_t* nw = static_cast<const uint16_t*>(kind == 0 ? a.q_w : a.k_w);
    float y[4][16];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint2 wv = *reinterpret_cast<const uint2*>(nw + 32 * mb + 8 * j + 4 * hf);
        const uint32_t ww[2] = {wv.x, wv.y};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t xw = px[mb][2 * j + h];
          // bf16(x * r), then bf16(that * w)
          const uint32_t nrm = cvt_pk_bf16(bf16_lo(xw) * inv_rms, bf16_hi(xw) * inv_rms);
          const uint32_t m = cvt_pk_bf16(bf16_lo(nrm) * bf16_lo(ww[h]), bf16_hi(nrm) * bf16_hi(ww[h]));
          y[mb][4 * j + 2 * h] = bf16_lo(m);
          y[mb][4 * j + 2 * h + 1] = bf16_hi(m);
        }
      }

    int pos = tv ? a.positions[t] : 0;
    pos = pos < 0 ? 0 : (pos >= a.max_position ? a.max_position - 1 : pos);
    const float* cs = a.cos_sin + (int64_t)pos * kHeadDim;
    uint32_t po[4][8];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * mb + 8 * j + 4 * hf;  // < 64; its partner is d0 + 64 (block mb + 2)
        const float4 c4 = *reinterpret_cast<const float4*>(cs + d0);
        const float4 s4 = *reinterpret_cast<const float4*>(cs + kHeadDim / 2 + d0);
        const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
        const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
        float o1[4], o2[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float y1 = y[mb][4 * j + e], y2 = y[mb + 2][4 * j + e];
          o1[e] = y1 * cv[e] - y2 * sv[e];
          o2[e] = y2 * cv[e] + y1 * sv[e];
        }
        po[mb][2 * j] = cvt_pk_bf16(o1[0], o1[1]);
        po[mb][2 * j + 1] = cvt_pk_bf16(o1[2], o1[3]);
        po[mb + 2][2 * j] = cvt_pk_bf16(o2[0], o2[1]);
        po[mb + 2][2 * j + 1] = cvt_pk_bf16(o2[2], o2[3]);
      }

    uint16_t* drow = nullptr;
    if (kind == 0) {
      if (tv) drow = static_cast<uint16_t*>(a.q_out) + ((int64_t)t * Hq + hidx) * kHeadDim;
    } else if (store_kv) {
      drow = static_cast<uint16_t*>(a.k_cache) + dst_row * kHeadDim;
    }
    if (drow != nullptr) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<uint2*>(drow + 32 * mb + 8 * j + 4 * hf) =
              make_uint2(po[mb][2 * j], po[mb][2 * j + 1]);
    }
  }
}

}  // namespace

hipError_t launch_qkv_proj(const QkvProjArgs& a, hipStream_t s) {
  const int heads = a.num_q_heads + 2 * a.num_kv_heads;
  if (a.num_tokens == 0) return hipSuccess;
  dim3 grid(heads / 2, (a.num_tokens + kPTok - 1) / kPTok);
  hipLaunchKernelGGL(qkv_proj_kernel, grid, dim3(kPThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace qil
