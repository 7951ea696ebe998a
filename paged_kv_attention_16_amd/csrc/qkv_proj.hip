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
// Work split: a workgroup owns 2 output heads (256 weight rows) and 64 TG
// tokens, one wavefront per (head, 64 tokens): TG = 4 (256 tokens, 8
// wavefronts) for large batches, TG = 2 (128 tokens, 4 wavefronts) for
// small ones.  Each wavefront computes the transposed block C^T = W X^T on
// v_mfma_f32_32x32x16_bf16 with the head's columns on the M side and tokens
// on the N side.  That puts one token per lane and, for each lane, 64 of the
// head's 128 values (the other 64 sit in lane l ^ 32): the RMSNorm sum of
// squares closes with one cross-half swap, and a value's RoPE partner
// (column + 64) sits in the same lane, two 32-row blocks further on.
//
//   * Both operands are K-contiguous (x rows and nn.Linear weight rows), so
//     64-value slices of rows go from memory straight into LDS with
//     global_load_lds (16 bytes per lane), 16-byte chunks XOR-swizzled per
//     row so that 16 lanes reading one chunk column hit 16 distinct bank
//     groups.  A ring of three (TG = 2) or two (TG = 4) slices keeps the next
//     slices in flight while one is multiplied; one barrier per slice.
//   * The slice's LDS reads are inline assembly with counted waits, so the
//     next k-step's operands are read while the current k-step's matrix
//     instructions run.
//   * The epilogue stages through LDS: the cos / sin rows of the
//     workgroup's tokens arrive by coalesced DMA, and each wavefront's output
//     rows leave as whole 256-byte rows.
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
constexpr int kPCols = 2 * kHeadDim;       // weight rows (output columns) per workgroup

// Workgroup shapes: TG groups of 64 tokens x 2 heads, one wavefront per
// (head, token group).  TG = 2: 128 tokens, 4 wavefronts, a three-stage
// ring (144 KB of LDS); TG = 4: 256 tokens, 8 wavefronts, two stages (128 KB),
// a third fewer operand bytes per flop for large batches.
template <int TG>
struct ProjCfg {
  static constexpr int kTok = 64 * TG;
  static constexpr int kWaves = 2 * TG;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kStages = TG == 2 ? 3 : 2;
  static constexpr int kWInstr = kPCols * kPRowBytes / 1024 / kWaves;  // 1-KB weight loads per wave per stage
  static constexpr int kXInstr = kTok * kPRowBytes / 1024 / kWaves;    // 1-KB activation loads per wave per stage
  static_assert(kWInstr * kWaves * 1024 == kPCols * kPRowBytes, "weight rows split evenly");
  static_assert(kXInstr * kWaves * 1024 == kTok * kPRowBytes, "activation rows split evenly");
};

template <int TG>
struct ProjLds {
  char w[ProjCfg<TG>::kStages][kPCols * kPRowBytes];
  char x[ProjCfg<TG>::kStages][ProjCfg<TG>::kTok * kPRowBytes];
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

// SPLIT: the workgroup covers the hidden slices of split blockIdx.z only and
// writes its fp32 partial sums to a.partials; qkv_proj_reduce_kernel adds the
// splits and applies the epilogue.
template <int TG, bool SPLIT>
__global__ __launch_bounds__(ProjCfg<TG>::kThreads) void qkv_proj_kernel(QkvProjArgs a) {
  using C = ProjCfg<TG>;
  constexpr int kPTok = C::kTok, kPStages = C::kStages, kPWInstr = C::kWInstr, kPXInstr = C::kXInstr;
  __shared__ __attribute__((aligned(1024))) ProjLds<TG> lds;

  const int tid = threadIdx.x;
  const int w = wave_uniform(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int hf = lane >> 5;
  const int pair = blockIdx.x;
  const int t0 = blockIdx.y * kPTok;
  const int n0 = pair * kPCols;  // first weight row of the workgroup
  const int T = a.num_tokens;
  const int nst_all = a.hidden / kPK;
  const int sbeg = SPLIT ? (int)((int64_t)blockIdx.z * nst_all / a.num_splits) : 0;
  const int nst = SPLIT ? (int)((int64_t)(blockIdx.z + 1) * nst_all / a.num_splits) - sbeg : nst_all;

  const char* xg = static_cast<const char*>(a.x);
  const char* wg = static_cast<const char*>(a.weight);

  // Loader role: 1-KB blocks of 8 LDS rows; lane l lands at byte 16 l of
  // the block, i.e. row 8 b + l/8, physical chunk l%8, so it fetches the
  // logical chunk that the swizzle puts there.
  const int lrow = lane >> 3;
  const int lpc = lane & 7;
  auto issue = [&](int st) __attribute__((always_inline)) {
    const int buf = st % kPStages;
    const int64_t kofs = (int64_t)(sbeg + st) * kPRowBytes;
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
  // One slice: the operands of k-step kk+2 are read from LDS while the
  // matrix instructions of k-step kk run (lanes 0-31 take k 16kk .. +7,
  // lanes 32-63 k 16kk+8 .. +15).  The reads and their waits are written
  // out: LDS reads complete in order, so the wait for k-step kk leaves the
  // six reads of the next k-step in flight, which the compiler's own
  // waits (a full drain before every use) would not.
  auto compute = [&](int st) __attribute__((always_inline)) {
    const int buf = st % kPStages;
    const uint32_t wa = (uint32_t)(uintptr_t)(&lds.w[buf][0] + (wrow0 + lq) * kPRowBytes);
    const uint32_t xa = (uint32_t)(uintptr_t)(&lds.x[buf][0] + (xrow0 + lq) * kPRowBytes);
    constexpr int KS = kPK / 16;
    bf16x8_t av[KS][4], bv[KS][2];
    auto read = [&](int kk) __attribute__((always_inline)) {
      const uint32_t pc = 16 * ((2 * kk + hf) ^ sw);
      // weight rows 32 mb + lq (4096 bytes per 32 rows), activation rows 32 nb + lq
      asm volatile("ds_read_b128 %0, %1" : "=v"(av[kk][0]) : "v"(wa + pc) : "memory");
      asm volatile("ds_read_b128 %0, %1 offset:4096" : "=v"(av[kk][1]) : "v"(wa + pc) : "memory");
      asm volatile("ds_read_b128 %0, %1 offset:8192" : "=v"(av[kk][2]) : "v"(wa + pc) : "memory");
      asm volatile("ds_read_b128 %0, %1 offset:12288" : "=v"(av[kk][3]) : "v"(wa + pc) : "memory");
      asm volatile("ds_read_b128 %0, %1" : "=v"(bv[kk][0]) : "v"(xa + pc) : "memory");
      asm volatile("ds_read_b128 %0, %1 offset:4096" : "=v"(bv[kk][1]) : "v"(xa + pc) : "memory");
    };
    // wait until at most 6 (one k-step) / 0 LDS reads are pending: k-step
    // kk's operands are in
    auto wait6 = [&](int kk) __attribute__((always_inline)) {
      asm volatile("s_waitcnt lgkmcnt(6)"
                   : "+v"(av[kk][0]), "+v"(av[kk][1]), "+v"(av[kk][2]), "+v"(av[kk][3]),
                     "+v"(bv[kk][0]), "+v"(bv[kk][1]) : : "memory");
    };
    auto wait0 = [&](int kk) __attribute__((always_inline)) {
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(av[kk][0]), "+v"(av[kk][1]), "+v"(av[kk][2]), "+v"(av[kk][3]),
                     "+v"(bv[kk][0]), "+v"(bv[kk][1]) : : "memory");
    };
    auto mma = [&](int kk) __attribute__((always_inline)) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[kk][mb], bv[kk][nb], acc[nb][mb], 0, 0, 0);
    };
    static_assert(KS == 4, "the pipeline below is written for four k-steps");
    // the scheduling fences keep each k-step's matrix instructions between
    // its wait and the next one
    read(0);
    read(1);
    wait6(0);
    read(2);
    __builtin_amdgcn_sched_barrier(0);
    mma(0);
    __builtin_amdgcn_sched_barrier(0);
    wait6(1);
    read(3);
    __builtin_amdgcn_sched_barrier(0);
    mma(1);
    __builtin_amdgcn_sched_barrier(0);
    wait6(2);
    __builtin_amdgcn_sched_barrier(0);
    mma(2);
    __builtin_amdgcn_sched_barrier(0);
    wait0(3);
    mma(3);
  };

  const int head = 2 * pair + (w & 1);
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int kind = head < Hq ? 0 : (head < Hq + Hkv ? 1 : 2);  // q, k, v
  const int hidx = kind == 0 ? head : (kind == 1 ? head - Hq : head - Hq - Hkv);

  // Ring: stage s sits in buffer s % kPStages.  At the top of iteration s
  // the wavefront's own loads of stage s are waited for (with three stages
  // stage s+1 may stay in flight), the barrier publishes everyone's, and
  // also marks that every wavefront has finished reading the buffer that
  // stage s + kPStages - 1 refills.
  constexpr int kPer = kPWInstr + kPXInstr;
#pragma unroll
  for (int p = 0; p < kPStages - 1; ++p)
    if (p < nst) issue(p);
  for (int s = 0; s < nst; ++s) {
    if (kPStages == 3 && s + 1 < nst) proj_wait_vmcnt<kPer>();
    else proj_wait_vmcnt<0>();
    // a bare barrier: __syncthreads() would also drain the stage still in flight
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // Nothing of this wavefront's is pending on the LDS counter here; the
    // explicit drain also retires scalar argument loads hoisted above the
    // loop (they return out of order, so while one may be pending every LDS
    // wait in the loop would have to be a full drain).
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    if (s + kPStages - 1 < nst) issue(s + kPStages - 1);
    compute(s);
  }

  if constexpr (SPLIT) {
    // fp32 partial sums of this split: 4 consecutive columns per store
    const int ncols_p = (Hq + 2 * Hkv) * kHeadDim;
    float* part = a.partials + (int64_t)blockIdx.z * T * ncols_p + head * kHeadDim;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int t = t0 + xrow0 + 32 * nb + lq;
      if (t >= T) continue;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<float4*>(part + (int64_t)t * ncols_p + 32 * mb + 8 * j + 4 * hf) =
              make_float4(acc[nb][mb][4 * j], acc[nb][mb][4 * j + 1], acc[nb][mb][4 * j + 2],
                          acc[nb][mb][4 * j + 3]);
    }
    return;
  }

  // ---- epilogue ---------------------------------------------------------
  // acc[nb][mb][v] is column 32 mb + 8 (v/4) + 4 hf + v%4 of this wave's head
  // for token t0 + 64 (w >> 1) + 32 nb + lq.  The LDS is free from here on;
  // it stages the cos / sin rows of the workgroup's tokens (read per lane,
  // written by whole rows) and then each wavefront's output rows (written
  // per lane, stored to memory by whole 256-byte rows).
  char* lbase = reinterpret_cast<char*>(&lds);
  const int ncols = (Hq + 2 * Hkv) * kHeadDim;
  const int P = 1 << a.log2_page;
  __syncthreads();  // every wavefront is done with the operand buffers

  // Metadata of the rows this lane moves below, requested first so its
  // latency hides behind the arithmetic: the slot of each staged output row
  // (k / v heads) and the position of each cos / sin row it loads.
  constexpr int kRowsPerWave = kPTok / C::kWaves;  // cos / sin rows per wave: 32, two per load
  int32_t row_slot[16], row_pos[kRowsPerWave / 2];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = t0 + xrow0 + 4 * i + (lane >> 4);
    row_slot[i] = (kind != 0 && t < T) ? a.slots[t] : -1;
  }
  const int head0 = 2 * pair;
  const bool any_rope = head0 < Hq + Hkv;  // the pair's first head is q or k
#pragma unroll
  for (int i = 0; i < kRowsPerWave / 2; ++i) {
    const int r = 2 * ((kRowsPerWave / 2) * w + i) + (lane >> 5);
    const int pos = any_rope ? a.positions[min(t0 + r, T - 1)] : 0;
    row_pos[i] = pos < 0 ? 0 : (pos >= a.max_position ? a.max_position - 1 : pos);
  }

  // the projection rounded to bf16, two columns per word: vals[nb][mb][i]
  // holds columns 32 mb + 8 (i/2) + 4 hf + 2 (i%2), +1
  uint32_t vals[2][4][8];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 8; ++i) vals[nb][mb][i] = cvt_pk_bf16(acc[nb][mb][2 * i], acc[nb][mb][2 * i + 1]);

  // Row staging: wavefront w owns 16 KB at 16 KB * w, its 64 token rows of
  // 256 bytes with 16-byte chunk c of row r at physical chunk c ^ (r % 16),
  // so the 32 rows a write instruction touches spread over all banks.
  char* wstage = lbase + 16384 * w;
  auto stage_rows = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int r = 32 * nb + lq;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = 4 * mb + j;
          *reinterpret_cast<uint2*>(wstage + r * 256 + 16 * (c ^ (r & 15)) + 8 * hf) =
              make_uint2(vals[nb][mb][2 * j], vals[nb][mb][2 * j + 1]);
        }
    }
  };
  // Store the staged rows: instruction i moves rows 4 i .. 4 i + 3, 16 lanes
  // (16 bytes each) per row; row_ptr(r) gives the row's destination or null.
  auto store_rows = [&](auto row_ptr) __attribute__((always_inline)) {
    const int p = lane & 15;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 4 * i + (lane >> 4);
      const uint4 v = *reinterpret_cast<const uint4*>(wstage + r * 256 + 16 * p);
      uint16_t* dst = row_ptr(i, r);
      if (dst != nullptr) *reinterpret_cast<uint4*>(dst + 8 * (p ^ (r & 15))) = v;
    }
  };

  if (a.qkv_out != nullptr) {
    stage_rows();
    store_rows([&](int, int r) -> uint16_t* {
      const int t = t0 + xrow0 + r;
      return t < T ? static_cast<uint16_t*>(a.qkv_out) + (int64_t)t * ncols + head * kHeadDim : nullptr;
    });
    __builtin_amdgcn_s_waitcnt(0xc07f);  // this wavefront's staging reads are done
  }

  // cos / sin rows of the workgroup's tokens, when either head is a q or k
  // head: row r (token t0 + r) is the 512-byte table row of its position,
  // 16-byte chunk c at physical chunk c ^ (r % 16); two rows per 1-KB load.
  if (any_rope) {
    __syncthreads();  // the qkv_out staging above is read
#pragma unroll
    for (int i = 0; i < kRowsPerWave / 2; ++i) {
      const int g = (kRowsPerWave / 2) * w + i;
      const int r = 2 * g + (lane >> 5);
      const int c = (lane & 31) ^ (r & 15);
      __builtin_amdgcn_global_load_lds(a.cos_sin + (int64_t)row_pos[i] * kHeadDim + 4 * c,
                                       (lds_char*)(lbase + 1024 * g), 16, 0, 0);
    }
    proj_wait_vmcnt<0>();
    __syncthreads();
  }

  if (kind != 2) {
    // q / k: RMSNorm over the head's 128 values, then RoPE; vals is
    // replaced by the rotated rows
    const uint16_t* nw = static_cast<const uint16_t*>(kind == 0 ? a.q_w : a.k_w);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float ss = 0.f;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float lo = bf16_lo(vals[nb][mb][i]), hi = bf16_hi(vals[nb][mb][i]);
          ss = fmaf(lo, lo, ss);
          ss = fmaf(hi, hi, ss);
        }
      ss = sum_halves32(ss);
      const float inv_rms = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + a.eps);
      const int r = xrow0 + 32 * nb + lq;  // row of the staged cos / sin
      const char* crow = lbase + r * 512;
      // one RoPE pair of column blocks at a time: block mb (columns < 64)
      // and block mb + 2 (their partners, 64 further)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        float y[2][16];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int b = mb + 2 * h2;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint2 wv = *reinterpret_cast<const uint2*>(nw + 32 * b + 8 * j + 4 * hf);
            const uint32_t ww[2] = {wv.x, wv.y};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint32_t xw = vals[nb][b][2 * j + h];
              // bf16(x * r), then bf16(that * w)
              const uint32_t nrm = cvt_pk_bf16(bf16_lo(xw) * inv_rms, bf16_hi(xw) * inv_rms);
              const uint32_t m = cvt_pk_bf16(bf16_lo(nrm) * bf16_lo(ww[h]), bf16_hi(nrm) * bf16_hi(ww[h]));
              y[h2][4 * j + 2 * h] = bf16_lo(m);
              y[h2][4 * j + 2 * h + 1] = bf16_hi(m);
            }
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int cc = 8 * mb + 2 * j + hf;  // cos chunk of columns 32 mb + 8 j + 4 hf .. +3
          const float4 c4 = *reinterpret_cast<const float4*>(crow + 16 * (cc ^ (r & 15)));
          const float4 s4 = *reinterpret_cast<const float4*>(crow + 16 * ((16 + cc) ^ (r & 15)));
          const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
          const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
          float o1[4], o2[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float y1 = y[0][4 * j + e], y2 = y[1][4 * j + e];
            o1[e] = y1 * cv[e] - y2 * sv[e];
            o2[e] = y2 * cv[e] + y1 * sv[e];
          }
          vals[nb][mb][2 * j] = cvt_pk_bf16(o1[0], o1[1]);
          vals[nb][mb][2 * j + 1] = cvt_pk_bf16(o1[2], o1[3]);
          vals[nb][mb + 2][2 * j] = cvt_pk_bf16(o2[0], o2[1]);
          vals[nb][mb + 2][2 * j + 1] = cvt_pk_bf16(o2[2], o2[3]);
        }
      }
    }
  }

  if (any_rope) __syncthreads();  // the staged cos / sin are read
  stage_rows();
  store_rows([&](int i, int r) -> uint16_t* {
    const int t = t0 + xrow0 + r;
    if (t >= T) return nullptr;
    if (kind == 0) return static_cast<uint16_t*>(a.q_out) + ((int64_t)t * Hq + hidx) * kHeadDim;
    const int32_t slot = row_slot[i];
    const int64_t page = slot >> a.log2_page;
    if (slot < 0 || page >= a.num_pages) return nullptr;  // -1 = skip; out of range never touched
    const int64_t row = ((page * Hkv + hidx) << a.log2_page) + (slot & (P - 1));
    return static_cast<uint16_t*>(kind == 1 ? a.k_cache : a.v_cache) + row * kHeadDim;
  });
}

// The split path's second kernel: the epilogue for one (token, head) row per
// 16 lanes, lane j holding columns 8 j .. 8 j + 7 (the first half of the head
// in lanes 0-7, so a value's RoPE partner sits 8 lanes away).  It adds the
// splits' partial sums in split order, rounds to bf16 as the layer's output,
// and applies the same arithmetic as the fused qil_kv_write to that row.
__global__ __launch_bounds__(256) void qkv_proj_reduce_kernel(QkvProjArgs a) {
  const int heads = a.num_q_heads + 2 * a.num_kv_heads;
  const int ncols = heads * kHeadDim;
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  if (row >= (int64_t)a.num_tokens * heads) return;  // whole 16-lane groups exit together
  const int t = (int)(row / heads);
  const int head = (int)(row - (int64_t)t * heads);
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int kind = head < Hq ? 0 : (head < Hq + Hkv ? 1 : 2);  // q, k, v
  const int hidx = kind == 0 ? head : (kind == 1 ? head - Hq : head - Hq - Hkv);

  float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const float* src = a.partials + (int64_t)t * ncols + head * kHeadDim + 8 * j;
  const int64_t split_stride = (int64_t)a.num_tokens * ncols;
  for (int z = 0; z < a.num_splits; ++z) {
    const float4 lo = *reinterpret_cast<const float4*>(src + z * split_stride);
    const float4 hi = *reinterpret_cast<const float4*>(src + z * split_stride + 4);
    x[0] += lo.x; x[1] += lo.y; x[2] += lo.z; x[3] += lo.w;
    x[4] += hi.x; x[5] += hi.y; x[6] += hi.z; x[7] += hi.w;
  }
  uint32_t px[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) px[i] = cvt_pk_bf16(x[2 * i], x[2 * i + 1]);
  if (a.qkv_out != nullptr)
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.qkv_out) + (int64_t)t * ncols + head * kHeadDim + 8 * j) =
        make_uint4(px[0], px[1], px[2], px[3]);

  uint16_t* dst = nullptr;
  if (kind == 0) {
    dst = static_cast<uint16_t*>(a.q_out) + ((int64_t)t * Hq + hidx) * kHeadDim;
  } else {
    const int32_t slot = a.slots[t];
    const int64_t page = slot >> a.log2_page;
    if (slot >= 0 && page < a.num_pages) {
      const int64_t prow = ((page * Hkv + hidx) << a.log2_page) + (slot & ((1 << a.log2_page) - 1));
      dst = static_cast<uint16_t*>(kind == 1 ? a.k_cache : a.v_cache) + prow * kHeadDim;
    }
  }
  if (kind == 2) {  // v: the rounded projection as it is
    if (dst != nullptr) *reinterpret_cast<uint4*>(dst + 8 * j) = make_uint4(px[0], px[1], px[2], px[3]);
    return;
  }

  // q / k: RMSNorm over the 16 lanes of the row, then RoPE
  float xr[8], ss = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xr[2 * i] = bf16_lo(px[i]);
    xr[2 * i + 1] = bf16_hi(px[i]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) ss = fmaf(xr[i], xr[i], ss);
  ss = row_sum16(ss);
  const float inv_rms = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + a.eps);
  const uint4 wraw = *reinterpret_cast<const uint4*>(
      static_cast<const uint16_t*>(kind == 0 ? a.q_w : a.k_w) + 8 * j);
  const uint32_t ww[4] = {wraw.x, wraw.y, wraw.z, wraw.w};
  float y[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // bf16(x * r), then bf16(that * w)
    const uint32_t n = cvt_pk_bf16(xr[2 * i] * inv_rms, xr[2 * i + 1] * inv_rms);
    const uint32_t m = cvt_pk_bf16(bf16_lo(n) * bf16_lo(ww[i]), bf16_hi(n) * bf16_hi(ww[i]));
    y[2 * i] = bf16_lo(m);
    y[2 * i + 1] = bf16_hi(m);
  }
  int pos = a.positions[t];
  pos = pos < 0 ? 0 : (pos >= a.max_position ? a.max_position - 1 : pos);
  const float* cs = a.cos_sin + (int64_t)pos * kHeadDim + 8 * (j & 7);
  const float4 c0 = *reinterpret_cast<const float4*>(cs);
  const float4 c1 = *reinterpret_cast<const float4*>(cs + 4);
  const float4 s0 = *reinterpret_cast<const float4*>(cs + kHeadDim / 2);
  const float4 s1 = *reinterpret_cast<const float4*>(cs + kHeadDim / 2 + 4);
  const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  const bool first_half = j < 8;
  uint32_t o32[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float r[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = 2 * i + h;
      const float partner = row_swap8(y[e]);
      // first half: y1*c - y2*s ; second half: y2*c + y1*s
      r[h] = first_half ? (y[e] * cv[e] - partner * sv[e]) : (y[e] * cv[e] + partner * sv[e]);
    }
    o32[i] = cvt_pk_bf16(r[0], r[1]);
  }
  if (dst != nullptr) *reinterpret_cast<uint4*>(dst + 8 * j) = make_uint4(o32[0], o32[1], o32[2], o32[3]);
}

}  // namespace

hipError_t launch_qkv_proj(const QkvProjArgs& a, hipStream_t s) {
  const int heads = a.num_q_heads + 2 * a.num_kv_heads;
  if (a.num_tokens == 0) return hipSuccess;
  if (a.num_splits > 1) {
    // split over hidden: partial sums, then their sum and the epilogue
    dim3 grid(heads / 2, (a.num_tokens + ProjCfg<2>::kTok - 1) / ProjCfg<2>::kTok, a.num_splits);
    hipLaunchKernelGGL((qkv_proj_kernel<2, true>), grid, dim3(ProjCfg<2>::kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)a.num_tokens * heads;
    hipLaunchKernelGGL(qkv_proj_reduce_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  // One pass: pick the workgroup shape with the shorter estimated time,
  // rounds of 256 CUs (one workgroup per CU) times the time of one round.
  // Measured on the Qwen3-8B shape, a round of 128-token workgroups takes
  // ~0.7 of a round of 256-token ones (they move more operand bytes per
  // flop): 2112 tokens run in one round of 216 256-token workgroups rather
  // than two of 408, while 1024 tokens run as one round of 192 128-token
  // workgroups rather than 96 256-token ones.  256 tokens win when their
  // estimate is no larger.
  const int64_t pairs = heads / 2;
  const int64_t rounds4 = (pairs * ((a.num_tokens + 255) / 256) + 255) / 256;
  const int64_t rounds2 = (pairs * ((a.num_tokens + 127) / 128) + 255) / 256;
  if (10 * rounds4 <= 7 * rounds2) {
    dim3 grid(heads / 2, (a.num_tokens + ProjCfg<4>::kTok - 1) / ProjCfg<4>::kTok);
    hipLaunchKernelGGL((qkv_proj_kernel<4, false>), grid, dim3(ProjCfg<4>::kThreads), 0, s, a);
  } else {
    dim3 grid(heads / 2, (a.num_tokens + ProjCfg<2>::kTok - 1) / ProjCfg<2>::kTok);
    hipLaunchKernelGGL((qkv_proj_kernel<2, false>), grid, dim3(ProjCfg<2>::kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace qil
