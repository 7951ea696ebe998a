// Chunked varlen causal prefill over the paged cache, on bf16 matrix cores:
// the device code, included by prefill.hip and mixed.hip.
//
// What is computed follows the "nano-vLLM learning note" Attention.forward
// prefill branch (with a cached prefix the keys come from the cache through
// the block tables) and prepare_prefill block (the new tokens of a request
// sit at positions num_cached .. num_cached + n - 1), and the "qwen-engine"
// README's flat varlen prefill (requests packed by cu_seqlens) and its note
// that prefill is compute-bound.
//
// One workgroup (8 wavefronts, two per SIMD) owns 256 query rows of one
// request and one KV head: 256/G consecutive new tokens times the G query
// heads that share the KV head (GQA packing), so each K/V tile fetched from
// HBM/L2 serves 256 rows.  Each wavefront owns 32 rows.  The workgroup walks
// key tiles of 64 keys up to its last visible key.  Whole query tiles over
// short contexts run as workgroups of 4 wavefronts (128 rows), two per CU;
// each row's arithmetic is the same in either shape.
//
//   * Tiles go from memory straight into LDS (global_load_lds, 16 bytes per
//     lane, no staging registers): K and V rows land row-major with the
//     16-byte chunks XOR-swizzled per row.  LDS is double-buffered: a tile's
//     loads are in flight while the previous tile is computed.  Each
//     wavefront keeps the page ids of its rows, one tile per lane, in a
//     register loaded once per 64 tiles.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys on the M side, query
//     rows on the N side), so that each lane owns one query row and the row
//     statistics of the online softmax stay per lane.
//   * The PV product O^T = V^T P^T reads V^T operands with
//     ds_read_b64_tr_b16, which transposes 4x16 blocks of row-major V on the
//     way out of LDS; P comes straight from the S^T accumulator registers,
//     rounded to bf16.
//   * Online softmax in base 2 with a lazy reference maximum: the output is
//     rescaled only when a row maximum grows by more than 2^8, so the weights
//     exp2(s - m_ref) stay below 256 and most tiles skip the rescale.  The
//     check runs once per 64-key tile, on the maximum of the whole tile and
//     before any weight of the tile is formed, so every weight added to O
//     and to the row sum is relative to the same reference.  The row sum
//     adds the same rounded weights that feed the PV product.  The
//     reference is an integer (the ceiling of the row maximum), so a weight
//     rounded to bf16 is the same bf16 value times a power of two whatever
//     the reference, and a rescale multiplies by an exact power of two: the
//     result does not depend on where the rescales fall, and pieces of one
//     row's keys (the split over keys) merge to the whole row's sums up to
//     the order of fp32 additions.
//   * Causal masking only on the diagonal band of tiles.
//   * Each 64-key tile runs as two 32-key halves: the first half's row
//     maximum sits next to the second half's QK^T matrix work, and the first
//     half's PV product next to the second half's exponentials.
// Block ids are laid out KV-head fastest, so with 8 KV heads all tiles of one
// KV head land on one XCD (workgroups are dealt to the 8 XCDs round robin)
// and its K/V stay in that XCD's L2.  Query tiles are issued last-first: the
// tiles with the most keys start earliest.
#pragma once
#include <type_traits>

#include "device_common.h"
#include "qil_internal.h"

namespace qil {
namespace {

constexpr int kBN = 64;        // keys per tile
constexpr float kLazyRescale = 8.0f;  // log2 of the largest weight allowed before rescaling

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) char lds_char;

// Row (M index) of accumulator register v held by lanes of half hf, for the
// 32x32 MFMA output: rows 8*(v/4) + 4*hf + v%4, column = lane % 32.
__device__ __forceinline__ int acc_row(int v, int hf) { return 8 * (v >> 2) + 4 * hf + (v & 3); }

// Physical 16-byte chunk of logical chunk c in row `row` of a K tile and of a
// V tile (256-byte rows, 16 chunks).  K: XOR with row mod 16, so the 16 rows
// read by a quarter wavefront hit 16 different chunk positions.  V: XOR with
// 4 * (row mod 4), so the 8 rows of a transposing read fall into four
// different 64-byte bank groups.
__device__ __forceinline__ int k_chunk(int row, int c) { return c ^ (row & 15); }
__device__ __forceinline__ int v_chunk(int row, int c) { return c ^ ((row & 3) << 2); }

// One 16-byte LDS-DMA load per lane (global_load_lds_dwordx4): lane l's
// bytes land at dst + 16 l.  Written as assembly so that the compiler does not
// track it.  With the builtin, the compiler cannot tell which of the two tile
// buffers a load writes, so before the current tile's first transposing read
// it waited for every load in flight, the next tile's included, and part of
// that tile's load latency sat inside the current tile (measured: 4-6 %
// on prefill-varlen and the 8B step's prefill).  The tile loop waits for its
// own loads (vmcnt 0 before each workgroup barrier).  The s_nop covers the
// wait state that a write of M0 needs before an LDS-DMA instruction.  No
// register is written.
__device__ __forceinline__ void lds_dma16(const char* src, lds_char* dst) {
  const unsigned m0 = (unsigned)(uintptr_t)dst;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}

// Maximum / sum over the two halves of a wavefront (lanes l and l ^ 32),
// with v_permlane32_swap instead of an LDS round trip.
__device__ __forceinline__ float max_halves(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// The split-over-keys path and the one-launch mixed step use workgroups of
// 8 wavefronts (256 query rows).  Whole query tiles also run as workgroups
// of 4 wavefronts (128 rows, two workgroups per CU) when the keys per tile
// are few (see launch_prefill).
constexpr int kWaves = 8;               // wavefronts per workgroup, 32 query rows each
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsWG = 32 * kWaves;    // query rows per workgroup

// LDS of one workgroup: [slot][K | V][64 rows x 256 bytes].
typedef char PrefillLds[2][2][kBN * 256];

// Key tiles [kt_begin, kt_end) of one query tile: KV head g, request r,
// query tile `tile`.  With part_o null the rows are final and go to a.out;
// otherwise this is one piece of a split tile, and each row's unnormalized
// output sums go to part_o (fp32, [256 rows][128]) with the row's integer
// reference maximum (log2 domain) and weight sum to part_ml (rows
// ml_row_stride pairs apart).  Every thread of the workgroup of W
// wavefronts (32 W query rows) calls it; `smem` is the workgroup's LDS.
// APPEND (whole tiles only): keys at the request's new positions come from
// a.k_new / a.v_new instead of the pools (other workgroups of the launch
// store those rows into the pools meanwhile).
template <int G, int W = kWaves, bool APPEND = false>
__device__ __forceinline__ void prefill_range(const PrefillArgs& a, int g, int r, int tile,
                                              int kt_begin, int kt_end, float* part_o,
                                              float* part_ml, int ml_row_stride, PrefillLds& smem) {
  static_assert(W == 4 || W == 8, "4 or 8 wavefronts");
  constexpr int kWGThreads = 64 * W;
  constexpr int kRowsPerWave = kBN / W;  // tile rows each wavefront loads
  constexpr int TQ = 32 * W / G;         // tokens per workgroup
  const int q0 = a.cu_seqlens[r];
  // rows of this request, kept inside [0, total_q)
  const int n = min(a.cu_seqlens[r + 1], a.total_q) - max(q0, 0);
  const int t0 = tile * TQ;
  if (q0 < 0 || t0 >= n) return;
  const int L = min(a.context_lens[r], a.max_context_len);
  const int prefix = L - n;
  const int tvalid = min(TQ, n - t0);
  const int kmax = prefix + t0 + tvalid;  // keys [0, kmax) are visible to some row
  const int ntiles = min(kmax > 0 ? (kmax + kBN - 1) / kBN : 0, kt_end);
  const int kt0 = kt_begin;
  const int pos_min = prefix + t0;

  const int tid = threadIdx.x;
  const int w = wave_uniform(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int hf = lane >> 5;
  const int Hq = a.num_q_heads;

  // This lane's query row.
  const int rho = 32 * w + lq;
  const int tok = rho / G;
  const int hh = rho % G;
  const bool row_valid = tok < tvalid;
  const int my_pos = prefix + t0 + min(tok, tvalid - 1);
  // Keys this wavefront's rows see: up to its last valid token's position.
  // A wavefront whose rows all lie past the tile's tokens (the last query
  // tile of a request) has none.
  const int wtok_lo = (32 * w) / G, wtok_hi = (32 * w + 31) / G;
  const bool wave_rows = wtok_lo < tvalid;
  const int wpos_max = prefix + t0 + min(wtok_hi, tvalid - 1);

  // Loader role.  Wavefront w fills rows 8w .. 8w+7 of the K and V tiles,
  // 4 rows (1 KB) per instruction: lane l lands at byte 16 l of that KB,
  // i.e. row 4m + l/16, physical chunk l%16, so it fetches the logical chunk
  // that belongs there.  Eight consecutive keys always share a page.
  const int32_t* bt_row = a.block_tables + (int64_t)r * a.bt_stride;
  const char* kpool = static_cast<const char*>(a.k_cache);
  const char* vpool = static_cast<const char*>(a.v_cache);
  const int P = 1 << a.log2_page;
  const int lrow = lane >> 4;   // row within a 4-row instruction
  const int lpc = lane & 15;    // physical chunk this lane fills

  // Lane i holds the page id of this wavefront's rows in tile base + i.
  int page_lane = -1;
  auto fetch_pages = [&](int base) __attribute__((always_inline)) {
    const int key = (base + lane) * kBN + kRowsPerWave * w;
    page_lane = key < L ? bt_row[key >> a.log2_page] : -1;
  };

  // The first page ids go out before the query rows, and both without a
  // branch (a row past the tile's tokens loads the last token's row and
  // zeroes it), so the first tile's loads wait only for the page ids while
  // the query loads are still in flight.
  fetch_pages(kt0 & ~63);

  bf16x8_t qreg[8];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           ((int64_t)(q0 + t0 + min(tok, tvalid - 1)) * Hq + g * G + hh) * kHeadDim;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint4 x = *reinterpret_cast<const uint4*>(qrow + 16 * t + 8 * hf);
      if (!row_valid) x = make_uint4(0, 0, 0, 0);
      qreg[t] = __builtin_bit_cast(bf16x8_t, x);
    }
  }


  // Rows past the context are never loaded; what they hold stands in for
  // them (their scores are masked, so their weight is exactly 0) and only has
  // to be finite: start from zeros.
  {
    uint4* zf = reinterpret_cast<uint4*>(&smem[0][0][0]);
    for (int i = tid; i < (int)(sizeof(PrefillLds) / 16); i += kWGThreads) zf[i] = make_uint4(0, 0, 0, 0);
  }

  auto issue_tile = [&](int kt, int buf) __attribute__((always_inline)) {
    const int page = __builtin_amdgcn_readlane(page_lane, kt & 63);
    if ((unsigned)page >= (unsigned)a.num_pages) return;  // absent page (uniform)
#pragma unroll
    for (int m2 = 0; m2 < kRowsPerWave / 4; ++m2) {
      const int row = kRowsPerWave * w + 4 * m2 + lrow;  // tile row this lane fills
      const int key = kt * kBN + row;
      const int64_t grow = (((int64_t)page * a.num_kv_heads + g) << a.log2_page) + (key & (P - 1));
      lds_char* kdst = (lds_char*)&smem[buf][0][0] + (kRowsPerWave * w + 4 * m2) * 256;
      lds_char* vdst = (lds_char*)&smem[buf][1][0] + (kRowsPerWave * w + 4 * m2) * 256;
      if (key < L) {
        const char* ksrc = kpool + grow * 256;
        const char* vsrc = vpool + grow * 256;
        if (APPEND && key >= prefix) {  // a new token: its row is an input of this call
          const int64_t t = (int64_t)q0 + (key - prefix);
          ksrc = static_cast<const char*>(a.k_new) + (t * a.k_new_stride + (int64_t)g * kHeadDim) * 2;
          vsrc = static_cast<const char*>(a.v_new) + (t * a.v_new_stride + (int64_t)g * kHeadDim) * 2;
        }
        lds_dma16(ksrc + 16 * k_chunk(row, lpc), kdst);
        lds_dma16(vsrc + 16 * v_chunk(row, lpc), vdst);
      }
    }
  };

  // Per-lane LDS offsets of the matrix operands.
  //  K operand (A of S^T, ds_read_b128): row 32b + lq, logical chunk 2t + hf.
  const int kx = lq & 15;
  //  V^T operand (A of O^T) by transposing reads: in each 16-lane group
  //  (q = lane/16) lane src = j + 4k supplies the 8-byte address of V row
  //  16s + 8i + 4(q/2) + k, dims 32db + 16(q%2) + 4j .. +3; the hardware hands
  //  lane o of the group the 4 keys at dim 32db + 16(q%2) + o.  Two reads
  //  (i = 0, 1) give the 8 keys 16s + 8(e/4) + 4hf + e%4 that the accumulator
  //  layout of P puts in element e of this lane's B operand.
  const int q16 = lane >> 4;
  const int src = lane & 15;
  const int vj = src & 3, vk = src >> 2;
  int vofs[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int row = 4 * (q16 >> 1) + vk;  // + 16s + 8i, which keeps row & 3
    const int c = 4 * db + 2 * (q16 & 1) + (vj >> 1);
    vofs[db] = row * 256 + 16 * v_chunk(row, c) + 8 * (vj & 1);
  }

  f32x16_t oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[i][v] = 0.f;
  float mref = -1.0e30f;  // base-2 domain
  float lrun = 0.f;
  const float qs = a.scale * kLog2e;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  const f32x16_t zero16 = {};

  // Operand fetches are separate from the matrix instructions that use them,
  // so a whole half-tile of LDS reads is in flight before its first MFMA.
  auto load_k = [&](int buf, int b, bf16x8_t (&kop)[8]) __attribute__((always_inline)) {
    const char* krow = &smem[buf][0][0] + (32 * b + lq) * 256;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      kop[t] = *reinterpret_cast<const bf16x8_t*>(krow + 16 * ((2 * t + hf) ^ kx));
  };
  auto qk = [&](const bf16x8_t (&kop)[8]) __attribute__((always_inline)) -> f32x16_t {
    f32x16_t acc = zero16;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[t], qreg[t], acc, 0, 0, 0);
    return acc;
  };
  auto load_v = [&](int buf, int b, bf16x8_t (&vop)[4][2]) __attribute__((always_inline)) {
    const lds_char* vbase = (const lds_char*)&smem[buf][1][0];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int s = 2 * b + s2;
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(vbase + vofs[db] + (16 * s) * 256));
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(vbase + vofs[db] + (16 * s + 8) * 256));
        const i16x8_t v8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        vop[db][s2] = __builtin_bit_cast(bf16x8_t, v8);
      }
    }
  };
  auto pv = [&](const bf16x8_t (&vop)[4][2], const bf16x8_t (&pb)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[db][s2], pb[s2], oacc[db], 0, 0, 0);
  };

  // Masked row maximum (raw scores) of a half.
  auto half_max = [&](auto mask_tag, f32x16_t& s, int kbase, float& mx) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      if (MASK && kbase + acc_row(v, hf) > my_pos) s[v] = -INFINITY;
      mx = fmaxf(mx, s[v]);
    }
  };
  // The lazy rescale, once per tile before any weight of the tile is formed
  // (a uniform branch, rarely taken).
  auto rescale = [&](float mx) __attribute__((always_inline)) {
    mx = max_halves(mx) * qs;
    if (__ballot(mx > mref + kLazyRescale) != 0) {
      asm volatile("" ::: "memory");  // keep the rare rescale a real branch
      // integer references: the correction 2^(mref - mnew) is exact (0 for
      // the first tile, where mref is still the -1e30 start value)
      const float mnew = fmaxf(mref, ceilf(mx));
      const float corr = ldexpf(1.0f, (int)fmaxf(mref - mnew, -200.0f));
      mref = mnew;
      lrun *= corr;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[i][v] *= corr;
    }
  };

  // Weights of a half as two bf16 B operands; the row sum takes them too.
  auto exp_half = [&](const f32x16_t& s, bf16x8_t (&pb)[2]) __attribute__((always_inline)) {
    const float neg = -mref;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      uint32_t pk[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = fast_exp2(fmaf(s[8 * s2 + 2 * i], qs, neg));
        const float p1 = fast_exp2(fmaf(s[8 * s2 + 2 * i + 1], qs, neg));
        pk[i] = cvt_pk_bf16(p0, p1);
        lrun = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[i]), ones, lrun, false);
      }
      const uint4 u = {pk[0], pk[1], pk[2], pk[3]};
      pb[s2] = __builtin_bit_cast(bf16x8_t, u);
    }
  };

  // One tile as two 32-key halves.  A wavefront without valid rows skips
  // every tile, and on the diagonal one skips the tiles that lie wholly past
  // its last row's position: their weights would all be exactly 0.  It still
  // loads its share of every tile and meets every barrier; the gain is the
  // LDS operand reads it leaves to the other wavefronts of the CU.
  auto compute = [&](auto mask_tag, int buf, int kt) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int kbase = kt * kBN;
    if (!wave_rows || (MASK && kbase > wpos_max)) return;  // uniform per wavefront
    bf16x8_t kop[8];
    bf16x8_t vop[4][2];
    bf16x8_t p0[2], p1[2];
    load_k(buf, 0, kop);
    f32x16_t s0 = qk(kop);
    // all eight operand reads first, then the eight MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    load_k(buf, 1, kop);
    float mx = -INFINITY;
    half_max(mask_tag, s0, kbase, mx);
    f32x16_t s1 = qk(kop);
    half_max(mask_tag, s1, kbase + 32, mx);
    rescale(mx);
    load_v(buf, 0, vop);
    exp_half(s0, p0);
    pv(vop, p0);
    load_v(buf, 1, vop);
    exp_half(s1, p1);
    pv(vop, p1);
  };

  // Tiles [0, nfree) lie wholly at or before the first token's position and
  // need no mask; the rest (the diagonal band) are masked.  Page ids are
  // fetched 64 tiles at a time from a multiple of 64, so lane i always holds
  // the page of tile (kt & ~63) + i.
  const int nfree = min(ntiles, (pos_min + 1) / kBN);
  auto tile_step = [&](auto mask_tag, int kt) __attribute__((always_inline)) {
    const int buf = (kt - kt0) & 1;
    if (kt + 1 < ntiles) {
      if (((kt + 1) & 63) == 0) fetch_pages(kt + 1);
      issue_tile(kt + 1, buf ^ 1);
    }
    compute(mask_tag, buf, kt);
    __builtin_amdgcn_s_waitcnt(0);  // this wavefront's loads of the next tile have landed
    __syncthreads();
  };
  if (kt0 < ntiles) {
    __syncthreads();  // the zero fill is complete before any load lands
    issue_tile(kt0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = kt0; kt < nfree; ++kt) tile_step(std::false_type{}, kt);
    for (int kt = max(nfree, kt0); kt < ntiles; ++kt) tile_step(std::true_type{}, kt);
  }

  const float ltot = sum_halves(lrun);
  if (!row_valid) return;
  if (part_o) {
    // one piece of a split tile: this row's unnormalized sums and (m, l)
    float* prow = part_o + rho * kHeadDim;
    if (hf == 0) *reinterpret_cast<float2*>(part_ml + 2 * rho * ml_row_stride) = make_float2(mref, ltot);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * db + 8 * q4 + 4 * hf;
        *reinterpret_cast<float4*>(prow + d0) =
            make_float4(oacc[db][4 * q4], oacc[db][4 * q4 + 1], oacc[db][4 * q4 + 2], oacc[db][4 * q4 + 3]);
      }
    return;
  }
  const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
  uint16_t* orow = static_cast<uint16_t*>(a.out) + ((int64_t)(q0 + t0 + tok) * Hq + g * G + hh) * kHeadDim;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * db + 8 * q4 + 4 * hf;
      uint2 st;
      st.x = cvt_pk_bf16(oacc[db][4 * q4] * inv, oacc[db][4 * q4 + 1] * inv);
      st.y = cvt_pk_bf16(oacc[db][4 * q4 + 2] * inv, oacc[db][4 * q4 + 3] * inv);
      *reinterpret_cast<uint2*>(orow + d0) = st;
    }
  }
}

// One whole query tile, z counted from the last tile (z = 0 is the tile with
// the most keys).
template <int G, int W = kWaves>
__device__ __forceinline__ void prefill_tile(const PrefillArgs& a, int n_qtiles, int g, int r,
                                             int z, PrefillLds& smem) {
  prefill_range<G, W>(a, g, r, n_qtiles - 1 - z, 0, 1 << 30, nullptr, nullptr, 0, smem);
}

// Copy workgroup `cb` of `ncb`: stores the new tokens' K and V rows into
// their pool slots, 16-byte chunks (32 per token and KV head: 16 of K, 16 of
// V), four per thread in flight, the workgroups striding over the flat chunk
// index.  A slot of -1 or past the pools stores nothing.
template <int W>
__device__ __forceinline__ void append_rows(const PrefillArgs& a, int cb, int ncb) {
  constexpr int T = 64 * W;
  const int64_t nchunks = (int64_t)a.total_q * a.num_kv_heads * 32;
  const int pmask = (1 << a.log2_page) - 1;
  char* kpool = static_cast<char*>(const_cast<void*>(a.k_cache));  // writable for this entry point
  char* vpool = static_cast<char*>(const_cast<void*>(a.v_cache));
  for (int64_t base = (int64_t)cb * 4 * T; base < nchunks; base += (int64_t)ncb * 4 * T) {
    uint4 val[4];
    char* dst[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t idx = base + u * T + threadIdx.x;
      dst[u] = nullptr;
      if (idx < nchunks) {
        const int c = (int)(idx & 31);
        const int64_t th = idx >> 5;
        const int h = (int)(th % a.num_kv_heads);
        const int64_t t = th / a.num_kv_heads;
        const bool isv = c >= 16;
        const int32_t slot = a.new_slots[t];
        const int64_t page = slot >> a.log2_page;
        val[u] = *reinterpret_cast<const uint4*>(
            static_cast<const char*>(isv ? a.v_new : a.k_new) +
            (t * (isv ? a.v_new_stride : a.k_new_stride) + (int64_t)h * kHeadDim) * 2 + 16 * (c & 15));
        if (slot >= 0 && page < a.num_pages)
          dst[u] = (isv ? vpool : kpool) +
                   (((page * a.num_kv_heads + h) << a.log2_page) + (slot & pmask)) * 256 + 16 * (c & 15);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (dst[u] != nullptr) *reinterpret_cast<uint4*>(dst[u]) = val[u];
  }
}

// W = 8: one workgroup per CU; W = 4: two per CU (two wavefronts per SIMD
// either way, at most 256 registers each).  With APPEND the grid has extra
// z-slices past n_qtiles whose workgroups copy the new rows into the pools;
// the dispatcher hands them out last, to CUs the longest tiles leave idle.
template <int G, int W, bool APPEND = false>
__global__ __launch_bounds__(64 * W, 2) void prefill_kernel(PrefillArgs a, int n_qtiles) {
  __shared__ __attribute__((aligned(1024))) PrefillLds smem;
  if (APPEND && (int)blockIdx.z >= n_qtiles) {
    const int slice = gridDim.x * gridDim.y;
    append_rows<W>(a, ((int)blockIdx.z - n_qtiles) * slice + blockIdx.y * gridDim.x + blockIdx.x,
                   ((int)gridDim.z - n_qtiles) * slice);
    return;
  }
  prefill_range<G, W, APPEND>(a, blockIdx.x, blockIdx.y, n_qtiles - 1 - (int)blockIdx.z, 0, 1 << 30,
                              nullptr, nullptr, 0, smem);
}

}  // namespace
}  // namespace qil
