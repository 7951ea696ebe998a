// Measured ceilings for the roofline: a streaming-read kernel (the HBM rate a
// plain kernel reaches), a loop of independent bf16 MFMAs (the matrix-core
// rate) and loops of LDS operand reads (the rate at which LDS feeds them).  Built into libqil_ceiling.so, used only by the benchmark; not part
// of the attention path.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// Each workgroup reads one contiguous chunk with non-temporal 16-byte loads,
// four per thread in flight; an XOR of the data keeps the loads alive.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* p, size_t n16,
                                                          uint32_t* sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b = (size_t)blockIdx.x * per;
  const size_t e = b + per < n16 ? b + per : n16;
  uint32_t acc = 0;
  for (size_t i = b + threadIdx.x; i < e; i += 4 * 256) {
    u32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t k = i + (size_t)u * 256;
      v[u] = k < e ? __builtin_nontemporal_load(p + k) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x & 255] = acc;  // practically never taken
}

// Four independent accumulator chains per wavefront of v_mfma_f32_32x32x16_bf16.
__global__ __launch_bounds__(256) void mfma_loop_kernel(float* sink, int iters) {
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (threadIdx.x + e));
    b[e] = (__bf16)(0.002f * (threadIdx.x - e));
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  const float s = c0[0] + c1[1] + c2[2] + c3[3];
  if (s == 1234.5f) sink[blockIdx.x & 255] = s;  // practically never taken
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// LDS reads the way an MFMA operand fetch issues them: 512-thread workgroups
// over a 64 KB buffer, each lane reading its own 256-byte row at an
// XOR-swizzled 16-byte chunk, 16 independent reads per batch, then one wait.
// TR = false: ds_read_b128 (16 bytes per lane); TR = true: the transposing
// ds_read_b64_tr_b16 (8 bytes per lane).  Every address stays in the buffer.
template <bool TR>
__global__ __launch_bounds__(512) void lds_read_kernel(uint32_t* sink, int iters) {
  __shared__ __attribute__((aligned(1024))) char lds[65536];
  for (int i = threadIdx.x; i < 65536 / 16; i += 512) reinterpret_cast<int4*>(lds)[i] = make_int4(i, 1, 2, 3);
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  uint32_t addr[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int row = (lane & 31) + 32 * (j & 1);            // < 64
    const int c = ((2 * (j >> 1) + (lane >> 5)) ^ (row & 15)) & 15;
    addr[j] = base + (w & 1) * 32768 + row * 256 + 16 * c;  // < 64 KB
  }
  i32x4_t acc = {0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
    if (!TR) {
      i32x4_t r[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) asm volatile("ds_read_b128 %0, %1" : "=v"(r[j]) : "v"(addr[j]) : "memory");
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int j = 0; j < 16; ++j) acc ^= r[j];
    } else {
      i16x4_t r[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r[j]) : "v"(addr[j]) : "memory");
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j & 3] ^= (int)(uint16_t)r[j][0] | ((int)r[j][1] << 16);
    }
  }
  if (acc[0] == 0x12345678 && acc[1] == 7) sink[blockIdx.x & 255] = (uint32_t)acc[2];  // practically never taken
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16) from device buffer `buf` once.  `sink` is a
// device buffer of 256 words.  Returns 0 or a hipError_t.
int qil_ceiling_stream_read(const void* buf, size_t bytes, void* sink, int32_t num_blocks,
                            void* stream) {
  if (!buf || !sink || bytes % 16 || num_blocks <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3(num_blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(buf),
                     bytes / 16, static_cast<uint32_t*>(sink));
  return (int)hipGetLastError();
}

// num_blocks workgroups of 4 wavefronts, each wavefront issuing 4 * iters
// MFMAs of 32x32x16 (32768 FLOP each).  `sink` as above.
int qil_ceiling_mfma_bf16(void* sink, int32_t num_blocks, int32_t iters, void* stream) {
  if (!sink || num_blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(num_blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<float*>(sink), iters);
  return (int)hipGetLastError();
}

// num_blocks workgroups of 8 wavefronts, each lane issuing 16 * iters LDS
// reads of 16 bytes (transposing = 0: ds_read_b128) or 8 bytes
// (transposing = 1: ds_read_b64_tr_b16).  `sink` as above.
int qil_ceiling_lds_read(int32_t transposing, void* sink, int32_t num_blocks, int32_t iters,
                         void* stream) {
  if (!sink || num_blocks <= 0 || iters <= 0 || (transposing != 0 && transposing != 1))
    return (int)hipErrorInvalidValue;
  if (transposing)
    hipLaunchKernelGGL(lds_read_kernel<true>, dim3(num_blocks), dim3(512), 0,
                       static_cast<hipStream_t>(stream), static_cast<uint32_t*>(sink), iters);
  else
    hipLaunchKernelGGL(lds_read_kernel<false>, dim3(num_blocks), dim3(512), 0,
                       static_cast<hipStream_t>(stream), static_cast<uint32_t*>(sink), iters);
  return (int)hipGetLastError();
}

}  // extern "C"
