// Matrix-core rate calibration: the rate the GPU sustains on v_mfma_f32_32x32x16_bf16 (the
// instruction of the decode's score and output products) when every SIMD issues independent
// products back to back, with no memory traffic and no other instructions in the way.  It is the
// compute ceiling the decode's roofline is read against, next to the data sheet's figure: a large
// library GEMM reaches well below it (its own loads and stores share the time).
//
// Each wave keeps four independent accumulators and issues `iters` x 4 products; lane 0 of wave w
// stores one word derived from the results at out[w], which keeps them live.
//
// Read-rate calibration: the rate HBM delivers to plain reads moved the way the decode moves its
// tiles (global_load_lds_dwordx4 into LDS, 36,864-byte chunks, three chunks in flight per
// workgroup), with nothing else to do: the memory ceiling the decode is read against, next to the
// data sheet's 8 TB/s (a device copy, which also writes, reaches less).
#include "mla_device.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

__global__ __launch_bounds__(256) void mfma_rate_kernel(float* out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (float)(threadIdx.x + i));
    b[i] = (__bf16)(1e-3f * (float)(8 - i));
  }
  f32x16 acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[c][j];
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

constexpr int kChunkBytes = 36 * 1024;   // one decode tile's bytes
constexpr int kChunkCopies = kChunkBytes / 1024 / 4;  // copies per wave per chunk (four waves)

#define LDS_AS __attribute__((address_space(3)))
__device__ __forceinline__ void dma16(const void* gaddr, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gaddr), "s"(lds)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Workgroup g reads chunks g, g + G, ... (G workgroups) through a four-slot LDS ring, three in
// flight; thread 0 XORs the first word of every chunk that lands into out[g].
__global__ __launch_bounds__(256) void read_rate_kernel(const char* __restrict__ buf, long long nchunks, int* out) {
  __shared__ __attribute__((aligned(1024))) char ring[4][kChunkBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long first = blockIdx.x, step = gridDim.x;
  const long long mine = first < nchunks ? (nchunks - first + step - 1) / step : 0;
  const unsigned ring0 = (unsigned)(uintptr_t)(LDS_AS char*)ring[0];
  auto issue = [&](long long k) {
    const char* src = buf + (size_t)(first + k * step) * kChunkBytes;
    const unsigned lds = ring0 + (unsigned)(k & 3) * kChunkBytes;
#pragma unroll
    for (int j = 0; j < kChunkCopies; ++j) {
      const int blk = wave * kChunkCopies + j;
      dma16(src + blk * 1024 + 16 * lane, lds + blk * 1024);
    }
  };
  for (long long k = 0; k < 3 && k < mine; ++k) issue(k);
  unsigned acc = 0;
  for (long long k = 0; k < mine; ++k) {
    // chunk k has landed once only the chunks issued after it are outstanding
    const long long younger = (mine - 1 - k) < 2 ? (mine - 1 - k) : 2;
    if (younger == 2) wait_vmcnt<2 * kChunkCopies>();
    else if (younger == 1) wait_vmcnt<kChunkCopies>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (threadIdx.x == 0) acc ^= *reinterpret_cast<const unsigned*>(ring[k & 3]);
    // slot (k + 3) & 3 held chunk k - 1, read before the barrier above
    if (k + 3 < mine) issue(k + 3);
  }
  wait_vmcnt<0>();
  if (threadIdx.x == 0) out[blockIdx.x] = (int)acc;
}

}  // namespace

hipError_t launch_read_rate(const void* buf, size_t bytes, int* out, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(read_rate_kernel, dim3(blocks), dim3(256), 0, s, (const char*)buf,
                     (long long)(bytes / kChunkBytes), out);
  return hipGetLastError();
}

hipError_t launch_mfma_rate(float* out, int blocks, int iters, hipStream_t s) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(256), 0, s, out, iters);
  return hipGetLastError();
}

}  // namespace mla
