// Matrix-core rate calibration: the rate the GPU sustains on v_mfma_f32_32x32x16_bf16 (the
// instruction of the decode's score and output products) when every SIMD issues independent
// products back to back, with no memory traffic and no other instructions in the way.  It is the
// compute ceiling the decode's roofline is read against, next to the data sheet's figure: a large
// library GEMM reaches well below it (its own loads and stores share the time).
//
// Each wave keeps four independent accumulators and issues `iters` x 4 products; lane 0 of wave w
// stores one word derived from the results at out[w], which keeps them live.
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

}  // namespace

hipError_t launch_mfma_rate(float* out, int blocks, int iters, hipStream_t s) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(256), 0, s, out, iters);
  return hipGetLastError();
}

}  // namespace mla
