// The ~6-bit cache (DeepSeek-V2 explainer, the audit after Step 8: deployed V2 keeps each cached
// number in about six bits, near 26 KB per token over 60 layers).  The pages give no format; here a
// number is an FP6 E2M3 code (sign, 2 exponent bits with bias 1, 3 mantissa bits: magnitudes
// 0, 1/8 .. 7/8, 1 .. 7.5) and each row carries one power-of-two scale 2^e, the smallest with the
// row's largest magnitude at most 7.5 * 2^e (e >= -126).  Codes round to nearest, ties to even.
//
// Page layout: 64 rows of 432 bytes (row code i at bits 6i .. 6i+5 of the row's little-endian bit
// string, which is also the operand layout of v_cvt_scalef32_pk32_bf16_fp6), then the 64 row
// scales as float32.  A stored number is code_value * 2^e exactly, and exactly a bf16 number.
//
// A row is quantized by one wave: lane l takes the 4-value groups l, l + 64, l + 128 (< 144) of
// the row, so a group's four codes are three whole bytes.
#include "mla_device.h"

namespace mla {
namespace {

constexpr int kGroups = kRow / 4;  // 144 groups of four numbers = three bytes

// Code of the E2M3 number nearest to y (|y| <= 7.5 after scaling; larger magnitudes saturate),
// ties to even.  Below 2 the grid step is 1/8 (the subnormals and the first binade share it), then
// 1/4 up to 4, then 1/2; the code is the grid index plus 0, 8 or 16, so an even index is an even
// mantissa.  Every product here is by a power of two, hence exact.
__device__ __forceinline__ uint32_t fp6_code(float y) {
  const float a = fminf(fabsf(y), 7.5f);
  uint32_t c;
  if (a < 2.0f) c = (uint32_t)__builtin_rintf(a * 8.0f);
  else if (a < 4.0f) c = 8u + (uint32_t)__builtin_rintf(a * 4.0f);
  else c = 16u + (uint32_t)__builtin_rintf(a * 2.0f);
  return c | (__float_as_uint(y) >> 31 << 5);
}

// Exponent of the row scale from the row's largest magnitude: with amax = m 2^k, m in [0.5, 1),
// amax <= 7.5 2^(k-3) exactly when m <= 0.9375, else 7.5 2^(k-2) holds.
__device__ __forceinline__ int fp6_row_exponent(float amax) {
  if (!(amax > 0.0f)) return -126;
  int k;
  const float m = frexpf(amax, &k);
  const int e = (m <= 0.9375f) ? k - 3 : k - 2;
  return e < -126 ? -126 : e;
}

// Quantizes the row whose groups this lane holds (x[j] = group l + 64 j, valid when l + 64 j < 144)
// into dst (432 bytes) and *scale.
__device__ __forceinline__ void quantize_row(const float (&x)[3][4], uint8_t* dst, float* scale) {
  const int lane = threadIdx.x & 63;
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (lane + 64 * j < kGroups)
#pragma unroll
      for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(x[j][i]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  const int e = fp6_row_exponent(amax);
  const float inv = __builtin_ldexpf(1.0f, -e);
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int g = lane + 64 * j;
    if (g >= kGroups) continue;
    uint32_t bits = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) bits |= fp6_code(x[j][i] * inv) << (6 * i);
    dst[3 * g] = (uint8_t)bits;
    dst[3 * g + 1] = (uint8_t)(bits >> 8);
    dst[3 * g + 2] = (uint8_t)(bits >> 16);
  }
  if (lane == 0) *scale = __builtin_ldexpf(1.0f, e);
}

template <typename T>
__device__ __forceinline__ void load_group(const T* src, float (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = Elem<T>::load(src, i);
}

// One wave per sequence: the row [c_new[b] | kpe_new[b]] is quantized into its slot.
template <typename T>
__global__ __launch_bounds__(64) void append_fp6_kernel(uint8_t* cache, const int32_t* block_table,
                                                        int max_blocks, const int32_t* positions,
                                                        const T* c_new, const T* kpe_new) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int pos = positions[b];
  const int page = block_table[(size_t)b * max_blocks + pos / kPage];
  const int slot = pos % kPage;
  float x[3][4];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int g = lane + 64 * j;
    if (g >= kGroups) continue;
    const T* src = (4 * g < kDc) ? c_new + (size_t)b * kDc + 4 * g : kpe_new + (size_t)b * kDr + (4 * g - kDc);
    load_group(src, x[j]);
  }
  uint8_t* pg = cache + (size_t)page * kFp6PageBytes;
  quantize_row(x, pg + slot * kFp6RowBytes, reinterpret_cast<float*>(pg + kPage * kFp6RowBytes) + slot);
}

// Whole pages: workgroup = 4 waves, one page per workgroup, wave w quantizes rows w, w + 4, ...
__global__ __launch_bounds__(256) void quantize_pages_fp6_kernel(const uint16_t* src, uint8_t* dst) {
  const size_t page = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint8_t* pg = dst + page * kFp6PageBytes;
  for (int t = wave; t < kPage; t += 4) {
    const uint16_t* row = src + (page * kPage + t) * kRow;
    float x[3][4];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int g = lane + 64 * j;
      if (g < kGroups) load_group(row + 4 * g, x[j]);
    }
    quantize_row(x, pg + t * kFp6RowBytes, reinterpret_cast<float*>(pg + kPage * kFp6RowBytes) + t);
  }
}

}  // namespace

hipError_t launch_append_fp6(void* cache, const int32_t* block_table, int max_blocks,
                             const int32_t* positions, const void* c_new, const void* kpe_new, int batch,
                             bool f32, hipStream_t s) {
  if (f32)
    hipLaunchKernelGGL(append_fp6_kernel<float>, dim3(batch), dim3(64), 0, s, (uint8_t*)cache, block_table,
                       max_blocks, positions, (const float*)c_new, (const float*)kpe_new);
  else
    hipLaunchKernelGGL(append_fp6_kernel<uint16_t>, dim3(batch), dim3(64), 0, s, (uint8_t*)cache, block_table,
                       max_blocks, positions, (const uint16_t*)c_new, (const uint16_t*)kpe_new);
  return hipGetLastError();
}

hipError_t launch_quantize_pages_fp6(const void* src, void* dst, int num_pages, hipStream_t s) {
  hipLaunchKernelGGL(quantize_pages_fp6_kernel, dim3(num_pages), dim3(256), 0, s, (const uint16_t*)src,
                     (uint8_t*)dst);
  return hipGetLastError();
}

}  // namespace mla
