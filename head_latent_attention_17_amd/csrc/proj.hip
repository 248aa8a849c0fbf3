// Cache append, and the fp32 (debug-mode) versions of the two per-head projections around the
// latent decode; the bf16 projections run on the matrix cores (proj_mfma.hip):
//   absorb:   q_lat = q_nope @ W_UK[h]    (the query moved into latent space; DeepSeek-V2 explainer, Step 6)
//   out-proj: out   = o_lat  @ W_UV[h]    (the value up-projection applied after the weighted sum, Step 6)
#include "mla_device.h"

namespace mla {

// ---------------------------------------------------------------------------------------------
// Append: one 1152-byte row per sequence, copied bit for bit into its page slot.
// ---------------------------------------------------------------------------------------------

template <typename T>
__global__ __launch_bounds__(128) void append_kernel(uint16_t* cache, const int32_t* block_table,
                                                     int max_blocks, const int32_t* positions,
                                                     const T* c_new, const T* kpe_new) {
  const int b = blockIdx.x;
  const int c = threadIdx.x;  // 16-byte chunk of the row: 0..63 latent, 64..71 RoPE key
  if (c >= kRow / 8) return;
  const int pos = positions[b];
  const int page = block_table[(size_t)b * max_blocks + pos / kPage];
  uint16_t* row = cache + ((size_t)page * kPage + (pos % kPage)) * kRow;
  uint16_t v[8];
  if constexpr (sizeof(T) == 2) {
    const T* src = (c < kDc / 8) ? c_new + (size_t)b * kDc + c * 8 : kpe_new + (size_t)b * kDr + (c - kDc / 8) * 8;
    *reinterpret_cast<uint4*>(v) = *reinterpret_cast<const uint4*>(src);
  } else {
    const float* src = (c < kDc / 8) ? c_new + (size_t)b * kDc + c * 8 : kpe_new + (size_t)b * kDr + (c - kDc / 8) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (uint16_t)(__float_as_uint(src[i]) >> 16);
  }
  *reinterpret_cast<uint4*>(row + c * 8) = *reinterpret_cast<const uint4*>(v);
}

hipError_t launch_append(void* cache, const int32_t* block_table, int max_blocks,
                         const int32_t* positions, const void* c_new, const void* kpe_new,
                         int batch, bool f32, hipStream_t s) {
  if (f32)
    hipLaunchKernelGGL(append_kernel<float>, dim3(batch), dim3(128), 0, s, (uint16_t*)cache,
                       block_table, max_blocks, positions, (const float*)c_new, (const float*)kpe_new);
  else
    hipLaunchKernelGGL(append_kernel<uint16_t>, dim3(batch), dim3(128), 0, s, (uint16_t*)cache,
                       block_table, max_blocks, positions, (const uint16_t*)c_new,
                       (const uint16_t*)kpe_new);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Absorb (vector ALU): one workgroup per (head, 64 latent columns); the 128 x 64 weight tile is
// staged in LDS as fp32 and applied to every sequence of the batch.
// ---------------------------------------------------------------------------------------------

template <typename T>
__global__ __launch_bounds__(256) void absorb_valu_kernel(const T* q, const T* w_uk, T* q_abs,
                                                          int batch, int heads) {
  __shared__ float w_s[kDnope][64];
  const int h = blockIdx.x;
  const int c0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  for (int i = tid; i < kDnope * 64; i += 256) {
    const int k = i / 64, n = i % 64;
    w_s[k][n] = Elem<T>::load(w_uk, ((size_t)h * kDnope + k) * kDc + c0 + n);
  }
  __syncthreads();
  const int n = tid & 63;
  for (int b = tid >> 6; b < batch; b += 4) {
    const size_t qb = ((size_t)b * heads + h) * kQdim;
    float acc = 0.f;
#pragma unroll 8
    for (int k = 0; k < kDnope; ++k) acc = fmaf(Elem<T>::load(q, qb + k), w_s[k][n], acc);
    Elem<T>::store(q_abs, ((size_t)b * heads + h) * kRow + c0 + n, acc);
  }
  if (blockIdx.y == 0) {  // q^R passes through unchanged
    for (int i = tid; i < batch * kDr; i += 256) {
      const int b = i / kDr, j = i % kDr;
      q_abs[((size_t)b * heads + h) * kRow + kDc + j] = q[((size_t)b * heads + h) * kQdim + kDnope + j];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Out-projection (vector ALU): one workgroup per (head, 32 output columns); the 512 x 32 weight
// tile sits in LDS as fp32 (64 KB).
// ---------------------------------------------------------------------------------------------

template <typename T>
__global__ __launch_bounds__(256) void out_proj_valu_kernel(const T* o_lat, const T* w_uv, T* out,
                                                            int batch, int heads) {
  extern __shared__ float w_dyn[];
  float (*w_s)[32] = reinterpret_cast<float (*)[32]>(w_dyn);
  const int h = blockIdx.x;
  const int c0 = blockIdx.y * 32;
  const int tid = threadIdx.x;
  for (int i = tid; i < kDc * 32; i += 256) {
    const int k = i / 32, n = i % 32;
    w_s[k][n] = Elem<T>::load(w_uv, ((size_t)h * kDc + k) * kDv + c0 + n);
  }
  __syncthreads();
  const int n = tid & 31;
  for (int b = tid >> 5; b < batch; b += 8) {
    const size_t ob = ((size_t)b * heads + h) * kDc;
    float acc = 0.f;
#pragma unroll 8
    for (int k = 0; k < kDc; ++k) acc = fmaf(Elem<T>::load(o_lat, ob + k), w_s[k][n], acc);
    Elem<T>::store(out, ((size_t)b * heads + h) * kDv + c0 + n, acc);
  }
}

hipError_t launch_absorb_mfma(const void* q, const void* w_uk, void* q_abs, int batch, int heads,
                              hipStream_t s);
hipError_t launch_out_proj_mfma(const void* o_lat, const void* w_uv, void* out, int batch, int heads,
                                hipStream_t s);

hipError_t launch_absorb(const void* q, const void* w_uk, void* q_abs, int batch, int heads,
                         bool f32, hipStream_t s) {
  if (!f32) return launch_absorb_mfma(q, w_uk, q_abs, batch, heads, s);
  // fp32 debug mode: vector ALU, fp32 products and sums
  hipLaunchKernelGGL(absorb_valu_kernel<float>, dim3(heads, kDc / 64), dim3(256), 0, s,
                     (const float*)q, (const float*)w_uk, (float*)q_abs, batch, heads);
  return hipGetLastError();
}

hipError_t launch_out_proj(const void* o_lat, const void* w_uv, void* out, int batch, int heads,
                           bool f32, hipStream_t s) {
  if (!f32) return launch_out_proj_mfma(o_lat, w_uv, out, batch, heads, s);
  // fp32 debug mode: vector ALU, fp32 products and sums
  hipLaunchKernelGGL(out_proj_valu_kernel<float>, dim3(heads, kDv / 32), dim3(256),
                     (size_t)kDc * 32 * sizeof(float), s, (const float*)o_lat, (const float*)w_uv,
                     (float*)out, batch, heads);
  return hipGetLastError();
}

}  // namespace mla
