// The producer side of the cache (DeepSeek-V2 explainer, Step 5, eq. 9: a token's hidden vector h is
// squeezed to the latent note c = W^DKV h, 5,120 -> 512; Step 7: the token also contributes one
// 64-dim key k^R, rotated by its position and shared by all heads).  The row [c | RoPE(W^KR h)] is
// written to the token's slot of the paged cache, as mla_cache_append writes a given row.
//
// Both products read weights far larger than the batch rows (5,120 x 576 bf16 = 5.9 MB), so the
// work is split along K: workgroup (k-chunk, 32 columns) multiplies 512 rows of h against a
// 512 x 32 slab of one weight matrix on the bf16 matrix cores and writes an fp32 partial tile; a
// second kernel sums the ten partials of each row, rotates the key in double precision and writes
// the bf16 row.  fp32 mode (a debug mode) computes the sums directly on the vector ALUs.
//
// Rotation (the pages give neither the frequencies nor the pairing; the plain rotary form): pair
// (2i, 2i + 1) of the key turns by position * base^(-2i / 64) radians.
#include "mla_device.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
#define LDS_AS __attribute__((address_space(3)))

constexpr int kDModel = 5120;
constexpr int kKChunk = 512;
constexpr int kKChunks = kDModel / kKChunk;  // 10

// One 16-byte-per-lane copy HBM -> LDS; the kernel waits for it explicitly (vmcnt(0) + barrier).
__device__ __forceinline__ void dma16(const void* gaddr, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gaddr), "s"(lds)
               : "memory", "m0");
}

// part[kc][b][col_off + n0 + j] = sum over k in chunk kc of h[b][k] w[k][n0 + j], j < 32, for the
// weight matrix w [5120][ldw].  Grid (10 chunks, ldw / 32 column blocks), 4 waves each taking a
// quarter of the chunk (8 k-steps); their partial tiles are summed through LDS.  MB 32-row batch
// blocks per pass.
template <int MB>
__global__ __launch_bounds__(256) void hidden_proj_kernel(const uint16_t* __restrict__ h,
                                                          const uint16_t* __restrict__ w, int ldw,
                                                          float* __restrict__ part, int batch,
                                                          int col_off) {
  constexpr int kSteps = kKChunk / 16 / 4;  // k-steps per wave
  __shared__ __attribute__((aligned(1024))) char slab[kKChunk * 64];
  __shared__ __attribute__((aligned(16))) float red[4][32 * 32];
  const int kc = blockIdx.x;
  const int n0 = blockIdx.y * 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  {
    // slab row r = weight row kc * 512 + r, 64 bytes (32 columns); copy i holds rows 16 i .. + 15
    const uint16_t* w0 = w + (size_t)kc * kKChunk * ldw + n0;
    const unsigned lds0 = (unsigned)(uintptr_t)(LDS_AS char*)slab;
#pragma unroll
    for (int i = wave; i < kKChunk * 64 / 1024; i += 4)
      dma16(w0 + (size_t)(16 * i + lane / 4) * ldw + 8 * (lane % 4), lds0 + i * 1024);
  }
  // Transposing reads of the B operand: rows 8 half + (lane % 16) / 4 (+ 4), 16-byte unit
  // 2 ((lane / 16) % 2) + (lane % 4) / 2, byte 8 (lane % 2); 64-byte rows put the four rows of one
  // 16-lane read on different banks.
  unsigned tr_off[2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int r = 8 * half + ((lane & 15) >> 2) + 4 * rd;
    const int u = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    tr_off[rd] = (unsigned)(uintptr_t)(LDS_AS char*)slab + r * 64 + 16 * u + 8 * (lane & 1);
  }
  bool first = true;
  for (int m0 = 0; m0 < batch; m0 += 32 * MB) {
    f32x16 acc[MB];
    bf16x8 aop[MB][kSteps];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      acc[mb] = f32x16{};
      const int row = m0 + 32 * mb + (lane & 31);
#pragma unroll
      for (int i = 0; i < kSteps; ++i) {
        const int ks = wave * kSteps + i;
        aop[mb][i] = bf16x8{};
        if (row < batch)
          aop[mb][i] = *reinterpret_cast<const bf16x8*>(h + (size_t)row * kDModel + kc * kKChunk + 16 * ks + 8 * half);
      }
    }
    if (first) {
      __builtin_amdgcn_s_waitcnt(0);  // every copy (and load) of this wave has landed
      __syncthreads();
      first = false;
    }
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      const int ks = wave * kSteps + i;
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS char*)(uintptr_t)tr_off[0] + ks * 16 * 64));
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS char*)(uintptr_t)tr_off[1] + ks * 16 * 64));
      const bf16x8 bop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[mb][i], bop, acc[mb], 0, 0, 0);
    }
    // acc lane l, register j: row 8 (j / 4) + 4 half + j % 4, column l % 32
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (m0 + 32 * mb >= batch) break;
#pragma unroll
      for (int j = 0; j < 16; ++j) red[wave][(8 * (j >> 2) + 4 * half + (j & 3)) * 32 + (lane & 31)] = acc[mb][j];
      __syncthreads();
      // 32 rows x 32 columns; thread t: row t / 8, columns 4 (t % 8) ..
      const int r = tid >> 3, c4 = 4 * (tid & 7);
      float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(&red[q][r * 32 + c4]);
        sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
      }
      const int row = m0 + 32 * mb + r;
      if (row < batch)
        *reinterpret_cast<float4*>(part + ((size_t)kc * batch + row) * kRow + col_off + n0 + c4) = sum;
      __syncthreads();
    }
  }
}

// fp32 mode: part[0][b][n] = sum_k h[b][k] W[k][n] over all 5,120 k, one thread per (b, n), in fp32.
__global__ __launch_bounds__(256) void hidden_proj_f32_kernel(const float* __restrict__ h,
                                                              const float* __restrict__ w_dkv,
                                                              const float* __restrict__ w_kr,
                                                              float* __restrict__ part, int batch) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  if (n >= kRow) return;
  const float* hr = h + (size_t)b * kDModel;
  float s = 0.f;
  if (n < kDc) {
    for (int k = 0; k < kDModel; ++k) s = fmaf(hr[k], w_dkv[(size_t)k * kDc + n], s);
  } else {
    for (int k = 0; k < kDModel; ++k) s = fmaf(hr[k], w_kr[(size_t)k * kDr + (n - kDc)], s);
  }
  part[(size_t)b * kRow + n] = s;
}

// Row b: sums the `chunks` partials, rotates the key by positions[b] and stores the bf16 row at
// block_table[b][p / 64], slot p % 64.  One workgroup of 576 threads (one per column) per row.
__global__ __launch_bounds__(576) void finish_row_kernel(const float* __restrict__ part, int chunks,
                                                         int batch, const int32_t* __restrict__ positions,
                                                         const int32_t* __restrict__ block_table,
                                                         int max_blocks, uint16_t* __restrict__ cache,
                                                         double base) {
  __shared__ float key[kDr];
  const int b = blockIdx.x;
  const int n = threadIdx.x;
  float s = 0.f;
  for (int c = 0; c < chunks; ++c) s += part[((size_t)c * batch + b) * kRow + n];
  const int pos = positions[b];
  if (n >= kDc) key[n - kDc] = s;
  __syncthreads();
  float v = s;
  if (n >= kDc) {
    const int i = (n - kDc) >> 1;
    const double angle = (double)pos * pow(base, -2.0 * i / kDr);
    double sn, cs;
    sincos(angle, &sn, &cs);
    const double x0 = key[2 * i], x1 = key[2 * i + 1];
    v = (float)(((n - kDc) & 1) ? x0 * sn + x1 * cs : x0 * cs - x1 * sn);
  }
  const int page = block_table[(size_t)b * max_blocks + pos / kPage];
  cache[((size_t)page * kPage + pos % kPage) * kRow + n] = f32_to_bf16(v);
}

}  // namespace

hipError_t launch_append_hidden(void* cache, const int32_t* block_table, int max_blocks,
                                 const int32_t* positions, const void* hidden, const void* w_dkv,
                                 const void* w_kr, double rope_base, int batch, float* part, bool f32,
                                 hipStream_t s) {
  int chunks = 1;
  if (f32) {
    hipLaunchKernelGGL(hidden_proj_f32_kernel, dim3((kRow + 255) / 256, batch), dim3(256), 0, s,
                       (const float*)hidden, (const float*)w_dkv, (const float*)w_kr, part, batch);
  } else {
    chunks = kKChunks;
    const uint16_t* H = (const uint16_t*)hidden;
    if (batch <= 32) {
      hipLaunchKernelGGL(hidden_proj_kernel<1>, dim3(kKChunks, kDc / 32), dim3(256), 0, s, H, (const uint16_t*)w_dkv, kDc, part, batch, 0);
      hipLaunchKernelGGL(hidden_proj_kernel<1>, dim3(kKChunks, kDr / 32), dim3(256), 0, s, H, (const uint16_t*)w_kr, kDr, part, batch, kDc);
    } else {
      hipLaunchKernelGGL(hidden_proj_kernel<2>, dim3(kKChunks, kDc / 32), dim3(256), 0, s, H, (const uint16_t*)w_dkv, kDc, part, batch, 0);
      hipLaunchKernelGGL(hidden_proj_kernel<2>, dim3(kKChunks, kDr / 32), dim3(256), 0, s, H, (const uint16_t*)w_kr, kDr, part, batch, kDc);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(finish_row_kernel, dim3(batch), dim3(kRow), 0, s, part, chunks, batch, positions,
                     block_table, max_blocks, (uint16_t*)cache, rope_base);
  return hipGetLastError();
}

}  // namespace mla
