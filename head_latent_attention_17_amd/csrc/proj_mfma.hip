// Per-head projections on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16):
//   absorb:   q_lat[b][h][:] = q_nope[b][h][:] (128) @ W_UK[h] (128 x 512)
//   out-proj: out[b][h][:]   = o_lat[b][h][:]  (512) @ W_UV[h] (512 x 128)
// (DeepSeek-V2 explainer, Step 6: the query side absorbs W_UK, the output side applies W_UV after
// the weighted sum.)  Both are C[b][n] = sum_k A[b][k] W[k][n] per head with M = batch; each weight
// matrix is read from HBM once per launch and is the dominant traffic, so the kernel streams W
// through LDS in 128-row chunks and applies every chunk to the whole batch.
//
// Work split: one workgroup per (head, 32 output columns), so every weight byte is fetched by
// exactly one workgroup and a launch has heads x N / 32 workgroups (2048 for the absorption, 512
// for the out-projection).  The workgroup's weight slab (K rows x 64 bytes) is copied HBM -> LDS
// in one go with global_load_lds_dwordx4 (16 rows per copy, no registers held), while the batch
// rows of A are fetched straight into registers.  The four waves split K (wave w takes k-steps
// w, w + 4, ...) and their partial 32 x 32 tiles are summed through LDS.
//
// Operands of v_mfma_f32_32x32x16_bf16: A (32 batch rows x 16 k) is 8 consecutive k of one row per
// lane, read from global memory; B (16 k x 32 columns) needs 8 consecutive k of one column per
// lane while W is stored with columns contiguous, so it comes out of the LDS slab with two 16-lane
// transposing reads (ds_read_b64_tr_b16), each giving a lane 4 consecutive rows of its column.
// Slab rows are 64 bytes, so the 4 rows x 32 bytes of one 16-lane read cover 256 consecutive
// bytes: no bank conflicts.
#include "mla_device.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
#define LDS_AS __attribute__((address_space(3)))

constexpr int kNT = 32;  // output columns per workgroup

// One 16-byte-per-lane copy HBM -> LDS: lane l's 16 bytes from gaddr land at LDS byte lds + 16 l.
// As asm the compiler does not track it; the kernel waits for it explicitly (vmcnt(0) + barrier).
// Vector loads complete in issue order, so the compiler's own counted waits for the A loads stay
// correct (they can only become stricter).
__device__ __forceinline__ void dma16(const void* gaddr, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gaddr), "s"(lds)
               : "memory", "m0");
}

// MB = 32-row batch blocks per pass.
template <int K, int N, int MB>
__global__ __launch_bounds__(256) void head_gemm_kernel(const uint16_t* __restrict__ a, int lda,
                                                        const uint16_t* __restrict__ w,
                                                        uint16_t* __restrict__ c, int ldc,
                                                        int batch, int heads) {
  constexpr int kSteps = K / 16;        // k-steps of the product
  constexpr int kPerWave = kSteps / 4;  // k-steps per wave
  __shared__ __attribute__((aligned(1024))) char slab[K * 64];
  __shared__ __attribute__((aligned(16))) float red[4][32 * 32];
  const int h = blockIdx.x;
  const int n0 = blockIdx.y * kNT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;

  // Weight slab: copy j of this wave moves rows 16 (4 j + wave) .. + 15, 64 bytes each.
  {
    const uint16_t* wh = w + (size_t)h * K * N + n0;
    const unsigned lds0 = (unsigned)(uintptr_t)(LDS_AS char*)slab;
#pragma unroll
    for (int j = 0; j < K / 64; ++j) {
      const int r0 = 16 * (4 * j + wave);
      dma16(wh + (size_t)(r0 + (lane >> 2)) * N + 8 * (lane & 3), lds0 + r0 * 64);
    }
  }
  if (K == kDnope && blockIdx.y == 0) {
    // absorption only: q^R passes through unchanged, q_abs[b][h][512:576] = q[b][h][128:192]
    for (int i = tid; i < batch * 8; i += 256) {
      const int r = i >> 3, part = i & 7;
      *reinterpret_cast<uint4*>(c + ((size_t)r * heads + h) * ldc + kDc + part * 8) =
          *reinterpret_cast<const uint4*>(a + ((size_t)r * heads + h) * lda + kDnope + part * 8);
    }
  }

  // Transposing-read address of this lane (row within a k-step, byte within a row): rows
  // 8 half + (lane % 16) / 4 (+ 4 for the second read), columns 16 ((lane / 16) % 2) + 4 (lane % 4).
  const unsigned tr_off = (unsigned)(uintptr_t)(LDS_AS char*)slab +
                          (8 * half + ((lane & 15) >> 2)) * 64 + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);

  for (int m0 = 0; m0 < batch; m0 += 32 * MB) {
    f32x16 acc[MB];
    bf16x8 aop[MB][kPerWave];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      acc[mb] = f32x16{};
      const int row = m0 + 32 * mb + (lane & 31);
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) {
        const int ks = wave + 4 * i;
        aop[mb][i] = bf16x8{};
        if (row < batch)
          aop[mb][i] = *reinterpret_cast<const bf16x8*>(a + ((size_t)row * heads + h) * lda + 16 * ks + 8 * half);
      }
    }
    if (m0 == 0) {
      __builtin_amdgcn_s_waitcnt(0);  // every copy (and load) of this wave has landed
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int ks = wave + 4 * i;
      const LDS_AS char* p0 = (const LDS_AS char*)(uintptr_t)tr_off + ks * 16 * 64;
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)p0);
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(p0 + 4 * 64));
      const bf16x8 bop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[mb][i], bop, acc[mb], 0, 0, 0);
    }
    // Sum the four waves' partial tiles: acc lane l, register j is row 8 (j / 4) + 4 half + j % 4,
    // column l % 32.  Thread t then owns row t / 8, columns 4 (t % 8) .. + 3.
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (m0 + 32 * mb >= batch) break;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        red[wave][(8 * (j >> 2) + 4 * half + (j & 3)) * 32 + (lane & 31)] = acc[mb][j];
      __syncthreads();
      const int r = tid >> 3, c4 = 4 * (tid & 7);
      float4 sum = *reinterpret_cast<const float4*>(&red[0][r * 32 + c4]);
#pragma unroll
      for (int q = 1; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(&red[q][r * 32 + c4]);
        sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
      }
      const int row = m0 + 32 * mb + r;
      if (row < batch) {
        uint2 packed;
        packed.x = (uint32_t)f32_to_bf16(sum.x) | ((uint32_t)f32_to_bf16(sum.y) << 16);
        packed.y = (uint32_t)f32_to_bf16(sum.z) | ((uint32_t)f32_to_bf16(sum.w) << 16);
        *reinterpret_cast<uint2*>(c + ((size_t)row * heads + h) * ldc + n0 + c4) = packed;
      }
      __syncthreads();
    }
  }
}

template <int K, int N>
void launch_gemm(const void* a, int lda, const void* w, void* c, int ldc, int batch, int heads, hipStream_t s) {
  const dim3 grid(heads, N / kNT);
  const uint16_t* A = (const uint16_t*)a;
  const uint16_t* W = (const uint16_t*)w;
  uint16_t* C = (uint16_t*)c;
  if (batch <= 32)
    hipLaunchKernelGGL((head_gemm_kernel<K, N, 1>), grid, dim3(256), 0, s, A, lda, W, C, ldc, batch, heads);
  else if (batch <= 64)
    hipLaunchKernelGGL((head_gemm_kernel<K, N, 2>), grid, dim3(256), 0, s, A, lda, W, C, ldc, batch, heads);
  else
    hipLaunchKernelGGL((head_gemm_kernel<K, N, 4>), grid, dim3(256), 0, s, A, lda, W, C, ldc, batch, heads);
}

}  // namespace

hipError_t launch_absorb_mfma(const void* q, const void* w_uk, void* q_abs, int batch, int heads,
                              hipStream_t s) {
  launch_gemm<kDnope, kDc>(q, kQdim, w_uk, q_abs, kRow, batch, heads, s);
  return hipGetLastError();
}

hipError_t launch_out_proj_mfma(const void* o_lat, const void* w_uv, void* out, int batch, int heads,
                                hipStream_t s) {
  launch_gemm<kDc, kDv>(o_lat, kDc, w_uv, out, kDv, batch, heads, s);
  return hipGetLastError();
}

}  // namespace mla
