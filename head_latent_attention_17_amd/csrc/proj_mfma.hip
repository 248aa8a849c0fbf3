// Per-head projections on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16):
//   absorb:   q_lat[b][h][:] = q_nope[b][h][:] (128) @ W_UK[h] (128 x 512)
//   out-proj: out[b][h][:]   = o_lat[b][h][:]  (512) @ W_UV[h] (512 x 128)
// (DeepSeek-V2 explainer, Step 6: the query side absorbs W_UK, the output side applies W_UV after
// the weighted sum.)  Both are C[b][n] = sum_k A[b][k] W[k][n] per head with M = batch; each weight
// matrix is read from HBM once per launch and is the dominant traffic, so the kernel streams W
// through LDS in 128-row chunks and applies every chunk to the whole batch.
//
// Operands of the 32x32x16 MFMA: A (batch rows x 16 k) comes straight from global memory, 8
// consecutive k per lane; B (16 k x 32 n) needs 8 consecutive k of one column n per lane, while W
// is stored with n contiguous, so it is fetched from the LDS copy of the chunk with two 16-lane
// transposing reads (ds_read_b64_tr_b16).  Rows of the LDS chunk are padded by 32 bytes so the
// four rows touched by one 16-lane read fall on different banks.
#include "mla_device.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
#define LDS_AS __attribute__((address_space(3)))

constexpr int kKChunk = 128;                 // W rows staged per step
constexpr int kNTile = 64;                   // W columns per workgroup
constexpr int kRowBytes = kNTile * 2 + 32;   // padded LDS row: 160 bytes
constexpr int kMaxMBlocks = 4;               // 32-row batch blocks held per wave (two waves per column block)

// One workgroup: head h, columns [n0, n0 + 64).  Wave w: column block (w & 1), batch blocks
// (w >> 1), (w >> 1) + 2, ...  Batches above 256 rows take further passes over W.
template <int K, int N>
__global__ __launch_bounds__(256) void head_gemm_kernel(const uint16_t* __restrict__ a, int lda,
                                                        const uint16_t* __restrict__ w,
                                                        uint16_t* __restrict__ c, int ldc,
                                                        int batch, int heads) {
  __shared__ __attribute__((aligned(16))) char wt[2][kKChunk * kRowBytes];
  const int h = blockIdx.x;
  const int n0 = blockIdx.y * kNTile;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int nb = wave & 1;
  const int mpar = wave >> 1;
  const uint16_t* wh = w + (size_t)h * K * N;
  if (K == kDnope && blockIdx.y == 0) {
    // absorption only: q^R passes through unchanged, q_abs[b][h][512:576] = q[b][h][128:192]
    for (int i = tid; i < batch * 8; i += 256) {
      const int r = i >> 3, part = i & 7;
      *reinterpret_cast<uint4*>(c + ((size_t)r * heads + h) * ldc + kDc + part * 8) =
          *reinterpret_cast<const uint4*>(a + ((size_t)r * heads + h) * lda + kDnope + part * 8);
    }
  }

  // transposing-read lane base: row k = 8 half + 4 r + (lane & 15) / 4, column 32 nb + 16 ((lane >> 4) & 1) + 4 (lane & 3)
  const int tr_row = 8 * half + ((lane & 15) >> 2);
  const int tr_col = 32 * nb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int tr_base = tr_row * kRowBytes + tr_col * 2;

  // W chunk staging: 128 rows x 64 columns = 1024 16-byte pieces, 4 per thread.  The next chunk is
  // fetched into registers before the current one is consumed and written to LDS afterwards.
  uint4 pre[4];
  auto fetch_chunk = [&](int kc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int piece = tid + 256 * i;
      pre[i] = *reinterpret_cast<const uint4*>(wh + (size_t)(kc + (piece >> 3)) * N + n0 + (piece & 7) * 8);
    }
  };
  auto store_chunk = [&](char* dst) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int piece = tid + 256 * i;
      *reinterpret_cast<uint4*>(dst + (piece >> 3) * kRowBytes + (piece & 7) * 16) = pre[i];
    }
  };

  for (int m0 = 0; m0 < batch; m0 += 32 * 2 * kMaxMBlocks) {
    f32x16 acc[kMaxMBlocks];
#pragma unroll
    for (int i = 0; i < kMaxMBlocks; ++i) acc[i] = f32x16{};
    fetch_chunk(0);
    store_chunk(wt[0]);
    for (int kc = 0; kc < K; kc += kKChunk) {
      const int buf = (kc / kKChunk) & 1;
      __syncthreads();
      const bool more = kc + kKChunk < K;
      if (more) fetch_chunk(kc + kKChunk);
      const LDS_AS char* tile = (const LDS_AS char*)wt[buf];
#pragma unroll
      for (int ks = 0; ks < kKChunk / 16; ++ks) {
        const LDS_AS char* p0 = tile + tr_base + ks * 16 * kRowBytes;
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)p0);
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(p0 + 4 * kRowBytes));
        const bf16x8 bop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int i = 0; i < kMaxMBlocks; ++i) {
          const int row = m0 + 32 * (mpar + 2 * i) + (lane & 31);
          bf16x8 aop = {};
          if (row < batch)
            aop = *reinterpret_cast<const bf16x8*>(a + ((size_t)row * heads + h) * lda + kc + ks * 16 + 8 * half);
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop, acc[i], 0, 0, 0);
        }
      }
      if (more) store_chunk(wt[buf ^ 1]);
    }
    // acc[i] lane l, register j: row 8 (j / 4) + 4 half + (j % 4) of the block, column l % 32
#pragma unroll
    for (int i = 0; i < kMaxMBlocks; ++i) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int row = m0 + 32 * (mpar + 2 * i) + 8 * (j >> 2) + 4 * half + (j & 3);
        if (row < batch)
          c[((size_t)row * heads + h) * ldc + n0 + 32 * nb + (lane & 31)] = f32_to_bf16(acc[i][j]);
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_absorb_mfma(const void* q, const void* w_uk, void* q_abs, int batch, int heads,
                              hipStream_t s) {
  hipLaunchKernelGGL((head_gemm_kernel<kDnope, kDc>), dim3(heads, kDc / kNTile), dim3(256), 0, s,
                     (const uint16_t*)q, kQdim, (const uint16_t*)w_uk, (uint16_t*)q_abs, kRow, batch,
                     heads);
  return hipGetLastError();
}

hipError_t launch_out_proj_mfma(const void* o_lat, const void* w_uv, void* out, int batch, int heads,
                                hipStream_t s) {
  hipLaunchKernelGGL((head_gemm_kernel<kDc, kDv>), dim3(heads, kDv / kNTile), dim3(256), 0, s,
                     (const uint16_t*)o_lat, kDc, (const uint16_t*)w_uv, (uint16_t*)out, kDv, batch,
                     heads);
  return hipGetLastError();
}

}  // namespace mla
