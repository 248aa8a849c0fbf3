// Per-head projections on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16):
//   absorb:   q_lat[b][h][:] = q_nope[b][h][:] (128) @ W_UK[h] (128 x 512)
//   out-proj: out[b][h][:]   = o_lat[b][h][:]  (512) @ W_UV[h] (512 x 128)
// (DeepSeek-V2 explainer, Step 6: the query side absorbs W_UK, the output side applies W_UV after
// the weighted sum.)  Both are C[b][n] = sum_k A[b][k] W[k][n] per head with M = batch; each weight
// matrix is read from HBM once per launch and is the dominant traffic, so each workgroup copies its
// slice of W to LDS once and applies it to the whole batch.
//
// Work split: one workgroup per (head, 32 NB output columns), so every weight byte is fetched by
// exactly one workgroup (the absorption's own kernel below: 512 or 256 workgroups; the
// out-projection: 512 with NB = 1).  The workgroup's weight slab (K rows x 64 NB bytes) is copied HBM -> LDS in one
// go with global_load_lds_dwordx4 (1 KB per copy, no registers held), while the batch rows of A are
// fetched straight into registers.  The four waves split the column blocks and K; partial tiles of
// one column block are summed through LDS.
//
// Operands of v_mfma_f32_32x32x16_bf16: A (32 batch rows x 16 k) is 8 consecutive k of one row per
// lane, read from global memory; B (16 k x 32 columns) needs 8 consecutive k of one column per
// lane while W is stored with columns contiguous, so it comes out of the LDS slab with two 16-lane
// transposing reads (ds_read_b64_tr_b16), each giving a lane 4 consecutive rows of its column.
// With 64-byte slab rows the 4 rows x 32 bytes of one 16-lane read cover 256 consecutive bytes: no
// bank conflicts; wider rows are swizzled to the same effect.
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

// MB = 32-row batch blocks per pass; NB = 32-column blocks per workgroup.  The four waves are NB
// column blocks x (4 / NB) slices of K; with more than one slice their partial tiles are summed
// through LDS.  A slab row is 64 NB bytes; for NB > 1 the 16-byte units of row r are stored XOR
// g(r) = 2 ((r 64 NB / 256) mod 4) so that the four rows of one transposing read fall on different
// banks.
template <int NB>
__device__ __forceinline__ int slab_swz(int r) {
  constexpr int U = 4 * NB;  // 16-byte units per slab row
  return NB == 1 ? 0 : ((2 * ((r * U / 16) & 3)) & (U - 1));
}

template <int K, int N, int MB, int NB>
__global__ __launch_bounds__(256) void head_gemm_kernel(const uint16_t* __restrict__ a, int lda,
                                                        const uint16_t* __restrict__ w,
                                                        uint16_t* __restrict__ c, int ldc,
                                                        int batch, int heads) {
  constexpr int KS = 4 / NB;            // K slices
  constexpr int RB = 64 * NB;           // slab row bytes
  constexpr int U = RB / 16;            // 16-byte units per slab row
  constexpr int kSteps = K / 16;        // k-steps of the product
  constexpr int kPerWave = kSteps / KS; // k-steps per wave
  constexpr int kCopies = K * RB / 1024;
  __shared__ __attribute__((aligned(1024))) char slab[K * RB];
  __shared__ __attribute__((aligned(16))) float red[KS > 1 ? 4 : 1][32 * 32];
  const int h = blockIdx.x;
  const int n0 = blockIdx.y * kNT * NB;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int cb = wave % NB;             // column block of this wave
  const int ksl = wave / NB;            // K slice of this wave

  // Weight slab: copy i moves 1024 / RB rows; lane l fetches unit (l % U) ^ g(row) of row l / U.
  {
    const uint16_t* wh = w + (size_t)h * K * N + n0;
    const unsigned lds0 = (unsigned)(uintptr_t)(LDS_AS char*)slab;
#pragma unroll
    for (int i = wave; i < kCopies; i += 4) {
      const int r = i * (1024 / RB) + lane / U;
      const int u = (lane % U) ^ slab_swz<NB>(r);
      dma16(wh + (size_t)r * N + 8 * u, lds0 + i * 1024);
    }
  }

  // Transposing reads: row 8 half + (lane % 16) / 4 of a k-step (+ 4 for the second read), logical
  // unit 4 cb + 2 ((lane / 16) % 2) + (lane % 4) / 2, byte 8 (lane % 2).  g(row) repeats every 16
  // rows, so a k-step is an immediate offset.
  unsigned tr_off[2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int r = 8 * half + ((lane & 15) >> 2) + 4 * rd;
    const int u = 4 * cb + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    tr_off[rd] = (unsigned)(uintptr_t)(LDS_AS char*)slab + r * RB + 16 * (u ^ slab_swz<NB>(r)) + 8 * (lane & 1);
  }

  for (int m0 = 0; m0 < batch; m0 += 32 * MB) {
    f32x16 acc[MB];
    bf16x8 aop[MB][kPerWave];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      acc[mb] = f32x16{};
      const int row = m0 + 32 * mb + (lane & 31);
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) {
        const int ks = ksl + KS * i;
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
      const int ks = ksl + KS * i;
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS char*)(uintptr_t)tr_off[0] + ks * 16 * RB));
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS char*)(uintptr_t)tr_off[1] + ks * 16 * RB));
      const bf16x8 bop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[mb][i], bop, acc[mb], 0, 0, 0);
    }
    // acc lane l, register j is row 8 (j / 4) + 4 half + j % 4, column l % 32 of this wave's block.
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (m0 + 32 * mb >= batch) break;
      if constexpr (KS == 1) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int row = m0 + 32 * mb + 8 * (j >> 2) + 4 * half + (j & 3);
          if (row < batch) c[((size_t)row * heads + h) * ldc + n0 + 32 * cb + (lane & 31)] = f32_to_bf16(acc[mb][j]);
        }
      } else {
        // Sum the K slices through LDS: thread t then owns row t / 8 of column block (t / 8) ..
#pragma unroll
        for (int j = 0; j < 16; ++j)
          red[wave][(8 * (j >> 2) + 4 * half + (j & 3)) * 32 + (lane & 31)] = acc[mb][j];
        __syncthreads();
        // 32 x 32 NB outputs, 256 threads: thread t covers column block t % NB, row (t / NB) % 32,
        // columns 4 ((t / (32 NB)) ..) in steps; done as NB x 32 rows x 8 groups of 4 columns.
#pragma unroll
        for (int e = tid; e < NB * 32 * 8; e += 256) {
          const int blk = e / (32 * 8), r = (e / 8) % 32, c4 = 4 * (e % 8);
          float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
          for (int q = 0; q < KS; ++q) {
            const float4 v = *reinterpret_cast<const float4*>(&red[q * NB + blk][r * 32 + c4]);
            sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
          }
          const int row = m0 + 32 * mb + r;
          if (row < batch) {
            uint2 packed;
            packed.x = (uint32_t)f32_to_bf16(sum.x) | ((uint32_t)f32_to_bf16(sum.y) << 16);
            packed.y = (uint32_t)f32_to_bf16(sum.z) | ((uint32_t)f32_to_bf16(sum.w) << 16);
            *reinterpret_cast<uint2*>(c + ((size_t)row * heads + h) * ldc + n0 + 32 * blk + c4) = packed;
          }
        }
        __syncthreads();
      }
    }
  }
}

// Absorption: one workgroup of NB waves per (head, 32 NB latent columns), wave w owning column
// block w over the whole K = 128, so no partial tiles are summed.  The batch rows' q_nope (256
// contiguous bytes each) are copied to LDS 64 rows at a time, 16 lanes per row, so that a copy
// touches four rows (eight 128-byte lines) where an operand load straight from memory touched 32
// rows 49 KB apart; their 16-byte units are XOR-swizzled by row so that the operand reads
// (ds_read_b128, 32 rows of one unit) hit 16 different bank groups.  Results pass through LDS and
// leave as 64 NB-byte row segments of q_abs.
// Slab rows of 256 or 512 bytes: the 16-byte units of row r are stored XOR 2 (r mod 4), so the four
// rows x 32 bytes of one 16-lane transposing read fall in one 128-byte span of distinct banks.
__device__ __forceinline__ int absorb_swz(int r) { return 2 * (r & 3); }

template <int NB>
__global__ __launch_bounds__(64 * NB) void absorb_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ w,
                                                         uint16_t* __restrict__ qa, int batch, int heads) {
  constexpr int K = kDnope, N = kDc;
  constexpr int RB = 64 * NB;            // slab row bytes
  constexpr int U = RB / 16;             // 16-byte units per slab row
  constexpr int kCopies = K * RB / 1024;
  constexpr int kRows = 64;              // batch rows per pass
  constexpr int OU = 4 * NB;             // 16-byte units of one output row segment
  __shared__ __attribute__((aligned(1024))) char slab[K * RB];
  __shared__ __attribute__((aligned(1024))) char arows[kRows * 256];
  __shared__ __attribute__((aligned(16))) uint16_t obuf[kRows * 32 * NB];
  const int h = blockIdx.x;
  const int n0 = blockIdx.y * 32 * NB;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const unsigned slab0 = (unsigned)(uintptr_t)(LDS_AS char*)slab;
  const unsigned arows0 = (unsigned)(uintptr_t)(LDS_AS char*)arows;

  {
    const uint16_t* wh = w + (size_t)h * K * N + n0;
#pragma unroll
    for (int i = wave; i < kCopies; i += NB) {
      const int r = i * (1024 / RB) + lane / U;
      const int u = (lane % U) ^ absorb_swz(r);
      dma16(wh + (size_t)r * N + 8 * u, slab0 + i * 1024);
    }
  }
  // Rows m0 .. m0 + 63 of q_nope: copy i moves rows 4 i .. 4 i + 3; copies past the batch are
  // skipped (those LDS rows feed only result rows that are never stored).
  auto copy_rows = [&](int m0) {
    const int rows = min(kRows, batch - m0);
    for (int i = wave; 4 * i < rows; i += NB) {
      const int rl = 4 * i + (lane >> 4);
      const int row = min(m0 + rl, batch - 1);
      const int u = (lane & 15) ^ (rl & 15);
      dma16(q + ((size_t)row * heads + h) * kQdim + 8 * u, arows0 + i * 1024);
    }
  };
  copy_rows(0);
  if (blockIdx.y == 0) {
    // q^R passes through unchanged: q_abs[b][h][512:576] = q[b][h][128:192]
    for (int i = tid; i < batch * 8; i += 64 * NB) {
      const int r = i >> 3, part = i & 7;
      *reinterpret_cast<uint4*>(qa + ((size_t)r * heads + h) * kRow + kDc + part * 8) =
          *reinterpret_cast<const uint4*>(q + ((size_t)r * heads + h) * kQdim + kDnope + part * 8);
    }
  }

  // Transposing reads of the slab, as in head_gemm_kernel: rows 8 half + (lane % 16) / 4 (+ 4),
  // logical unit 4 w + 2 ((lane / 16) % 2) + (lane % 4) / 2, byte 8 (lane % 2); the swizzle repeats
  // every 16 rows, so a k-step is an immediate offset.
  unsigned tr_off[2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int r = 8 * half + ((lane & 15) >> 2) + 4 * rd;
    const int u = 4 * wave + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    tr_off[rd] = slab0 + r * RB + 16 * (u ^ absorb_swz(r)) + 8 * (lane & 1);
  }

  for (int m0 = 0;;) {
    __builtin_amdgcn_s_waitcnt(0);  // every copy of this wave has landed
    __syncthreads();
    const bool two = batch - m0 > 32;
    f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < K / 16; ++ks) {
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS char*)(uintptr_t)tr_off[0] + ks * 16 * RB));
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS char*)(uintptr_t)tr_off[1] + ks * 16 * RB));
      const bf16x8 bop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      // A operand: row (lane % 32) of the block, unit 2 ks + half
      const int au = ((2 * ks + half) ^ (lane & 15)) * 16;
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&arows[(lane & 31) * 256 + au]);
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bop, acc[0], 0, 0, 0);
      if (two) {
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&arows[(32 + (lane & 31)) * 256 + au]);
        acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bop, acc[1], 0, 0, 0);
      }
    }
    // acc lane l, register j: row 8 (j / 4) + 4 half + j % 4 of the block, column l % 32 of block w
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      if (mb == 1 && !two) break;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        obuf[(32 * mb + 8 * (j >> 2) + 4 * half + (j & 3)) * 32 * NB + 32 * wave + (lane & 31)] = f32_to_bf16(acc[mb][j]);
    }
    __syncthreads();
    const int rows = min(kRows, batch - m0);
    for (int e = tid; e < rows * OU; e += 64 * NB) {
      const int rl = e / OU, u = e % OU;
      *reinterpret_cast<uint4*>(qa + ((size_t)(m0 + rl) * heads + h) * kRow + n0 + 8 * u) =
          *reinterpret_cast<const uint4*>(&obuf[rl * 32 * NB + 8 * u]);
    }
    m0 += kRows;
    if (m0 >= batch) break;
    copy_rows(m0);  // every wave is past this pass's operand reads (the barrier above)
  }
}

// Column blocks per workgroup, measured on the MI355X at batch 4 to 128 with weights that do not
// stay in the Infinity Cache between calls.  Out-projection: one (512 workgroups, four K slices),
// against one to sixteen.  Absorption (60 weight copies in turn, per call): 256 columns per
// workgroup (256 workgroups of eight waves) above 32 rows, 7.8 us at batch 64 and 10.9 us at 128
// against 8.1 / 11.7 us with 128 columns and 8.4 / 12.4 us with 64; 128 columns (512 workgroups
// of four waves) up to 32 rows, 6.1 us at batch 32 against 6.3 / 6.1 us.
#ifndef MLA_NB_OUT
#define MLA_NB_OUT 1
#endif

template <int K, int N, int NB>
void launch_gemm(const void* a, int lda, const void* w, void* c, int ldc, int batch, int heads, hipStream_t s) {
  const dim3 grid(heads, N / (kNT * NB));
  const uint16_t* A = (const uint16_t*)a;
  const uint16_t* W = (const uint16_t*)w;
  uint16_t* C = (uint16_t*)c;
  if (batch <= 32)
    hipLaunchKernelGGL((head_gemm_kernel<K, N, 1, NB>), grid, dim3(256), 0, s, A, lda, W, C, ldc, batch, heads);
  else if (batch <= 64)
    hipLaunchKernelGGL((head_gemm_kernel<K, N, 2, NB>), grid, dim3(256), 0, s, A, lda, W, C, ldc, batch, heads);
  else
    hipLaunchKernelGGL((head_gemm_kernel<K, N, 4, NB>), grid, dim3(256), 0, s, A, lda, W, C, ldc, batch, heads);
}

}  // namespace

hipError_t launch_absorb_mfma(const void* q, const void* w_uk, void* q_abs, int batch, int heads,
                              hipStream_t s) {
  const uint16_t* Q = (const uint16_t*)q;
  const uint16_t* W = (const uint16_t*)w_uk;
  uint16_t* QA = (uint16_t*)q_abs;
  if (batch <= 32)
    hipLaunchKernelGGL(absorb_kernel<4>, dim3(heads, kDc / 128), dim3(256), 0, s, Q, W, QA, batch, heads);
  else
    hipLaunchKernelGGL(absorb_kernel<8>, dim3(heads, kDc / 256), dim3(512), 0, s, Q, W, QA, batch, heads);
  return hipGetLastError();
}

hipError_t launch_out_proj_mfma(const void* o_lat, const void* w_uv, void* out, int batch, int heads,
                                hipStream_t s) {
  launch_gemm<kDc, kDv, MLA_NB_OUT>(o_lat, kDc, w_uv, out, kDv, batch, heads, s);
  return hipGetLastError();
}

}  // namespace mla
