// Output projection to the hidden width (DeepSeek-V2 explainer, Step 6: the heads' outputs,
// concatenated, are mixed by W^O; W^UV is applied before it, after the weighted sum).
//   hidden[b][n] = sum_k x[b][k] W^O[k][n],  x = out[b] flattened head-major (K = heads * 128),
//   W^O [K][5120] input-major, n < 5120.
// The weights (K x 5,120 bf16: 168 MB at 128 heads) dwarf the batch rows, so the product streams
// them once.  Split along K: workgroup (K chunk of 1,024, 64-column block) walks its chunk in four
// 256-row slabs, each copied HBM -> LDS one slab ahead (LDS-direct loads, double-buffered) and
// multiplied on the bf16 matrix cores against the batch rows, which come from global memory one
// slab ahead into registers; the two K halves of its four waves are summed through LDS into an
// fp32 partial tile.  A second kernel sums the partials in chunk order and rounds to bf16.  Batches
// above 64 rows go through in groups of 64 (each group streams the weights again).
// Batches up to 32 take a wide form instead (dense_proj4_kernel): 128-column blocks whose copies
// move 256 contiguous bytes of each of 4 rows (DRAM sees 256-byte runs instead of 64-byte ones), each
// wave owning 32 columns over the whole chunk.
// fp32 mode (a debug mode) computes each output directly on the vector ALUs.
#include "mla_device.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
#define LDS_AS __attribute__((address_space(3)))

constexpr int kN = 5120;                 // hidden width
constexpr int kSlab = 256;               // weight rows per slab
constexpr int kChunk = 1024;             // weight rows per workgroup
constexpr int kSlabs = kChunk / kSlab;
constexpr int kSteps = kSlab / 16 / 2;   // k-steps per wave and slab (two K halves)

__device__ __forceinline__ void dma16(const void* gaddr, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gaddr), "s"(lds)
               : "memory", "m0");
}

// s_waitcnt vmcnt(n) leaving the other counters alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// part[kc][b][n0 + j] = sum over k in chunk kc of x[b][k] w[k][n0 + j], j < 64, for batch rows
// m0 .. m0 + 32 MB - 1 of each group.  Grid (K / 1024, 5120 / 64).
template <int MB>
__global__ __launch_bounds__(256) void dense_proj_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ w, int K,
                                                         float* __restrict__ part, int batch) {
  // a slab: two planes of 32 columns, 256 rows of 64 bytes each
  __shared__ __attribute__((aligned(1024))) char slab[2][2][kSlab * 64];
  __shared__ __attribute__((aligned(16))) float red[2][32 * 64];
  const int kc = blockIdx.x;
  const int n0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int tile = wave & 1, kh = wave >> 1;
  const uint16_t* wk = w + (size_t)kc * kChunk * kN + n0;
  // copy j of a slab: plane j / 16, rows 16 (j % 16) .. + 15; lane -> row + lane / 4, unit lane % 4
  auto issue_slab = [&](int s, int buf) __attribute__((always_inline)) {
    const unsigned lds0 = (unsigned)(uintptr_t)(LDS_AS char*)&slab[buf][0][0];
#pragma unroll
    for (int j = wave; j < 2 * kSlab / 16; j += 4) {
      const int t = j / (kSlab / 16), i = j % (kSlab / 16);
      dma16(wk + (size_t)(kSlab * s + 16 * i + lane / 4) * kN + 32 * t + 8 * (lane % 4),
            lds0 + t * kSlab * 64 + i * 1024);
    }
  };
  constexpr int kCopies = 2 * kSlab / 16 / 4;  // per wave and slab
  // Transposing reads of the B operand (as in the producer's projection): rows 8 half + (lane % 16)
  // / 4 (+ 4), 16-byte unit 2 ((lane / 16) % 2) + (lane % 4) / 2, byte 8 (lane % 2).
  unsigned tr_off[2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int r = 8 * half + ((lane & 15) >> 2) + 4 * rd;
    const int u = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    tr_off[rd] = (unsigned)(r * 64 + 16 * u + 8 * (lane & 1) + tile * kSlab * 64);
  }
  for (int m0 = 0; m0 < batch; m0 += 32 * MB) {
    f32x16 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16{};
    bf16x8 a_cur[MB][kSteps], a_nxt[MB][kSteps];
    auto load_a = [&](int s, bf16x8 (&a)[MB][kSteps]) __attribute__((always_inline)) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        // Rows past the batch load the last row instead (their sums are never stored): every load
        // is issued, so the counted wait below knows how many are in flight.
        const int row = min(m0 + 32 * mb + (lane & 31), batch - 1);
#pragma unroll
        for (int i = 0; i < kSteps; ++i)
          a[mb][i] = *reinterpret_cast<const bf16x8*>(
              x + (size_t)row * K + kc * kChunk + kSlab * s + 16 * (kh * kSteps + i) + 8 * half);
      }
    };
    __syncthreads();  // the previous group's last slab reads and reduction are done
    issue_slab(0, 0);
    load_a(0, a_cur);
#pragma unroll
    for (int s = 0; s < kSlabs; ++s) {
      if (s + 1 < kSlabs) {
        issue_slab(s + 1, (s + 1) & 1);
        load_a(s + 1, a_nxt);
        // slab s has landed once only slab s + 1's copies and rows may be outstanding
        wait_vmcnt<kCopies + MB * kSteps>();
      } else {
        wait_vmcnt<0>();
      }
      __syncthreads();
      const unsigned base = (unsigned)(uintptr_t)(LDS_AS char*)&slab[s & 1][0][0];
#pragma unroll
      for (int i = 0; i < kSteps; ++i) {
        const int ks = kh * kSteps + i;
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS char*)(uintptr_t)(base + tr_off[0]) + ks * 16 * 64));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS char*)(uintptr_t)(base + tr_off[1]) + ks * 16 * 64));
        const bf16x8 bop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_cur[mb][i], bop, acc[mb], 0, 0, 0);
      }
      __syncthreads();  // every wave is done with this buffer before slab s + 2 refills it
      if (s + 1 < kSlabs) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i = 0; i < kSteps; ++i) a_cur[mb][i] = a_nxt[mb][i];
      }
    }
    // acc lane l, register j: row 8 (j / 4) + 4 half + j % 4, column l % 32 of the wave's plane
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (m0 + 32 * mb >= batch) break;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        red[kh][(8 * (j >> 2) + 4 * half + (j & 3)) * 64 + 32 * tile + (lane & 31)] = acc[mb][j];
      __syncthreads();
      const int r = tid >> 3, c8 = 8 * (tid & 7);
      const int row = m0 + 32 * mb + r;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float4 a = *reinterpret_cast<const float4*>(&red[0][r * 64 + c8 + 4 * q]);
        const float4 b = *reinterpret_cast<const float4*>(&red[1][r * 64 + c8 + 4 * q]);
        if (row < batch)
          *reinterpret_cast<float4*>(part + ((size_t)kc * batch + row) * kN + n0 + c8 + 4 * q) =
              make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
      }
      __syncthreads();
    }
  }
}

#ifndef MLA_OP4_CHUNK
#define MLA_OP4_CHUNK 1024
#endif
constexpr int kChunk4 = MLA_OP4_CHUNK;   // weight rows per workgroup (wide form)
// 32-row slabs (16 KB of LDS a workgroup with both buffers) let every workgroup of the grid be
// resident at once: 45.6 against 54.0 us at batch 32 and 40.2 against 44.1 us at batch 4 with
// 128-row slabs (64 KB, two workgroups a compute unit, so the grid's last fifth ran as a second
// round); 16-row slabs spend more on barriers than they gain (60.5 us).
#ifndef MLA_OP4_SLAB
#define MLA_OP4_SLAB 32
#endif
constexpr int kSlab4 = MLA_OP4_SLAB;     // weight rows per slab (wide form)
constexpr int kRow4 = 256;               // slab row bytes: 128 columns

// Wide form for batches up to 32: workgroup (K chunk, 128-column block), the chunk walked in slabs
// of kSlab4 rows, double-buffered; each copy moves 4 rows x 256 contiguous bytes (16-byte unit u of slab row r stored at unit u ^ 2 (r mod 4), so that the
// four rows of a transposing read fall on different banks); wave w owns columns 32 w .. 32 w + 31
// over the whole chunk, so no K halves are summed.  part[kc][b][n], as the narrow form.
__global__ __launch_bounds__(256) void dense_proj4_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ w, int K,
                                                          float* __restrict__ part, int batch) {
  __shared__ __attribute__((aligned(1024))) char slab[2][kSlab4 * kRow4];
  const int kc = blockIdx.x;
  const int n0 = blockIdx.y * 128;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const uint16_t* wk = w + (size_t)kc * kChunk4 * kN + n0;
  constexpr int kCopies = kSlab4 * kRow4 / 1024 / 4;   // per wave and slab
  constexpr int kSteps4 = kSlab4 / 16;                 // k-steps per slab
  static_assert(kCopies >= 1 && kChunk4 % kSlab4 == 0, "whole copies per wave, whole slabs per chunk");
  auto swz = [](int r) { return 2 * (r & 3); };
  auto issue_slab = [&](int s, int buf) __attribute__((always_inline)) {
    const unsigned lds0 = (unsigned)(uintptr_t)(LDS_AS char*)&slab[buf][0];
#pragma unroll
    for (int jj = 0; jj < kCopies; ++jj) {
      const int j = wave + 4 * jj;
      const int r = 4 * j + lane / 16;
      const int u = (lane % 16) ^ swz(r);
      dma16(wk + (size_t)(kSlab4 * s + r) * kN + 8 * u, lds0 + j * 1024);
    }
  };
  unsigned tr_off[2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int r = 8 * half + ((lane & 15) >> 2) + 4 * rd;
    const int u = 4 * wave + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    tr_off[rd] = (unsigned)(r * kRow4 + 16 * (u ^ swz(r)) + 8 * (lane & 1));
  }
  constexpr int kSlabs4 = kChunk4 / kSlab4;
  f32x16 acc = {};
  bf16x8 a_cur[kSteps4], a_nxt[kSteps4];
  const int row = min(lane & 31, batch - 1);   // rows past the batch repeat the last (never stored)
  auto load_a = [&](int s, bf16x8 (&a)[kSteps4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kSteps4; ++i)
      a[i] = *reinterpret_cast<const bf16x8*>(x + (size_t)row * K + kc * kChunk4 + kSlab4 * s + 16 * i + 8 * half);
  };
  issue_slab(0, 0);
  load_a(0, a_cur);
#pragma unroll 1
  for (int s = 0; s < kSlabs4; ++s) {
    if (s + 1 < kSlabs4) {
      issue_slab(s + 1, (s + 1) & 1);
      load_a(s + 1, a_nxt);
      wait_vmcnt<kCopies + kSteps4>();   // slab s (and its rows) have landed
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    const unsigned base = (unsigned)(uintptr_t)(LDS_AS char*)&slab[s & 1][0];
#pragma unroll
    for (int i = 0; i < kSteps4; ++i) {
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS char*)(uintptr_t)(base + tr_off[0]) + i * 16 * kRow4));
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS char*)(uintptr_t)(base + tr_off[1]) + i * 16 * kRow4));
      const bf16x8 bop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_cur[i], bop, acc, 0, 0, 0);
    }
    __syncthreads();  // every wave is done with this buffer before slab s + 2 refills it
    if (s + 1 < kSlabs4) {
#pragma unroll
      for (int i = 0; i < kSteps4; ++i) a_cur[i] = a_nxt[i];
    }
  }
  // acc lane l, register j: row 8 (j / 4) + 4 half + j % 4, column l % 32 of the wave's block
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = 8 * (j >> 2) + 4 * half + (j & 3);
    if (r < batch) part[((size_t)kc * batch + r) * kN + n0 + 32 * wave + (lane & 31)] = acc[j];
  }
}

// hidden[b][n] = sum over chunks (in order) of part[c][b][n], rounded to bf16; 4 outputs a thread.
__global__ __launch_bounds__(256) void dense_finish_kernel(const float* __restrict__ part, int chunks,
                                                           int batch, uint16_t* __restrict__ out) {
  const int b = blockIdx.y;
  const int n = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (n >= kN) return;
  // The partials' loads go out eight at a time before any is added (the sum still runs in chunk
  // order), instead of one memory round trip per chunk.
  constexpr int kGroup = 8;
  float4 s = make_float4(-0.f, -0.f, -0.f, -0.f);   // -0 + x is x for every x
  for (int c0 = 0; c0 < chunks; c0 += kGroup) {
    float4 v[kGroup];
#pragma unroll
    for (int u = 0; u < kGroup; ++u)
      if (c0 + u < chunks) v[u] = *reinterpret_cast<const float4*>(part + ((size_t)(c0 + u) * batch + b) * kN + n);
#pragma unroll
    for (int u = 0; u < kGroup; ++u)
      if (c0 + u < chunks) {
        s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
      }
  }
  uint2 packed;
  packed.x = (uint32_t)f32_to_bf16(s.x) | ((uint32_t)f32_to_bf16(s.y) << 16);
  packed.y = (uint32_t)f32_to_bf16(s.z) | ((uint32_t)f32_to_bf16(s.w) << 16);
  *reinterpret_cast<uint2*>(out + (size_t)b * kN + n) = packed;
}

// fp32 mode: one thread per output, fp32 arithmetic.
__global__ __launch_bounds__(256) void dense_f32_kernel(const float* __restrict__ x, const float* __restrict__ w,
                                                        int K, float* __restrict__ out) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  if (n >= kN) return;
  const float* xr = x + (size_t)b * K;
  float s = 0.f;
  for (int k = 0; k < K; ++k) s = fmaf(xr[k], w[(size_t)k * kN + n], s);
  out[(size_t)b * kN + n] = s;
}

}  // namespace

size_t out_proj_hidden_workspace_bytes(int batch, int heads) {
  const int chunk = kChunk4 < kChunk ? kChunk4 : kChunk;   // the form with more partials
  return (size_t)(heads * kDv / chunk) * (size_t)batch * kN * sizeof(float);
}

hipError_t launch_out_proj_hidden(const void* out, const void* w_o, void* hidden, int batch, int heads,
                                  float* part, bool f32, hipStream_t s) {
  const int K = heads * kDv;
  if (f32) {
    hipLaunchKernelGGL(dense_f32_kernel, dim3(kN / 256, batch), dim3(256), 0, s, (const float*)out,
                       (const float*)w_o, K, (float*)hidden);
    return hipGetLastError();
  }
  int chunks = K / kChunk;
  const dim3 grid(chunks, kN / 64);
  if (batch <= 32 && K % kChunk4 == 0) {
    chunks = K / kChunk4;
    hipLaunchKernelGGL(dense_proj4_kernel, dim3(chunks, kN / 128), dim3(256), 0, s, (const uint16_t*)out,
                       (const uint16_t*)w_o, K, part, batch);
  } else if (batch <= 32)
    hipLaunchKernelGGL(dense_proj_kernel<1>, grid, dim3(256), 0, s, (const uint16_t*)out, (const uint16_t*)w_o, K,
                       part, batch);
  else
    hipLaunchKernelGGL(dense_proj_kernel<2>, grid, dim3(256), 0, s, (const uint16_t*)out, (const uint16_t*)w_o, K,
                       part, batch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dense_finish_kernel, dim3(kN / 4 / 256, batch), dim3(256), 0, s, part, chunks, batch,
                     (uint16_t*)hidden);
  return hipGetLastError();
}

}  // namespace mla
