// The producer side of the cache (DeepSeek-V2 explainer, Step 5, eq. 9: a token's hidden vector h is
// squeezed to the latent note c = W^DKV h, 5,120 -> 512; Step 7: the token also contributes one
// 64-dim key k^R, rotated by its position and shared by all heads).  The row [c | RoPE(W^KR h)] is
// written to the token's slot of the paged cache, as mla_cache_append writes a given row.
//
// Both products read weights far larger than the batch rows (5,120 x 576 bf16 = 5.9 MB), so the
// work is split along K: workgroup (k-chunk, 64-column block) multiplies the batch rows of h against
// a 256 x 64 slab of one weight matrix on the bf16 matrix cores and writes an fp32 partial tile; one
// launch covers both matrices (eight column blocks of W^DKV, one of W^KR).  A second kernel sums the
// twenty partials of each row, rotates the key in double precision and writes the bf16 row.  fp32
// mode (a debug mode) computes the sums directly on the vector ALUs.
//
// Rotation (the pages give neither the frequencies nor the pairing; the plain rotary form): pair
// (2i, 2i + 1) of the key turns by position * base^(-2i / 64) radians.
#include <cmath>

#include "mla_device.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
#define LDS_AS __attribute__((address_space(3)))

constexpr int kDModel = 5120;
constexpr int kKc = 256;                   // rows of the weight slab one workgroup multiplies
constexpr int kKChunks = kDModel / kKc;    // partial sums per output
static_assert(kKChunks == kAppendChunks, "the workspace holds one partial row per chunk");
constexpr int kColBlocks = kDc / 64 + 1;   // 8 blocks of W^DKV, then W^KR

// One 16-byte-per-lane copy HBM -> LDS; the kernel waits for it explicitly (vmcnt(0) + barrier).
__device__ __forceinline__ void dma16(const void* gaddr, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gaddr), "s"(lds)
               : "memory", "m0");
}

// part[kc][b][col0 + j] = sum over k in chunk kc of h[b][k] w[k][n0 + j], j < 64, where column
// block cb < 8 is columns 64 cb .. of W^DKV [5120][512] (col0 = n0) and cb = 8 is all of W^KR
// [5120][64] (col0 = 512).  Grid (20 chunks, 9 column blocks).  The slab is held as two planes of
// 32 columns (64-byte rows); wave w multiplies plane w % 2 over k-half w / 2, and the two k-halves
// are summed through LDS.  MB 32-row batch blocks per pass.
template <int MB>
__global__ __launch_bounds__(256) void hidden_proj_kernel(const uint16_t* __restrict__ h,
                                                          const uint16_t* __restrict__ w_dkv,
                                                          const uint16_t* __restrict__ w_kr,
                                                          float* __restrict__ part, int batch) {
  constexpr int kSteps = kKc / 16 / 2;  // k-steps per wave
  __shared__ __attribute__((aligned(1024))) char slab[2][kKc * 64];
  __shared__ __attribute__((aligned(16))) float red[2][32 * 64];
  const int kc = blockIdx.x;
  const bool kr = blockIdx.y == kColBlocks - 1;
  const uint16_t* w = kr ? w_kr : w_dkv;
  const int ldw = kr ? kDr : kDc;
  const int n0 = kr ? 0 : 64 * blockIdx.y;
  const int col0 = kr ? kDc : n0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  {
    // copy j: plane j / 16, rows 16 (j % 16) .. + 15; lane -> row + lane / 4, 16-byte unit lane % 4
    const uint16_t* w0 = w + (size_t)kc * kKc * ldw + n0;
    const unsigned lds0 = (unsigned)(uintptr_t)(LDS_AS char*)&slab[0][0];
#pragma unroll
    for (int j = wave; j < 2 * kKc / 16; j += 4) {
      const int t = j / (kKc / 16), i = j % (kKc / 16);
      dma16(w0 + (size_t)(16 * i + lane / 4) * ldw + 32 * t + 8 * (lane % 4), lds0 + t * kKc * 64 + i * 1024);
    }
  }
  const int tile = wave & 1, kh = wave >> 1;
  // Transposing reads of the B operand: rows 8 half + (lane % 16) / 4 (+ 4), 16-byte unit
  // 2 ((lane / 16) % 2) + (lane % 4) / 2, byte 8 (lane % 2); 64-byte rows put the four rows of one
  // 16-lane read on different banks.
  unsigned tr_off[2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int r = 8 * half + ((lane & 15) >> 2) + 4 * rd;
    const int u = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    tr_off[rd] = (unsigned)(uintptr_t)(LDS_AS char*)&slab[tile][0] + r * 64 + 16 * u + 8 * (lane & 1);
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
        const int ks = kh * kSteps + i;
        aop[mb][i] = bf16x8{};
        if (row < batch)
          aop[mb][i] = *reinterpret_cast<const bf16x8*>(h + (size_t)row * kDModel + kc * kKc + 16 * ks + 8 * half);
      }
    }
    if (first) {
      __builtin_amdgcn_s_waitcnt(0);  // every copy (and load) of this wave has landed
      __syncthreads();
      first = false;
    }
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      const int ks = kh * kSteps + i;
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS char*)(uintptr_t)tr_off[0] + ks * 16 * 64));
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS char*)(uintptr_t)tr_off[1] + ks * 16 * 64));
      const bf16x8 bop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[mb][i], bop, acc[mb], 0, 0, 0);
    }
    // acc lane l, register j: row 8 (j / 4) + 4 half + j % 4, column l % 32 of the wave's plane
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (m0 + 32 * mb >= batch) break;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        red[kh][(8 * (j >> 2) + 4 * half + (j & 3)) * 64 + 32 * tile + (lane & 31)] = acc[mb][j];
      __syncthreads();
      // 32 rows x 64 columns; thread t: row t / 8, columns 8 (t % 8) .. + 7
      const int r = tid >> 3, c8 = 8 * (tid & 7);
      const int row = m0 + 32 * mb + r;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float4 a = *reinterpret_cast<const float4*>(&red[0][r * 64 + c8 + 4 * q]);
        const float4 b = *reinterpret_cast<const float4*>(&red[1][r * 64 + c8 + 4 * q]);
        if (row < batch)
          *reinterpret_cast<float4*>(part + ((size_t)kc * batch + row) * kRow + col0 + c8 + 4 * q) =
              make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
      }
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

// Per-pair rotation frequencies base^(-2i / 64), i < 32, computed on the host in double precision.
struct RopeFreqs {
  double inv[kDr / 2];
};

// Row b: sums the CH partials in chunk order, rotates the key by positions[b] and stores the bf16
// row at block_table[b][p / 64], slot p % 64.  One workgroup per row; thread g owns columns
// 4 g .. 4 g + 3, so a key thread holds two whole rotation pairs.  Every partial load is issued
// before the angles are worked out, so the trigonometry runs while the loads are in flight.
template <int CH>
__global__ __launch_bounds__(192) void finish_row_kernel(const float* __restrict__ part, int batch,
                                                         const int32_t* __restrict__ positions,
                                                         const int32_t* __restrict__ block_table,
                                                         int max_blocks, uint16_t* __restrict__ cache,
                                                         RopeFreqs freqs) {
  const int b = blockIdx.x;
  const int g = threadIdx.x;
  if (g >= kRow / 4) return;
  float4 v[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) v[c] = *reinterpret_cast<const float4*>(part + ((size_t)c * batch + b) * kRow + 4 * g);
  const int pos = positions[b];
  const int page = block_table[(size_t)b * max_blocks + pos / kPage];
  double cs[2] = {1.0, 1.0}, sn[2] = {0.0, 0.0};
  if (4 * g >= kDc) {
    // pairs 2 j and 2 j + 1; the frequencies are picked with uniform indices so that they stay in
    // scalar registers (a per-lane index into the kernel arguments would be a vector load)
    const int j = g - kDc / 4;
    double f[2] = {0.0, 0.0};
#pragma unroll
    for (int u = 0; u < kDr / 4; ++u)
      if (j == u) {
        f[0] = freqs.inv[2 * u];
        f[1] = freqs.inv[2 * u + 1];
      }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      // angle mod 2 pi by the two-constant Cody-Waite split of 2 pi (|k| < 2^29 for any int position)
      const double angle = (double)pos * f[q];
      const double k = rint(angle * 0.15915494309189535);
      const double r = fma(-k, 2.4492935982947064e-16, fma(-k, 6.283185307179586, angle));
      sincos(r, &sn[q], &cs[q]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  float s[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
#pragma unroll
  for (int c = 1; c < CH; ++c) {
    s[0] += v[c].x; s[1] += v[c].y; s[2] += v[c].z; s[3] += v[c].w;
  }
  if (4 * g >= kDc) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const double x0 = s[2 * q], x1 = s[2 * q + 1];
      s[2 * q] = (float)(x0 * cs[q] - x1 * sn[q]);
      s[2 * q + 1] = (float)(x0 * sn[q] + x1 * cs[q]);
    }
  }
  uint2 packed;
  packed.x = (uint32_t)f32_to_bf16(s[0]) | ((uint32_t)f32_to_bf16(s[1]) << 16);
  packed.y = (uint32_t)f32_to_bf16(s[2]) | ((uint32_t)f32_to_bf16(s[3]) << 16);
  *reinterpret_cast<uint2*>(cache + ((size_t)page * kPage + pos % kPage) * kRow + 4 * g) = packed;
}

}  // namespace

hipError_t launch_append_hidden(void* cache, const int32_t* block_table, int max_blocks,
                                 const int32_t* positions, const void* hidden, const void* w_dkv,
                                 const void* w_kr, double rope_base, int batch, float* part, bool f32,
                                 hipStream_t s) {
  if (f32) {
    hipLaunchKernelGGL(hidden_proj_f32_kernel, dim3((kRow + 255) / 256, batch), dim3(256), 0, s,
                       (const float*)hidden, (const float*)w_dkv, (const float*)w_kr, part, batch);
  } else {
    const uint16_t* H = (const uint16_t*)hidden;
    const uint16_t* Wd = (const uint16_t*)w_dkv;
    const uint16_t* Wr = (const uint16_t*)w_kr;
    if (batch <= 32)
      hipLaunchKernelGGL(hidden_proj_kernel<1>, dim3(kKChunks, kColBlocks), dim3(256), 0, s, H, Wd, Wr, part, batch);
    else
      hipLaunchKernelGGL(hidden_proj_kernel<2>, dim3(kKChunks, kColBlocks), dim3(256), 0, s, H, Wd, Wr, part, batch);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  RopeFreqs freqs;
  for (int i = 0; i < kDr / 2; ++i) freqs.inv[i] = std::pow(rope_base, -2.0 * i / kDr);
  if (f32)
    hipLaunchKernelGGL(finish_row_kernel<1>, dim3(batch), dim3(192), 0, s, part, batch, positions, block_table,
                       max_blocks, (uint16_t*)cache, freqs);
  else
    hipLaunchKernelGGL(finish_row_kernel<kKChunks>, dim3(batch), dim3(192), 0, s, part, batch, positions,
                       block_table, max_blocks, (uint16_t*)cache, freqs);
  return hipGetLastError();
}

}  // namespace mla
