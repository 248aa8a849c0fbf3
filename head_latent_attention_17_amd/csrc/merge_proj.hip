// The split merge and the value up-projection in one kernel (bf16):
//   o_lat[b][h] = sum_s (2^(m_s - M) l_s / L) x_s      (the pieces of sequence b, M = max_s m_s,
//                                                      L = sum_s 2^(m_s - M) l_s)
//   out[b][h]   = bf16(o_lat[b][h]) @ W_UV[h]          (512 -> 128, fp32 accumulation)
// (DeepSeek-V2 explainer, Step 6: W^UV is applied once, after the weighted sum of latent notes.)
// The merge follows the log-sum-exp combination of partial softmax sums; x_s is a piece's sum
// already divided by its own softmax sum l_s, as the matrix-core decode leaves it (bf16), with the
// range of units holding each sequence in the table that kernel writes.
//
// One workgroup of sixteen waves per (head, 64 output columns): it starts copying its 512 x 64 slab
// of W_UV into LDS (64 KB, LDS-direct loads, no registers held); each wave reads the unit ranges of
// its rows (every sixteenth row of a group of 64), then streams their pieces, ten at a time in
// flight (16 bytes of the piece per lane and the piece's (max, sum) pair), folding each row in with
// a running maximum and leaving it in an LDS buffer in bf16; four waves then multiply the rows
// against the slab on the matrix cores (v_mfma_f32_32x32x16_bf16).  So a launch waits for about
// three rounds of memory latency.  Every W_UV byte is read once per launch; each sequence's pieces
// are read by the two workgroups of a head, which sit on the same XCD.  Batches above 64 go through
// in groups of 64 rows with the slab kept.  Heads must be a multiple of 8.
#include <type_traits>

#include "mla_device.h"

namespace mla {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
#define LDS_AS __attribute__((address_space(3)))
#define CONST_AS __attribute__((address_space(4)))

constexpr int kCols = 64;                 // output columns per workgroup
constexpr int kSlabRow = kCols * 2;       // bytes per k-row of the W_UV slab
constexpr int kGroupRows = 64;            // batch rows per pass
constexpr int kApitch = kDc * 2 + 16;     // bf16 row pitch of the merged rows: rows step across banks
constexpr int kChunk = 10;                // pieces in flight per lane
constexpr int kWaves = 16;                // waves per workgroup: more pieces in flight per compute unit
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = kGroupRows / kWaves;
constexpr int kMaxUnits = 1024;           // units the liveness mask covers

// One 16-byte-per-lane copy HBM -> LDS: lane l's 16 bytes from gaddr land at LDS byte lds + 16 l.
// The kernel waits for it explicitly (vmcnt(0) + barrier) before the slab is read.
__device__ __forceinline__ void dma16(const void* gaddr, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gaddr), "s"(lds)
               : "memory", "m0");
}

// 16-byte units of slab row r are stored XOR 2 ((r / 2) mod 4), so that the four rows of one
// transposing read fall on different banks.
__device__ __forceinline__ int slab_swz(int r) { return 2 * ((r >> 1) & 3); }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ uint4 pack8(const float* x) {
  uint4 v;
  v.x = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
  v.y = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
  v.z = (uint32_t)f32_to_bf16(x[4]) | ((uint32_t)f32_to_bf16(x[5]) << 16);
  v.w = (uint32_t)f32_to_bf16(x[6]) | ((uint32_t)f32_to_bf16(x[7]) << 16);
  return v;
}

__global__ __launch_bounds__(kThreads, 1) void merge_out_proj_kernel(DecodeParams p, const uint16_t* __restrict__ w_uv,
                                                                      uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) char slab[kDc * kSlabRow];   // 64 KB
  __shared__ __attribute__((aligned(16))) char rows[kGroupRows * kApitch];  // 65 KB
  __shared__ __attribute__((aligned(16))) float red[2][32 * 32];           // K-half partial tiles
  __shared__ long long total_pages_s;
  __shared__ uint32_t live_bits[kMaxUnits / 32];
  // Workgroup i runs on XCD i mod 8: the two halves of a head are i and i + 8, so that the second
  // reads the head's pieces from the L2 the first filled.
  const int xi = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int h = (j >> 1) * 8 + xi;
  const int n0 = (j & 1) * kCols;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const bool writer = n0 == 0;   // one workgroup of a head writes o_lat and lse
  uint16_t* o_lat = static_cast<uint16_t*>(p.o_lat);
  auto slot = [&](int w, int b) { return ((size_t)w + b) * p.heads + h; };

  // W_UV[h][:, n0 .. n0 + 63]: copy i moves 8 rows; lane l fetches unit (l % 8) ^ swz(row) of row l / 8.
  {
    const uint16_t* wh = w_uv + (size_t)h * kDc * kDv + n0;
    const unsigned lds0 = (unsigned)(uintptr_t)(LDS_AS char*)slab;
    for (int i = wave; i < kDc * kSlabRow / 1024; i += kWaves) {
      const int r = i * 8 + lane / 8;
      const int u = (lane % 8) ^ slab_swz(r);
      dma16(wh + (size_t)r * kDv + 8 * u, lds0 + i * 1024);
    }
  }
  if (wave == 0) {  // total pages: a unit with no page (more units than pages) wrote no piece
    const long long P = total_pages(p.seq_lens, p.batch);
    if (lane == 0) total_pages_s = P;
  }
  for (int i = tid; i < kMaxUnits / 32; i += kThreads) live_bits[i] = 0;
  __syncthreads();
  const long long P = total_pages_s;
  const bool all_live = P >= p.num_units;
  if (!all_live) {  // which units hold a page, worked out once
    for (int w = tid; w < p.num_units; w += kThreads)
      if (unit_start(P, p.num_units, w) != unit_start(P, p.num_units, w + 1)) atomicOr(&live_bits[w >> 5], 1u << (w & 31));
    __syncthreads();
  }
  auto live = [&](int w) { return all_live || ((live_bits[w >> 5] >> (w & 31)) & 1u); };

  // B operand (slab, transposed reads): rows 8 half + (lane % 16) / 4 (+ 4) of a k-step, logical
  // unit 4 cb + 2 ((lane / 16) % 2) + (lane % 4) / 2, byte 8 (lane % 2); a k-step is 16 rows.
  auto b_addr = [&](int cb, int rd) {
    const int r = 8 * half + ((lane & 15) >> 2) + 4 * rd;
    const int u = 4 * cb + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    return (unsigned)(uintptr_t)(LDS_AS char*)slab + r * kSlabRow + 16 * (u ^ slab_swz(r)) + 8 * (lane & 1);
  };

  for (int g0 = 0; g0 < p.batch; g0 += kGroupRows) {
    const int nrows = min(kGroupRows, p.batch - g0);
    // ---- merge: wave w takes rows w, w + 16, ... (kRowsPerWave at most).  Their unit ranges are read
    // first, all at once; then their pieces stream through in order, kChunk in flight (16 bytes of the
    // piece per lane and its (max, sum) pair, the same address in every lane; indices past the end
    // repeat the last piece, unused), each row folded in with a running maximum and flushed (bf16)
    // when its last piece is in.
    {
      // lane k (< kRowsPerWave) holds row w + 16 k's first unit and unit count; read back with
      // readlane for a wave-uniform k (a register array indexed at run time would go to scratch)
      int wf_v = 0, n_v = 0;
      {
        const int r = wave + kWaves * min(lane, kRowsPerWave - 1);
        const int b = g0 + min(r, nrows - 1);
        const int len = p.seq_lens[b];
        const int4 d = *reinterpret_cast<const int4*>(p.seq_units + 4 * b);
        if (lane < kRowsPerWave && r < nrows && len > 0) {
          wf_v = d.x;
          n_v = d.y - d.x + 1;
        }
      }
      auto wf_of = [&](int k) { return __builtin_amdgcn_readlane(wf_v, k); };
      auto n_of = [&](int k) { return __builtin_amdgcn_readlane(n_v, k); };
      int cnt = 0;
#pragma unroll
      for (int k = 0; k < kRowsPerWave; ++k) cnt += n_of(k);
      float acc[8];
      float mx = -INFINITY, sum = 0.f;
      int cur = -1;   // row (k) being folded
      auto flush = [&](int k) {
        const int r = wave + kWaves * k;
        const int nk = n_of(k);
        const float inv = nk ? 1.f / sum : 0.f;
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = acc[i] * inv;
        const uint4 v = pack8(x);
        *reinterpret_cast<LDS_AS u32x4*>((LDS_AS char*)rows + r * kApitch + 16 * lane) = u32x4{v.x, v.y, v.z, v.w};
        if (writer) {
          const int b = g0 + r;
          if (o_lat) *reinterpret_cast<uint4*>(o_lat + ((size_t)b * p.heads + h) * kDc + 8 * lane) = v;
          if (p.lse && lane == 0)
            p.lse[(size_t)b * p.heads + h] = nk ? (mx + log2f(sum)) * 0.69314718055994531f : -INFINITY;
        }
      };
      auto start_row = [&](int k) {
        cur = k;
        mx = -INFINITY;
        sum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
      };
      // item i -> (row k, piece s): rows in order, their pieces in order
      auto item = [&](int i, int& k, int& s) {
        k = 0;
        s = i;
#pragma unroll
        for (int kk = 0; kk < kRowsPerWave - 1; ++kk) {
          const int nk = n_of(kk);
          if (k == kk && s >= nk) {
            s -= nk;
            k = kk + 1;
          }
        }
      };
      // rows with no piece (empty sequences, or past the batch) are flushed as zeros up front
#pragma unroll
      for (int k = 0; k < kRowsPerWave; ++k) {
        if (wave + kWaves * k < nrows && n_of(k) == 0) {
          start_row(k);
          flush(k);
        }
      }
      for (int c = 0; c < cnt; c += kChunk) {
        int kk[kChunk], ww[kChunk];
        uint4 v[kChunk];
        float2 ml[kChunk];
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
          int k, s;
          item(min(c + u, cnt - 1), k, s);
          kk[u] = k;
          ww[u] = wf_of(k) + s;
          const size_t sl = slot(ww[u], g0 + wave + kWaves * k);
          v[u] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.ws_o + sl * kDc) + 8 * lane);
          ml[u] = *reinterpret_cast<const float2*>(p.ws_ml + 2 * sl);
        }
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
          if (c + u < cnt) {
            if (kk[u] != cur) {
              if (cur >= 0) flush(cur);
              start_row(kk[u]);
            }
            if (live(ww[u])) {
              if (ml[u].x > mx) {   // a new running maximum: the sums so far are scaled down
                const float r = exp2f(mx - ml[u].x);
                sum *= r;
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] *= r;
                mx = ml[u].x;
              }
              const float wt = exp2f(ml[u].x - mx) * ml[u].y;
              sum += wt;
              const uint32_t q[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                acc[2 * i] = fmaf(wt, bf16_lo(q[i]), acc[2 * i]);
                acc[2 * i + 1] = fmaf(wt, bf16_hi(q[i]), acc[2 * i + 1]);
              }
            }
          }
        }
      }
      if (cur >= 0) flush(cur);
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wave's slab copies (first group) and stores have landed
    __syncthreads();

    // ---- projection on the first four waves: tiles of 32 rows x 32 columns; with one row block the
    // two K halves of each column block go to two waves and are summed through LDS
    const int nblk = (nrows + 31) / 32;
    const int tiles = 2 * nblk;          // 2 or 4
    const int ksplit = 4 / tiles;        // 2 or 1
    const int t = wave % tiles, kpart = wave / tiles;
    const int mb = t >> 1, cb = t & 1;
    f32x16 acc = {};
    if (wave < 4) {
      const int ks0 = kpart * (32 / ksplit), ks1 = ks0 + 32 / ksplit;
      const unsigned a_base = (unsigned)(uintptr_t)(LDS_AS char*)rows + (32 * mb + (lane & 31)) * kApitch + 16 * half;
      const unsigned b0 = b_addr(cb, 0), b1 = b_addr(cb, 1);
      for (int ks = ks0; ks < ks1; ++ks) {
        const bf16x8 a = *reinterpret_cast<const LDS_AS bf16x8*>((LDS_AS char*)(uintptr_t)(a_base + 32 * ks));
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS char*)(uintptr_t)b0 + ks * 16 * kSlabRow));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS char*)(uintptr_t)b1 + ks * 16 * kSlabRow));
        const bf16x8 bop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, acc, 0, 0, 0);
      }
      // acc lane l, register j: row 8 (j / 4) + 4 half + j % 4 of the tile, column l % 32
      if (ksplit == 2 && kpart == 1) {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) red[cb][(8 * (jj >> 2) + 4 * half + (jj & 3)) * 32 + (lane & 31)] = acc[jj];
      }
    }
    __syncthreads();
    if (wave < 4 && kpart == 0) {
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int rr = 8 * (jj >> 2) + 4 * half + (jj & 3);
        float x = acc[jj];
        if (ksplit == 2) x += red[cb][rr * 32 + (lane & 31)];
        const int row = 32 * mb + rr;
        if (row < nrows)
          out[((size_t)(g0 + row) * p.heads + h) * kDv + n0 + 32 * cb + (lane & 31)] = f32_to_bf16(x);
      }
    }
    __syncthreads();   // the rows buffer and the partial tiles are reused by the next group
  }
}

}  // namespace

// Sixteen waves take a row each at a time; with fewer than sixteen sequences (a few long ones, many
// pieces each) most of them would idle, and the separate merge spreads those pieces wider.
bool merge_out_proj_supported(const DecodeParams& p) {
  return p.heads % 8 == 0 && p.batch >= kWaves && p.num_units <= kMaxUnits;
}

hipError_t launch_merge_out_proj(const DecodeParams& p, const void* w_uv, void* out, hipStream_t s) {
  if (!p.partial_bf16 || !p.seq_units || !merge_out_proj_supported(p)) return hipErrorNotSupported;
  hipLaunchKernelGGL(merge_out_proj_kernel, dim3(2 * p.heads), dim3(kThreads), 0, s, p, (const uint16_t*)w_uv,
                     (uint16_t*)out);
  return hipGetLastError();
}

}  // namespace mla
