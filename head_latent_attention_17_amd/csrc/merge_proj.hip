// The split merge and the value up-projection in one kernel (bf16):
//   o_lat[b][h] = sum_s (2^(m_s - M) l_s / L) x_s      (the pieces of sequence b, M = max_s m_s,
//                                                      L = sum_s 2^(m_s - M) l_s)
//   out[b][h]   = bf16(o_lat[b][h]) @ W_UV[h]          (512 -> 128, fp32 accumulation)
// (DeepSeek-V2 explainer, Step 6: W^UV is applied once, after the weighted sum of latent notes.)
// The merge follows the log-sum-exp combination of partial softmax sums; x_s is a piece's sum
// already divided by its own softmax sum l_s, as the matrix-core decode leaves it (bf16), with the
// range of units holding each sequence in the table that kernel writes.
//
// Two workgroups of sixteen waves per head, each taking every other group of 32 batch rows and all
// 128 output columns, so that every piece is read exactly once.  A workgroup starts copying the
// head's whole W_UV (512 x 128, 128 KB) into LDS (LDS-direct loads, no registers held); each wave
// reads the unit ranges of its two rows, then loads all of their pieces at once, ten in flight
// (16 bytes of the piece per lane and its (max, sum) pair), folding each row in with a running
// maximum and leaving it in a 32 KB buffer of bf16 rows; four waves then multiply the rows against
// the slab on the matrix cores (v_mfma_f32_32x32x16_bf16), one 32-column block each.  The slab and
// the rows buffer fill the 160 KB of LDS.  The two workgroups of a head sit on the same XCD, so the
// second reads W_UV from the L2 the first filled.  Heads must be a multiple of 8.
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

constexpr int kCols = kDv;                 // output columns per workgroup: all of them
constexpr int kSlabRow = kCols * 2;        // bytes per k-row of the W_UV slab
constexpr int kGroupRows = 32;             // batch rows per pass
constexpr int kRowBytes = kDc * 2;         // bf16 bytes of a merged row
constexpr int kChunk = 10;                 // pieces in flight per lane
constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = kGroupRows / kWaves;   // 2
static_assert(kDc * kSlabRow + kGroupRows * kRowBytes <= 160 * 1024, "slab + rows fill the LDS");

// One 16-byte-per-lane copy HBM -> LDS: lane l's 16 bytes from gaddr land at LDS byte lds + 16 l.
// The kernel waits for it explicitly (vmcnt(0) + barrier) before the slab is read.
__device__ __forceinline__ void dma16(const void* gaddr, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gaddr), "s"(lds)
               : "memory", "m0");
}

// 16-byte unit u of slab k-row r is stored at unit u ^ 2 (r mod 4): the four rows of one
// transposing read (32 bytes each) then fall on eight different 16-byte bank groups.
__device__ __forceinline__ int slab_swz(int r) { return 2 * (r & 3); }
// 16-byte chunk c of merged row r is stored at chunk c ^ (r mod 16): the row reads of the A operand
// (16 rows, one chunk) fall on sixteen different bank groups.
__device__ __forceinline__ unsigned row_off(int r, int c) { return (unsigned)(r * kRowBytes + 16 * (c ^ (r & 15))); }

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
  __shared__ __attribute__((aligned(1024))) char slab[kDc * kSlabRow];      // 128 KB
  __shared__ __attribute__((aligned(1024))) char rows[kGroupRows * kRowBytes];  // 32 KB
  // Workgroup i runs on XCD i mod 8: the two workgroups of a head are i and i + 8.
  const int xi = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int h = (j >> 1) * 8 + xi;
  const int first_group = j & 1;   // groups first_group, first_group + 2, ...
  if (first_group * kGroupRows >= p.batch) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  uint16_t* o_lat = static_cast<uint16_t*>(p.o_lat);
  auto slot = [&](int w, int b) { return ((size_t)w + b) * p.heads + h; };

  // W_UV[h]: copy i moves k-rows 4 i .. 4 i + 3; lane l fetches unit (l % 16) ^ swz(row) of row 4 i + l / 16.
  {
    const uint16_t* wh = w_uv + (size_t)h * kDc * kDv;
    const unsigned lds0 = (unsigned)(uintptr_t)(LDS_AS char*)slab;
    for (int i = wave; i < kDc * kSlabRow / 1024; i += kWaves) {
      const int r = i * 4 + lane / 16;
      const int u = (lane % 16) ^ slab_swz(r);
      dma16(wh + (size_t)r * kDv + 8 * u, lds0 + i * 1024);
    }
  }

  // B operand (slab, transposed reads): rows 8 half + (lane % 16) / 4 (+ 4) of a k-step, logical
  // unit 4 cb + 2 ((lane / 16) % 2) + (lane % 4) / 2, byte 8 (lane % 2); a k-step is 16 rows.
  auto b_addr = [&](int cb, int rd) {
    const int r = 8 * half + ((lane & 15) >> 2) + 4 * rd;
    const int u = 4 * cb + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    return (unsigned)(uintptr_t)(LDS_AS char*)slab + r * kSlabRow + 16 * (u ^ slab_swz(r)) + 8 * (lane & 1);
  };

  bool slab_ready = false;
  for (int gi = first_group; gi * kGroupRows < p.batch; gi += 2) {
    const int g0 = gi * kGroupRows;
    const int nrows = min(kGroupRows, p.batch - g0);
    // ---- merge: wave w takes rows w and w + 16.  Their unit ranges are read first; then all their
    // pieces stream through in order, kChunk in flight (16 bytes of the piece per lane and its
    // (max, sum) pair, the same address in every lane; indices past the end repeat the last piece,
    // unused), each row folded in with a running maximum and flushed (bf16) when its last piece is in.
    {
      // lane k (< kRowsPerWave) holds row w + 16 k's first unit and unit count; read back with
      // readlane for a wave-uniform k (a register array indexed at run time would go to scratch)
      int wf_v = 0, n_v = 0, dead_v = 0;
      {
        const int r = wave + kWaves * min(lane, kRowsPerWave - 1);
        const int b = g0 + min(r, nrows - 1);
        const int len = p.seq_lens[b];
        const int4 d = *reinterpret_cast<const int4*>(p.seq_units + 4 * b);
        if (lane < kRowsPerWave && r < nrows && len > 0) {
          wf_v = d.x;
          n_v = d.y - d.x + 1;
          dead_v = d.z ? 0 : 1;   // some unit of the call holds no page (more units than pages)
        }
      }
      auto wf_of = [&](int k) { return __builtin_amdgcn_readlane(wf_v, k); };
      auto n_of = [&](int k) { return __builtin_amdgcn_readlane(n_v, k); };
      int cnt = 0;
#pragma unroll
      for (int k = 0; k < kRowsPerWave; ++k) cnt += n_of(k);
      // With units that hold no page, those inside a sequence's range wrote no piece: they are
      // skipped, found from the page count (only then worked out).
      const bool all_live = __builtin_amdgcn_ballot_w64(dead_v != 0) == 0;
      long long P = 0;
      if (!all_live) P = total_pages(p.seq_lens, p.batch);
      auto live = [&](int w) {
        return all_live || unit_start(P, p.num_units, w) != unit_start(P, p.num_units, w + 1);
      };
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
        *reinterpret_cast<LDS_AS u32x4*>((LDS_AS char*)rows + row_off(r, lane)) = u32x4{v.x, v.y, v.z, v.w};
        const int b = g0 + r;
        if (o_lat) *reinterpret_cast<uint4*>(o_lat + ((size_t)b * p.heads + h) * kDc + 8 * lane) = v;
        if (p.lse && lane == 0)
          p.lse[(size_t)b * p.heads + h] = nk ? (mx + log2f(sum)) * 0.69314718055994531f : -INFINITY;
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
      // rows with no piece (empty sequences) are flushed as zeros up front; rows past the batch
      // are zeros in the buffer (the projection reads them; their outputs are not stored)
#pragma unroll
      for (int k = 0; k < kRowsPerWave; ++k) {
        const int r = wave + kWaves * k;
        if (r < nrows && n_of(k) == 0) {
          start_row(k);
          flush(k);
        } else if (r >= nrows) {
          *reinterpret_cast<LDS_AS u32x4*>((LDS_AS char*)rows + row_off(r, lane)) = u32x4{0u, 0u, 0u, 0u};
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
    if (!slab_ready) {
      __builtin_amdgcn_s_waitcnt(0);   // this wave's slab copies have landed
      slab_ready = true;
    }
    __syncthreads();

    // ---- projection on the first four waves: column block cb = wave, 32 rows x 32 columns over
    // the whole K (32 MFMAs)
    if (wave < kCols / 32) {
      const int cb = wave;
      f32x16 acc = {};
      const unsigned rbase = (unsigned)(uintptr_t)(LDS_AS char*)rows;
      const unsigned b0 = b_addr(cb, 0), b1 = b_addr(cb, 1);
      const int rr = lane & 31;
#pragma unroll 4
      for (int ks = 0; ks < kDc / 16; ++ks) {
        const bf16x8 a = *reinterpret_cast<const LDS_AS bf16x8*>((LDS_AS char*)(uintptr_t)(rbase + row_off(rr, 2 * ks + half)));
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS char*)(uintptr_t)b0 + ks * 16 * kSlabRow));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS char*)(uintptr_t)b1 + ks * 16 * kSlabRow));
        const bf16x8 bop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, acc, 0, 0, 0);
      }
      // acc lane l, register jj: row 8 (jj / 4) + 4 half + jj % 4 of the group, column l % 32
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int row = 8 * (jj >> 2) + 4 * half + (jj & 3);
        if (row < nrows)
          out[((size_t)(g0 + row) * p.heads + h) * kDv + 32 * cb + (lane & 31)] = f32_to_bf16(acc[jj]);
      }
    }
    __syncthreads();   // the rows buffer is reused by the next group
  }
}

}  // namespace

// Sixteen waves take two rows each; with fewer than sixteen sequences (a few long ones, many pieces
// each) most of them would idle, and the separate merge spreads those pieces wider.
bool merge_out_proj_supported(const DecodeParams& p) {
  return p.heads % 8 == 0 && p.batch >= kWaves;
}

hipError_t launch_merge_out_proj(const DecodeParams& p, const void* w_uv, void* out, hipStream_t s) {
  if (!p.partial_bf16 || !p.seq_units || !merge_out_proj_supported(p)) return hipErrorNotSupported;
  hipLaunchKernelGGL(merge_out_proj_kernel, dim3(2 * p.heads), dim3(kThreads), 0, s, p, (const uint16_t*)w_uv,
                     (uint16_t*)out);
  return hipGetLastError();
}

}  // namespace mla
