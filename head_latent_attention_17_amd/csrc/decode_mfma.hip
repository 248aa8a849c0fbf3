// Latent-space decode attention on the bf16 matrix cores of gfx950 (v_mfma_f32_32x32x16_bf16).
//
// What is computed (DeepSeek-V2 explainer, Steps 6-8): for every head h of sequence b,
//   S[t][h] = q_abs[b][h] . row_t        (576-long: latent score + RoPE score, one dot product)
//   P       = softmax_t(scale * S)       (online, base 2)
//   O[d][h] = sum_t P[h][t] * row_t[d]   (d < 512: the weighted sum of latent notes)
// All heads of a sequence share every cached row (the row is per token, not per head), so heads
// form the N dimension of both products and each row is read from HBM once per launch.
//
// Workgroup = 4 waves x 32 heads = 128 heads, one workgroup per compute unit (64 and 32 heads: the
// waves' columns repeat heads, see head_of; 16 heads run decode_h16_kernel, below, on the 16-wide
// matrix instruction).  Per 32-token tile:
//   scores  S^T[t][h] = K . Q^T   M = 32 tokens, N = 32 heads, K = 576  (36 MFMAs per wave)
//   output  O^T[d][h] = V^T . P^T M = 32 dims,   N = 32 heads, K = 32   (16 blocks x 2 MFMAs)
// Q stays in VGPRs for a whole segment; O^T (32 x 512 fp32 per wave) stays in the 256 AGPRs.  The
// S^T accumulator layout (lane = head, registers = tokens) is already the B-operand layout of the
// second product, so P never leaves its lane; V^T comes out of the token-major LDS tile with
// ds_read_b64_tr_b16, a 16-lane transposing read.
//
// Pipelining.  Tiles stream HBM -> LDS with global_load_lds_dwordx4 through a 4-stage ring, three
// tiles ahead of the one being processed.  The prologue puts three tiles in flight; after that each
// wave issues its nine copies of tile it + 3 one per four score MFMAs of tile it + 1.  With one wave
// per SIMD nothing hides a stall, so one iteration overlaps two tiles: after the wait for tile it + 1
// (counted vmcnt, then a barrier), the score MFMAs of tile it + 1 carry the softmax of tile it (its
// maximum, the rescale decision and the first eight exponentials), then the output product of tile
// it carries the last eight.  LDS operands are prefetched: the score operand 3 k-steps ahead, the
// output operand 4 d-blocks ahead.  The softmax rescale of O is lazy: the reference maximum only
// moves when a tile's maximum exceeds it by more than 2^8.
//
// Tile layout in LDS.  A tile is 32 tokens x 72 chunks of 16 bytes, stored as 36 blocks of
// 8 tokens x 8 chunks, 1 KB each (block = 9 (t / 8) + c / 8), so one global_load_lds_dwordx4 fills
// one block.  Inside a block, chunk c of token t sits at slot
//   8 ((t mod 8) ^ g) + ((c mod 8) ^ sigma(t mod 8)),  g = (t / 8) mod 2,
//   sigma(x) = 2 (x mod 4) + (x / 4) mod 2.
// With it, the 16 lanes of one row read of the score operand (16 tokens, one chunk) and of one
// transposing read (4 tokens x 2 chunks) always land on 16 different 16-byte bank groups.
//
// The file also holds the decode over the ~6-bit cache (decode_fp6_kernel, below): the same work
// split, ring and softmax, with operands converted from the codes in registers; and the 16-head
// decode (decode_h16_kernel, at the end).
#include "mla_device.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(6 * sizeof(unsigned)))) unsigned u32x6;
typedef __attribute__((__vector_size__(16 * sizeof(unsigned)))) unsigned u32x16;
typedef __attribute__((__vector_size__(3 * sizeof(unsigned)))) unsigned u32x3;
typedef __attribute__((__vector_size__(3 * sizeof(int)))) int i32x3;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
#define LDS_AS __attribute__((address_space(3)))
#define CONST_AS __attribute__((address_space(4)))

constexpr int kTileTok = 32;
constexpr int kChunks = kRow / 8;                    // 72 16-byte chunks per row
constexpr int kCG = kChunks / 8;                     // 9 chunk groups
constexpr int kBlocks = kTileTok / 8 * kCG;          // 36 blocks of 8 tokens x 8 chunks
constexpr int kWaves = 4;                            // waves of the bf16 kernel, 32 heads each
constexpr int kTileBytes = kBlocks * 1024;           // 36,864
constexpr int kStages = 4;                           // tiles it .. it+3
static_assert((kStages & (kStages - 1)) == 0, "stage index by mask");
__device__ __forceinline__ int stage_of(int t) { return t & (kStages - 1); }  // stage of tile t
constexpr float kRescaleThreshold = 8.0f;            // base-2 headroom before O is rescaled
#ifndef MLA_KAHEAD
#define MLA_KAHEAD 3
#endif
#ifndef MLA_VAHEAD
#define MLA_VAHEAD 4
#endif
constexpr int kKAhead = MLA_KAHEAD;                  // score operand prefetch depth (k-steps)
constexpr int kVAhead = MLA_VAHEAD;                  // output operand prefetch depth (d-blocks)

__device__ __forceinline__ int sigma(int x) { return ((x & 3) << 1) | ((x >> 2) & 1); }

// Byte offset inside a tile of chunk c of token t.
__device__ __forceinline__ int tile_offset(int t, int c) {
  const int tg = t >> 3, tl = t & 7, cl = c & 7;
  const int slot = 8 * (tl ^ (tg & 1)) + (cl ^ sigma(tl));
  return ((tg * kCG + (c >> 3)) * 64 + slot) * 16;
}

// s_waitcnt lgkmcnt(0) leaving the other counters alone.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14)); }

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Score MFMAs with their accumulator pinned to VGPRs: the 32 x 512 output accumulator of each wave
// takes all 256 AGPRs.  Hazards the compiler cannot see through asm are padded explicitly: two
// wait states before each MFMA (a VALU write of an operand may precede it) and, after the last,
// enough for a VALU access of the 8-pass result (the drain ties itself to the accumulator so
// nothing touching it is scheduled earlier).
__device__ __forceinline__ void mfma_v_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// The same without the leading wait states, for loops whose MFMA operands come only from LDS reads
// (waited by lgkmcnt), from registers no vector-ALU instruction wrote within the last two
// instructions, and from the previous MFMA's accumulator (the hardware forwards that one).
__device__ __forceinline__ void mfma_v_first_nw(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v_nw(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v_drain(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
}
// Output MFMAs with their accumulator pinned to AGPRs ("+a"): left to itself the compiler turns the
// loop-carried 256-register accumulator into VGPR copies and spills.
__device__ __forceinline__ void mfma_a(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_a_nw(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// acc = 0, produced by the matrix core itself (0 x 0 + 0) so it lands in AGPRs.
__device__ __forceinline__ void mfma_a_zero(f32x16& acc, const bf16x8& zero) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc) : "v"(zero));
}
// Wait states before anything other than an MFMA reads the output accumulators.
__device__ __forceinline__ void mfma_a_drain(f32x16* o) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]),
                 "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]),
                 "+a"(o[12]), "+a"(o[13]), "+a"(o[14]), "+a"(o[15]));
}

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Lane id as an opaque asm result: addresses derived from it where they are used cannot be hoisted
// out of the tile loop, where they would hold VGPRs for its whole length.
__device__ __forceinline__ int lane_id() {
  int ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  return ln;
}

// Block-table entries and lengths are read through the constant address space so they become
// scalar loads (lgkmcnt).  A vector load here would be ordered behind the in-flight LDS DMA and its
// wait would drain the whole ring.  Neither array is written while a launch runs.
__device__ __forceinline__ int ld_const(const int32_t* ptr, size_t i) {
  return ((const CONST_AS int32_t*)ptr)[i];
}

// Maxima of scores (finite or -inf) as single instructions: fmaxf would first quiet possible
// signalling NaNs of every operand it cannot prove canonical, one extra instruction each.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// max / sum of a value and its copy in lane l ^ 32
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Walks the 32-token tiles of one work unit (pages [pg0, pg1) of the concatenated batch) in order.
// Every field is wave-uniform and lives in scalar registers.
struct TileCursor {
  const int32_t* lens;
  int sh;         // the cut's grain: 1 << sh tokens (32 under the weighted cut, else 64, a page)
  int pg0, pg1;   // the unit's global range, in grains
  int b;          // current sequence
  int before;     // grains of sequences [0, b)
  int len, np;    // tokens / grains of sequence b
  int t;          // first token of the current tile
  int t_end;      // end token of the current segment
  bool valid;
  bool all_live;  // every unit holds at least one grain

  __device__ __forceinline__ void load_seq() {
    len = ld_const(lens, b);
    np = (int)(((unsigned)max(len, 0) + (1u << sh) - 1) >> sh);
  }
  // Sets t / t_end for sequence b, skipping sequences with no tokens.
  __device__ __forceinline__ void enter() {
    while (np == 0) {
      ++b;
      load_seq();
    }
    const int p0 = max(pg0 - before, 0);
    const int p1 = min(pg1 - before, np);
    t = p0 << sh;
    t_end = min(p1 << sh, len);
  }
  // a / d for a >= 0, d > 0: a 32-bit division when `small` (operands below 2^32), else 64-bit.
  static __device__ __forceinline__ long long udiv(long long a, long long d, bool small) {
    return small ? (long long)((unsigned)a / (unsigned)d) : a / d;
  }
  // Unit w's range from a batch of at most 64 NCH sequences held in registers (lane i of chunk c
  // holds sequence 64 c + i): the cost-weighted tile cut with at least 8 tiles per unit (every unit
  // then holds a tile), else the plain page cut [floor(w P / W), floor((w + 1) P / W)).
  template <int NCH>
  __device__ __forceinline__ void init_resident(const DecodeParams& p, int w) {
    const int W = p.num_units;
    const int ln = threadIdx.x & 63;
    int len_c[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) len_c[c] = 64 * c + ln < p.batch ? max(p.seq_lens[64 * c + ln], 0) : 0;
    // tiles per sequence, inclusive scans of tiles and of non-empty sequences across the chunks
    int nt_c[NCH], tin_c[NCH], nc_c[NCH];
    int tb = 0, nb = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      nt_c[c] = (len_c[c] + 31) >> 5;
      const int ti = wave_incl_scan(nt_c[c]), ni = wave_incl_scan(nt_c[c] > 0 ? 1 : 0);
      tin_c[c] = tb + ti;
      nc_c[c] = nb + ni;
      tb = __builtin_amdgcn_readlane(tin_c[c], 63);
      nb = __builtin_amdgcn_readlane(nc_c[c], 63);
    }
    const int T = tb;
    int unit_incl[NCH], unit_n[NCH];  // the cut's grains per sequence and their inclusive scan
    if (weighted_cut(T, W)) {
      sh = 5;
      const bool small = ((long long)T + (long long)kSegmentCostTiles * p.batch + 1) * W < (1LL << 32);
      const long long cw = udiv((long long)w * T, W, small);
      // walls around cw: the last at or before it (k0) and the first after it (k1)
      int A0 = 0, n0 = 0, k0 = 0, A1 = T, n1 = nb, k1 = p.batch;
      bool found1 = false;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int sl = tin_c[c] - nt_c[c];
        const bool wall = nt_c[c] > 0 && udiv((udiv((long long)sl * W + T - 1, T, small)) * T, W, small) == sl;
        const unsigned long long lo = __ballot(wall && sl <= cw);
        const unsigned long long hi = __ballot(wall && sl > cw);
        if (!found1 && lo) {
          const int f = 63 - __clzll((long long)lo);
          A0 = __builtin_amdgcn_readlane(sl, f);
          n0 = __builtin_amdgcn_readlane(nc_c[c], f);
          k0 = 64 * c + f;
        }
        if (!found1 && hi) {
          const int f = __ffsll((long long)hi) - 1;
          A1 = __builtin_amdgcn_readlane(sl, f);
          n1 = __builtin_amdgcn_readlane(nc_c[c], f) - 1;
          k1 = 64 * c + f;
          found1 = true;
        }
      }
      const long long wa0 = udiv((long long)A0 * W + T - 1, T, small);
      const long long wa1 = found1 ? udiv((long long)A1 * W + T - 1, T, small) : W;
      const long long V = (A1 - A0) + (long long)kSegmentCostTiles * (n1 - n0);
      // the tile at virtual position x: the first sequence of the stretch whose tiles end past x
      auto tile_at = [&](long long x) __attribute__((always_inline)) {
        int r = A1;
        bool done = x >= V;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const int sl = tin_c[c] - nt_c[c];
          const int vs = sl - A0 + kSegmentCostTiles * (nc_c[c] - n0);  // virtual start of the lane's tiles
          const int bi = 64 * c + ln;
          const unsigned long long h = __ballot(!done && bi >= k0 && bi < k1 && nt_c[c] > 0 && vs + nt_c[c] > x);
          if (h) {
            const int f = __ffsll((long long)h) - 1;
            r = __builtin_amdgcn_readlane(sl, f) + max((int)x - __builtin_amdgcn_readlane(vs, f), 0);
            done = true;
          }
        }
        return r;
      };
      pg0 = uni(tile_at(udiv((w - wa0) * V, wa1 - wa0, small)));
      pg1 = uni(tile_at(udiv((w - wa0 + 1) * V, wa1 - wa0, small)));
      all_live = true;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        unit_incl[c] = tin_c[c];
        unit_n[c] = nt_c[c];
      }
    } else {
      sh = 6;
      int pb = 0;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        unit_n[c] = (len_c[c] + kPage - 1) / kPage;
        unit_incl[c] = pb + wave_incl_scan(unit_n[c]);
        pb = __builtin_amdgcn_readlane(unit_incl[c], 63);
      }
      const int P = pb;
      pg0 = uni((int)((long long)w * P / W));
      pg1 = uni((int)((long long)(w + 1) * P / W));
      all_live = P >= W;
    }
    valid = pg0 < pg1;
    if (!valid) return;
    // the sequence holding the unit's first grain
    bool found = false;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const unsigned long long h = __ballot(!found && 64 * c + ln < p.batch && unit_incl[c] > pg0);
      if (h) {
        const int f = __ffsll((long long)h) - 1;
        b = 64 * c + f;
        before = __builtin_amdgcn_readlane(unit_incl[c] - unit_n[c], f);
        found = true;
      }
    }
    b = uni(b);
    before = uni(before);
  }
  __device__ __forceinline__ void init(const DecodeParams& p, int w) {
    lens = p.seq_lens;
    const int W = p.num_units;
    if (p.batch <= 64) {
      init_resident<1>(p, w);
    } else if (p.batch <= 256) {
      init_resident<4>(p, w);
    } else {
      const int T = uni((int)total_tiles(p.seq_lens, p.batch));
      if (weighted_cut(T, W)) {
        sh = 5;
        long long t0, t1;
        weighted_unit_range(p.seq_lens, p.batch, W, w, T, t0, t1);
        pg0 = uni((int)t0);
        pg1 = uni((int)t1);
        all_live = true;
      } else {
        sh = 6;
        const int P = uni((int)total_pages(p.seq_lens, p.batch));
        pg0 = uni((int)((long long)w * P / W));
        pg1 = uni((int)((long long)(w + 1) * P / W));
        all_live = P >= W;
      }
      valid = pg0 < pg1;
      if (!valid) return;
      int bb;
      long long bf;
      locate_unit(p.seq_lens, p.batch, pg0, sh, bb, bf);
      b = uni(bb);
      before = uni((int)bf);
    }
    if (!valid) return;
    load_seq();
    enter();
  }
  __device__ __forceinline__ void advance() {
    t += kTileTok;
    if (t < t_end) return;
    before += np;
    if (before >= pg1) {
      valid = false;
      return;
    }
    ++b;
    load_seq();
    enter();
  }
  __device__ __forceinline__ bool last() const { return t + kTileTok >= t_end; }
};

// One 16-byte-per-lane copy HBM -> LDS (global_load_lds_dwordx4): lane l's 16 bytes from
// gbase + voff land at LDS byte lds + 16 l.  Issued as asm so that the compiler does not track it:
// it would otherwise wait for every such copy in flight before any LDS read it cannot prove
// disjoint, draining the ring each tile.  The kernel orders these copies itself (counted vmcnt
// waits plus a barrier before a stage is read or refilled).  No register is written.
__device__ __forceinline__ void dma16(const char* gbase, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(gbase), "s"(lds)
               : "memory", "m0");
}
// The same for 4 bytes a lane (global_load_lds_dword): they land at LDS byte lds + 4 l.
__device__ __forceinline__ void dma4(const char* gbase, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(gbase), "s"(lds)
               : "memory", "m0");
}

// Copy j of a wave's token group: lane l's 16 bytes from gbase + voff + 128 j land at LDS byte
// lds + 1024 j + 16 l.  The instruction offset (128 j) is added to the LDS address as well, so M0
// takes lds + 896 j: one scalar add per copy.  j must fold to a constant.
__device__ __forceinline__ void dma16_group(const char* gbase, unsigned voff, unsigned lds, int j) {
  if (j == 0) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(gbase), "s"(lds)
                 : "memory", "m0");
  } else {
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%4"
                 :
                 : "v"(voff), "s"(gbase), "s"(lds), "i"(896 * j), "i"(128 * j)
                 : "memory", "m0", "scc");
  }
}

// The same copy from a per-lane 64-bit address: lane l's 16 bytes from addr + 128 j land at LDS byte
// lds + 16 l (lds the block's own address; M0 takes lds - 128 j).  j must fold to a constant.
__device__ __forceinline__ void dma16_addr(uint64_t addr, unsigned lds, int j) {
  if (j == 0) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(addr), "s"(lds)
                 : "memory", "m0");
  } else {
    asm volatile("s_add_u32 m0, %1, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%3"
                 :
                 : "v"(addr), "s"(lds), "i"(-128 * j), "i"(128 * j)
                 : "memory", "m0", "scc");
  }
}

// Kept tokens read in place: the byte address of the cache row of list entry
// min(8 g + tl, nt - 1) of the tile at cursor c (entries are token positions, read through the
// block table).  The 16 list and table reads are wave-uniform scalar loads; each lane then selects
// the row of its token-in-group tl.
__device__ __forceinline__ uint64_t topk_row_addr(const DecodeParams& p, const TileCursor& c, int g, int nt,
                                                  int tl) {
  const size_t lb = (size_t)c.b * p.pos_stride + c.t;
  const size_t tb = (size_t)c.b * p.max_blocks;
  int r = 0;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const unsigned pos = (unsigned)ld_const(p.positions, lb + min(8 * g + kk, nt - 1));
    const int row = ld_const(p.block_table, tb + pos / kPage) * kPage + (int)(pos % kPage);
    r = (kk == 0 || tl == kk) ? row : r;
  }
  return (uint64_t)(uintptr_t)p.cache + (uint64_t)(unsigned)r * (kRow * 2);
}

// DMA of one tile: wave w fills blocks [w * per, (w + 1) * per).  For a full tile the per-lane part
// of every source address is one of two lane constants (token-group parity); a ragged tile (fewer
// than 32 tokens) re-reads its last valid row in place of the missing ones.
template <bool TOPK>
__device__ __forceinline__ void issue_tile(const DecodeParams& p, const TileCursor& c,
                                           LDS_AS char* stage, int wave) {
  constexpr int kPer = kBlocks / kWaves;
  const int nt = min(kTileTok, c.t_end - c.t);
  const unsigned lds = (unsigned)(uintptr_t)stage;
  int ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  if constexpr (TOPK) {  // the wave's token groups, each lane's row looked up through the list
#pragma unroll
    for (int g = 0; g < kPer / kCG; ++g) {
      const int tg = wave * (kPer / kCG) + g;
      const int tl = (ln >> 3) ^ (tg & 1);
      const uint64_t ra = topk_row_addr(p, c, tg, nt, tl) + (unsigned)(((ln & 7) ^ sigma(tl)) * 16);
#pragma unroll
      for (int cg = 0; cg < kCG; ++cg) dma16_addr(ra, lds + (tg * kCG + cg) * 1024, cg);
    }
    return;
  }
  const int page = ld_const(p.block_table, (size_t)c.b * p.max_blocks + (unsigned)c.t / kPage);
  const char* base = reinterpret_cast<const char*>(p.cache) +
                     ((size_t)page * kPage + ((unsigned)c.t % kPage)) * (kRow * 2);
  if (nt == kTileTok) {
    // slot (lane / 8, lane % 8) of a block holds token-in-group (lane / 8) ^ parity and
    // chunk-in-group (lane % 8) ^ sigma(token-in-group)
    int lane_off[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int tl = (ln >> 3) ^ par;
      lane_off[par] = tl * (kRow * 2) + ((ln & 7) ^ sigma(tl)) * 16;
    }
    // wave w copies token group w
    const char* gb = base + wave * 8 * (kRow * 2);
#pragma unroll
    for (int j = 0; j < kPer; ++j) dma16_group(gb, (unsigned)lane_off[wave & 1], lds + wave * kPer * 1024, j);
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int blk = wave * kPer + j;
      const int tg = blk / kCG, cg = blk % kCG;
      const int tl = (ln >> 3) ^ (tg & 1);
      const int cl = (ln & 7) ^ sigma(tl);
      const int tt = min(8 * tg + tl, nt - 1);
      dma16(base, (unsigned)(tt * (kRow * 2) + (8 * cg + cl) * 16), lds + blk * 1024);
    }
  }
}

// Score operand for k-step ks: 8 consecutive latent dims (16 ks + 8 half ..) of token (lane % 32).
// tk = tile + this lane's offset for ks = 0; the chunk 2 (ks % 4) + half of chunk group ks / 4 only
// flips bits 5-6 of the offset (the swizzle XORs the chunk's upper bits with a lane constant) and
// the chunk group is 1 KB per step.
__device__ __forceinline__ bf16x8 k_operand(unsigned tk, int ks) {
  const unsigned a = tk ^ (32u * (ks & 3));
  return *reinterpret_cast<const LDS_AS bf16x8*>((const LDS_AS char*)(uintptr_t)a + 1024 * (ks >> 2));
}

// Output operand for d-block db and token half m: 8 tokens of one latent dim, gathered by two
// 16-lane transposing reads (token rows 16 m + 8 r + 4 half + (lane % 16) / 4, r = 0, 1).  tv =
// tile + this lane's offset for db 0, r 0; odd d-blocks flip bit 6 of the offset (chunk bit 2), the
// second token group of a half flips bit 7 (token-group parity in the swizzle), the column group
// db / 2 and the token half are whole blocks (immediates).
__device__ __forceinline__ bf16x8 v_operand(unsigned tv, int db, int m) {
  const unsigned a = tv ^ (64u * (db & 1));
  const LDS_AS char* p0 = (const LDS_AS char*)(uintptr_t)a + ((2 * m) * kCG + (db >> 1)) * 1024;
  const LDS_AS char* p1 = (const LDS_AS char*)(uintptr_t)(a ^ 128u) + ((2 * m + 1) * kCG + (db >> 1)) * 1024;
  const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)p0);
  const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)p1);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Workgroups go to the eight XCDs round-robin (workgroup i to XCD i mod 8), each XCD with its own
// L2.  Consecutive work units, which hold neighbouring pages and mostly the same sequence, are
// placed on one XCD so that they share its L2 for that sequence's query and block-table lines.
__device__ __forceinline__ int xcd_unit(int id, int n) {
  const int per = n / 8, rem = n % 8, x = id % 8;
  return x * per + min(x, rem) + id / 8;
}

template <bool TOPK>
__global__ __launch_bounds__(kWaves * 64, 1) void decode_mfma_kernel(DecodeParams p) {
  constexpr int kPer = kBlocks / kWaves;  // copies per wave per tile
  __shared__ __attribute__((aligned(1024))) char ring[kStages][kTileBytes];
  // Target of the copies a unit issues after its last tile: they keep the count of copies per tile
  // fixed, which the counted waits rely on, and nothing reads them.
  __shared__ __attribute__((aligned(1024))) char sink[kPer * 1024];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;       // which K half of the MFMA operands this lane holds
  const int l32 = lane & 31;
  const int w = uni(xcd_unit(blockIdx.x, gridDim.x));

  TileCursor ld, cp;
  ld.init(p, w);
  cp = ld;
  if (!cp.valid) return;

  // Score operand base: token l32, chunk half.  Output operand base: token 4 half + (lane % 16) / 4,
  // chunk 2 ((lane / 16) % 2) + (lane % 4) / 2, byte 8 (lane % 2).  The per-step XORs above touch
  // bits the swizzle alone sets, and every stage starts on a 1 KB boundary, so they may be applied
  // after adding the stage base.
  const unsigned k_off = (unsigned)tile_offset(l32, half);
  const unsigned v_off = (unsigned)(tile_offset(4 * half + ((lane & 15) >> 2),
                                                2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) + 8 * (lane & 1));

  // The query of a segment lives in VGPRs for the whole segment (36 x 8 bf16 per lane).
  const uint16_t* qa = static_cast<const uint16_t*>(p.q_abs);
  bf16x8 q[36];
  // Head of accumulator column c (0 .. 31) of this wave: (32 wave + c) mod H.  Below 128 heads
  // the columns repeat heads: same query, same data, so bit-identical results, and every store they
  // make writes the same bits to the same place as the first copy's.  (Heads are powers of two.)
  auto head_of = [&](int c) __attribute__((always_inline)) { return (wave * 32 + c) & (p.heads - 1); };
  auto load_q = [&](int b) __attribute__((always_inline)) {
    const int ln = lane_id();
    const uint16_t* qrow = qa + ((size_t)b * p.heads + head_of(ln & 31)) * kRow + 8 * (ln >> 5);
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) q[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks);
  };
  // The first segment's query is requested ahead of the first copies, so that waiting for it does
  // not wait for them.
  load_q(cp.b);

  // Prologue: three tiles in flight.
  int issued = 0;
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) {
    if (ld.valid) {
      issue_tile<TOPK>(p, ld, (LDS_AS char*)ring[s], wave);
      ld.advance();
      ++issued;
    }
  }
  // Loads complete in issue order: with at most the prologue's copies outstanding (capped at the
  // counter's 63, which only waits for more), the query has landed.
  if (issued >= 3) wait_vmcnt<(3 * kPer < 63 ? 3 * kPer : 63)>();
  else if (issued == 2) wait_vmcnt<(2 * kPer < 63 ? 2 * kPer : 63)>();
  else wait_vmcnt<(kPer < 63 ? kPer : 63)>();
  // Waits until the copies of tile `t` (this wave's part) have landed, then for every wave.
  // Vector loads complete in issue order: it is enough to let the tiles issued after it stay in
  // flight.
  auto tile_ready = [&](int t) __attribute__((always_inline)) {
    const int younger = issued - t - 1;
    if (younger >= 2) wait_vmcnt<(2 * kPer < 63 ? 2 * kPer : 63)>();
    else if (younger == 1) wait_vmcnt<(kPer < 63 ? kPer : 63)>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  };

  // Scores of a ragged tile (n < 32 tokens) with the tokens past the end at -inf, so that they take
  // no weight.  Lane half h, register j holds token 8 (j / 4) + 4 h + j % 4.
  auto tail_masked = [&](const f32x16& s, int n) __attribute__((always_inline)) {
    f32x16 r;
    const int hf = lane_id() >> 5;
#pragma unroll
    for (int j = 0; j < 16; ++j) r[j] = ((j >> 2) * 8 + hf * 4 + (j & 3) >= n) ? -INFINITY : s[j];
    return r;
  };

  const float scale = p.scale_log2;
  int it = 0;  // tile index within the unit
  bool first_segment = true;
  while (cp.valid) {  // one segment: the part of sequence b inside this unit
    const int b = cp.b;
    if (threadIdx.x == 0) {  // the merge reads the range of units that hold sequence b from here
      if (cp.t == 0) {
        p.seq_units[4 * b] = w;
        p.seq_units[4 * b + 2] = cp.all_live ? 1 : 0;
      }
      if (cp.t_end == cp.len) p.seq_units[4 * b + 1] = w;
    }
    if (!first_segment) {
      load_q(b);
      // Wait here, once per segment: left to the compiler, the wait for Q would sit inside the tile
      // loop and drain the copy ring on every tile.
      wait_vmcnt<0>();
    }
    first_segment = false;
    f32x16 o[16];
    {
      const bf16x8 zero = {};
#pragma unroll
      for (int i = 0; i < 16; ++i) mfma_a_zero(o[i], zero);
    }
    float m_ref = -INFINITY;  // base-2 reference maximum (same in lanes l and l ^ 32)
    float l_sum = 0.f;        // this lane's share of the softmax denominator
    bool fresh = true;

    // Scores of the segment's first tile, on their own.
    f32x16 s_cur;
    {
      tile_ready(it);
      const unsigned tk = (unsigned)(uintptr_t)(LDS_AS char*)ring[stage_of(it)] + k_off;
      bf16x8 ka[kKAhead + 1];
#pragma unroll
      for (int ks = 0; ks < kKAhead; ++ks) ka[ks] = k_operand(tk, ks);
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) {
        if (ks + kKAhead < 36) ka[(ks + kKAhead) % (kKAhead + 1)] = k_operand(tk, ks + kKAhead);
        if (ks == 0) mfma_v_first(s_cur, ka[0], q[0]); else mfma_v(s_cur, ka[ks % (kKAhead + 1)], q[ks]);
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma_v_drain(s_cur);
      const int n0 = min(kTileTok, cp.t_end - cp.t);
      if (n0 < kTileTok) s_cur = tail_masked(s_cur, n0);
    }

    bool last;
    do {  // tile `it`: its softmax and output product, overlapped with the next tile's scores
      last = cp.last();
      cp.advance();
      // Copies of tile it + 3 into the stage of tile it - 1.  With four waves, each wave copies one
      // token group (nine 1 KB blocks), one block per four score MFMAs below: 36 copies at once
      // would queue in the address unit and hold every wave for hundreds of cycles.  A ragged tile
      // repeats its last row in place of the missing ones; after the unit's last tile the copies
      // go to the sink (from the first page, which always exists).  The addresses are worked out
      // before the wait below, so that the block-table read overlaps it; the copies start after it.
      const char* sp_base = reinterpret_cast<const char*>(p.cache);
      unsigned sp_lane = 0, sp_lds = 0;
      uint64_t sp_addr = 0;  // kept tokens: this lane's full source address
      int sp_page = 0, sp_tok = 0;
      bool sp_have = false;
      {
        const int ln = lane_id();
        const int tl = (ln >> 3) ^ (wave & 1);
        const unsigned cl16 = (unsigned)((ln & 7) ^ sigma(tl)) * 16u;
        sp_have = ld.valid;
        if (ld.valid) {
          const int ntl = min(kTileTok, ld.t_end - ld.t);
          if constexpr (TOPK) {
            sp_addr = topk_row_addr(p, ld, wave, ntl, tl) + cl16;
          } else {
            sp_page = ld_const(p.block_table, (size_t)ld.b * p.max_blocks + (unsigned)ld.t / kPage);
            sp_tok = (int)((unsigned)ld.t % kPage);
            sp_lane = (unsigned)min(8 * wave + tl, ntl - 1) * (kRow * 2) + cl16;
          }
          sp_lds = (unsigned)(uintptr_t)(LDS_AS char*)ring[stage_of(it + kStages - 1)] + wave * kPer * 1024;
          ld.advance();
        } else {
          sp_lane = (unsigned)(8 * wave + tl) * (kRow * 2) + cl16;
          sp_addr = (uint64_t)(uintptr_t)sp_base + sp_lane;
          sp_lds = (unsigned)(uintptr_t)(LDS_AS char*)sink;
        }
      }
      // The next tile must be in LDS before its scores start; the barrier also frees the stage of
      // tile it - 1.
      tile_ready(last ? it : it + 1);
      ++issued;
      if constexpr (TOPK) {
        asm volatile("" : "+v"(sp_addr));
      } else {
        asm volatile("" : "+s"(sp_page));  // the page is first needed here, behind the wait
        if (sp_have) sp_base += ((size_t)sp_page * kPage + sp_tok) * (kRow * 2);
      }
      auto spread_copy = [&](int j) __attribute__((always_inline)) {
        if constexpr (TOPK) dma16_addr(sp_addr, sp_lds + 1024 * j, j);
        else dma16_group(sp_base, sp_lane, sp_lds, j);
      };

      // ---- softmax of tile it (base 2), lane = head, registers = tokens, spread over the next
      // tile's score MFMAs -------------------------------------------------------------------------
      float mt, ls0 = 0.f, ls1 = 0.f, alpha = 1.f;
      bool rescale = false;
      bf16x8 pb0, pb1;
      // exponent j of the tile (token slot j of the accumulator), two running sums
      auto softmax_exp = [&](int j) __attribute__((always_inline)) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s_cur[j], scale, -m_ref));
        if (j & 1) ls1 += e; else ls0 += e;
        if (j < 8) pb0[j] = (__bf16)e; else pb1[j - 8] = (__bf16)e;
      };
      auto softmax_step = [&](int k) __attribute__((always_inline)) {
        if (k == 0) {
          mt = max3(max3(s_cur[0], s_cur[1], s_cur[2]), max3(s_cur[3], s_cur[4], s_cur[5]),
                    max2(s_cur[6], s_cur[7]));
        } else if (k == 1) {
          mt = max3(max3(mt, s_cur[8], s_cur[9]), max3(s_cur[10], s_cur[11], s_cur[12]),
                    max3(s_cur[13], s_cur[14], s_cur[15]));
        } else if (k == 2) {
          mt = max_halves(mt) * scale;
        } else if (k == 3) {
          if (fresh) {
            m_ref = mt;
            fresh = false;
          } else if (__ballot(mt > m_ref + kRescaleThreshold)) {
            // Rare (the running maximum jumped by more than 2^8): the reference moves and O is
            // scaled by alpha after the score MFMAs, before this tile's product is added.
            const float m_new = fmaxf(m_ref, mt);
            alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
            m_ref = m_new;
            l_sum *= alpha;
            rescale = true;
          }
        } else if (k >= 4 && k < 4 + 8) {
          softmax_exp(k - 4);
        }
      };

      f32x16 s_nxt;
      if (!last) {
        // scores of tile it + 1 into s_nxt, one softmax step of tile it after each MFMA
        const unsigned tk = (unsigned)(uintptr_t)(LDS_AS char*)ring[stage_of(it + 1)] + k_off;
        bf16x8 ka[kKAhead + 1];
#pragma unroll
        for (int ks = 0; ks < kKAhead; ++ks) ka[ks] = k_operand(tk, ks);
#pragma unroll
        for (int ks = 0; ks < 36; ++ks) {
          if (ks + kKAhead < 36) ka[(ks + kKAhead) % (kKAhead + 1)] = k_operand(tk, ks + kKAhead);
          if (ks == 0) mfma_v_first_nw(s_nxt, ka[0], q[0]); else mfma_v_nw(s_nxt, ka[ks % (kKAhead + 1)], q[ks]);
          softmax_step(ks);
          if ((ks & 3) == 0) spread_copy(ks >> 2);
          __builtin_amdgcn_sched_barrier(0);
        }
        mfma_v_drain(s_nxt);
      } else {
#pragma unroll
        for (int k = 0; k < 12; ++k) softmax_step(k);
#pragma unroll
        for (int j = 0; j < kCG; ++j) spread_copy(j);
      }

      if (__builtin_expect(rescale, 0)) {
        // The accumulators make a round trip through this piece's own workspace slot, which its
        // final write overwrites anyway, so scaling them never holds more than one block in VGPRs.
        mfma_a_drain(o);
        const int ln = lane_id();
        float* slot = p.ws_o + (((size_t)w + b) * p.heads + head_of(ln & 31)) * kDc + 4 * (ln >> 5);
#pragma unroll
        for (int db = 0; db < 16; ++db) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<float4*>(slot + 32 * db + 8 * g) =
                make_float4(o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]);
        }
        asm volatile("" ::: "memory");  // the values must come back from memory
#pragma unroll
        for (int db = 0; db < 16; ++db) {
          f32x16 t;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 v = *reinterpret_cast<const float4*>(slot + 32 * db + 8 * g);
            t[4 * g] = v.x * alpha;
            t[4 * g + 1] = v.y * alpha;
            t[4 * g + 2] = v.z * alpha;
            t[4 * g + 3] = v.w * alpha;
          }
          o[db] = t;
          __builtin_amdgcn_sched_barrier(0);
        }
        // Q is read again from memory: redefining it here frees its 144 VGPRs for this block
        // instead of leaving the register allocator to spill it around the hot loop.
        load_q(b);
        wait_vmcnt<0>();
      }

      // ---- output of tile it: O^T += V^T . P^T, first the 16 tokens of pb0 for every d-block,
      // then those of pb1 (the exponents of pb1 are computed during the first pass); operands
      // kVAhead MFMAs ahead.
      {
        const unsigned tv = (unsigned)(uintptr_t)(LDS_AS char*)ring[stage_of(it)] + v_off;
        bf16x8 va[kVAhead + 1];
#pragma unroll
        for (int i = 0; i < kVAhead; ++i) va[i] = v_operand(tv, i & 15, i >> 4);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int nx = i + kVAhead;
          if (nx < 32) va[nx % (kVAhead + 1)] = v_operand(tv, nx & 15, nx >> 4);
          if (i == 0) mfma_a(o[0], va[0], pb0);                     // pb0 was just written
          else if (i < 16) mfma_a_nw(o[i], va[i % (kVAhead + 1)], pb0);
          else if (i == 16) mfma_a(o[0], va[16 % (kVAhead + 1)], pb1);
          else mfma_a_nw(o[i & 15], va[i % (kVAhead + 1)], pb1);
          if (i < 8) softmax_exp(8 + i);
          if (i == 8) l_sum += ls0 + ls1;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (!last) {  // the second half of tile it's scores was needed until here
        const int nn = min(kTileTok, cp.t_end - cp.t);  // cp holds tile it + 1 now
        s_cur = nn < kTileTok ? tail_masked(s_nxt, nn) : s_nxt;
      }
      ++it;
    } while (!last);

    // ---- end of segment: the piece's sum, divided by its softmax sum, is stored in bf16 (half the
    // bytes of the fp32 sum; the merge weighs it by that sum again) with (reference max, sum).
    const float l_tot = sum_halves(l_sum);
    const float inv = 1.f / l_tot;
    mfma_a_drain(o);
    const int ln = lane_id();
    const size_t part = ((size_t)w + b) * p.heads + head_of(ln & 31);
    // four sums of one lane, divided by the softmax sum, rounded to bf16 (nearest even)
    auto packed_out = [&](int db, int g) __attribute__((always_inline)) {
      const bf16x4 v = {(__bf16)(o[db][4 * g] * inv), (__bf16)(o[db][4 * g + 1] * inv),
                        (__bf16)(o[db][4 * g + 2] * inv), (__bf16)(o[db][4 * g + 3] * inv)};
      return __builtin_bit_cast(u32x2, v);
    };
    {
      // Rows go through LDS and leave as 256-byte quarter rows: written straight from the
      // accumulator layout, each store would write 8-byte pieces of 32 rows (about 20,000 cycles
      // for a unit's stores instead of about 6,500).  Once every wave is done with the last tile
      // its stage is free: each wave takes 32 heads x 128 dims of it, padded by 16 bytes per row
      // against bank conflicts, and passes its rows through a quarter at a time.
      constexpr int kPad = 256 + 16;
      __builtin_amdgcn_s_barrier();
      LDS_AS char* region = (LDS_AS char*)ring[stage_of(it - 1)] + wave * 32 * kPad;
      const int hw = ln & 31, hl = ln >> 5;
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<LDS_AS u32x2*>(region + hw * kPad + (32 * d + 8 * g + 4 * hl) * 2) = packed_out(4 * qt + d, g);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int h = 4 * k + (ln >> 4);
          const u32x4 v = *reinterpret_cast<const LDS_AS u32x4*>(region + h * kPad + (ln & 15) * 16);
          const size_t ph = ((size_t)w + b) * p.heads + head_of(h);
          *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.ws_o + ph * kDc) + 128 * qt + 8 * (ln & 15)) = v;
        }
      }
    }
    if (ln < 32) *reinterpret_cast<float2*>(p.ws_ml + 2 * part) = make_float2(m_ref, l_tot);
  }
  // No copy into LDS may still be in flight when the workgroup ends.
  wait_vmcnt<0>();
}

// ---- ~6-bit cache, read from its codes -----------------------------------------------------------
// A tile of 32 rows lands in LDS as 40 sixteen-byte slots per row (row stride 640 bytes): slot p of
// row t holds code chunk c (codes 16 c .. 16 c + 15, 12 bytes, copied as 16 bytes from the packed
// row, so that every chunk starts on a 16-byte boundary), c = (p & ~7) | ((p & 7) ^ f6swz(t)); slots
// whose c is 36 or more are padding.  The rows' fp32 scales follow at byte 20,480.
//   scores: lane (token t, half h) converts codes 64 j + 32 h .. + 31 of its token (chunks 4 j + 2 h
//     and + 1, two 12-byte reads) with v_cvt_scalef32_pk32_bf16_fp6 and the row's scale (exact:
//     code x 2^e), giving its A operands of k-steps 4 j .. 4 j + 3; the query is loaded in the same
//     k order (dims 64 j + 32 h + 8 i of k-step 4 j + i).
//   output: ds_read_b96_tr_b6 gives each lane of a 16-lane group one code column (one latent dim)
//     of the 16 rows whose addresses the group's lanes supply: lanes of half h supply tokens
//     4 h + 8 (e / 4) + e % 4, e = 0 .. 15, the order of the probabilities the lane holds, and two
//     d-blocks' reads convert at scale 1 into the A operands of both output MFMAs of both blocks.
//     The rows' scales 2^e_t move onto the probabilities instead (exact in bf16 but for values
//     below 2^-125, which add nothing).
// The swizzle f6swz spreads the 32 rows of a score read over 8 slots per 8 rows and the 16 rows of
// one transposing read over pairs of slots.
constexpr int kF6Slots = 40;                        // 16-byte slots per row in LDS
constexpr int kF6RowStride = kF6Slots * 16;         // 640
constexpr int kF6ScaleOff = kTileTok * kF6RowStride;  // 20,480: the rows' fp32 scales
constexpr int kF6DataCopies = kTileTok * kF6Slots / 64;  // 20 copies of 64 slots per tile

__device__ __forceinline__ int f6swz(int t) { return (t & 3) | ((((t >> 2) ^ (t >> 3)) & 1) << 2); }

// Byte offset, inside a packed ~6-bit page row block, of the source of LDS slot g (0 .. 1,279) of a
// tile: row min(g / 40, nt - 1), chunk c (chunk 0 for padding slots).
__device__ __forceinline__ unsigned f6_src_off(int g, int nt) {
  const int t = g / kF6Slots, slot = g % kF6Slots;
  int c = (slot & ~7) | ((slot & 7) ^ f6swz(t));
  if (c >= kRow / 16) c = 0;
  return (unsigned)(min(t, nt - 1) * kFp6RowBytes + 12 * c);
}

template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void decode_fp6_kernel(DecodeParams p) {
  constexpr int kDataPer = kF6DataCopies / NW;      // 5 (four waves) or 10 (two waves)
  constexpr int kPer = kDataPer + 1;                // plus this wave's rows' scales
  constexpr int kScaleRows = kTileTok / NW;         // scales this wave copies
  static_assert(kF6DataCopies % NW == 0, "whole copies per wave");
  __shared__ __attribute__((aligned(1024))) char ring[kStages][kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sink[1024];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int w = uni(xcd_unit(blockIdx.x, gridDim.x));

  TileCursor ld, cp;
  ld.init(p, w);
  cp = ld;
  if (!cp.valid) return;

  // Score operand: row l32, chunk pair 4 j + 2 half: two lane offsets (j even / odd); the second
  // chunk of a pair is the slot XOR 1 (byte XOR 16), and j / 2 adds 128 bytes.
  unsigned ko[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) ko[par] = (unsigned)(l32 * kF6RowStride + 16 * ((4 * par + 2 * half) ^ f6swz(l32)));
  // Output operand: this lane supplies the row of token 4 (lane / 32) + 8 (e / 4) + e % 4, e = lane
  // % 16, for chunk 2 db + (lane / 16) % 2; four lane offsets (db % 4), db / 4 adds 128 bytes.
  unsigned vo[4];
  {
    const int e = lane & 15, g = lane >> 4;
    const int tv = 4 * (g >> 1) + 8 * (e >> 2) + (e & 3);
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4) vo[d4] = (unsigned)(tv * kF6RowStride + 16 * ((2 * d4 + (g & 1)) ^ f6swz(tv)));
  }
  // Source offsets of this wave's data copies for a full tile (row 0 = the tile's first row).
  unsigned so[kDataPer];
#pragma unroll
  for (int j = 0; j < kDataPer; ++j) so[j] = f6_src_off(64 * (wave * kDataPer + j) + lane, kTileTok);

  const uint16_t* qa = static_cast<const uint16_t*>(p.q_abs);
  bf16x8 q[36];
  auto load_q = [&](int b) __attribute__((always_inline)) {
    const int ln = lane_id();
    const uint16_t* qrow = qa + ((size_t)b * p.heads + wave * 32 + (ln & 31)) * kRow + 32 * (ln >> 5);
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) q[ks] = *reinterpret_cast<const bf16x8*>(qrow + 64 * (ks >> 2) + 8 * (ks & 3));
  };
  load_q(cp.b);

  // Copies of the tile at cursor c into LDS stage `lds` (sink when !have): data copy j of this wave,
  // then (j == kDataPer) its rows' scales.  j must fold to a constant.
  auto copy = [&](bool have, const char* pb, int slot0, int nt, unsigned lds, int j) __attribute__((always_inline)) {
    const char* rows = pb + (size_t)slot0 * kFp6RowBytes;
    if (j < kDataPer) {
      const unsigned off = (have && nt < kTileTok) ? f6_src_off(64 * (wave * kDataPer + j) + lane_id(), nt) : so[j];
      dma16(rows, off, have ? lds + 1024 * (wave * kDataPer + j) : (unsigned)(uintptr_t)(LDS_AS char*)sink);
    } else {
      const int ln = lane_id();
      if (ln < kScaleRows) {
        const int r = wave * kScaleRows + ln;
        dma4(pb + kPage * kFp6RowBytes, (unsigned)(4 * (slot0 + min(r, nt - 1))),
             have ? lds + kF6ScaleOff + 4 * wave * kScaleRows : (unsigned)(uintptr_t)(LDS_AS char*)sink);
      }
    }
  };
  auto page_of_ld = [&]() __attribute__((always_inline)) {
    return reinterpret_cast<const char*>(p.cache) +
           (size_t)ld_const(p.block_table, (size_t)ld.b * p.max_blocks + (unsigned)ld.t / kPage) * kFp6PageBytes;
  };

  int issued = 0;
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) {
    if (ld.valid) {
      const char* pb = page_of_ld();
      const int slot0 = (int)((unsigned)ld.t % kPage), nt = min(kTileTok, ld.t_end - ld.t);
#pragma unroll
      for (int j = 0; j < kPer; ++j) copy(true, pb, slot0, nt, (unsigned)(uintptr_t)(LDS_AS char*)ring[s], j);
      ld.advance();
      ++issued;
    }
  }
  if (issued >= 3) wait_vmcnt<3 * kPer>();
  else if (issued == 2) wait_vmcnt<2 * kPer>();
  else wait_vmcnt<kPer>();
  auto tile_ready = [&](int t) __attribute__((always_inline)) {
    const int younger = issued - t - 1;
    if (younger >= 2) wait_vmcnt<2 * kPer>();
    else if (younger == 1) wait_vmcnt<kPer>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  };
  auto tail_masked = [&](const f32x16& s, int n) __attribute__((always_inline)) {
    f32x16 r;
    const int hf = lane_id() >> 5;
#pragma unroll
    for (int j = 0; j < 16; ++j) r[j] = ((j >> 2) * 8 + hf * 4 + (j & 3) >= n) ? -INFINITY : s[j];
    return r;
  };
  // Score operands of k-steps 4 j .. 4 j + 3 from stage st: two 12-byte reads and a conversion.
  auto k_conv_read = [&](unsigned st, int j, u32x6& codes) __attribute__((always_inline)) {
    const LDS_AS char* a = (const LDS_AS char*)(uintptr_t)(st + ko[j & 1] + 128 * (j >> 1));
    const u32x3 c0 = *reinterpret_cast<const LDS_AS u32x3*>(a);
    const u32x3 c1 = *reinterpret_cast<const LDS_AS u32x3*>((const LDS_AS char*)(uintptr_t)((st + ko[j & 1] + 128 * (j >> 1)) ^ 16u));
    codes = u32x6{c0[0], c0[1], c0[2], c1[0], c1[1], c1[2]};
  };
  // 32 codes -> 32 bf16 (times the exponent of sc).  Written as asm: the compiler's builtin for this
  // conversion returned its first element in every position when probed on the GPU.
  auto cvt32 = [&](const u32x6& codes, float sc) __attribute__((always_inline)) {
    u32x16 v;
    asm volatile("v_cvt_scalef32_pk32_bf16_fp6 %0, %1, %2" : "=&v"(v) : "v"(codes), "v"(sc));
    return v;
  };
  // The same with wait states after it, for a result that an MFMA reads next.
  auto cvt32_w = [&](const u32x6& codes, float sc) __attribute__((always_inline)) {
    u32x16 v;
    asm volatile("v_cvt_scalef32_pk32_bf16_fp6 %0, %1, %2\n\ts_nop 4" : "=&v"(v) : "v"(codes), "v"(sc));
    return v;
  };
  auto op4 = [](const u32x16& v, int i) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, u32x4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]});
  };
  // Score product of the tile in stage st into s (36 MFMAs, conversions one group ahead); `step(ks)`
  // runs after each MFMA.
  auto scores = [&](unsigned st, f32x16& sacc, auto&& step) __attribute__((always_inline)) {
    const float sc = *reinterpret_cast<const LDS_AS float*>((const LDS_AS char*)(uintptr_t)(st + kF6ScaleOff + 4 * l32));
    u32x6 cd;
    k_conv_read(st, 0, cd);
    u32x16 cur = cvt32_w(cd, sc);
#pragma unroll
    for (int j = 0; j < 9; ++j) {
      u32x16 nxt;
      if (j + 1 < 9) k_conv_read(st, j + 1, cd);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ks = 4 * j + i;
        if (ks == 0) mfma_v_first(sacc, op4(cur, 0), q[0]);
        else mfma_v(sacc, op4(cur, i), q[ks]);
        step(ks);
        if (i == 1 && j + 1 < 9) nxt = cvt32(cd, sc);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (j + 1 < 9) cur = nxt;
    }
    mfma_v_drain(sacc);
  };
  auto no_step = [](int) __attribute__((always_inline)) {};

  const float scale = p.scale_log2;
  int it = 0;
  bool first_segment = true;
  while (cp.valid) {
    const int b = cp.b;
    if (threadIdx.x == 0) {
      if (cp.t == 0) {
        p.seq_units[4 * b] = w;
        p.seq_units[4 * b + 2] = cp.all_live ? 1 : 0;
      }
      if (cp.t_end == cp.len) p.seq_units[4 * b + 1] = w;
    }
    if (!first_segment) {
      load_q(b);
      wait_vmcnt<0>();
    }
    first_segment = false;
    f32x16 o[16];
    {
      const bf16x8 zero = {};
#pragma unroll
      for (int i = 0; i < 16; ++i) mfma_a_zero(o[i], zero);
    }
    float m_ref = -INFINITY;
    float l_sum = 0.f;
    bool fresh = true;

    f32x16 s_cur;
    {
      tile_ready(it);
      scores((unsigned)(uintptr_t)(LDS_AS char*)ring[stage_of(it)], s_cur, no_step);
      const int n0 = min(kTileTok, cp.t_end - cp.t);
      if (n0 < kTileTok) s_cur = tail_masked(s_cur, n0);
    }

    bool last;
    do {
      last = cp.last();
      cp.advance();
      // copies of tile it + 3 into the stage of tile it - 1 (the sink after the unit's last tile),
      // spread over the score MFMAs below
      const bool sp_have = ld.valid;
      const char* sp_pb = reinterpret_cast<const char*>(p.cache);
      int sp_slot0 = 0, sp_nt = kTileTok;
      if (sp_have) {
        sp_pb = page_of_ld();
        sp_slot0 = (int)((unsigned)ld.t % kPage);
        sp_nt = min(kTileTok, ld.t_end - ld.t);
        ld.advance();
      }
      const unsigned sp_lds = (unsigned)(uintptr_t)(LDS_AS char*)ring[stage_of(it + kStages - 1)];
      tile_ready(last ? it : it + 1);
      ++issued;
      asm volatile("" : "+s"(sp_pb));
      auto spread_copy = [&](int ks) __attribute__((always_inline)) {
        constexpr int kEvery = 32 / kPer;   // six copies: every 5 k-steps; eleven: every 2
#pragma unroll
        for (int j = 0; j < kPer; ++j)
          if (ks == kEvery * j) copy(sp_have, sp_pb, sp_slot0, sp_nt, sp_lds, j);
      };

      // probabilities of tile it carry the tokens' scales 2^e_t: this lane's 16 tokens are
      // 4 half + 8 k + 0 .. 3, k = 0 .. 3, four consecutive scales read together one group ahead
      const unsigned sb = (unsigned)(uintptr_t)(LDS_AS char*)ring[stage_of(it)] + kF6ScaleOff + 16 * half;
      auto tsc_read = [&](int k) __attribute__((always_inline)) {
        return *reinterpret_cast<const LDS_AS f32x4*>((const LDS_AS char*)(uintptr_t)(sb + 32 * k));
      };
      f32x4 tsc_cur = tsc_read(0), tsc_nxt = tsc_read(1);
      float mt, ls0 = 0.f, ls1 = 0.f, alpha = 1.f;
      bool rescale = false;
      bf16x8 pb0, pb1;
      auto softmax_exp = [&](int j) __attribute__((always_inline)) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s_cur[j], scale, -m_ref));
        if (j & 1) ls1 += e; else ls0 += e;
        const float pe = e * tsc_cur[j & 3];
        if (j < 8) pb0[j] = (__bf16)pe; else pb1[j - 8] = (__bf16)pe;
        if ((j & 3) == 3 && j < 15) {
          tsc_cur = tsc_nxt;
          if (j + 5 < 16) tsc_nxt = tsc_read((j + 5) >> 2);
        }
      };
      auto softmax_step = [&](int k) __attribute__((always_inline)) {
        if (k == 0) {
          mt = max3(max3(s_cur[0], s_cur[1], s_cur[2]), max3(s_cur[3], s_cur[4], s_cur[5]),
                    max2(s_cur[6], s_cur[7]));
        } else if (k == 1) {
          mt = max3(max3(mt, s_cur[8], s_cur[9]), max3(s_cur[10], s_cur[11], s_cur[12]),
                    max3(s_cur[13], s_cur[14], s_cur[15]));
        } else if (k == 2) {
          mt = max_halves(mt) * scale;
        } else if (k == 3) {
          if (fresh) {
            m_ref = mt;
            fresh = false;
          } else if (__ballot(mt > m_ref + kRescaleThreshold)) {
            const float m_new = fmaxf(m_ref, mt);
            alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
            m_ref = m_new;
            l_sum *= alpha;
            rescale = true;
          }
        } else if (k >= 4 && k < 4 + 16) {  // all 16 probabilities before the output product
          softmax_exp(k - 4);
        } else if (k == 4 + 16) {
          l_sum += ls0 + ls1;
        }
      };

      f32x16 s_nxt;
      if (!last) {
        scores((unsigned)(uintptr_t)(LDS_AS char*)ring[stage_of(it + 1)], s_nxt, [&](int ks) __attribute__((always_inline)) {
          softmax_step(ks);
          spread_copy(ks);
        });
      } else {
#pragma unroll
        for (int k = 0; k < 21; ++k) softmax_step(k);
#pragma unroll
        for (int ks = 0; ks < 32; ++ks) spread_copy(ks);
      }

      if (__builtin_expect(rescale, 0)) {
        mfma_a_drain(o);
        const int ln = lane_id();
        float* slot = p.ws_o + (((size_t)w + b) * p.heads + wave * 32 + (ln & 31)) * kDc + 4 * (ln >> 5);
#pragma unroll
        for (int db = 0; db < 16; ++db) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<float4*>(slot + 32 * db + 8 * g) =
                make_float4(o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]);
        }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int db = 0; db < 16; ++db) {
          f32x16 t;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 v = *reinterpret_cast<const float4*>(slot + 32 * db + 8 * g);
            t[4 * g] = v.x * alpha;
            t[4 * g + 1] = v.y * alpha;
            t[4 * g + 2] = v.z * alpha;
            t[4 * g + 3] = v.w * alpha;
          }
          o[db] = t;
          __builtin_amdgcn_sched_barrier(0);
        }
        load_q(b);
        wait_vmcnt<0>();
      }

      // output of tile it: per pair of d-blocks, two transposing reads and one conversion at scale
      // 1 give the A operands of four MFMAs; the next pair is read two pairs ahead and converted
      // while the current pair's MFMAs run, so no MFMA reads a register the conversion just wrote
      {
        const unsigned tv = (unsigned)(uintptr_t)(LDS_AS char*)ring[stage_of(it)];
        auto vread = [&](int db) __attribute__((always_inline)) {
          return __builtin_amdgcn_ds_read_tr6_b96_v3i32(
              (LDS_AS i32x3*)((LDS_AS char*)(uintptr_t)(tv + vo[db & 3] + 128 * (db >> 2))));
        };
        auto pair_codes = [](const i32x3& a, const i32x3& c) __attribute__((always_inline)) {
          return u32x6{(unsigned)a[0], (unsigned)a[1], (unsigned)a[2], (unsigned)c[0], (unsigned)c[1], (unsigned)c[2]};
        };
        i32x3 r0 = vread(0), r1 = vread(1);
        u32x16 vcur = cvt32_w(pair_codes(r0, r1), 1.0f);
        r0 = vread(2);
        r1 = vread(3);
#pragma unroll
        for (int pr = 0; pr < 8; ++pr) {
          const int d0 = 2 * pr, d1 = 2 * pr + 1;
          u32x16 vnxt;
          mfma_a(o[d0], op4(vcur, 0), pb0);
          mfma_a_nw(o[d1], op4(vcur, 2), pb0);
          if (pr + 1 < 8) {
            vnxt = cvt32(pair_codes(r0, r1), 1.0f);
            if (pr + 2 < 8) {
              r0 = vread(2 * pr + 4);
              r1 = vread(2 * pr + 5);
            }
          }
          mfma_a_nw(o[d0], op4(vcur, 1), pb1);
          mfma_a_nw(o[d1], op4(vcur, 3), pb1);
          if (pr + 1 < 8) vcur = vnxt;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (!last) {
        const int nn = min(kTileTok, cp.t_end - cp.t);
        s_cur = nn < kTileTok ? tail_masked(s_nxt, nn) : s_nxt;
      }
      ++it;
    } while (!last);

    const float l_tot = sum_halves(l_sum);
    const float inv = 1.f / l_tot;
    mfma_a_drain(o);
    const int ln = lane_id();
    const size_t part = ((size_t)w + b) * p.heads + wave * 32 + (ln & 31);
    auto packed_out = [&](int db, int g) __attribute__((always_inline)) {
      const bf16x4 v = {(__bf16)(o[db][4 * g] * inv), (__bf16)(o[db][4 * g + 1] * inv),
                        (__bf16)(o[db][4 * g + 2] * inv), (__bf16)(o[db][4 * g + 3] * inv)};
      return __builtin_bit_cast(u32x2, v);
    };
    {
      constexpr int kPad = 256 + 16;
      __builtin_amdgcn_s_barrier();
      LDS_AS char* region = (LDS_AS char*)ring[stage_of(it - 1)] + wave * 32 * kPad;
      const int hw = ln & 31, hl = ln >> 5;
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<LDS_AS u32x2*>(region + hw * kPad + (32 * d + 8 * g + 4 * hl) * 2) = packed_out(4 * qt + d, g);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int h = 4 * k + (ln >> 4);
          const u32x4 v = *reinterpret_cast<const LDS_AS u32x4*>(region + h * kPad + (ln & 15) * 16);
          const size_t ph = ((size_t)w + b) * p.heads + wave * 32 + h;
          *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.ws_o + ph * kDc) + 128 * qt + 8 * (ln & 15)) = v;
        }
      }
    }
    if (ln < 32) *reinterpret_cast<float2*>(p.ws_ml + 2 * part) = make_float2(m_ref, l_tot);
  }
  wait_vmcnt<0>();
}

// ---- 16 heads: heads are the 16-wide dimension of v_mfma_f32_16x16x32_bf16 -------------------
// Each wave computes the scores of the whole tile for all 16 heads (two 16-token blocks x 18
// k-steps, S^T[t][h] = K . Q^T with the query in 72 VGPRs) and a quarter of the output product (its
// 128 latent dims: eight 16-dim blocks over the tile's 32 tokens, O^T[d][h] += V^T . P^T), so the
// query is loaded once per wave and each piece is stored once, where the four-wave 32-column
// kernel would repeat every head eight times.  The score accumulators give lane l head l % 16 and
// tokens 4 g .. 4 g + 3 of each block (g = l / 16): its eight probabilities are the B operand of
// the output product with the tokens in the order {4 g .. 4 g + 3, 16 + 4 g .. 16 + 4 g + 3}, and
// the V^T operand reads the same tokens with two transposing reads.  The four waves work out the
// same softmax (online, base 2, O rescaled whenever a head's maximum rises).  Work units are ranges
// of 32-token tiles: the plain cut of the batch's tiles over min(units, tiles) units, so every unit
// holds a tile and small batches spread over more workgroups than they have pages.  Pieces,
// per-sequence unit table, tile ring and the list mode (TOPK: kept tokens read in place) are those
// of the kernel above.
template <bool TOPK>
__global__ __launch_bounds__(kWaves * 64, 1) void decode_h16_kernel(DecodeParams p) {
  constexpr int kPer = kBlocks / kWaves;  // copies per wave per tile
  typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4v;
  __shared__ __attribute__((aligned(1024))) char ring[kStages][kTileBytes];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = uni(xcd_unit(blockIdx.x, gridDim.x));
  TileCursor ld;
  ld.lens = p.seq_lens;
  ld.sh = 5;
  ld.valid = true;
  ld.all_live = true;
  if (p.batch <= 64) {
    // One read of the lengths (lane b holds sequence b's) gives the tile count, the unit's first
    // sequence and that sequence's length: no second pass and no scalar reload of the length.
    const int lane = threadIdx.x & 63;
    const int len_l = lane < p.batch ? max(p.seq_lens[lane], 0) : 0;
    const long long nt = tiles_of(len_l);
    const long long incl = wave_incl_scan_i64(nt);
    const long long T = readlane_i64(incl, 63);
    const int W = (int)min((long long)gridDim.x, T);
    if (w >= W) return;
    ld.pg0 = uni((int)((long long)w * T / W));
    ld.pg1 = uni((int)((long long)(w + 1) * T / W));
    const unsigned long long hit = __ballot(lane < p.batch && incl > ld.pg0);
    const int first = __ffsll((long long)hit) - 1;
    ld.b = uni(first);
    ld.before = uni((int)readlane_i64(incl - nt, first));
    ld.len = __builtin_amdgcn_readlane(len_l, first);
    ld.np = tiles_of(ld.len);
  } else {
    const long long T = total_tiles(p.seq_lens, p.batch);
    const int W = (int)min((long long)gridDim.x, T);
    if (w >= W) return;
    ld.pg0 = uni((int)((long long)w * T / W));
    ld.pg1 = uni((int)((long long)(w + 1) * T / W));
    int bb;
    long long bf;
    locate_unit(p.seq_lens, p.batch, ld.pg0, 5, bb, bf);
    ld.b = uni(bb);
    ld.before = uni((int)bf);
    ld.load_seq();
  }
  ld.enter();
  TileCursor cp = ld;

  // Per-lane LDS offsets inside a tile (lane = 16 g + j).  Score operand of k-step ks: token
  // 16 blk + j, latent dims 32 ks + 8 g ..: chunk 4 ks + g, whose odd k-steps flip bit 6 of the
  // offset and whose chunk group ks / 2 is a whole block.  Output operand of d-block i: dims
  // 128 wave + 16 i + 4 (j % 4) .. of tokens 4 g + j / 4 (first read) and 16 + 4 g + j / 4 (second
  // read, 18 blocks on): chunk 16 wave + 2 i + (j % 4) / 2, byte 8 (j % 2); i flips bits 5-6 and
  // i / 4 is a whole block.
  const int ln0 = lane_id();
  const int g = ln0 >> 4, j = ln0 & 15;
  const unsigned k_base0 = (unsigned)tile_offset(j, g);
  const unsigned k_base1 = (unsigned)tile_offset(16 + j, g);
  const unsigned v_base = (unsigned)(tile_offset(4 * g + (j >> 2), 16 * wave + ((j & 3) >> 1)) + 8 * (j & 1));
  auto lds16 = [](unsigned a) __attribute__((always_inline)) {
    return *reinterpret_cast<const LDS_AS bf16x8*>((const LDS_AS char*)(uintptr_t)a);
  };
  auto lds_tr = [](unsigned a) __attribute__((always_inline)) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS char*)(uintptr_t)a));
  };

  const uint16_t* qa = static_cast<const uint16_t*>(p.q_abs);
  bf16x8 q[18];
  auto load_q = [&](int b) __attribute__((always_inline)) {
    const int ln = lane_id();
    const uint16_t* qrow = qa + ((size_t)b * 16 + (ln & 15)) * kRow + 8 * (ln >> 4);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) q[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
  };
  load_q(cp.b);

  int issued = 0;
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) {
    if (ld.valid) {
      issue_tile<TOPK>(p, ld, (LDS_AS char*)ring[s], wave);
      ld.advance();
      ++issued;
    }
  }
  // Loads complete in issue order: with at most the prologue's copies outstanding, Q has landed.
  if (issued >= 3) wait_vmcnt<3 * kPer>();
  else if (issued == 2) wait_vmcnt<2 * kPer>();
  else wait_vmcnt<kPer>();
  // The copies are invisible to the compiler, so it cannot tell that this wait covered the query: it
  // would wait for its loads again inside the tile loop, before every score MFMA of every tile (and,
  // counting the copies too, drain the ring each time).  Using Q here puts those waits here, once.
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) asm volatile("" : : "v"(q[ks]));
  auto tile_ready = [&](int t) __attribute__((always_inline)) {
    const int younger = issued - t - 1;
    if (younger >= 2) wait_vmcnt<2 * kPer>();
    else if (younger == 1) wait_vmcnt<kPer>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  };

  const float scale = p.scale_log2;
  const unsigned ring0 = (unsigned)(uintptr_t)(LDS_AS char*)ring[0];
  int it = 0;
  bool first_segment = true;
  while (cp.valid) {  // one segment: the part of sequence b inside this unit
    const int b = cp.b;
    if (threadIdx.x == 0) {
      if (cp.t == 0) {
        p.seq_units[4 * b] = w;
        p.seq_units[4 * b + 2] = 1;
      }
      if (cp.t_end == cp.len) p.seq_units[4 * b + 1] = w;
    }
    if (!first_segment) {
      load_q(b);
      wait_vmcnt<0>();
    }
    first_segment = false;
    f32x4v o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = f32x4v{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;  // base-2 running maximum of this lane's head
    float l_run = 0.f;        // this lane's share of the softmax sum
    bool last;
    do {
      last = cp.last();
      // The barrier also frees the stage of tile it - 1 for the copies of tile it + 3.  (Spread one
      // per two score k-steps, as in the kernel above, they measured slower here: 161-165 against
      // 148 us at 4 x 131,072 tokens.)
      tile_ready(it);
      if (ld.valid) {
        issue_tile<TOPK>(p, ld, (LDS_AS char*)ring[stage_of(it + kStages - 1)], wave);
        ld.advance();
        ++issued;
      }
      const unsigned tb = ring0 + (unsigned)stage_of(it) * kTileBytes;
      f32x4v s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        const unsigned d = 64u * (ks & 1), blk = 1024u * (ks >> 1);
        const bf16x8 a0 = lds16(((tb + k_base0) ^ d) + blk);
        const bf16x8 a1 = lds16(((tb + k_base1) ^ d) + blk);
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, q[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, q[ks], s1, 0, 0, 0);
      }
      // softmax of the tile: tokens past the segment's end (a ragged last tile) take no weight
      const int n = min(kTileTok, cp.t_end - cp.t);
      float v[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = 4 * g + i < n ? s0[i] * scale : -INFINITY;
        v[4 + i] = 16 + 4 * g + i < n ? s1[i] * scale : -INFINITY;
      }
      float mx = max3(max3(v[0], v[1], v[2]), max3(v[3], v[4], v[5]), max2(v[6], v[7]));
      mx = max2(mx, __shfl_xor(mx, 16, 64));
      mx = max_halves(mx);
      if (mx > m_run) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - mx);  // 0 for the first tile
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] *= alpha;
        m_run = mx;
      }
      bf16x8 pb;
      float ls = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float e = __builtin_amdgcn_exp2f(v[i] - m_run);
        ls += e;
        pb[i] = (__bf16)e;
      }
      l_run += ls;
      // output: this wave's eight d-blocks
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const unsigned a = ((tb + v_base) ^ (32u * (i & 3))) + 1024u * (i >> 2);
        const s16x4 v0 = lds_tr(a);
        const s16x4 v1 = lds_tr(a + 18 * 1024);
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        o[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[i], 0, 0, 0);
      }
      cp.advance();
      ++it;
    } while (!last);

    // The piece: this wave's 128 dims of each head, divided by the head's softmax sum, in bf16
    // (lane 16 g + j: head j, dims 128 wave + 16 i + 4 g .. + 3), with (maximum, sum) per head.
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot = sum_halves(l_tot);
    const float inv = 1.f / l_tot;
    const size_t part = ((size_t)w + b) * 16 + j;
    uint16_t* po = reinterpret_cast<uint16_t*>(p.ws_o + part * kDc) + 128 * wave + 4 * g;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bf16x4 x = {(__bf16)(o[i][0] * inv), (__bf16)(o[i][1] * inv), (__bf16)(o[i][2] * inv),
                        (__bf16)(o[i][3] * inv)};
      *reinterpret_cast<u32x2*>(po + 16 * i) = __builtin_bit_cast(u32x2, x);
    }
    if (wave == 0 && g == 0) *reinterpret_cast<float2*>(p.ws_ml + 2 * part) = make_float2(m_run, l_tot);
  }
  // No copy into LDS may still be in flight when the workgroup ends.
  wait_vmcnt<0>();
}

}  // namespace

bool mfma_supported(const DecodeParams& p) {
  return p.heads == 128 || p.heads == 64 || p.heads == 32 || p.heads == 16;
}

hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t s) {
  if (p.fp6) {
    if (p.positions) return hipErrorNotSupported;
    switch (p.heads) {
      case 128: hipLaunchKernelGGL((decode_fp6_kernel<4>), dim3(p.num_units), dim3(256), 0, s, p); break;
      case 64: hipLaunchKernelGGL((decode_fp6_kernel<2>), dim3(p.num_units), dim3(128), 0, s, p); break;
      default: return hipErrorNotSupported;
    }
    return hipGetLastError();
  }
  if (!mfma_supported(p)) return hipErrorNotSupported;
  if (p.heads == 16) {
    if (p.positions)
      hipLaunchKernelGGL(decode_h16_kernel<true>, dim3(p.num_units), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(decode_h16_kernel<false>, dim3(p.num_units), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  // Every head count runs four waves: below 128 heads their columns repeat heads, which spreads the
  // tile copies over four waves instead of leaving them to H / 32.
  if (p.positions)
    hipLaunchKernelGGL((decode_mfma_kernel<true>), dim3(p.num_units), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<false>), dim3(p.num_units), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
