// Latent-space decode attention on the bf16 matrix cores of gfx950 (v_mfma_f32_32x32x16_bf16).
//
// What is computed (DeepSeek-V2 explainer, Steps 6-8): for every head h of sequence b,
//   S[t][h] = q_abs[b][h] . row_t        (576-long: latent score + RoPE score, one dot product)
//   P       = softmax_t(scale * S)       (online, base 2)
//   O[d][h] = sum_t P[h][t] * row_t[d]   (d < 512: the weighted sum of latent notes)
// All heads of a sequence share every cached row (the row is per token, not per head), so heads
// form the N dimension of both products and each row is read from HBM once per launch.
//
// Workgroup = 4 waves x 32 heads = 128 heads, one workgroup per compute unit.  Per 32-token tile:
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
// ~6-bit cache (FP6 template argument).  Pages hold 6-bit E2M3 codes with one power-of-two scale
// per row, so every stored number is exactly a bf16 number.  Each wave copies its own rows of a
// tile (32 / waves rows: codes and scales, 13.6 KB per tile in all) into a wave-private 3-stage
// LDS ring, four tiles ahead (a stage is free once its tile is converted), and converts them with
// v_cvt_scalef32_pk32_bf16_fp6 (32 codes per instruction, the scale's exponent applied exactly)
// into the same swizzled bf16 tile layout, two tiles ahead, spread over the output product.  The bf16 ring then has three stages (the tile whose
// output product runs, the tile whose scores run, the tile being converted) and everything after it
// is the bf16 path unchanged.  Reading only the codes, the conversion needs no barrier of its own:
// a wave converts exactly the rows it copied, and the barrier that opens each iteration publishes
// the converted tile.
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
#define LDS_AS __attribute__((address_space(3)))
#define CONST_AS __attribute__((address_space(4)))

constexpr int kTileTok = 32;
constexpr int kChunks = kRow / 8;                    // 72 16-byte chunks per row
constexpr int kCG = kChunks / 8;                     // 9 chunk groups
constexpr int kBlocks = kTileTok / 8 * kCG;          // 36 blocks of 8 tokens x 8 chunks
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
  int pg0, pg1;   // the unit's global page range
  int b;          // current sequence
  int before;     // pages of sequences [0, b)
  int len, np;    // tokens / pages of sequence b
  int t;          // first token of the current tile
  int t_end;      // end token of the current segment
  bool valid;
  bool all_live;  // every unit holds at least one page

  __device__ __forceinline__ void load_seq() {
    len = ld_const(lens, b);
    np = (int)(((unsigned)max(len, 0) + kPage - 1) / kPage);
  }
  // Sets t / t_end for sequence b, skipping sequences with no tokens.
  __device__ __forceinline__ void enter() {
    while (np == 0) {
      ++b;
      load_seq();
    }
    const int p0 = max(pg0 - before, 0);
    const int p1 = min(pg1 - before, np);
    t = p0 * kPage;
    t_end = min(p1 * kPage, len);
  }
  __device__ __forceinline__ void init(const DecodeParams& p, int w) {
    lens = p.seq_lens;
    if (p.batch <= 64) {
      // One pass: lane i holds sequence i's page count, an inclusive scan gives both the total and
      // the sequence holding the unit's first page.
      const int ln = threadIdx.x & 63;
      const int np_l = ln < p.batch ? (int)(((unsigned)max(p.seq_lens[ln], 0) + kPage - 1) / kPage) : 0;
      int incl = np_l;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int n = __shfl_up(incl, o, 64);
        if (ln >= o) incl += n;
      }
      const int P = __builtin_amdgcn_readlane(incl, 63);
      pg0 = uni((int)((long long)w * P / p.num_units));
      pg1 = uni((int)((long long)(w + 1) * P / p.num_units));
      all_live = P >= p.num_units;
      valid = pg0 < pg1;
      if (!valid) return;
      const unsigned long long hit = __ballot(ln < p.batch && incl > pg0);
      b = uni(__ffsll((long long)hit) - 1);
      before = __builtin_amdgcn_readlane(incl - np_l, b);
    } else {
      const int P = uni((int)total_pages(p.seq_lens, p.batch));
      pg0 = uni((int)((long long)w * P / p.num_units));
      pg1 = uni((int)((long long)(w + 1) * P / p.num_units));
      all_live = P >= p.num_units;
      valid = pg0 < pg1;
      if (!valid) return;
      int bb;
      long long bf;
      locate_page(p.seq_lens, p.batch, pg0, bb, bf);
      b = uni(bb);
      before = uni((int)bf);
    }
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
template <int NW, bool TOPK>
__device__ __forceinline__ void issue_tile(const DecodeParams& p, const TileCursor& c,
                                           LDS_AS char* stage, int wave) {
  constexpr int kPer = kBlocks / NW;
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
    if constexpr (NW == 4) {  // wave w copies token group w
      const char* gb = base + wave * 8 * (kRow * 2);
#pragma unroll
      for (int j = 0; j < kPer; ++j) dma16_group(gb, (unsigned)lane_off[wave & 1], lds + wave * kPer * 1024, j);
    } else {
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int blk = wave * kPer + j;
        const int tg = blk / kCG, cg = blk % kCG;
        dma16(base + tg * 8 * (kRow * 2) + cg * 128, (unsigned)lane_off[tg & 1], lds + blk * 1024);
      }
    }
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

// ---- ~6-bit cache ---------------------------------------------------------------------------------
// Per wave and tile: rows R w .. R w + R - 1 (R = 32 / waves), copied as their contiguous codes
// (432 bytes a row, every 16-byte piece inside one row) then their R scales; converted as units of
// 32 codes (24 bytes) each, 18 to a row.
template <int NW>
struct Fp6Geom {
  static constexpr int kRows = kTileTok / NW;
  static constexpr int kDataBytes = kRows * kFp6RowBytes;            // 3,456 / 6,912 / 13,824
  static constexpr int kDataCopies = (kDataBytes + 1023) / 1024;     // 4 / 7 / 14, the last partial
  static constexpr int kCopies = kDataCopies + 1;                    // plus one for the scales
  static constexpr int kWaveBytes = kDataBytes + kRows * 4;
  static constexpr int kUnits = kRows * (kRow / 32);                 // 144 / 288 / 576
  static constexpr int kRounds = (kUnits + 63) / 64;                 // 3 / 5 / 9
  // Rounds inside the 32 steps of the output product, from step 4: loaded at 4 + kRoundStep k,
  // converted and stored two steps later, one unit in flight at a time.
  static constexpr int kRoundStep = 28 / kRounds > 8 ? 8 : 28 / kRounds;   // 8 / 5 / 3
  static_assert(kRoundStep >= 3 && 4 + kRoundStep * (kRounds - 1) + 2 < 32, "rounds fit the product");
  // Copies inside the 36 score steps: copy j at step 2 + kCopyStep j.
  static constexpr int kCopyStep = 32 / kCopies;                                    // 6 / 4 / 2
  static_assert(2 + kCopyStep * (kCopies - 1) < 36, "copies fit the score product");
};
constexpr int kFp6Stages = 3;

// One 4-byte-per-lane copy HBM -> LDS: lane l's dword from gbase + voff lands at LDS byte lds + 4 l.
__device__ __forceinline__ void dma4(const char* gbase, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(gbase), "s"(lds)
               : "memory", "m0");
}

// Copy j (< kCopies) of this wave's part of one tile (tile rows start at page slot slot0, nt valid
// rows) into its region `lds` of an fp6 stage: copies 0 .. kDataCopies - 1 move 1 KB of codes each
// (the last one partly), the final copy the scales.  A ragged tile repeats its last valid row for
// the missing ones, so every converted number is finite.  Some lane is active in every copy, so
// each is one instruction for the counted waits.  j must fold to a constant.
template <int NW>
__device__ __forceinline__ void issue_copy6(const char* page_base, int slot0, int nt, unsigned lds, int wave, int j) {
  using G = Fp6Geom<NW>;
  const int ln = lane_id();
  const int r0 = wave * G::kRows;
  if (j < G::kDataCopies) {
    const int o = 1024 * j + 16 * ln;
    if (j < G::kDataCopies - 1 || o < G::kDataBytes) {
      const int r = o / kFp6RowBytes;
      const int rr = min(r0 + r, nt - 1);
      dma16(page_base, (unsigned)((slot0 + rr) * kFp6RowBytes + (o - r * kFp6RowBytes)), lds + 1024 * j);
    }
  } else if (ln < G::kRows) {
    dma4(page_base, (unsigned)(kPage * kFp6RowBytes + 4 * (slot0 + min(r0 + ln, nt - 1))), lds + G::kDataBytes);
  }
}

// One conversion unit in flight: 32 codes and the row scale.
struct Fp6Unit {
  u32x6 codes;
  float scale;
};

// Loads unit u of this wave's rows from its fp6 region (unit u: row u % R, codes 32 (u / R) ..,
// R = rows per wave).  Rows vary fastest across lanes: 16 lanes then write 8 or 16 different rows,
// which the tile swizzle spreads over the bank groups (two lanes per group with 8 rows, one with
// 16), where 16 units of one row would land on two groups.  Units are numbered lane + 64 k for
// round k, the lane taken from lane_id() so that the address arithmetic stays where it is used
// instead of holding registers across the tile loop.
template <int NW>
__device__ __forceinline__ Fp6Unit fp6_load(unsigned region, int k) {
  using G = Fp6Geom<NW>;
  const int u = lane_id() + 64 * k;
  const int r = u % G::kRows, g = u / G::kRows;
  const LDS_AS char* src = (const LDS_AS char*)(uintptr_t)region + r * kFp6RowBytes + 24 * g;
  const u32x2 a = *reinterpret_cast<const LDS_AS u32x2*>(src);
  const u32x2 b = *reinterpret_cast<const LDS_AS u32x2*>(src + 8);
  const u32x2 c = *reinterpret_cast<const LDS_AS u32x2*>(src + 16);
  Fp6Unit x;
  x.codes = u32x6{a[0], a[1], b[0], b[1], c[0], c[1]};
  x.scale = *reinterpret_cast<const LDS_AS float*>((const LDS_AS char*)(uintptr_t)region + G::kDataBytes + 4 * r);
  return x;
}

// Converts a unit (only the scale's exponent is applied, so code * 2^e exactly) and writes its 32
// bf16 numbers, chunks 4 g .. 4 g + 3 of its row, into the swizzled bf16 tile at `stage` (1 KB
// aligned).  Those four chunks share a block and differ only in the two low chunk bits, which the
// swizzle XORs with a row constant: chunk 4 g + j sits at the offset of chunk 4 g XOR 16 j.  The
// conversion is written as asm: the compiler's builtin for it returned its first element in every
// position.
template <int NW>
__device__ __forceinline__ void fp6_store(const Fp6Unit& x, int k, unsigned stage, int wave) {
  using G = Fp6Geom<NW>;
  u32x16 v;
  asm("v_cvt_scalef32_pk32_bf16_fp6 %0, %1, %2" : "=&v"(v) : "v"(x.codes), "v"(x.scale));
  const int u = lane_id() + 64 * k;
  const int r = u % G::kRows, g = u / G::kRows;
  const unsigned a0 = stage + (unsigned)tile_offset(wave * G::kRows + r, 4 * g);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<LDS_AS u32x4*>((LDS_AS char*)(uintptr_t)(a0 ^ (16u * j))) =
        u32x4{v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
}

// Whole-tile conversion (prologue): every unit of this wave's rows.
template <int NW>
__device__ __forceinline__ void fp6_convert_all(unsigned region, unsigned stage, int wave) {
  using G = Fp6Geom<NW>;
  const int ln = lane_id();
#pragma unroll
  for (int k = 0; k < G::kRounds; ++k) {
    if (ln + 64 * k < G::kUnits) fp6_store<NW>(fp6_load<NW>(region, k), k, stage, wave);
  }
}

// Workgroups go to the eight XCDs round-robin (workgroup i to XCD i mod 8), each XCD with its own
// L2.  Consecutive work units, which hold neighbouring pages and mostly the same sequence, are
// placed on one XCD so that they share its L2 for that sequence's query and block-table lines.
__device__ __forceinline__ int xcd_unit(int id, int n) {
  const int per = n / 8, rem = n % 8, x = id % 8;
  return x * per + min(x, rem) + id / 8;
}

template <int NW, bool FP6, bool TOPK>
__global__ __launch_bounds__(NW * 64, 1) void decode_mfma_kernel(DecodeParams p) {
  static_assert(!(FP6 && TOPK), "kept tokens are read from bf16 rows");
  constexpr int kPer = kBlocks / NW;  // copies per wave per tile
  using G6 = Fp6Geom<NW>;
  __shared__ __attribute__((aligned(1024))) char ring[FP6 ? 3 : kStages][kTileBytes];
  // Target of the copies a four-wave unit issues after its last tile: they keep the count of copies
  // per tile fixed, which the counted waits rely on, and nothing reads them.
  __shared__ __attribute__((aligned(1024))) char sink[(!FP6 && NW == 4) ? kPer * 1024 : 16];
  // ~6-bit cache: the waves' private copy regions, three tiles' worth.
  __shared__ __attribute__((aligned(16))) char ring6[FP6 ? kFp6Stages * NW * G6::kWaveBytes : 16];
  auto stg = [](int t) __attribute__((always_inline)) { return FP6 ? t % 3 : stage_of(t); };

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
  // Head of accumulator column c (0 .. 31) of this wave.  With 16 heads the columns 16 .. 31 repeat
  // heads 0 .. 15: same query, same data, so bit-identical results, and every store they make
  // writes the same bits to the same place as the real head's.  (Heads are powers of two.)
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
  // ~6-bit cache: this wave's fp6 region for tile t, and the copies of the tile at cursor `ld`
  const unsigned r6 = (unsigned)(uintptr_t)(LDS_AS char*)ring6 + wave * G6::kWaveBytes;
  auto region6 = [&](int t) __attribute__((always_inline)) {
    return r6 + (unsigned)((t % kFp6Stages) * NW * G6::kWaveBytes);
  };
  auto issue6 = [&](int page) __attribute__((always_inline)) {
    const char* pb = reinterpret_cast<const char*>(p.cache) + (size_t)page * kFp6PageBytes;
    const int slot0 = (int)((unsigned)ld.t % kPage), nt = min(kTileTok, ld.t_end - ld.t);
    const unsigned lds = region6(issued);
#pragma unroll
    for (int j = 0; j < G6::kCopies; ++j) issue_copy6<NW>(pb, slot0, nt, lds, wave, j);
    ld.advance();
    ++issued;
  };
  if constexpr (FP6) {
#pragma unroll
    for (int s = 0; s < kFp6Stages; ++s) {
      if (ld.valid) issue6(ld_const(p.block_table, (size_t)ld.b * p.max_blocks + (unsigned)ld.t / kPage));
    }
    // Tiles 0 and 1 are converted here, the rest two tiles ahead inside the loop.  Once tile 0 is
    // converted its stage takes tile 3, so the copies run four tiles ahead of the tile whose output
    // product runs.  Loads complete in issue order, so the query has landed once tile 0 has.
    constexpr int C = G6::kCopies;
    if (issued >= 3) wait_vmcnt<2 * C>();
    else if (issued == 2) wait_vmcnt<C>();
    else wait_vmcnt<0>();
    fp6_convert_all<NW>(region6(0), (unsigned)(uintptr_t)(LDS_AS char*)ring[0], wave);
    if (ld.valid) issue6(ld_const(p.block_table, (size_t)ld.b * p.max_blocks + (unsigned)ld.t / kPage));
    if (issued >= 2) {
      if (issued >= 4) wait_vmcnt<2 * C>();
      else if (issued == 3) wait_vmcnt<C>();
      else wait_vmcnt<0>();
      fp6_convert_all<NW>(region6(1), (unsigned)(uintptr_t)(LDS_AS char*)ring[1], wave);
    }
  } else {
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) {
      if (ld.valid) {
        issue_tile<NW, TOPK>(p, ld, (LDS_AS char*)ring[s], wave);
        ld.advance();
        ++issued;
      }
    }
    // Loads complete in issue order: with at most the prologue's copies outstanding (capped at the
    // counter's 63, which only waits for more), the query has landed.
    if (issued >= 3) wait_vmcnt<(3 * kPer < 63 ? 3 * kPer : 63)>();
    else if (issued == 2) wait_vmcnt<(2 * kPer < 63 ? 2 * kPer : 63)>();
    else wait_vmcnt<(kPer < 63 ? kPer : 63)>();
  }
  // Waits until the copies of tile `t` (this wave's part) have landed, then for every wave.
  // Vector loads complete in issue order: it is enough to let the tiles issued after it stay in
  // flight.
  auto tile_ready = [&](int t) __attribute__((always_inline)) {
    if constexpr (FP6) {  // the tile was converted by every wave: their LDS writes, then the barrier
      wait_lgkmcnt0();
      __builtin_amdgcn_s_barrier();
      return;
    }
    const int younger = issued - t - 1;
    if (younger >= 2) wait_vmcnt<(2 * kPer < 63 ? 2 * kPer : 63)>();
    else if (younger == 1) wait_vmcnt<(kPer < 63 ? kPer : 63)>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  };
  // Refills the stage of the tile before `t` (every wave is past it) with the next tile.
  auto refill = [&](int t) __attribute__((always_inline)) {
    if (ld.valid) {
      issue_tile<NW, TOPK>(p, ld, (LDS_AS char*)ring[stg(t + kStages - 1)], wave);
      ld.advance();
      ++issued;
    }
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
      const unsigned tk = (unsigned)(uintptr_t)(LDS_AS char*)ring[stg(it)] + k_off;
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
      // The ~6-bit cache copies a twelfth of the bytes per wave and issues them all at once.
      const char* sp_base = reinterpret_cast<const char*>(p.cache);
      unsigned sp_lane = 0, sp_lds = 0;
      uint64_t sp_addr = 0;  // kept tokens: this lane's full source address
      int sp_page = 0, sp_tok = 0;
      bool sp_have = false;
      if constexpr (FP6) {
        // The converted tile it + 1 is published by the barrier; the block-table read for the
        // copies of tile it + 4 (into the stage of tile it + 1, converted last iteration) is issued
        // after this wave's own LDS writes are done, so that it overlaps the barrier instead of
        // being waited for before it.
        wait_lgkmcnt0();
        __builtin_amdgcn_sched_barrier(0);
        sp_have = ld.valid;
        if (ld.valid) {
          sp_page = ld_const(p.block_table, (size_t)ld.b * p.max_blocks + (unsigned)ld.t / kPage);
          sp_tok = (int)((unsigned)ld.t % kPage);
          sp_lane = (unsigned)min(kTileTok, ld.t_end - ld.t);   // valid rows of the tile
          sp_lds = region6(issued);
          ld.advance();
          ++issued;
        }
        __builtin_amdgcn_s_barrier();
        asm volatile("" : "+s"(sp_page));  // the page is first needed behind the barrier
        if (sp_have) sp_base += (size_t)sp_page * kFp6PageBytes;
      } else if constexpr (NW == 4) {
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
      if constexpr (!FP6) {
        tile_ready(last ? it : it + 1);
        if constexpr (NW == 4 && TOPK) {
          ++issued;
          asm volatile("" : "+v"(sp_addr));
        } else if constexpr (NW == 4) {
          ++issued;
          asm volatile("" : "+s"(sp_page));  // the page is first needed here, behind the wait
          if (sp_have) sp_base += ((size_t)sp_page * kPage + sp_tok) * (kRow * 2);
        } else {
          refill(it);
        }
      }
      auto spread_copy = [&](int j) __attribute__((always_inline)) {
        if constexpr (NW == 4 && TOPK) dma16_addr(sp_addr, sp_lds + 1024 * j, j);
        else if constexpr (NW == 4 && !FP6) dma16_group(sp_base, sp_lane, sp_lds, j);
      };
      // ~6-bit cache: copy j of tile it + 4 (spread over the score product like the bf16 copies)
      auto copy6 = [&](int j) __attribute__((always_inline)) {
        if constexpr (FP6) {
          if (sp_have) issue_copy6<NW>(sp_base, sp_tok, (int)sp_lane, sp_lds, wave, j);
        }
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
        const unsigned tk = (unsigned)(uintptr_t)(LDS_AS char*)ring[stg(it + 1)] + k_off;
        bf16x8 ka[kKAhead + 1];
#pragma unroll
        for (int ks = 0; ks < kKAhead; ++ks) ka[ks] = k_operand(tk, ks);
#pragma unroll
        for (int ks = 0; ks < 36; ++ks) {
          if (ks + kKAhead < 36) ka[(ks + kKAhead) % (kKAhead + 1)] = k_operand(tk, ks + kKAhead);
          if (ks == 0) mfma_v_first_nw(s_nxt, ka[0], q[0]); else mfma_v_nw(s_nxt, ka[ks % (kKAhead + 1)], q[ks]);
          softmax_step(ks);
          if ((ks & 3) == 0) spread_copy(ks >> 2);
          if constexpr (FP6) {
            if (ks >= 2 && (ks - 2) % G6::kCopyStep == 0 && (ks - 2) / G6::kCopyStep < G6::kCopies)
              copy6((ks - 2) / G6::kCopyStep);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        mfma_v_drain(s_nxt);
      } else {
#pragma unroll
        for (int k = 0; k < 12; ++k) softmax_step(k);
#pragma unroll
        for (int j = 0; j < kCG; ++j) spread_copy(j);
#pragma unroll
        for (int j = 0; j < G6::kCopies; ++j) copy6(j);
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
        const unsigned tv = (unsigned)(uintptr_t)(LDS_AS char*)ring[stg(it)] + v_off;
        // ~6-bit cache: tile it + 2 is converted here, its stage free since the barrier above
        const bool conv = FP6 && it + 2 < issued;
        const unsigned cv_src = FP6 ? region6(it + 2) : 0u;
        const unsigned cv_dst = FP6 ? (unsigned)(uintptr_t)(LDS_AS char*)ring[stg(it + 2)] : 0u;
        Fp6Unit cbuf;
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
          if constexpr (FP6) {
            if (conv) {
              if (i == 4) {  // this wave's copies of tile it + 2 have landed (those of it + 3, it + 4 may not)
                if (it + 4 < issued) wait_vmcnt<2 * G6::kCopies>();
                else if (it + 3 < issued) wait_vmcnt<G6::kCopies>();
                else wait_vmcnt<0>();
              }
#pragma unroll
              for (int k = 0; k < G6::kRounds; ++k) {
                const int at = 4 + k * G6::kRoundStep;
                const bool mine = lane + 64 * k < G6::kUnits;
                if (i == at && mine) cbuf = fp6_load<NW>(cv_src, k);
                if (i == at + 2 && mine) fp6_store<NW>(cbuf, k, cv_dst, wave);
              }
            }
          }
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
      LDS_AS char* region = (LDS_AS char*)ring[stg(it - 1)] + wave * 32 * kPad;
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

}  // namespace

bool mfma_supported(const DecodeParams& p) {
  return p.heads == 128 || p.heads == 64 || p.heads == 32 || p.heads == 16;
}

hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t s) {
  if (p.fp6) {
    if (p.positions) return hipErrorNotSupported;
    // No one-wave variant: with its conversion the compiler keeps that kernel's output accumulators
    // in memory across the tile loop, which the unpadded MFMA wrappers above do not allow.
    switch (p.heads) {
      case 128: hipLaunchKernelGGL((decode_mfma_kernel<4, true, false>), dim3(p.num_units), dim3(256), 0, s, p); break;
      case 64: hipLaunchKernelGGL((decode_mfma_kernel<2, true, false>), dim3(p.num_units), dim3(128), 0, s, p); break;
      default: return hipErrorNotSupported;
    }
    return hipGetLastError();
  }
  if (p.positions) {
    switch (p.heads) {
      case 128: hipLaunchKernelGGL((decode_mfma_kernel<4, false, true>), dim3(p.num_units), dim3(256), 0, s, p); break;
      case 64: hipLaunchKernelGGL((decode_mfma_kernel<2, false, true>), dim3(p.num_units), dim3(128), 0, s, p); break;
      case 32:
      case 16: hipLaunchKernelGGL((decode_mfma_kernel<1, false, true>), dim3(p.num_units), dim3(64), 0, s, p); break;
      default: return hipErrorNotSupported;
    }
    return hipGetLastError();
  }
  switch (p.heads) {
    case 128: hipLaunchKernelGGL((decode_mfma_kernel<4, false, false>), dim3(p.num_units), dim3(256), 0, s, p); break;
    case 64: hipLaunchKernelGGL((decode_mfma_kernel<2, false, false>), dim3(p.num_units), dim3(128), 0, s, p); break;
    case 32:
    case 16: hipLaunchKernelGGL((decode_mfma_kernel<1, false, false>), dim3(p.num_units), dim3(64), 0, s, p); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace mla
