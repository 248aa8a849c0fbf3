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
// tiles ahead of the one being processed.  With one wave per SIMD, LDS latency (well over 100
// cycles under load) is the main stall, so both products prefetch their LDS operands: the score
// product 4 k-steps ahead (4 x 32 MFMA cycles of cover), the output product two d-blocks ahead,
// and the first output operands are requested before the softmax so its vector ALU work covers
// their latency.  The softmax rescale of O is lazy: the reference maximum only moves when a tile's
// maximum exceeds it by more than 2^8.
//
// Tile layout in LDS.  A tile is 32 tokens x 72 chunks of 16 bytes, stored as 36 blocks of
// 8 tokens x 8 chunks, 1 KB each (block = 9 (t / 8) + c / 8), so one global_load_lds_dwordx4 fills
// one block.  Inside a block, chunk c of token t sits at slot
//   8 ((t mod 8) ^ g) + ((c mod 8) ^ sigma(t mod 8)),  g = (t / 8) mod 2,
//   sigma(x) = 2 (x mod 4) + (x / 4) mod 2.
// With it, the 16 lanes of one row read of the score operand (16 tokens, one chunk) and of one
// transposing read (4 tokens x 2 chunks) always land on 16 different 16-byte bank groups.
#include "mla_device.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
#define LDS_AS __attribute__((address_space(3)))
#define CONST_AS __attribute__((address_space(4)))

constexpr int kTileTok = 32;
constexpr int kChunks = kRow / 8;                    // 72 16-byte chunks per row
constexpr int kCG = kChunks / 8;                     // 9 chunk groups
constexpr int kBlocks = kTileTok / 8 * kCG;          // 36 blocks of 8 tokens x 8 chunks
constexpr int kTileBytes = kBlocks * 1024;           // 36,864
constexpr int kStages = 4;                           // tiles it .. it+3
constexpr float kRescaleThreshold = 8.0f;            // base-2 headroom before O is rescaled
constexpr int kKAhead = 4;                           // score operand prefetch depth (k-steps)

__device__ __forceinline__ int sigma(int x) { return ((x & 3) << 1) | ((x >> 2) & 1); }

// Byte offset inside a tile of chunk c of token t.
__device__ __forceinline__ int tile_offset(int t, int c) {
  const int tg = t >> 3, tl = t & 7, cl = c & 7;
  const int slot = 8 * (tl ^ (tg & 1)) + (cl ^ sigma(tl));
  return ((tg * kCG + (c >> 3)) * 64 + slot) * 16;
}

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

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
__device__ __forceinline__ void mfma_v_drain(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
}
// Output MFMAs with their accumulator pinned to AGPRs ("+a"): left to itself the compiler turns the
// loop-carried 256-register accumulator into VGPR copies and spills.
__device__ __forceinline__ void mfma_a(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
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

// Block-table entries and lengths are read through the constant address space so they become
// scalar loads (lgkmcnt).  A vector load here would be ordered behind the in-flight LDS DMA and its
// wait would drain the whole ring.  Neither array is written while a launch runs.
__device__ __forceinline__ int ld_const(const int32_t* ptr, size_t i) {
  return ((const CONST_AS int32_t*)ptr)[i];
}

// max / sum of a value and its copy in lane l ^ 32
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

  __device__ __forceinline__ void load_seq() {
    len = ld_const(lens, b);
    np = (len + kPage - 1) / kPage;
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
    const int P = uni((int)total_pages(p.seq_lens, p.batch));
    pg0 = uni((int)((long long)w * P / p.num_units));
    pg1 = uni((int)((long long)(w + 1) * P / p.num_units));
    valid = pg0 < pg1;
    if (!valid) return;
    int bb;
    long long bf;
    locate_page(p.seq_lens, p.batch, pg0, bb, bf);
    b = uni(bb);
    before = uni((int)bf);
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

// DMA of one tile: wave w fills blocks [w * per, (w + 1) * per).  For a full tile the per-lane part
// of every source address is one of two lane constants (token-group parity); a ragged tile (fewer
// than 32 tokens) re-reads its last valid row in place of the missing ones.
template <int NW>
__device__ __forceinline__ void issue_tile(const DecodeParams& p, const TileCursor& c,
                                           LDS_AS char* stage, int wave, const int* lane_off) {
  constexpr int kPer = kBlocks / NW;
  const int page = ld_const(p.block_table, (size_t)c.b * p.max_blocks + c.t / kPage);
  const int nt = min(kTileTok, c.t_end - c.t);
  const char* base = reinterpret_cast<const char*>(p.cache) +
                     ((size_t)page * kPage + (c.t % kPage)) * (kRow * 2);
  const unsigned lds = (unsigned)(uintptr_t)stage;
  if (nt == kTileTok) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int blk = wave * kPer + j;
      const int tg = blk / kCG, cg = blk % kCG;
      dma16(base + tg * 8 * (kRow * 2) + cg * 128, (unsigned)lane_off[tg & 1], lds + blk * 1024);
    }
  } else {
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
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

// Score operand for k-step ks = 4 g + i: 8 consecutive latent dims of this lane's token.
__device__ __forceinline__ bf16x8 k_operand(const LDS_AS char* tile, const int* k_base, int ks) {
  return *reinterpret_cast<const LDS_AS bf16x8*>(tile + k_base[ks & 3] + 1024 * (ks >> 2));
}

// Output operand for d-block db and token half m: 8 tokens of one latent dim, gathered by two
// 16-lane transposing reads (token rows 16 m + 8 r + 4 half + (lane % 16) / 4, r = 0, 1).
__device__ __forceinline__ bf16x8 v_operand(const LDS_AS char* tile, const int* v_base, int db, int m) {
  const LDS_AS char* p0 = tile + v_base[db & 1] + ((2 * m) * kCG + (db >> 1)) * 1024;
  const LDS_AS char* p1 = tile + v_base[2 + (db & 1)] + ((2 * m + 1) * kCG + (db >> 1)) * 1024;
  const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)p0);
  const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)p1);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void decode_mfma_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char ring[kStages][kTileBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;       // which K half of the MFMA operands this lane holds
  const int l32 = lane & 31;
  const int head = wave * 32 + l32; // head of this lane's score / output column
  const int w = blockIdx.x;

  TileCursor ld, cp;
  ld.init(p, w);
  cp = ld;
  if (!cp.valid) return;

  // DMA lane constants: slot (lane / 8, lane % 8) of a block holds token-in-group
  // (lane / 8) ^ parity and chunk-in-group (lane % 8) ^ sigma(token-in-group).
  int lane_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int tl = (lane >> 3) ^ par;
    lane_off[par] = tl * (kRow * 2) + ((lane & 7) ^ sigma(tl)) * 16;
  }
  // Score operand bases: token l32, chunk 2 ks + half; per k-step the rest is an immediate.
  int k_base[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) k_base[i] = tile_offset(l32, 2 * i + half);
  // Transposing-read bases, [r][e]: token 8 r + 4 half + (lane % 16) / 4 of a 16-token half, chunk
  // 4 e + 2 ((lane / 16) % 2) + (lane % 4) / 2 of a two-block column group, byte 8 (lane % 2); the
  // token group itself is added as an immediate.
  int v_base[4];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      v_base[r * 2 + e] = tile_offset(8 * r + 4 * half + ((lane & 15) >> 2),
                                      4 * e + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) +
                          8 * (lane & 1) - r * kCG * 1024;

  // Prologue: three tiles in flight.
  int issued = 0;
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) {
    if (ld.valid) {
      issue_tile<NW>(p, ld, (LDS_AS char*)ring[s], wave, lane_off);
      ld.advance();
      ++issued;
    }
  }

  const uint16_t* qa = static_cast<const uint16_t*>(p.q_abs);
  const float scale = p.scale_log2;
  int it = 0;
  while (cp.valid) {  // one segment: the part of sequence b inside this unit
    const int b = cp.b;
    bf16x8 q[36];
    {
      const uint16_t* qrow = qa + ((size_t)b * p.heads + head) * kRow + 8 * half;
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) q[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks);
      // Wait here, once per segment: left to the compiler, the wait for Q would sit inside the tile
      // loop and drain the DMA ring on every tile.
      wait_vmcnt<0>();
    }
    f32x16 o[16];
    {
      const bf16x8 zero = {};
#pragma unroll
      for (int i = 0; i < 16; ++i) mfma_a_zero(o[i], zero);
    }
    float m_ref = -INFINITY;  // base-2 reference maximum (same in lanes l and l ^ 32)
    float l_sum = 0.f;        // this lane's share of the softmax denominator
    bool fresh = true;
    bool last;

    do {  // one 32-token tile
      const int stage = it % kStages;
      {
        // This wave's DMA for tile `it` must have landed.  Vector loads complete in issue order, so
        // it is enough to allow exactly the DMA of the tiles issued after it to stay in flight
        // (later stores only make the wait longer).
        constexpr int kPer = kBlocks / NW;
        const int younger = issued - it - 1;
        if (younger >= 2) wait_vmcnt<(2 * kPer < 63 ? 2 * kPer : 63)>();
        else if (younger == 1) wait_vmcnt<(kPer < 63 ? kPer : 63)>();
        else wait_vmcnt<0>();
      }
      __builtin_amdgcn_s_barrier();
      const LDS_AS char* tile = (const LDS_AS char*)ring[stage];
      // the first score operands go out before the DMA and cursor work, which covers their latency
      bf16x8 ka[kKAhead + 1];
#pragma unroll
      for (int ks = 0; ks < kKAhead; ++ks) ka[ks] = k_operand(tile, k_base, ks);
      // Every wave is done with tile it-1: refill its stage.
      if (ld.valid) {
        issue_tile<NW>(p, ld, (LDS_AS char*)ring[(it + kStages - 1) % kStages], wave, lane_off);
        ld.advance();
        ++issued;
      }
      const int nt = min(kTileTok, cp.t_end - cp.t);
      last = cp.last();
      cp.advance();

      // ---- scores: S^T = K . Q^T ---------------------------------------------------------------
      f32x16 s;
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) {
        if (ks + kKAhead < 36) ka[(ks + kKAhead) % (kKAhead + 1)] = k_operand(tile, k_base, ks + kKAhead);
        if (ks == 0) mfma_v_first(s, ka[0], q[0]); else mfma_v(s, ka[ks % (kKAhead + 1)], q[ks]);
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- softmax (base 2), lane = head, registers = tokens ------------------------------------
      // The output operands of the first two d-blocks are requested first.
      bf16x8 va[3][2];
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        va[db][0] = v_operand(tile, v_base, db, 0);
        va[db][1] = v_operand(tile, v_base, db, 1);
      }
      mfma_v_drain(s);
      if (nt < kTileTok) {  // ragged tile: tokens past the end take no weight
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int tok = (j >> 2) * 8 + half * 4 + (j & 3);
          if (tok >= nt) s[j] = -INFINITY;
        }
      }
      float mt = fmaxf(fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7]))),
                       fmaxf(fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11])), fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15]))));
      mt = max_halves(mt) * scale;
      if (fresh) {
        m_ref = mt;
        fresh = false;
      } else if (__ballot(mt > m_ref + kRescaleThreshold)) {
        // Rare (the running maximum jumped by more than 2^8): O is scaled before this tile's
        // product is added.  The accumulators make a round trip through this piece's own
        // workspace slot, which its final write overwrites anyway, so scaling them never holds
        // more than one block in VGPRs.
        const float m_new = fmaxf(m_ref, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
        m_ref = m_new;
        l_sum *= alpha;
        mfma_a_drain(o);
        float* slot = p.ws_o + (((size_t)w + b) * p.heads + head) * kDc + 4 * half;
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
      }
      bf16x8 pb0, pb1;
      {
        float ls = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float e = __builtin_amdgcn_exp2f(fmaf(s[j], scale, -m_ref));
          ls += e;
          if (j < 8) pb0[j] = (__bf16)e; else pb1[j - 8] = (__bf16)e;
        }
        l_sum += ls;
      }

      // ---- output: O^T += V^T . P^T (operands two d-blocks ahead) -----------------------------
#pragma unroll
      for (int db = 0; db < 16; ++db) {
        if (db + 2 < 16) {
          va[(db + 2) % 3][0] = v_operand(tile, v_base, db + 2, 0);
          va[(db + 2) % 3][1] = v_operand(tile, v_base, db + 2, 1);
        }
        mfma_a(o[db], va[db % 3][0], pb0);
        mfma_a(o[db], va[db % 3][1], pb1);
        __builtin_amdgcn_sched_barrier(0);
      }
      ++it;
    } while (!last);

    // ---- end of segment: the un-normalised sum leaves straight from the accumulators; the merge
    // kernel divides by the softmax sum.
    const float l_tot = sum_halves(l_sum);
    mfma_a_drain(o);
    const size_t part = ((size_t)w + b) * p.heads + head;
    float* orow = p.ws_o + part * kDc + 4 * half;
#pragma unroll
    for (int db = 0; db < 16; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(orow + 32 * db + 8 * g) =
            make_float4(o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]);
    }
    if (half == 0) *reinterpret_cast<float2*>(p.ws_ml + 2 * part) = make_float2(m_ref, l_tot);
  }
}

}  // namespace

bool mfma_supported(const DecodeParams& p) { return p.heads == 128 || p.heads == 64 || p.heads == 32; }

hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t s) {
  switch (p.heads) {
    case 128: hipLaunchKernelGGL(decode_mfma_kernel<4>, dim3(p.num_units), dim3(256), 0, s, p); break;
    case 64: hipLaunchKernelGGL(decode_mfma_kernel<2>, dim3(p.num_units), dim3(128), 0, s, p); break;
    case 32: hipLaunchKernelGGL(decode_mfma_kernel<1>, dim3(p.num_units), dim3(64), 0, s, p); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace mla
