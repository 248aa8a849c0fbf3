// Latent-space decode attention on the bf16 matrix cores of gfx950 (v_mfma_f32_32x32x16_bf16).
//
// What is computed (DeepSeek-V2 explainer, Steps 6-8): for every head h of sequence b,
//   S[t][h] = q_abs[b][h] . row_t        (576-long: latent score + RoPE score, one dot product)
//   P       = softmax_t(scale * S)       (online, base 2)
//   O[d][h] = sum_t P[h][t] * row_t[d]   (d < 512: the weighted sum of latent notes)
// All heads of a sequence share every cached row (the row is per token, not per head), so heads
// form the N dimension of both products and each row is read from HBM once per launch.
//
// Workgroup = 32 heads per wave; 4 waves (one per SIMD) cover 128 heads.  Per 32-token tile:
//   scores  S^T[t][h] = K . Q^T   M = 32 tokens, N = 32 heads, K = 576  (36 MFMAs)
//   output  O^T[d][h] = V^T . P^T M = 32 dims,   N = 32 heads, K = 32   (16 blocks x 2 MFMAs)
// Q stays in VGPRs for the whole segment; O^T (32 x 512 fp32 per wave) stays in accumulators.
// The S^T accumulator layout (lane = head, registers = tokens) is already the B-operand layout of
// the second product, so P never leaves its lane; V^T comes out of the token-major LDS tile with
// ds_read_b64_tr_b16, a 16-lane transposing read.
//
// Tiles are streamed HBM -> LDS with global_load_lds_dwordx4 through a 4-stage ring (4 x 36 KB),
// so no VGPRs are spent on staging.  Within a tile, 16-byte chunk c of token t is stored at chunk
// slot t*72 + (c ^ sigma(t)), sigma(t) = 2 (t mod 4) + ((t / 4) mod 2), which keeps both the
// row reads of the score product and the transposing reads of the output product free of LDS bank
// conflicts.  The softmax rescale of O is lazy: the reference maximum only moves when a tile's
// maximum exceeds it by more than 8 (base 2), so the rescale of 256 accumulators is rare.
#include "mla_device.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
#define LDS_AS __attribute__((address_space(3)))

constexpr int kTileTok = 32;
constexpr int kChunks = kRow / 8;                   // 72 16-byte chunks per row
constexpr int kTileChunks = kTileTok * kChunks;     // 2304
constexpr int kTileBytes = kTileChunks * 16;        // 36,864
constexpr int kStages = 4;  // the wait in the tile loop assumes at most 2 younger tiles
static_assert(kStages - 2 == 2, "tile-loop wait counts at most two younger tiles");
constexpr float kRescaleThreshold = 8.0f;           // base-2 headroom before O is rescaled

__device__ __forceinline__ int sigma(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Score MFMAs with their accumulator pinned to VGPRs.  The 32 x 512 output accumulator of each
// wave takes all 256 AGPRs, so the score accumulator must live in VGPRs; the builtin would place it
// in AGPRs as well.  Hazards the compiler cannot see through asm are padded explicitly: two wait
// states before each MFMA (a VALU write of an operand may precede it) and, after the last one,
// enough wait states for a VALU read of the 8-pass result (the final s_nop block ties itself to
// the accumulator so nothing reading it is scheduled earlier).
__device__ __forceinline__ void mfma_v_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v_drain(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
}

// Output MFMAs with their accumulator pinned to AGPRs ("+a"): left to itself the compiler turns
// the loop-carried 256-register accumulator into VGPR copies and spills.
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
// scalar loads (lgkmcnt).  A vector load here would be ordered behind the in-flight LDS DMA and
// its wait would drain the whole ring.  Neither array is written while a launch runs.
#define CONST_AS __attribute__((address_space(4)))
__device__ __forceinline__ int ld_const(const int32_t* ptr, size_t i) {
  return ((const CONST_AS int32_t*)ptr)[i];
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
  __device__ __forceinline__ bool first() const { return t == max(pg0 - before, 0) * kPage; }
  __device__ __forceinline__ bool last() const { return t + kTileTok >= t_end; }
  __device__ __forceinline__ bool complete() const { return before >= pg0 && before + np <= pg1; }
  __device__ __forceinline__ int slot() const { return before < pg0 ? 0 : (before == pg0 ? 0 : 1); }
};

template <int NW>
__device__ __forceinline__ void issue_tile(const DecodeParams& p, const TileCursor& c,
                                           LDS_AS char* stage, int wave) {
  constexpr int kPerWave = kTileChunks / 64 / NW;
  const int page = ld_const(p.block_table, (size_t)c.b * p.max_blocks + c.t / kPage);
  const int nt = min(kTileTok, c.t_end - c.t);
  const char* base = reinterpret_cast<const char*>(p.cache) +
                     ((size_t)page * kPage + (c.t % kPage)) * (kRow * 2);
  // The per-lane offsets below are loop invariant for full tiles; recomputing them, from a lane id
  // rebuilt with mbcnt, keeps them out of long-lived VGPRs (a reloaded spill here would have to
  // wait for every DMA in flight).
  int ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int inst = wave * kPerWave + j;
    const int pos = inst * 64 + ln;
    const int t = pos / kChunks;
    const int slot = pos - t * kChunks;
    const int chunk = slot ^ sigma(t);
    const int tt = min(t, nt - 1);  // rows past the end re-read the last valid row (masked later)
    const unsigned off = (unsigned)(tt * (kRow * 2) + chunk * 16);
    __builtin_amdgcn_global_load_lds(base + off, (LDS_AS void*)(stage + inst * 1024), 16, 0, 0);
  }
}

// Score operand for k-step ks: 8 consecutive latent dims of this lane's token.
__device__ __forceinline__ bf16x8 k_operand(const LDS_AS char* tile, const int* k_base, int ks) {
  return *reinterpret_cast<const LDS_AS bf16x8*>(tile + k_base[ks & 3] + 128 * (ks >> 2));
}

// Output operand for d-block db and token half m: 8 tokens of one latent dim, gathered by two
// 16-lane transposing reads.
__device__ __forceinline__ bf16x8 v_operand(const LDS_AS char* tile, const int* v_base, int db, int m) {
  const LDS_AS char* vp = tile + v_base[db & 1] + 128 * (db >> 1) + (16 * m) * (kChunks * 16);
  const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)vp);
  const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(vp + 8 * kChunks * 16));
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

  // Prologue: put the first kStages-1 tiles in flight.
  int issued = 0;
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) {
    if (ld.valid) {
      issue_tile<NW>(p, ld, (LDS_AS char*)ring[s], wave);
      ld.advance();
      ++issued;
    }
  }

  const uint16_t* qa = static_cast<const uint16_t*>(p.q_abs);

  // Per-lane constant parts of the LDS addresses; the rest of every address is an immediate.
  // Score operand, k-step ks = 4 g + i: chunk (2 ks + half) ^ sigma(token) = 8 g + 2 (i ^ (sig >> 1))
  // + (half ^ (sig & 1)), so four lane bases (one per i) cover all 36 k-steps.
  const int k_sig = sigma(l32);
  int k_base[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    k_base[i] = (l32 * kChunks + 2 * (i ^ (k_sig >> 1)) + (half ^ (k_sig & 1))) * 16;
  // Transposing reads: token 16 m + 8 r + v_tok, chunk (4 db + v_chunk) ^ sigma(v_tok); with
  // db = 2 k + e that is 8 k + 4 (e ^ (sig >> 2)) + ((v_chunk ^ sig) & 3): two lane bases.
  const int v_tok = 4 * half + ((lane & 15) >> 2);
  const int v_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int v_sig = sigma(v_tok);
  int v_base[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
    v_base[e] = (v_tok * kChunks + 4 * (e ^ (v_sig >> 2)) + ((v_chunk ^ v_sig) & 3)) * 16 + 8 * (lane & 1);

  int it = 0;
  while (cp.valid) {  // one segment: the part of sequence b inside this unit
    const int b = cp.b;
    bf16x8 q[36];
    {
      const uint16_t* qrow = qa + ((size_t)b * p.heads + head) * kRow + 8 * half;
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) q[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks);
    }
    f32x16 o[16];
    {
      const bf16x8 zero = {};
#pragma unroll
      for (int i = 0; i < 16; ++i) mfma_a_zero(o[i], zero);
    }
    float m_ref = -INFINITY;  // base-2 reference maximum (identical in lanes l and l^32)
    float l_sum = 0.f;        // this lane's share of the softmax denominator
    bool fresh = true;
    bool last;

    do {  // one 32-token tile
      const int stage = it % kStages;
      {
        // This wave's DMA for tile `it` must have landed.  Vector loads complete in issue order,
        // so it is enough to allow exactly the DMA of the tiles issued after it to stay in
        // flight (later stores only make the wait longer).
        constexpr int kPerWave = kTileChunks / 64 / NW;
        const int younger = issued - it - 1;
        if (younger >= 2) wait_vmcnt<(2 * kPerWave < 63 ? 2 * kPerWave : 63)>();
        else if (younger == 1) wait_vmcnt<(kPerWave < 63 ? kPerWave : 63)>();
        else wait_vmcnt<0>();
      }
      __builtin_amdgcn_s_barrier();
      // All waves are past their reads of tile it-1: its stage may be refilled.
      if (ld.valid) {
        issue_tile<NW>(p, ld, (LDS_AS char*)ring[(it + kStages - 1) % kStages], wave);
        ld.advance();
        ++issued;
      }
      const int nt = min(kTileTok, cp.t_end - cp.t);
      const LDS_AS char* tile = (const LDS_AS char*)ring[stage];

      // ---- scores: S^T = K . Q^T -----------------------------------------------------------
      // Software pipeline: the LDS read for k-step ks+2 is issued before the MFMA of k-step ks.
      f32x16 s;
      bf16x8 ka[3];
      ka[0] = k_operand(tile, k_base, 0);
      ka[1] = k_operand(tile, k_base, 1);
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) {
        if (ks + 2 < 36) ka[(ks + 2) % 3] = k_operand(tile, k_base, ks + 2);
        if (ks == 0) mfma_v_first(s, ka[0], q[0]); else mfma_v(s, ka[ks % 3], q[ks]);
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma_v_drain(s);

      // ---- online softmax (base 2), lane = head, registers = tokens -----------------------
      float mt = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int tok = (j >> 2) * 8 + half * 4 + (j & 3);
        const float v = (tok < nt) ? s[j] * p.scale_log2 : -INFINITY;
        s[j] = v;
        mt = fmaxf(mt, v);
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      if (__ballot(fresh || (mt > m_ref + kRescaleThreshold))) {
        const float m_new = fmaxf(m_ref, mt);
        if (!fresh) {
          const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
          l_sum *= alpha;
          // Rare (the running maximum jumped by more than 2^8): the accumulators make a round
          // trip through this piece's own workspace slot, which its final write overwrites
          // anyway, so that scaling them never holds more than one block in VGPRs.
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
        m_ref = m_new;
        fresh = false;
      }
      bf16x8 pb0, pb1;
      float ls = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float e = __builtin_amdgcn_exp2f(s[j] - m_ref);
        ls += e;
        if (j < 8) pb0[j] = (__bf16)e; else pb1[j - 8] = (__bf16)e;
      }
      l_sum += ls;

      // ---- output: O^T += V^T . P^T ----------------------------------------------------------
      // Same pipelining: the two A operands of d-block db+1 are read while db's MFMAs issue.
      bf16x8 va[2][2];
      va[0][0] = v_operand(tile, v_base, 0, 0);
      va[0][1] = v_operand(tile, v_base, 0, 1);
#pragma unroll
      for (int db = 0; db < 16; ++db) {
        if (db + 1 < 16) {
          va[(db + 1) & 1][0] = v_operand(tile, v_base, db + 1, 0);
          va[(db + 1) & 1][1] = v_operand(tile, v_base, db + 1, 1);
        }
        mfma_a(o[db], va[db & 1][0], pb0);
        mfma_a(o[db], va[db & 1][1], pb1);
        __builtin_amdgcn_sched_barrier(0);
      }
      last = cp.last();
      cp.advance();
      ++it;
    } while (!last);

    // ---- end of segment: the un-normalised sum leaves straight from the accumulators; the merge
    // kernel divides by the softmax sum (keeps VALU work, and VGPRs, off the 256 accumulators).
    const float l_tot = l_sum + __shfl_xor(l_sum, 32, 64);
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
