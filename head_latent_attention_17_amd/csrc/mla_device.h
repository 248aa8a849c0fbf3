// Device-side helpers shared by the libmla kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {

// ---------------------------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16, round to nearest even (finite inputs; NaN is kept a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Element loads/stores for the two activation types (bf16 bits or fp32).
template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};

// ---------------------------------------------------------------------------------------------
// Wave64 inclusive scans, every lane active.  Within each row of 16 lanes by data-parallel moves
// (row_shr 1, 2, 4, 8: lane i adds lane i - s of its row; lanes shifted in from outside the row read
// 0), then each row adds the totals of the rows below it, read from lanes 15, 31 and 47.  Register
// moves only, where a shuffle (ds_bpermute) would make six dependent trips through the LDS crossbar.
// ---------------------------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ int row_shifted(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, true);
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  v += row_shifted<0x111>(v);
  v += row_shifted<0x112>(v);
  v += row_shifted<0x114>(v);
  v += row_shifted<0x118>(v);
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

template <int CTRL>
__device__ __forceinline__ long long row_shifted_i64(long long v) {
  const unsigned lo = (unsigned)row_shifted<CTRL>((int)(unsigned)v);
  const unsigned hi = (unsigned)row_shifted<CTRL>((int)(unsigned)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

__device__ __forceinline__ long long readlane_i64(long long v, int lane) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)v, lane);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)((unsigned long long)v >> 32), lane);
  return (long long)(((unsigned long long)hi << 32) | lo);
}

__device__ __forceinline__ long long wave_incl_scan_i64(long long v) {
  v += row_shifted_i64<0x111>(v);
  v += row_shifted_i64<0x112>(v);
  v += row_shifted_i64<0x114>(v);
  v += row_shifted_i64<0x118>(v);
  const long long r0 = readlane_i64(v, 15);
  const long long r1 = readlane_i64(v, 31);
  const long long r2 = readlane_i64(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// Sum over the wave, the same in every lane.
__device__ __forceinline__ long long wave_sum_i64(long long v) {
  return readlane_i64(wave_incl_scan_i64(v), 63);
}

// ---------------------------------------------------------------------------------------------
// Work units.  The pages of all sequences, concatenated in sequence order, are cut into
// `num_units` ranges [floor(w P / W), floor((w+1) P / W)), P = sum_b ceil(len_b / 64) (the vector-ALU
// decode, and the matrix-core decode below 8 tiles per unit); with more tiles the matrix-core decode
// cuts 32-token tiles by cost instead (below).  Every wave of every workgroup derives the same
// boundaries from seq_lens alone, so no host sync and no planning launch are needed.
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ int pages_of(int len) { return (int)(((unsigned)max(len, 0) + kPage - 1) / kPage); }

__device__ __forceinline__ long long unit_start(long long total_pages, int num_units, int w) {
  return (long long)w * total_pages / num_units;
}

// Unit holding global page p (the largest w with unit_start(w) <= p).
__device__ __forceinline__ int unit_of_page(long long total_pages, int num_units, long long p) {
  return (int)(((p + 1) * (long long)num_units - 1) / total_pages);
}

// Total pages of the batch (wave-uniform result).
__device__ __forceinline__ long long total_pages(const int32_t* seq_lens, int batch) {
  const int lane = threadIdx.x & 63;
  long long s = 0;
  for (int b = lane; b < batch; b += 64) s += pages_of(seq_lens[b]);
  return wave_sum_i64(s);
}

// Pages of sequences [0, b) (wave-uniform result).
__device__ __forceinline__ long long pages_before(const int32_t* seq_lens, int b) {
  const int lane = threadIdx.x & 63;
  long long s = 0;
  for (int i = lane; i < b; i += 64) s += pages_of(seq_lens[i]);
  return wave_sum_i64(s);
}

// First sequence whose pages reach past global page `p`, and the pages before it
// (wave-uniform).  Requires p < total pages.
__device__ __forceinline__ void locate_page(const int32_t* seq_lens, int batch, long long p,
                                            int& b_out, long long& before_out) {
  const int lane = threadIdx.x & 63;
  long long base = 0;
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int b = b0 + lane;
    const long long np = (b < batch) ? pages_of(seq_lens[b]) : 0;
    const long long incl = base + wave_incl_scan_i64(np);
    const unsigned long long hit = __ballot(b < batch && incl > p);
    if (hit) {
      const int first = __ffsll((long long)hit) - 1;
      const long long incl_first = __shfl(incl, first, 64);
      const long long np_first = __shfl(np, first, 64);
      b_out = b0 + first;
      before_out = incl_first - np_first;
      return;
    }
    base = __shfl(incl, 63, 64);
  }
  b_out = batch;
  before_out = base;
}

// Cost-weighted cut (the matrix-core decode's units), in tiles of 32 tokens.  A wave that moves on
// to another sequence inside its unit pays about five tiles for it: the new query queues behind the
// copies in flight, the finished piece is stored, and the first tile's scores run on their own.
// Walls: a sequence start that the plain cut floor(w T / W) already puts on a unit boundary costs
// nothing extra and stays a boundary.  Between two walls, the units that the plain cut gives that
// stretch cut it into equal lengths of a virtual line on which every other non-empty sequence
// spans kSegmentCostTiles positions for its start, then one per tile; a cut at virtual position x
// goes to the tile where x falls, or to the first tile of the sequence whose start positions hold
// x.  Used with at least 8 tiles per unit: every unit then spans at least 7 virtual positions, more
// than a start's cost, so it always holds a tile (and every cut stays inside its stretch).
constexpr int kSegmentCostTiles = 5;
__device__ __forceinline__ int tiles_of(int len) { return (int)(((unsigned)max(len, 0) + 31) / 32); }
__device__ __forceinline__ bool weighted_cut(long long total_tiles, int num_units) {
  return total_tiles >= 8LL * num_units;
}
// Whether tile position s is a boundary of the plain cut of T tiles into W units.
__device__ __forceinline__ bool plain_boundary(long long s, long long T, int W) {
  const long long w = (s * W + T - 1) / T;
  return w * T / W == s;
}
// First unit of the plain cut that starts at or after tile s.
__device__ __forceinline__ long long plain_unit_at(long long s, long long T, int W) { return (s * W + T - 1) / T; }

// Total tiles of the batch (wave-uniform result).
__device__ __forceinline__ long long total_tiles(const int32_t* seq_lens, int batch) {
  const int lane = threadIdx.x & 63;
  long long s = 0;
  for (int b = lane; b < batch; b += 64) s += tiles_of(seq_lens[b]);
  return wave_sum_i64(s);
}

// Unit w's tile range [t0, t1) under the weighted cut, for a batch of any size (wave-uniform).  Two
// passes over seq_lens: the walls around the plain cut of unit w, then the tiles at its two cuts.
__device__ __forceinline__ void weighted_unit_range(const int32_t* seq_lens, int batch, int W, int w,
                                                    long long T, long long& t0, long long& t1) {
  const int lane = threadIdx.x & 63;
  const long long cw = (long long)w * T / W;
  long long A0 = 0, A1 = T, n0 = 0, n1 = 0;  // walls; non-empty sequences up to A0's, before A1's
  int k0 = 0, k1 = batch;
  long long sbase = 0, nbase = 0;
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int b = b0 + lane;
    const long long nt = b < batch ? tiles_of(seq_lens[b]) : 0;
    const long long s = sbase + wave_incl_scan_i64(nt) - nt;
    const long long nc = nbase + wave_incl_scan_i64(nt > 0 ? 1 : 0);
    const bool wall = nt > 0 && plain_boundary(s, T, W);
    const unsigned long long lo = __ballot(wall && s <= cw);
    if (lo) {
      const int f = 63 - __clzll((long long)lo);
      A0 = __shfl(s, f, 64);
      n0 = __shfl(nc, f, 64);
      k0 = b0 + f;
    }
    const unsigned long long hi = __ballot(wall && s > cw);
    sbase = __shfl(s + nt, 63, 64);
    nbase = __shfl(nc, 63, 64);
    if (hi) {
      const int f = __ffsll((long long)hi) - 1;
      A1 = __shfl(s, f, 64);
      n1 = __shfl(nc, f, 64) - 1;
      k1 = b0 + f;
      break;
    }
  }
  if (k1 == batch) n1 = nbase;
  const long long wa0 = plain_unit_at(A0, T, W), wa1 = k1 < batch ? plain_unit_at(A1, T, W) : W;
  const long long V = (A1 - A0) + kSegmentCostTiles * (n1 - n0);
  const long long x0 = (w - wa0) * V / (wa1 - wa0), x1 = (w - wa0 + 1) * V / (wa1 - wa0);
  t0 = A1;
  t1 = A1;
  bool need0 = x0 < V, need1 = x1 < V;
  sbase = 0;
  nbase = 0;
  for (int b0 = 0; b0 < k1 && (need0 || need1); b0 += 64) {
    const int b = b0 + lane;
    const long long nt = b < batch ? tiles_of(seq_lens[b]) : 0;
    const long long s = sbase + wave_incl_scan_i64(nt) - nt;
    const long long nc = nbase + wave_incl_scan_i64(nt > 0 ? 1 : 0);
    const long long vs = s - A0 + kSegmentCostTiles * (nc - n0);  // virtual start of b's tiles
    const bool in = b >= k0 && b < k1 && nt > 0;
    if (need0) {
      const unsigned long long h = __ballot(in && vs + nt > x0);
      if (h) {
        const int f = __ffsll((long long)h) - 1;
        const long long d = x0 - __shfl(vs, f, 64);
        t0 = __shfl(s, f, 64) + (d > 0 ? d : 0);
        need0 = false;
      }
    }
    if (need1) {
      const unsigned long long h = __ballot(in && vs + nt > x1);
      if (h) {
        const int f = __ffsll((long long)h) - 1;
        const long long d = x1 - __shfl(vs, f, 64);
        t1 = __shfl(s, f, 64) + (d > 0 ? d : 0);
        need1 = false;
      }
    }
    sbase = __shfl(s + nt, 63, 64);
    nbase = __shfl(nc, 63, 64);
  }
}

// First sequence whose `1 << sh`-token units reach past global unit `p`, and the units before it
// (wave-uniform).  Requires p < the batch's total.
__device__ __forceinline__ void locate_unit(const int32_t* seq_lens, int batch, long long p, int sh,
                                            int& b_out, long long& before_out) {
  const int lane = threadIdx.x & 63;
  long long base = 0;
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int b = b0 + lane;
    const long long np = (b < batch) ? (long long)(((unsigned)max(seq_lens[b], 0) + (1u << sh) - 1) >> sh) : 0;
    const long long incl = base + wave_incl_scan_i64(np);
    const unsigned long long hit = __ballot(b < batch && incl > p);
    if (hit) {
      const int first = __ffsll((long long)hit) - 1;
      b_out = b0 + first;
      before_out = __shfl(incl, first, 64) - __shfl(np, first, 64);
      return;
    }
    base = __shfl(incl, 63, 64);
  }
  b_out = batch;
  before_out = base;
}

// One piece of a work unit: the pages [page0, page1) of sequence b that fall in the unit.
struct Segment {
  int b;
  int page0, page1;     // local page indices within sequence b
  int len;              // tokens of sequence b
  bool complete;        // the unit holds all of sequence b
  int slot;             // partial-result slot (0: the unit's first segment, 1: its last)
};

// Walks the segments of one unit.  All lanes of all waves run it identically.
struct SegmentWalker {
  const int32_t* seq_lens;
  int batch;
  long long unit_begin, unit_end, pos, before;
  int b;

  __device__ __forceinline__ void init(const int32_t* lens, int nb, int num_units, int w) {
    seq_lens = lens;
    batch = nb;
    const long long P = total_pages(lens, nb);
    unit_begin = P ? unit_start(P, num_units, w) : 0;
    unit_end = P ? unit_start(P, num_units, w + 1) : 0;
    pos = unit_begin;
    b = nb;
    before = 0;
    if (unit_begin < unit_end) locate_page(lens, nb, unit_begin, b, before);
  }

  __device__ __forceinline__ bool next(Segment& s) {
    if (pos >= unit_end) return false;
    int len = seq_lens[b];
    long long np = pages_of(len);
    while (np == 0 || before + np <= pos) {  // skip empty sequences
      before += np;
      ++b;
      len = seq_lens[b];
      np = pages_of(len);
    }
    const long long stop = (before + np < unit_end) ? before + np : unit_end;
    s.b = b;
    s.page0 = (int)(pos - before);
    s.page1 = (int)(stop - before);
    s.len = len;
    s.complete = (s.page0 == 0) && (s.page1 == (int)np);
    s.slot = (pos == unit_begin) ? 0 : 1;
    pos = stop;
    return true;
  }
};

// Units that hold sequence b: [wf, wl], from the table the matrix-core kernel writes, else derived
// from seq_lens.  A unit in that range holds no page (and wrote nothing) only when there are more
// units than pages.
struct SeqUnits {
  int wf, wl, W;
  bool all_live;
  long long P;
  __device__ __forceinline__ bool live(int w) const {
    return all_live || unit_start(P, W, w) != unit_start(P, W, w + 1);
  }
};

// The table's entry of sequence b, read together with its length (one memory round trip instead of
// two; the entry of an empty sequence is never written and never used).
__device__ __forceinline__ int4 seq_units_entry(const DecodeParams& p, int b) {
  return p.seq_units ? *reinterpret_cast<const int4*>(p.seq_units + 4 * b) : make_int4(0, 0, 0, 0);
}

__device__ __forceinline__ SeqUnits seq_units_of(const DecodeParams& p, int b, long long np, int4 d) {
  SeqUnits u;
  u.W = p.num_units;
  u.P = 0;
  if (p.seq_units) {
    u.wf = d.x;
    u.wl = d.y;
    u.all_live = d.z != 0;
    if (!u.all_live) u.P = total_pages(p.seq_lens, p.batch);
  } else {
    u.P = total_pages(p.seq_lens, p.batch);
    const long long before = pages_before(p.seq_lens, b);
    u.wf = unit_of_page(u.P, u.W, before);
    u.wl = unit_of_page(u.P, u.W, before + np - 1);
    u.all_live = u.P >= u.W;
  }
  return u;
}

}  // namespace mla
