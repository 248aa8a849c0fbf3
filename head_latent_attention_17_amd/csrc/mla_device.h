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
// Wave64 reductions / scans (ds_swizzle-free: __shfl_* lower to ds_bpermute)
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ long long wave_sum_i64(long long v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ long long wave_incl_scan_i64(long long v) {
  const int lane = threadIdx.x & 63;
  for (int o = 1; o < 64; o <<= 1) {
    long long n = __shfl_up(v, o, 64);
    if (lane >= o) v += n;
  }
  return v;
}

// ---------------------------------------------------------------------------------------------
// Work units.  The pages of all sequences, concatenated in sequence order, are cut into
// `num_units` ranges [floor(w P / W), floor((w+1) P / W)), P = sum_b ceil(len_b / 64).  Every
// wave of every workgroup derives the same boundaries from seq_lens alone, so no host sync and no
// planning launch are needed.
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

}  // namespace mla
