// Attention over the top-k tokens of a cheap index ("DeepSeek (AI)" wiki, "KV cache data movement
// minimization": retrieval is bandwidth-bound, so each token also carries a cheap index vector; a
// decode query scores all of them, keeps the k best, and attention reads only those rows).
// Reading: an index vector is 128 int8 numbers, so a score is an exact integer; ties go to the
// earlier position; a sequence of at most k tokens keeps them all.
//
//   scoring   s_t = q_index[b] . i_t for t < len_b (8 lanes per token, 16 bytes and four
//             v_dot4_i32_i8 each), written as int32, with a histogram of the high bits of the
//             order-preserving key s_t + 2^21 (4,096 bins, counted in LDS per 1,024-token chunk).
//   select    a two-pass radix select over many workgroups: the high bin holding the k-th largest
//             key, then a 2,048-bin histogram of the low bits inside it, give the k-th largest key
//             T and how many keys equal to T are kept (the earliest ones).
//   write     per chunk, keys above T and equal to T are counted; each chunk's output offset is
//             the kept count of the chunks before it (two sums, since equal keys are kept in
//             position order), and each chunk writes its kept positions, in increasing order.
//   short     with at most 16,384 tokens per block table, scoring is followed by one workgroup
//             per sequence that does both passes and the write in LDS (two launches, and no
//             global histogram to clear).
//   gather    copies the kept rows into compact pages (sequence b owns pages b P .. b P + P - 1,
//             P = ceil(k / 64)) and writes their block table, so that mla_decode runs over them
//             unchanged.  mla_decode_topk reads the same rows in place instead (the decode
//             kernel's list mode), with the same result.
#include "mla_device.h"

namespace mla {
namespace {

constexpr int kIndexDim = 128;
constexpr int kChunk = 1024;          // positions per workgroup in the selection passes (and scoring)
constexpr int kBins1 = 4096;          // key >> 11: keys are score + 2^21, in [0, 2^22]
constexpr int kBins2 = 2048;          // key & 2047
constexpr int kSmallMax = 16384;      // block tables up to this many tokens: one workgroup per sequence
constexpr int kSmallThreads = 1024;

// Workspace layout (int32), per sequence b:
//   scores [B][stride]; hist1 [B][4096]; hist2 [B][2048]; pick [B][4] (hi bin, left after it,
//   threshold key T, keys equal to T to keep; T = -1 keeps every token); chunk [B][nchunks][2]
//   (keys above T, keys equal to T).
struct TopkWs {
  int32_t* scores;
  int32_t* hist1;
  int32_t* hist2;
  int32_t* pick;
  int32_t* chunk;
  int stride, nchunks;
};

__device__ __forceinline__ int key_of(int32_t s) { return s + (1 << 21); }

__global__ __launch_bounds__(256) void topk_clear_kernel(TopkWs w) {
  const int b = blockIdx.x;
  for (int i = threadIdx.x; i < kBins1; i += 256) w.hist1[(size_t)b * kBins1 + i] = 0;
  for (int i = threadIdx.x; i < kBins2; i += 256) w.hist2[(size_t)b * kBins2 + i] = 0;
}

// Scores of the CH-token chunk blockIdx.x of sequence b (8 lanes per token, 32 tokens per step),
// plus the histogram of their high key bits, gathered in LDS and added to the sequence's histogram.
// CH (a multiple of 256, at most the selection chunk) is smaller when the batch has few chunks, so
// that the grid still fills the compute units.
template <int CH, bool HIST>
__global__ __launch_bounds__(256) void index_score_kernel(const int8_t* __restrict__ index_cache,
                                                          const int32_t* __restrict__ block_table, int max_blocks,
                                                          const int32_t* __restrict__ seq_lens,
                                                          const int8_t* __restrict__ q_index, TopkWs w) {
  static_assert(CH % 256 == 0 && CH <= kChunk, "whole rounds of eight 32-token steps");
  __shared__ int hist[kBins1];
  const int b = blockIdx.y;
  const int len = seq_lens[b];
  const int t0 = blockIdx.x * CH;
  if (t0 >= len) return;
  if constexpr (HIST) {
    for (int i = threadIdx.x; i < kBins1; i += 256) hist[i] = 0;
    __syncthreads();
  }
  const int part = threadIdx.x & 7;  // 16-byte part of the vector
  const int4 q = *reinterpret_cast<const int4*>(q_index + (size_t)b * kIndexDim + 16 * part);
  int32_t* __restrict__ scores = w.scores + (size_t)b * w.stride;
  // eight steps of 32 tokens at a time: all their loads are issued before any score is stored
  for (int s0 = 0; s0 < CH / 32; s0 += 8) {
    int4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      // a 32-token step lies inside one page (chunks start on page boundaries, two steps a page),
      // so its page id is the same for the whole workgroup: a scalar load
      const int step = s0 + u;
      const int t = t0 + step * 32 + (threadIdx.x >> 3);
      v[u] = make_int4(0, 0, 0, 0);
      if (t0 + step * 32 < len) {
        const int page = ((const __attribute__((address_space(4))) int32_t*)block_table)[(size_t)b * max_blocks + (t0 >> 6) + (step >> 1)];
        if (t < len)
          v[u] = *reinterpret_cast<const int4*>(index_cache + ((size_t)page * kPage + t % kPage) * kIndexDim + 16 * part);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = t0 + (s0 + u) * 32 + (threadIdx.x >> 3);
      int sc = 0;
      sc = __builtin_amdgcn_sdot4(v[u].x, q.x, sc, false);
      sc = __builtin_amdgcn_sdot4(v[u].y, q.y, sc, false);
      sc = __builtin_amdgcn_sdot4(v[u].z, q.z, sc, false);
      sc = __builtin_amdgcn_sdot4(v[u].w, q.w, sc, false);
      sc += __shfl_xor(sc, 1, 64);
      sc += __shfl_xor(sc, 2, 64);
      sc += __shfl_xor(sc, 4, 64);
      if (t < len && part == 0) {
        scores[t] = sc;
        if constexpr (HIST) atomicAdd(&hist[key_of(sc) >> 11], 1);
      }
    }
  }
  if constexpr (HIST) {
    __syncthreads();
    for (int i = threadIdx.x; i < kBins1; i += 256)
      if (hist[i]) atomicAdd(&w.hist1[(size_t)b * kBins1 + i], hist[i]);
  }
}

// Inclusive scan over a workgroup of NT threads (one value each) through the wave totals in LDS;
// the workgroup total goes to *total.
template <int NT>
__device__ __forceinline__ int block_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int i = 0; i < NT / 64; ++i) {
      const int x = wsum[i];
      wsum[i] = acc;
      acc += x;
    }
    *total = acc;
  }
  __syncthreads();
  const int r = v + wsum[wave];
  __syncthreads();  // wsum is reused by the next scan
  return r;
}

// Finds, from the top, the bin where the running count reaches `need` (pass 1: need = k; pass 2:
// what pass 1 left).  NT threads, thread i owns bins [i NB / NT, (i + 1) NB / NT) counted from the
// top; exactly one thread writes the result.
template <int NB, int NT = 256>
__device__ __forceinline__ void pick_bin(const int32_t* hist, int need, int* out_bin, int* out_left) {
  __shared__ int wsum[NT / 64];
  __shared__ int tot;
  constexpr int per = NB / NT;
  const int i = threadIdx.x;
  // thread i takes bins counted from the top: (NT - 1 - i) per .. + per - 1, scanned top first
  const int hi_bin = NB - 1 - i * per;
  int mine = 0;
  for (int j = 0; j < per; ++j) mine += hist[hi_bin - j];
  const int incl = block_scan<NT>(mine, wsum, &tot);
  const int before = incl - mine;  // keys in the bins above this thread's range
  if (before < need && incl >= need) {
    int cum = before, d = hi_bin;
    for (int j = 0; j < per; ++j, --d) {
      if (cum + hist[d] >= need) break;
      cum += hist[d];
    }
    *out_bin = d;
    *out_left = need - cum;
  }
}

// Histogram of the low key bits of the keys in the high bin that holds the k-th largest key.
// Every workgroup finds that bin from the high-bit histogram; the first one of each sequence
// records it (bin, keys still needed inside it), or -1 when the sequence keeps every token.
__global__ __launch_bounds__(256) void topk_hist2_kernel(const int32_t* __restrict__ seq_lens, int k, TopkWs w) {
  __shared__ int hist[kBins2];
  __shared__ int d1_s, left_s;
  const int b = blockIdx.y;
  const int len = max(seq_lens[b], 0);
  const int t0 = blockIdx.x * kChunk;
  int* pk = w.pick + 4 * b;
  if (len <= k) {
    if (blockIdx.x == 0 && threadIdx.x == 0) { pk[0] = -1; pk[1] = 0; pk[2] = -1; pk[3] = 0; }
    return;
  }
  pick_bin<kBins1>(w.hist1 + (size_t)b * kBins1, k, &d1_s, &left_s);
  __syncthreads();
  const int d1 = d1_s;
  if (blockIdx.x == 0 && threadIdx.x == 0) { pk[0] = d1; pk[1] = left_s; }
  if (t0 >= len) return;
  for (int i = threadIdx.x; i < kBins2; i += 256) hist[i] = 0;
  __syncthreads();
  for (int t = t0 + threadIdx.x; t < min(t0 + kChunk, len); t += 256) {
    const int key = key_of(w.scores[(size_t)b * w.stride + t]);
    if ((key >> 11) == d1) atomicAdd(&hist[key & 2047], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kBins2; i += 256)
    if (hist[i]) atomicAdd(&w.hist2[(size_t)b * kBins2 + i], hist[i]);
}

// Per chunk: keys above the k-th largest key T and keys equal to it (every token counts as above
// when the sequence keeps them all).  Every workgroup finds T from the low-bit histogram; the first
// one of each sequence records it with the number of keys equal to T that are kept.
__global__ __launch_bounds__(256) void topk_count_kernel(const int32_t* __restrict__ seq_lens, TopkWs w) {
  __shared__ int red[2][4];
  __shared__ int d2_s, left_s;
  const int b = blockIdx.y;
  const int c = blockIdx.x;
  const int len = max(seq_lens[b], 0);
  int* pk = w.pick + 4 * b;
  const int d1 = pk[0];
  int T = -1;
  if (d1 >= 0) {
    pick_bin<kBins2>(w.hist2 + (size_t)b * kBins2, pk[1], &d2_s, &left_s);
    __syncthreads();
    T = (d1 << 11) | d2_s;
    if (c == 0 && threadIdx.x == 0) { pk[2] = T; pk[3] = left_s; }
  }
  int gt = 0, eq = 0;
  for (int t = c * kChunk + threadIdx.x; t < min((c + 1) * kChunk, len); t += 256) {
    const int key = T < 0 ? 1 : key_of(w.scores[(size_t)b * w.stride + t]);
    gt += key > T;
    eq += key == T;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    gt += __shfl_xor(gt, o, 64);
    eq += __shfl_xor(eq, o, 64);
  }
  if ((threadIdx.x & 63) == 0) { red[0][threadIdx.x >> 6] = gt; red[1][threadIdx.x >> 6] = eq; }
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t* ch = w.chunk + ((size_t)b * w.nchunks + c) * 2;
    ch[0] = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    ch[1] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  }
}

// Writes the kept positions of chunk blockIdx.x in increasing order.  The kept keys before a
// position are all the keys above T before it plus min(need_eq, keys equal to T before it), since
// the equal keys are kept in position order; the earlier chunks' two counts are summed, and one scan
// of the pair (above T, equal to T) inside the chunk (each at most 1,024: they share one int) adds
// the rest.
__global__ __launch_bounds__(kChunk) void topk_write_kernel(const int32_t* __restrict__ seq_lens, int k, TopkWs w,
                                                            int32_t* __restrict__ positions,
                                                            int32_t* __restrict__ counts) {
  __shared__ int wsum[kChunk / 64];
  __shared__ int red[2][kChunk / 64];
  __shared__ int tot[1];
  const int b = blockIdx.y;
  const int c = blockIdx.x;
  const int len = max(seq_lens[b], 0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (c == 0 && threadIdx.x == 0) counts[b] = min(len, k);
  if (c * kChunk >= len) return;
  const int T = w.pick[4 * b + 2], need_eq = w.pick[4 * b + 3];
  int g = 0, e = 0;
  for (int cc = threadIdx.x; cc < c; cc += kChunk) {
    const int32_t* ch = w.chunk + ((size_t)b * w.nchunks + cc) * 2;
    g += ch[0];
    e += ch[1];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    g += __shfl_xor(g, o, 64);
    e += __shfl_xor(e, o, 64);
  }
  if (lane == 0) { red[0][wave] = g; red[1][wave] = e; }
  const int t = c * kChunk + threadIdx.x;
  const int key = t < len ? (T < 0 ? 1 : key_of(w.scores[(size_t)b * w.stride + t])) : -2;
  const int pair = (key > T ? 1 : 0) | (key == T ? 1 << 16 : 0);
  const int before = block_scan<kChunk>(pair, wsum, &tot[0]) - pair;  // its barriers publish red too
  int gt_before = 0, eq_before = 0;
#pragma unroll
  for (int i = 0; i < kChunk / 64; ++i) { gt_before += red[0][i]; eq_before += red[1][i]; }
  const int eq_rank = eq_before + (before >> 16);
  const int take = key > T || (key == T && eq_rank < need_eq);
  const int at = gt_before + (before & 0xffff) + min(need_eq, eq_rank);
  if (take) positions[(size_t)b * k + at] = t;
}

// The selection for one sequence in one workgroup, for block tables of at most kSmallMax tokens:
// its scores (written by the scoring kernel) are staged in LDS, both radix passes count in LDS, and
// the kept positions are written in increasing order (each thread owns a run of consecutive
// positions; one scan places the runs).  Same result as the multi-workgroup passes: the k highest keys, ties to the earlier
// position.
__global__ __launch_bounds__(kSmallThreads) void topk_select_small_kernel(const int32_t* __restrict__ seq_lens,
                                                                         int k, TopkWs w,
                                                                         int32_t* __restrict__ positions,
                                                                         int32_t* __restrict__ counts) {
  __shared__ int32_t sc[kSmallMax];
  __shared__ int32_t hist[kBins1];
  __shared__ int wsum[kSmallThreads / 64];
  __shared__ int tot[1];
  __shared__ int d_s, left_s;
  const int b = blockIdx.x;
  const int len = max(seq_lens[b], 0);
  const int tid = threadIdx.x;
  if (tid == 0) counts[b] = min(len, k);
  int32_t* out = positions + (size_t)b * k;
  if (len <= k) {  // every token is kept
    for (int t = tid; t < len; t += kSmallThreads) out[t] = t;
    return;
  }
  for (int i = tid; i < kBins1; i += kSmallThreads) hist[i] = 0;
  __syncthreads();
  {
    const int32_t* src = w.scores + (size_t)b * w.stride;
    int v[kSmallMax / kSmallThreads];
#pragma unroll
    for (int u = 0; u < kSmallMax / kSmallThreads; ++u) {
      const int t = tid + u * kSmallThreads;
      v[u] = t < len ? src[t] : 0;
    }
#pragma unroll
    for (int u = 0; u < kSmallMax / kSmallThreads; ++u) {
      const int t = tid + u * kSmallThreads;
      if (t < len) {
        sc[t] = v[u];
        atomicAdd(&hist[key_of(v[u]) >> 11], 1);
      }
    }
  }
  __syncthreads();
  pick_bin<kBins1, kSmallThreads>(hist, k, &d_s, &left_s);
  __syncthreads();
  const int d1 = d_s, left1 = left_s;
  for (int i = tid; i < kBins2; i += kSmallThreads) hist[i] = 0;
  __syncthreads();
  for (int t = tid; t < len; t += kSmallThreads) {
    const int key = key_of(sc[t]);
    if ((key >> 11) == d1) atomicAdd(&hist[key & 2047], 1);
  }
  __syncthreads();
  pick_bin<kBins2, kSmallThreads>(hist, left1, &d_s, &left_s);
  __syncthreads();
  const int T = (d1 << 11) | d_s, need_eq = left_s;
  // Thread i owns the J consecutive positions from J i, its keys held in registers (-1 where there
  // is no token: below every key).  The keys kept before its run are those above T plus the first
  // need_eq keys equal to T in position order, so one scan of the pair (above T, equal to T) places
  // every run: start = above + min(need_eq, equal).  Both counts are at most 2^14 and share one int.
  constexpr int kJ = kSmallMax / kSmallThreads;
  const int J = (len + kSmallThreads - 1) / kSmallThreads;
  const int t0 = tid * J, t1 = min(t0 + J, len);
  int key[kJ];
  int gt_mine = 0, eq_mine = 0;
#pragma unroll
  for (int u = 0; u < kJ; ++u) {
    key[u] = u < J && t0 + u < t1 ? key_of(sc[t0 + u]) : -1;
    gt_mine += key[u] > T;
    eq_mine += key[u] == T;
  }
  const int pair = gt_mine | (eq_mine << 16);
  const int before = block_scan<kSmallThreads>(pair, wsum, &tot[0]) - pair;
  int eq_rank = before >> 16;
  int at = (before & 0xffff) + min(need_eq, eq_rank);
#pragma unroll
  for (int u = 0; u < kJ; ++u) {
    if (key[u] > T || (key[u] == T && eq_rank < need_eq)) out[at++] = t0 + u;
    eq_rank += key[u] == T;
  }
}

// Row i < counts[b] of sequence b: 72 lanes of 16 bytes from its page to compact page
// b * P + i / 64, slot i % 64.  The first row's workgroup also writes the compact block table.
__global__ __launch_bounds__(128) void gather_rows_kernel(const uint16_t* __restrict__ cache,
                                                          const int32_t* __restrict__ block_table, int max_blocks,
                                                          const int32_t* __restrict__ positions,
                                                          const int32_t* __restrict__ counts, int k, int pk,
                                                          uint16_t* __restrict__ out, int32_t* __restrict__ out_bt) {
  const int i = blockIdx.x;
  const int b = blockIdx.y;
  const int c = threadIdx.x;
  if (i == 0)
    for (int j = c; j < pk; j += 128) out_bt[(size_t)b * pk + j] = b * pk + j;
  if (c >= kRow / 8 || i >= counts[b]) return;
  const int t = positions[(size_t)b * k + i];
  const int page = block_table[(size_t)b * max_blocks + t / kPage];
  const uint4 v = *reinterpret_cast<const uint4*>(cache + ((size_t)page * kPage + t % kPage) * kRow + 8 * c);
  *reinterpret_cast<uint4*>(out + (((size_t)b * pk + i / kPage) * kPage + i % kPage) * kRow + 8 * c) = v;
}

}  // namespace

static TopkWs topk_ws(void* base, int batch, int max_blocks) {
  TopkWs w;
  w.stride = max_blocks * kPage;
  w.nchunks = (w.stride + kChunk - 1) / kChunk;
  int32_t* p = static_cast<int32_t*>(base);
  w.scores = p;
  p += (size_t)batch * w.stride;
  w.hist1 = p;
  p += (size_t)batch * kBins1;
  w.hist2 = p;
  p += (size_t)batch * kBins2;
  w.pick = p;
  p += (size_t)batch * 4;
  w.chunk = p;
  return w;
}

size_t index_topk_workspace_bytes(int batch, int max_blocks) {
  const size_t stride = (size_t)max_blocks * kPage;
  const size_t nchunks = (stride + kChunk - 1) / kChunk;
  return (size_t)batch * (stride + kBins1 + kBins2 + 4 + 2 * nchunks) * sizeof(int32_t);
}

hipError_t launch_index_topk(const int8_t* index_cache, const int32_t* block_table, int max_blocks,
                             const int32_t* seq_lens, const int8_t* q_index, int batch, int k, int32_t* positions,
                             int32_t* counts, void* workspace, hipStream_t s) {
  const TopkWs w = topk_ws(workspace, batch, max_blocks);
  const dim3 chunks(w.nchunks, batch);
  // Scoring chunks: 1,024 tokens, or 256 while that grid would hold fewer than two workgroups per
  // compute unit (32 x 4,096 tokens: 12.0 -> 7.6 us).  Halving the chunks of a 516-workgroup grid
  // (4 x 131,072 tokens) made scoring slower (20.1 -> 22.2 us): more workgroups flush their
  // histograms into the same few hot bins.
  const bool small_chunks = (long long)w.nchunks * batch < 2 * kNumCUs;
  if ((long long)max_blocks * kPage <= kSmallMax) {
    // Short block tables: scoring alone, then one workgroup per sequence selects (two launches, no
    // global histograms to clear).
    if (small_chunks)
      hipLaunchKernelGGL((index_score_kernel<kChunk / 4, false>), dim3(4 * w.nchunks, batch), dim3(256), 0, s,
                         index_cache, block_table, max_blocks, seq_lens, q_index, w);
    else
      hipLaunchKernelGGL((index_score_kernel<kChunk, false>), chunks, dim3(256), 0, s, index_cache, block_table,
                         max_blocks, seq_lens, q_index, w);
    hipLaunchKernelGGL(topk_select_small_kernel, dim3(batch), dim3(kSmallThreads), 0, s, seq_lens, k, w, positions,
                       counts);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(topk_clear_kernel, dim3(batch), dim3(256), 0, s, w);
  if (small_chunks)
    hipLaunchKernelGGL((index_score_kernel<kChunk / 4, true>), dim3(4 * w.nchunks, batch), dim3(256), 0, s,
                       index_cache, block_table, max_blocks, seq_lens, q_index, w);
  else
    hipLaunchKernelGGL((index_score_kernel<kChunk, true>), chunks, dim3(256), 0, s, index_cache, block_table,
                       max_blocks, seq_lens, q_index, w);
  hipLaunchKernelGGL(topk_hist2_kernel, chunks, dim3(256), 0, s, seq_lens, k, w);
  hipLaunchKernelGGL(topk_count_kernel, chunks, dim3(256), 0, s, seq_lens, w);
  hipLaunchKernelGGL(topk_write_kernel, chunks, dim3(kChunk), 0, s, seq_lens, k, w, positions, counts);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* cache, const int32_t* block_table, int max_blocks,
                              const int32_t* positions, const int32_t* counts, int batch, int k, void* out,
                              int32_t* out_bt, hipStream_t s) {
  const int pk = (k + kPage - 1) / kPage;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(k, batch), dim3(128), 0, s, (const uint16_t*)cache, block_table,
                     max_blocks, positions, counts, k, pk, (uint16_t*)out, out_bt);
  return hipGetLastError();
}

}  // namespace mla
