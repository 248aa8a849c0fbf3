// Optional device-side check of the paging inputs (enabled per call by MLA_DEBUG_CHECKS=1): every
// block-table entry that a call will dereference must name a page in [0, num_pages), every length
// must fit the table row (decode), every append position must fall inside it (append), every kept
// count must be at most k and every kept position must fall inside the table row (top-k decode).
// The check reads only entries inside the table's [batch][max_blocks] extent, so a bad table is reported
// without touching the cache.  It synchronises the stream to read its verdict, which is why it is
// a debug mode and not part of the asynchronous path.
#include "mla_device.h"

namespace mla {
namespace {

__device__ int g_table_fault;  // set to 1 by any thread that finds a bad entry

__global__ void reset_fault_kernel() { g_table_fault = 0; }

// One workgroup per sequence.  mode 0: lens[b] tokens attended (pages [0, ceil(len / 64)) used);
// mode 1: lens[b] is an append position (page lens[b] / 64 used).
__global__ void check_table_kernel(const int32_t* __restrict__ bt, int max_blocks,
                                   const int32_t* __restrict__ lens, int num_pages, int mode) {
  const int b = blockIdx.x;
  const long long v = lens[b];
  const long long cap = (long long)max_blocks * kPage;
  bool bad = false;
  if (mode == 0) {
    if (v < 0 || v > cap) {
      bad = true;
    } else {
      const int np = (int)((v + kPage - 1) / kPage);
      for (int j = threadIdx.x; j < np; j += blockDim.x) {
        const int page = bt[(size_t)b * max_blocks + j];
        if (page < 0 || page >= num_pages) bad = true;
      }
    }
  } else if (threadIdx.x == 0) {
    if (v < 0 || v >= cap) {
      bad = true;
    } else {
      const int page = bt[(size_t)b * max_blocks + (int)(v / kPage)];
      bad = page < 0 || page >= num_pages;
    }
  }
  if (bad) g_table_fault = 1;
}

// One workgroup per sequence: counts[b] in [0, k]; each of its first counts[b] positions inside the
// table row, naming a page in [0, num_pages).
__global__ void check_positions_kernel(const int32_t* __restrict__ bt, int max_blocks,
                                       const int32_t* __restrict__ positions, const int32_t* __restrict__ counts,
                                       int k, int num_pages) {
  const int b = blockIdx.x;
  const int n = counts[b];
  bool bad = n < 0 || n > k;
  if (!bad) {
    const long long cap = (long long)max_blocks * kPage;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const int pos = positions[(size_t)b * k + i];
      if (pos < 0 || pos >= cap) {
        bad = true;
      } else {
        const int page = bt[(size_t)b * max_blocks + pos / kPage];
        if (page < 0 || page >= num_pages) bad = true;
      }
    }
  }
  if (bad) g_table_fault = 1;
}

hipError_t read_fault(hipStream_t s, bool* bad) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int fault = 0;
  e = hipMemcpyFromSymbolAsync(&fault, HIP_SYMBOL(g_table_fault), sizeof(int), 0, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess) *bad = fault != 0;
  return e;
}

}  // namespace

hipError_t check_positions(const int32_t* block_table, int max_blocks, const int32_t* positions,
                           const int32_t* counts, int batch, int k, int num_pages, hipStream_t s, bool* bad) {
  *bad = false;
  hipLaunchKernelGGL(reset_fault_kernel, dim3(1), dim3(1), 0, s);
  hipLaunchKernelGGL(check_positions_kernel, dim3(batch), dim3(64), 0, s, block_table, max_blocks, positions,
                     counts, k, num_pages);
  return read_fault(s, bad);
}

hipError_t check_tables(const int32_t* block_table, int max_blocks, const int32_t* lens, int batch,
                        int num_pages, bool append, hipStream_t s, bool* bad) {
  *bad = false;
  hipLaunchKernelGGL(reset_fault_kernel, dim3(1), dim3(1), 0, s);
  hipLaunchKernelGGL(check_table_kernel, dim3(batch), dim3(64), 0, s, block_table, max_blocks, lens,
                     num_pages, append ? 1 : 0);
  return read_fault(s, bad);
}

}  // namespace mla
