// C ABI of libmla: host-side validation, workspace sizing and dispatch.  No device code here;
// every check runs before any HIP call, so argument errors are reported without a GPU.
#include "../../include/mla.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "mla_internal.h"

namespace mla {

int auto_units(int batch, int heads, int max_blocks, bool f32) {
  // Enough ranges to give every compute unit work, but never more ranges than grains: pages, or
  // 32-token tiles for the 16-head matrix-core kernel, which cuts tiles.  The
  // matrix-core kernels (bf16) run one workgroup per compute unit; the fp32 debug kernel splits each
  // range further by 8-head groups, so at 16 heads it takes twice the ranges.
  long long grains_bound = (long long)batch * (long long)max_blocks;
  if (heads == 16 && !f32) grains_bound *= 2;
  long long units = (f32 && heads < 32) ? 2 * kNumCUs : kNumCUs;
  if (units > grains_bound) units = grains_bound;
  if (units < 1) units = 1;
  return (int)units;
}

// One partial result per (unit, sequence) piece.  Pieces are numbered unit + sequence, which grows
// strictly along the page order, so units + batch slots always suffice.  Then 16 bytes per sequence
// for the range of units that hold it.
size_t workspace_bytes(int batch, int heads, int units) {
  const size_t parts = ((size_t)units + (size_t)batch) * (size_t)heads;
  return parts * (size_t)kDc * sizeof(float) + parts * 2 * sizeof(float) + (size_t)batch * 4 * sizeof(int);
}

// Twenty fp32 partial rows of 576 per sequence (the split of the 5,120-long products).
size_t append_hidden_workspace_bytes(int batch) { return (size_t)batch * kAppendChunks * kRow * sizeof(float); }

bool debug_checks_enabled() {
  const char* v = getenv("MLA_DEBUG_CHECKS");
  return v && strcmp(v, "1") == 0;
}

}  // namespace mla

using namespace mla;

static bool valid_dtype(mla_dtype d) { return d == MLA_BF16 || d == MLA_F32; }
static bool valid_heads(int h) { return h == 16 || h == 32 || h == 64 || h == 128; }

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is null";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE: invalid or inconsistent size";
    case MLA_ERR_DTYPE: return "MLA_ERR_DTYPE: unknown dtype";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: page_size must be 64, heads in {16,32,64,128} (64 or 128 and bf16 for the ~6-bit cache)";
    case MLA_ERR_BLOCK_TABLE: return "MLA_ERR_BLOCK_TABLE: block table entry out of range";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: a HIP launch failed";
    case MLA_ERR_SCRATCH: return "MLA_ERR_SCRATCH: these sizes need more scratch than mla_decode_noalloc's fixed device buffer holds";
    default: return "unknown mla_status";
  }
}

int mla_abi_version(void) { return 108; }

size_t mla_decode_workspace_size(int batch, int num_heads, int max_blocks_per_seq, int num_splits,
                                 mla_dtype dtype) {
  if (batch < 0 || max_blocks_per_seq < 1 || num_splits < 0 || !valid_heads(num_heads) ||
      !valid_dtype(dtype))
    return 0;
  const int units = num_splits ? num_splits : auto_units(batch, num_heads, max_blocks_per_seq, dtype == MLA_F32);
  return workspace_bytes(batch, num_heads, units);
}

mla_status mla_cache_append(void* kv_cache, int num_pages, int page_size, const int32_t* block_table,
                            int max_blocks_per_seq, const int32_t* positions, const void* c_new,
                            const void* kpe_new, int batch, mla_dtype dtype, hipStream_t stream) {
  if (!valid_dtype(dtype)) return MLA_ERR_DTYPE;
  if (page_size != kPage) return MLA_ERR_UNSUPPORTED;
  if (batch < 0 || num_pages < 0 || max_blocks_per_seq < 1) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (num_pages < 1) return MLA_ERR_SHAPE;
  if (!kv_cache || !block_table || !positions || !c_new || !kpe_new) return MLA_ERR_NULL;
  if (debug_checks_enabled()) {
    bool bad = false;
    if (check_tables(block_table, max_blocks_per_seq, positions, batch, num_pages, true, stream, &bad) != hipSuccess)
      return MLA_ERR_HIP;
    if (bad) return MLA_ERR_BLOCK_TABLE;
  }
  hipError_t e = launch_append(kv_cache, block_table, max_blocks_per_seq, positions, c_new, kpe_new,
                               batch, dtype == MLA_F32, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

size_t mla_cache_append_hidden_workspace_size(int batch, mla_dtype dtype) {
  if (batch < 0 || !valid_dtype(dtype)) return 0;
  return append_hidden_workspace_bytes(batch);
}

mla_status mla_cache_append_hidden(void* kv_cache, int num_pages, int page_size, const int32_t* block_table,
                                   int max_blocks_per_seq, const int32_t* positions, const void* hidden,
                                   const void* w_dkv, const void* w_kr, float rope_base, int batch,
                                   void* workspace, size_t workspace_bytes_given, mla_dtype dtype,
                                   hipStream_t stream) {
  if (!valid_dtype(dtype)) return MLA_ERR_DTYPE;
  if (page_size != kPage) return MLA_ERR_UNSUPPORTED;
  if (batch < 0 || num_pages < 0 || max_blocks_per_seq < 1) return MLA_ERR_SHAPE;
  if (!(rope_base > 1.0f) || !isfinite(rope_base)) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (num_pages < 1) return MLA_ERR_SHAPE;
  if (!kv_cache || !block_table || !positions || !hidden || !w_dkv || !w_kr) return MLA_ERR_NULL;
  if (!workspace || workspace_bytes_given < append_hidden_workspace_bytes(batch)) return MLA_ERR_WORKSPACE;
  if (debug_checks_enabled()) {
    bool bad = false;
    if (check_tables(block_table, max_blocks_per_seq, positions, batch, num_pages, true, stream, &bad) != hipSuccess)
      return MLA_ERR_HIP;
    if (bad) return MLA_ERR_BLOCK_TABLE;
  }
  hipError_t e = launch_append_hidden(kv_cache, block_table, max_blocks_per_seq, positions, hidden, w_dkv,
                                      w_kr, (double)rope_base, batch, static_cast<float*>(workspace),
                                      dtype == MLA_F32, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_absorb_q(const void* q, const void* w_uk, void* q_abs, int batch, int num_heads,
                        mla_dtype dtype, hipStream_t stream) {
  if (!valid_dtype(dtype)) return MLA_ERR_DTYPE;
  if (batch < 0) return MLA_ERR_SHAPE;
  if (!valid_heads(num_heads)) return MLA_ERR_UNSUPPORTED;
  if (batch == 0) return MLA_OK;
  if (!q || !w_uk || !q_abs) return MLA_ERR_NULL;
  hipError_t e = launch_absorb(q, w_uk, q_abs, batch, num_heads, dtype == MLA_F32, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_out_proj(const void* o_lat, const void* w_uv, void* out, int batch, int num_heads,
                        mla_dtype dtype, hipStream_t stream) {
  if (!valid_dtype(dtype)) return MLA_ERR_DTYPE;
  if (batch < 0) return MLA_ERR_SHAPE;
  if (!valid_heads(num_heads)) return MLA_ERR_UNSUPPORTED;
  if (batch == 0) return MLA_OK;
  if (!o_lat || !w_uv || !out) return MLA_ERR_NULL;
  hipError_t e = launch_out_proj(o_lat, w_uv, out, batch, num_heads, dtype == MLA_F32, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

// workspace == nullptr with noalloc: the library's fixed scratch array stands in for the workspace.
static mla_status decode_common(const void* q_abs, const void* kv_cache, int num_pages, int page_size,
                                const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                                int batch, int num_heads, float softmax_scale, void* o_lat, float* lse,
                                void* workspace, size_t workspace_bytes_given, int num_splits, mla_dtype dtype,
                                bool fp6, hipStream_t stream, bool noalloc = false) {
  if (!valid_dtype(dtype)) return MLA_ERR_DTYPE;
  if (page_size != kPage) return MLA_ERR_UNSUPPORTED;
  if (!valid_heads(num_heads)) return MLA_ERR_UNSUPPORTED;
  if (fp6 && (dtype != MLA_BF16 || num_heads < 64)) return MLA_ERR_UNSUPPORTED;
  if (batch < 0 || num_pages < 0 || max_blocks_per_seq < 1 || num_splits < 0) return MLA_ERR_SHAPE;
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!q_abs || !kv_cache || !block_table || !seq_lens || !o_lat) return MLA_ERR_NULL;
  const int units = num_splits ? num_splits : auto_units(batch, num_heads, max_blocks_per_seq, dtype == MLA_F32);
  const size_t need = workspace_bytes(batch, num_heads, units);
  if (noalloc) {
    if (need > kNoAllocScratchBytes) return MLA_ERR_SCRATCH;
    if (noalloc_scratch(&workspace) != hipSuccess) return MLA_ERR_HIP;
  } else if (!workspace || workspace_bytes_given < need) {
    return MLA_ERR_WORKSPACE;
  }
  if (debug_checks_enabled()) {
    bool bad = false;
    if (check_tables(block_table, max_blocks_per_seq, seq_lens, batch, num_pages, false, stream, &bad) != hipSuccess)
      return MLA_ERR_HIP;
    if (bad) return MLA_ERR_BLOCK_TABLE;
  }

  DecodeParams p;
  p.q_abs = q_abs;
  p.cache = static_cast<const uint16_t*>(kv_cache);
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.o_lat = o_lat;
  p.lse = lse;
  p.ws_o = static_cast<float*>(workspace);
  p.ws_ml = p.ws_o + ((size_t)units + batch) * num_heads * kDc;
  p.seq_units = reinterpret_cast<int*>(p.ws_ml + ((size_t)units + batch) * num_heads * 2);
  p.fp6 = fp6 ? 1 : 0;
  p.positions = nullptr;
  p.pos_stride = 0;
  p.num_pages = num_pages;
  p.max_blocks = max_blocks_per_seq;
  p.batch = batch;
  p.heads = num_heads;
  p.num_units = units;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.partial_bf16 = 0;  // chosen with the kernel in launch_decode
  hipError_t e = launch_decode(p, dtype == MLA_F32, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_decode(const void* q_abs, const void* kv_cache, int num_pages, int page_size,
                      const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                      int batch, int num_heads, float softmax_scale, void* o_lat, float* lse,
                      void* workspace, size_t workspace_bytes_given, int num_splits, mla_dtype dtype,
                      hipStream_t stream) {
  return decode_common(q_abs, kv_cache, num_pages, page_size, block_table, max_blocks_per_seq, seq_lens, batch,
                       num_heads, softmax_scale, o_lat, lse, workspace, workspace_bytes_given, num_splits, dtype,
                       false, stream);
}

// Paths that merge into o_lat before projecting (the fp32 debug mode, and bf16 at 16 heads where the
// vector-ALU decode leaves fp32 pieces) keep o_lat behind the decode's workspace when the caller
// passes none: room for it in fp32.
static size_t decode_out_proj_extra(int batch, int num_heads, mla_dtype) {
  return (size_t)batch * num_heads * kDc * sizeof(float);
}

size_t mla_decode_out_proj_workspace_size(int batch, int num_heads, int max_blocks_per_seq, int num_splits,
                                          mla_dtype dtype) {
  const size_t base = mla_decode_workspace_size(batch, num_heads, max_blocks_per_seq, num_splits, dtype);
  return base ? base + decode_out_proj_extra(batch, num_heads, dtype) : 0;
}

mla_status mla_decode_out_proj(const void* q_abs, const void* kv_cache, int num_pages, int page_size,
                               const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                               int batch, int num_heads, float softmax_scale, const void* w_uv, void* out,
                               void* o_lat, float* lse, void* workspace, size_t workspace_bytes_given,
                               int num_splits, mla_dtype dtype, hipStream_t stream) {
  if (!valid_dtype(dtype)) return MLA_ERR_DTYPE;
  if (page_size != kPage) return MLA_ERR_UNSUPPORTED;
  if (!valid_heads(num_heads)) return MLA_ERR_UNSUPPORTED;
  if (batch < 0 || num_pages < 0 || max_blocks_per_seq < 1 || num_splits < 0) return MLA_ERR_SHAPE;
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!q_abs || !kv_cache || !block_table || !seq_lens || !w_uv || !out) return MLA_ERR_NULL;
  const int units = num_splits ? num_splits : auto_units(batch, num_heads, max_blocks_per_seq, dtype == MLA_F32);
  const size_t base = workspace_bytes(batch, num_heads, units);
  if (!workspace || workspace_bytes_given < base + decode_out_proj_extra(batch, num_heads, dtype))
    return MLA_ERR_WORKSPACE;
  if (debug_checks_enabled()) {
    bool bad = false;
    if (check_tables(block_table, max_blocks_per_seq, seq_lens, batch, num_pages, false, stream, &bad) != hipSuccess)
      return MLA_ERR_HIP;
    if (bad) return MLA_ERR_BLOCK_TABLE;
  }
  DecodeParams p;
  p.q_abs = q_abs;
  p.cache = static_cast<const uint16_t*>(kv_cache);
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.o_lat = o_lat;
  p.lse = lse;
  p.ws_o = static_cast<float*>(workspace);
  p.ws_ml = p.ws_o + ((size_t)units + batch) * num_heads * kDc;
  p.seq_units = reinterpret_cast<int*>(p.ws_ml + ((size_t)units + batch) * num_heads * 2);
  p.fp6 = 0;
  p.positions = nullptr;
  p.pos_stride = 0;
  p.num_pages = num_pages;
  p.max_blocks = max_blocks_per_seq;
  p.batch = batch;
  p.heads = num_heads;
  p.num_units = units;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.partial_bf16 = 0;
  hipError_t e;
  const bool f32 = dtype == MLA_F32;
  if (f32 || !mfma_supported(p) || !merge_out_proj_supported(p)) {  // the two calls in turn
    if (!p.o_lat) p.o_lat = static_cast<char*>(workspace) + base;
    e = launch_decode(p, f32, stream);
    if (e == hipSuccess) e = launch_out_proj(p.o_lat, w_uv, out, batch, num_heads, f32, stream);
  } else {  // the matrix-core decode's bf16 pieces, merged and projected in one kernel
    e = launch_decode_pieces(p, false, stream);
    if (e == hipSuccess) e = launch_merge_out_proj(p, w_uv, out, stream);
  }
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

size_t mla_decode_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

mla_status mla_calibrate_mfma(float* out, int blocks, int iters, hipStream_t stream) {
  if (!out) return MLA_ERR_NULL;
  if (blocks < 1 || iters < 1) return MLA_ERR_SHAPE;
  return launch_mfma_rate(out, blocks, iters, stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_calibrate_read(const void* buf, size_t bytes, int* out, int blocks, hipStream_t stream) {
  if (!buf || !out) return MLA_ERR_NULL;
  if (blocks < 1 || bytes == 0 || bytes % (36 * 1024) != 0) return MLA_ERR_SHAPE;
  return launch_read_rate(buf, bytes, out, blocks, stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_decode_noalloc(const void* q_abs, const void* kv_cache, int num_pages, int page_size,
                              const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                              int batch, int num_heads, float softmax_scale, void* o_lat, float* lse,
                              int num_splits, mla_dtype dtype, hipStream_t stream) {
  return decode_common(q_abs, kv_cache, num_pages, page_size, block_table, max_blocks_per_seq, seq_lens, batch,
                       num_heads, softmax_scale, o_lat, lse, nullptr, 0, num_splits, dtype, false, stream, true);
}

mla_status mla_decode_fp6(const void* q_abs, const void* kv_cache6, int num_pages, int page_size,
                          const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                          int batch, int num_heads, float softmax_scale, void* o_lat, float* lse,
                          void* workspace, size_t workspace_bytes_given, int num_splits, mla_dtype dtype,
                          hipStream_t stream) {
  return decode_common(q_abs, kv_cache6, num_pages, page_size, block_table, max_blocks_per_seq, seq_lens, batch,
                       num_heads, softmax_scale, o_lat, lse, workspace, workspace_bytes_given, num_splits, dtype,
                       true, stream);
}

mla_status mla_cache_append_fp6(void* kv_cache6, int num_pages, int page_size, const int32_t* block_table,
                                int max_blocks_per_seq, const int32_t* positions, const void* c_new,
                                const void* kpe_new, int batch, mla_dtype dtype, hipStream_t stream) {
  if (!valid_dtype(dtype)) return MLA_ERR_DTYPE;
  if (page_size != kPage) return MLA_ERR_UNSUPPORTED;
  if (batch < 0 || num_pages < 0 || max_blocks_per_seq < 1) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (num_pages < 1) return MLA_ERR_SHAPE;
  if (!kv_cache6 || !block_table || !positions || !c_new || !kpe_new) return MLA_ERR_NULL;
  if (debug_checks_enabled()) {
    bool bad = false;
    if (check_tables(block_table, max_blocks_per_seq, positions, batch, num_pages, true, stream, &bad) != hipSuccess)
      return MLA_ERR_HIP;
    if (bad) return MLA_ERR_BLOCK_TABLE;
  }
  hipError_t e = launch_append_fp6(kv_cache6, block_table, max_blocks_per_seq, positions, c_new, kpe_new, batch,
                                   dtype == MLA_F32, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_cache_quantize_fp6(const void* kv_cache, void* kv_cache6, int num_pages, int page_size,
                                  hipStream_t stream) {
  if (page_size != kPage) return MLA_ERR_UNSUPPORTED;
  if (num_pages < 0) return MLA_ERR_SHAPE;
  if (num_pages == 0) return MLA_OK;
  if (!kv_cache || !kv_cache6) return MLA_ERR_NULL;
  hipError_t e = launch_quantize_pages_fp6(kv_cache, kv_cache6, num_pages, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

size_t mla_out_proj_hidden_workspace_size(int batch, int num_heads, mla_dtype dtype) {
  if (batch < 0 || !valid_heads(num_heads) || !valid_dtype(dtype)) return 0;
  return dtype == MLA_F32 ? 0 : out_proj_hidden_workspace_bytes(batch, num_heads);
}

mla_status mla_out_proj_hidden(const void* out, const void* w_o, void* hidden, int batch, int num_heads,
                               void* workspace, size_t workspace_bytes_given, mla_dtype dtype,
                               hipStream_t stream) {
  if (!valid_dtype(dtype)) return MLA_ERR_DTYPE;
  if (batch < 0) return MLA_ERR_SHAPE;
  if (!valid_heads(num_heads)) return MLA_ERR_UNSUPPORTED;
  if (batch == 0) return MLA_OK;
  if (!out || !w_o || !hidden) return MLA_ERR_NULL;
  const bool f32 = dtype == MLA_F32;
  if (!f32 && (!workspace || workspace_bytes_given < out_proj_hidden_workspace_bytes(batch, num_heads)))
    return MLA_ERR_WORKSPACE;
  hipError_t e = launch_out_proj_hidden(out, w_o, hidden, batch, num_heads, static_cast<float*>(workspace), f32,
                                        stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

size_t mla_index_topk_workspace_size(int batch, int max_blocks_per_seq) {
  if (batch < 0 || max_blocks_per_seq < 1) return 0;
  return index_topk_workspace_bytes(batch, max_blocks_per_seq);
}

mla_status mla_index_topk(const int8_t* index_cache, int num_pages, int page_size, const int32_t* block_table,
                          int max_blocks_per_seq, const int32_t* seq_lens, const int8_t* q_index, int batch, int k,
                          int32_t* positions, int32_t* counts, void* workspace, size_t workspace_bytes_given,
                          hipStream_t stream) {
  if (page_size != kPage) return MLA_ERR_UNSUPPORTED;
  if (batch < 0 || num_pages < 0 || max_blocks_per_seq < 1 || k < 1) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!index_cache || !block_table || !seq_lens || !q_index || !positions || !counts) return MLA_ERR_NULL;
  if (!workspace || workspace_bytes_given < index_topk_workspace_bytes(batch, max_blocks_per_seq))
    return MLA_ERR_WORKSPACE;
  if (debug_checks_enabled()) {
    bool bad = false;
    if (check_tables(block_table, max_blocks_per_seq, seq_lens, batch, num_pages, false, stream, &bad) != hipSuccess)
      return MLA_ERR_HIP;
    if (bad) return MLA_ERR_BLOCK_TABLE;
  }
  hipError_t e = launch_index_topk(index_cache, block_table, max_blocks_per_seq, seq_lens, q_index, batch, k,
                                   positions, counts, workspace, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_gather_rows(const void* kv_cache, int num_pages, int page_size, const int32_t* block_table,
                           int max_blocks_per_seq, const int32_t* positions, const int32_t* counts, int batch,
                           int k, void* out_cache, int32_t* out_block_table, hipStream_t stream) {
  if (page_size != kPage) return MLA_ERR_UNSUPPORTED;
  if (batch < 0 || num_pages < 0 || max_blocks_per_seq < 1 || k < 1) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!kv_cache || !block_table || !positions || !counts || !out_cache || !out_block_table) return MLA_ERR_NULL;
  if (debug_checks_enabled()) {
    bool bad = false;
    if (check_positions(block_table, max_blocks_per_seq, positions, counts, batch, k, num_pages, stream, &bad) !=
        hipSuccess)
      return MLA_ERR_HIP;
    if (bad) return MLA_ERR_BLOCK_TABLE;
  }
  hipError_t e = launch_gather_rows(kv_cache, block_table, max_blocks_per_seq, positions, counts, batch, k, out_cache,
                                    out_block_table, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

size_t mla_decode_topk_workspace_size(int batch, int num_heads, int k) {
  if (batch < 0 || k < 1 || !valid_heads(num_heads)) return 0;
  const int kept_pages = (int)(((long long)k + kPage - 1) / kPage);
  return workspace_bytes(batch, num_heads, auto_units(batch, num_heads, kept_pages, false));
}

mla_status mla_decode_topk(const void* q_abs, const void* kv_cache, int num_pages, int page_size,
                           const int32_t* block_table, int max_blocks_per_seq, const int32_t* positions,
                           const int32_t* counts, int batch, int k, int num_heads, float softmax_scale,
                           void* o_lat, float* lse, void* workspace, size_t workspace_bytes_given,
                           hipStream_t stream) {
  if (page_size != kPage) return MLA_ERR_UNSUPPORTED;
  if (!valid_heads(num_heads)) return MLA_ERR_UNSUPPORTED;
  if (batch < 0 || num_pages < 0 || max_blocks_per_seq < 1 || k < 1) return MLA_ERR_SHAPE;
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (num_pages < 1) return MLA_ERR_SHAPE;
  if (!q_abs || !kv_cache || !block_table || !positions || !counts || !o_lat) return MLA_ERR_NULL;
  const int kept_pages = (int)(((long long)k + kPage - 1) / kPage);
  const int units = auto_units(batch, num_heads, kept_pages, false);
  const size_t need = workspace_bytes(batch, num_heads, units);
  if (!workspace || workspace_bytes_given < need) return MLA_ERR_WORKSPACE;
  if (debug_checks_enabled()) {
    bool bad = false;
    if (check_positions(block_table, max_blocks_per_seq, positions, counts, batch, k, num_pages, stream, &bad) !=
        hipSuccess)
      return MLA_ERR_HIP;
    if (bad) return MLA_ERR_BLOCK_TABLE;
  }

  DecodeParams p;
  p.q_abs = q_abs;
  p.cache = static_cast<const uint16_t*>(kv_cache);
  p.block_table = block_table;
  p.seq_lens = counts;  // each sequence's list of kept tokens is what it attends to
  p.o_lat = o_lat;
  p.lse = lse;
  p.ws_o = static_cast<float*>(workspace);
  p.ws_ml = p.ws_o + ((size_t)units + batch) * num_heads * kDc;
  p.seq_units = reinterpret_cast<int*>(p.ws_ml + ((size_t)units + batch) * num_heads * 2);
  p.fp6 = 0;
  p.positions = positions;
  p.pos_stride = k;
  p.num_pages = num_pages;
  p.max_blocks = max_blocks_per_seq;
  p.batch = batch;
  p.heads = num_heads;
  p.num_units = units;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.partial_bf16 = 0;
  hipError_t e = launch_decode(p, false, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
