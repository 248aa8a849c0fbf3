// Internal interface between the C-ABI layer (mla_api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

constexpr int kDc = 512;      // latent width
constexpr int kDr = 64;       // decoupled RoPE width
constexpr int kDnope = 128;   // per-head content query/key width
constexpr int kDv = 128;      // per-head value width
constexpr int kRow = 576;     // cached numbers per token
constexpr int kQdim = 192;    // [q_nope | q_pe]
constexpr int kPage = 64;     // tokens per page
constexpr int kNumCUs = 256;  // MI355X compute units (used only to pick the automatic split)
constexpr int kAppendChunks = 20;  // 5,120 / 256: partial sums per output of the producer products
constexpr int kFp6RowBytes = kRow * 6 / 8;                       // 432: a row of 6-bit codes
constexpr int kFp6PageBytes = kPage * kFp6RowBytes + kPage * 4;  // 27,904: rows, then fp32 scales
constexpr size_t kNoAllocScratchBytes = (size_t)128 << 20;       // mla_decode_noalloc's fixed scratch

// Everything a decode launch needs.  Pointers are device pointers.
struct DecodeParams {
  const void* q_abs;
  const uint16_t* cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* o_lat;
  float* lse;          // may be null
  float* ws_o;         // [units + batch][heads][512] fp32 slots of the partial outputs
  float* ws_ml;        // [units + batch][heads][2] fp32 (base-2 reference max, softmax sum)
  int* seq_units;      // [batch][4]: first unit, last unit, every unit holds a page (1 / 0), unused;
                       // written by the matrix-core kernel, which sets it (null: the merges
                       // derive the unit range from seq_lens)
  int partial_bf16;    // 0: fp32 un-normalised sums; 1: bf16 sums already divided by the
                       // softmax sum, in the first half of each slot (set by launch_decode)
  int fp6;            // 1: cache holds ~6-bit pages (kFp6PageBytes each), 0: bf16 rows
  // Attention over kept tokens in place (null: every token): sequence b attends to the tokens at
  // positions[b * pos_stride + i], i < seq_lens[b] (here the kept counts), each read through the
  // block table; its pages are then runs of 64 list entries.
  const int32_t* positions;
  int pos_stride;
  int num_pages;
  int max_blocks;
  int batch;
  int heads;
  int num_units;
  float scale_log2;    // softmax_scale * log2(e)
};

int auto_units(int batch, int heads, int max_blocks, bool f32);
size_t workspace_bytes(int batch, int heads, int units);

// Launchers: return hipSuccess or the launch error.
hipError_t launch_append(void* cache, const int32_t* block_table, int max_blocks,
                         const int32_t* positions, const void* c_new, const void* kpe_new,
                         int batch, bool f32, hipStream_t s);
hipError_t launch_absorb(const void* q, const void* w_uk, void* q_abs, int batch, int heads,
                         bool f32, hipStream_t s);
hipError_t launch_out_proj(const void* o_lat, const void* w_uv, void* out, int batch, int heads,
                           bool f32, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, bool f32, hipStream_t s);
// The bf16 matrix-core decode handles these sizes (the rest run on the vector-ALU kernel).
bool mfma_supported(const DecodeParams& p);
// The decode kernel alone: leaves each piece in the workspace (p.partial_bf16 and p.seq_units set
// to what the kernel wrote) for a merge to finish.
hipError_t launch_decode_pieces(DecodeParams& p, bool f32, hipStream_t s);
// Merge of the pieces and the W_UV projection in one kernel (bf16): out [B][H][128], o_lat and lse
// written when non-null.  Heads must be a multiple of 8.
hipError_t launch_merge_out_proj(const DecodeParams& p, const void* w_uv, void* out, hipStream_t s);
bool merge_out_proj_supported(const DecodeParams& p);
// Producer side: rows [h W_DKV | RoPE(h W_KR)] written at positions[b]; part is the fp32 workspace
// of append_hidden_workspace_bytes(batch).
hipError_t launch_append_hidden(void* cache, const int32_t* block_table, int max_blocks,
                                const int32_t* positions, const void* hidden, const void* w_dkv,
                                const void* w_kr, double rope_base, int batch, float* part, bool f32,
                                hipStream_t s);
size_t append_hidden_workspace_bytes(int batch);
// ~6-bit cache: quantize and write one row per sequence; quantize whole bf16 pages.
hipError_t launch_append_fp6(void* cache, const int32_t* block_table, int max_blocks,
                             const int32_t* positions, const void* c_new, const void* kpe_new, int batch,
                             bool f32, hipStream_t s);
hipError_t launch_quantize_pages_fp6(const void* src, void* dst, int num_pages, hipStream_t s);
// Output projection to the hidden width: hidden [B][5120] = out [B][heads * 128] @ W^O; part is the
// fp32 workspace of out_proj_hidden_workspace_bytes(batch, heads) (heads >= 16).
hipError_t launch_out_proj_hidden(const void* out, const void* w_o, void* hidden, int batch, int heads,
                                  float* part, bool f32, hipStream_t s);
size_t out_proj_hidden_workspace_bytes(int batch, int heads);
// Top-k over a cheap int8 index and the gather of the kept rows into compact pages.
hipError_t launch_index_topk(const int8_t* index_cache, const int32_t* block_table, int max_blocks,
                             const int32_t* seq_lens, const int8_t* q_index, int batch, int k, int32_t* positions,
                             int32_t* counts, void* workspace, hipStream_t s);
hipError_t launch_gather_rows(const void* cache, const int32_t* block_table, int max_blocks,
                              const int32_t* positions, const int32_t* counts, int batch, int k, void* out,
                              int32_t* out_bt, hipStream_t s);
size_t index_topk_workspace_bytes(int batch, int max_blocks);

// Device-side check of kept-token lists: counts[b] in [0, k], every listed position inside the
// table row and naming a page in [0, num_pages); synchronises s.
hipError_t check_positions(const int32_t* block_table, int max_blocks, const int32_t* positions,
                           const int32_t* counts, int batch, int k, int num_pages, hipStream_t s, bool* bad);
// Device-side check of block-table entries and lengths (append = false) or append positions
// (append = true); synchronises s.  *bad is set when an entry is out of range.
hipError_t check_tables(const int32_t* block_table, int max_blocks, const int32_t* lens, int batch,
                        int num_pages, bool append, hipStream_t s, bool* bad);
// Matrix-core rate kernel: `blocks` workgroups of four waves, each wave `iters` x 4 independent
// v_mfma_f32_32x32x16_bf16; out holds one float per wave (blocks * 4).
hipError_t launch_mfma_rate(float* out, int blocks, int iters, hipStream_t s);
hipError_t launch_read_rate(const void* buf, size_t bytes, int* out, int blocks, hipStream_t s);
// Device address of this device's fixed scratch array (kNoAllocScratchBytes), looked up on the first
// call on each device; allocates nothing.
hipError_t noalloc_scratch(void** out);
// MLA_DEBUG_CHECKS=1 in the environment, read at every call.
bool debug_checks_enabled();

}  // namespace mla
