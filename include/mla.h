/*
 * mla.h -- C ABI of libmla: Multi-head Latent Attention (MLA) decode over a paged latent cache,
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (DeepSeek-V2, as the "DeepSeek-V2" explainer on aiany.app lays it out):
 *   - Step 5, eq. 9: every token leaves one latent note c (d_c = 512 numbers) per layer; per-head
 *     keys and values are functions of it, k_h = W_UK[h] c and v_h = W_UV[h]^T c.
 *   - Step 6: a score q_nope . k_h equals (W_UK[h]^T q_nope) . c, so the query is moved into latent
 *     space once and the keys are never built; W_UV is applied after the weighted sum.
 *   - Step 7: position rides a separate 64-number rotated key k^R shared by all heads, scored by a
 *     per-head 64-number q^R; the two scores add inside the softmax.
 *   - Step 8: the cache therefore holds 512 + 64 = 576 numbers per token per layer.
 * The pages give no API; the arguments below follow the problem as posed there: a cache of
 * per-token notes plus RoPE strips, addressed through a block table, per-sequence lengths and a
 * softmax scale.
 *
 * Fixed sizes: d_c = 512, d_R = 64, d_nope = d_v = 128, cache row = 576, page = 64 tokens.
 *
 * Layouts (all row-major, all device memory owned by the caller):
 *   kv_cache     bf16 [num_pages][64][576]; row = [c (512) | k^R (64)], 1152 bytes
 *   block_table  int32 [batch][max_blocks_per_seq]; token t of sequence b lives in page
 *                block_table[b][t / 64], slot t % 64.  Entries for blocks a sequence does not use
 *                are never read (any value, -1 by convention).
 *   q            [batch][heads][192] = [q_nope (128) | q^R (64)]; q^R and k^R arrive rotated
 *   w_uk         [heads][128][512]  (k_h = W_UK[h] c)
 *   w_uv         [heads][512][128]  (v_h = c^T W_UV[h])
 *   q_abs        [batch][heads][576] = [W_UK[h]^T q_nope | q^R]
 *   o_lat        [batch][heads][512] = sum_t p_t c_t
 *   out          [batch][heads][128] = o_lat W_UV[h]
 *   lse          fp32 [batch][heads]: natural log of sum_t exp(scale * q_abs . row_t)
 * Element type of q, w_uk, w_uv, q_abs, o_lat, out, c_new, kpe_new: bf16 for MLA_BF16, fp32 for
 * MLA_F32 (a debug mode with fp32 intermediates; the cache stays bf16 in both modes).
 *
 * Conventions:
 *   - Every call is asynchronous on the caller's stream (0 = the null stream).  The library never
 *     synchronises and never allocates; scratch memory comes from a caller workspace (for
 *     mla_decode_noalloc, from a fixed device array inside the library).
 *   - Every entry point validates its arguments on the host before launching anything and returns a
 *     negative mla_status on error, without touching any buffer.  Launch failures are reported as
 *     MLA_ERR_HIP.  Nothing is thrown across the ABI.
 *   - Device-side contents (block-table entries, lengths, positions, kept counts) are trusted: an
 *     entry outside [0, num_pages) or a length above max_blocks_per_seq * 64 is undefined
 *     behaviour.  With the environment variable MLA_DEBUG_CHECKS=1 (read at every call), every
 *     call that reads the block table (the appends, the decodes, mla_index_topk, mla_gather_rows)
 *     first checks on the device every entry it would use, synchronises the stream to read the
 *     verdict, and returns MLA_ERR_BLOCK_TABLE, launching nothing else, if one is out of range.
 *   - Calls that share a workspace must be ordered on one stream.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,         /* a required pointer is null */
  MLA_ERR_SHAPE = -2,        /* a size is negative, zero where it must not be, or inconsistent */
  MLA_ERR_DTYPE = -3,        /* unknown mla_dtype */
  MLA_ERR_WORKSPACE = -4,    /* workspace missing or smaller than mla_decode_workspace_size() */
  MLA_ERR_UNSUPPORTED = -5,  /* page_size != 64, or heads not in {16, 32, 64, 128} */
  MLA_ERR_BLOCK_TABLE = -6,  /* device-side check (MLA_DEBUG_CHECKS=1): bad table entry or length */
  MLA_ERR_HIP = -7,          /* a HIP launch failed */
  MLA_ERR_SCRATCH = -8       /* mla_decode_noalloc: the sizes need more than its fixed scratch buffer */
} mla_status;

typedef enum { MLA_BF16 = 0, MLA_F32 = 1 } mla_dtype;

#define MLA_D_C 512
#define MLA_D_R 64
#define MLA_D_NOPE 128
#define MLA_D_V 128
#define MLA_ROW 576
#define MLA_PAGE_SIZE 64

/* Human-readable name of a status code; never null. */
const char* mla_status_string(int status);

/* ABI version of this header (major * 100 + minor). */
int mla_abi_version(void);

/*
 * Bytes of workspace mla_decode needs for these sizes (0 on invalid arguments).
 * num_splits is the number of work units the batch's tokens are cut into (0 = automatic: the value
 * mla_decode would choose): equal page ranges, or with at least 8 tiles of 32 tokens per unit, tile
 * ranges cut so that a unit that starts another sequence holds fewer tiles.  At 16 heads (bf16) the
 * units are equal ranges of 32-token tiles, at most one unit per tile.  The result does not depend
 * on the sequence lengths.
 */
size_t mla_decode_workspace_size(int batch, int num_heads, int max_blocks_per_seq, int num_splits,
                                 mla_dtype dtype);

/*
 * Append one token per sequence to the paged cache (explainer Step 2: the note of a token already
 * read never changes, so it is stored once; Step 8: the stored row is [c | k^R]).
 * For each b: row [c_new[b] (512) | kpe_new[b] (64)] is copied bit for bit to logical position
 * positions[b] (the length before the append): page block_table[b][positions[b] / 64], slot
 * positions[b] % 64.  c_new / kpe_new are bf16 for MLA_BF16 and fp32 holding bf16-representable
 * values for MLA_F32 (their low 16 bits must then be zero; they are dropped).  seq_lens is not
 * touched: the caller adds one after the append.  Sequences appending to the same page slot race.
 */
mla_status mla_cache_append(void* kv_cache, int num_pages, int page_size, const int32_t* block_table,
                            int max_blocks_per_seq, const int32_t* positions, const void* c_new,
                            const void* kpe_new, int batch, mla_dtype dtype, hipStream_t stream);

/*
 * The producer side of the cache (explainer Step 5, eq. 9: the hidden vector is squeezed to the
 * latent note c = W^DKV h, 5,120 -> 512; Step 7: the token also contributes one 64-dim key k^R,
 * rotated by its position and shared by all heads).  For each b, with p = positions[b] (the length
 * before the append), the row [hidden[b] @ w_dkv (512) | RoPE_p(hidden[b] @ w_kr) (64)] is rounded
 * to bf16 (nearest even) and written to page block_table[b][p / 64], slot p % 64.
 *   hidden  [batch][5120], w_dkv [5120][512], w_kr [5120][64]: bf16 for MLA_BF16 (fp32 accumulation),
 *           fp32 arrays holding bf16-representable values for MLA_F32 (fp32 arithmetic throughout).
 *   RoPE_p  (a reading: the pages give neither frequencies nor pairing) turns pair (2i, 2i + 1) by
 *           p * rope_base^(-2i / 64) radians, computed in double precision; rope_base > 1 (10000 is
 *           the plain rotary choice), no context-extension rescaling.
 *   workspace: at least mla_cache_append_hidden_workspace_size(batch, dtype) bytes of device
 *           memory, contents irrelevant, used only during the call (stream-ordered).
 * Errors as mla_cache_append, plus MLA_ERR_SHAPE for a bad rope_base and MLA_ERR_WORKSPACE.  With
 * MLA_DEBUG_CHECKS=1 the positions and table entries are checked as for mla_cache_append.
 */
size_t mla_cache_append_hidden_workspace_size(int batch, mla_dtype dtype);
mla_status mla_cache_append_hidden(void* kv_cache, int num_pages, int page_size, const int32_t* block_table,
                                   int max_blocks_per_seq, const int32_t* positions, const void* hidden,
                                   const void* w_dkv, const void* w_kr, float rope_base, int batch,
                                   void* workspace, size_t workspace_bytes, mla_dtype dtype,
                                   hipStream_t stream);

/*
 * Absorb the content query into latent space (explainer Step 6):
 *   q_abs[b][h][0:512]   = q[b][h][0:128] @ W_UK[h]     (fp32 accumulation)
 *   q_abs[b][h][512:576] = q[b][h][128:192]             (q^R passes through, explainer Step 7)
 */
mla_status mla_absorb_q(const void* q, const void* w_uk, void* q_abs, int batch, int num_heads,
                        mla_dtype dtype, hipStream_t stream);

/*
 * Decode attention in latent space for one query per sequence, all heads (explainer Steps 6-7):
 *   s_t   = softmax_scale * (q_abs[b][h] . row_t),  t = 0 .. seq_lens[b]-1   (576-long dot)
 *   o_lat = sum_t softmax(s)_t * c_t                                          (512 wide)
 *   lse   = log sum_t exp(s_t)                                                (natural log)
 * The tokens of all sequences are cut into num_splits ranges (0 = automatic; the cut is described at
 * mla_decode_workspace_size); each range is reduced by one workgroup and sequences cut across
 * ranges are combined with a log-sum-exp merge.
 * Results do not depend on num_splits beyond rounding; equal arguments give bit-identical results.
 * A sequence of length 0 gives o_lat = 0 and lse = -inf.  lse may be null.
 * workspace must hold mla_decode_workspace_size(batch, num_heads, max_blocks_per_seq, num_splits,
 * dtype) bytes; its contents on entry are ignored.
 */
mla_status mla_decode(const void* q_abs, const void* kv_cache, int num_pages, int page_size,
                      const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                      int batch, int num_heads, float softmax_scale, void* o_lat, float* lse,
                      void* workspace, size_t workspace_bytes, int num_splits, mla_dtype dtype,
                      hipStream_t stream);

/*
 * mla_decode and mla_out_proj in one call (explainer Step 6: the values are never built per token;
 * W_UV is applied once, after the weighted sum of the latent notes):
 *   out[b][h] = o_lat[b][h] @ W_UV[h],  o_lat as mla_decode computes it.
 * The split merge and the projection run as one kernel (bf16), so o_lat need not go through
 * memory: o_lat [batch][heads][512] and lse [batch][heads] are written only when non-null.  out
 * [batch][heads][128], w_uv [heads][512][128]; element types as for mla_decode / mla_out_proj (fp32
 * for MLA_F32, where the two run one after the other, as they do in bf16 at 16 heads).  In bf16, o_lat is rounded to bf16 before
 * the projection, as when it passes through memory between the two calls; results agree with
 * mla_decode followed by mla_out_proj within rounding.  workspace: at least
 * mla_decode_out_proj_workspace_size(...) bytes, contents on entry ignored.  Errors as mla_decode,
 * plus MLA_ERR_NULL for a null w_uv or out.
 */
size_t mla_decode_out_proj_workspace_size(int batch, int num_heads, int max_blocks_per_seq, int num_splits,
                                          mla_dtype dtype);
mla_status mla_decode_out_proj(const void* q_abs, const void* kv_cache, int num_pages, int page_size,
                               const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                               int batch, int num_heads, float softmax_scale, const void* w_uv, void* out,
                               void* o_lat, float* lse, void* workspace, size_t workspace_bytes,
                               int num_splits, mla_dtype dtype, hipStream_t stream);

/*
 * mla_decode without a workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  Arguments, results and
 * errors are those of mla_decode, minus workspace and workspace_bytes: the scratch space comes from
 * a fixed device array inside the library, mla_decode_noalloc_max_bytes() bytes (128 MiB) on every
 * GPU the library runs on, held from the moment the library's code is loaded on that GPU until the
 * process ends.  Sizes whose mla_decode_workspace_size() exceeds it return MLA_ERR_SCRATCH before
 * anything is launched (at 128 heads and the automatic split: up to 253 sequences).  The call
 * allocates nothing; its first call on a device looks up that device's array once.  Every call on
 * one GPU shares that GPU's array: calls that may overlap on one GPU (two streams, two threads)
 * race and must be ordered by the caller.  No part of the array needs to start at zero; each call
 * writes what it later reads.  Results are bit-identical to mla_decode's for equal arguments.
 */
size_t mla_decode_noalloc_max_bytes(void);
mla_status mla_decode_noalloc(const void* q_abs, const void* kv_cache, int num_pages, int page_size,
                              const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                              int batch, int num_heads, float softmax_scale, void* o_lat, float* lse,
                              int num_splits, mla_dtype dtype, hipStream_t stream);

/*
 * The ~6-bit cache (explainer, the audit after Step 8: deployed V2 keeps each cached number in about
 * six bits, near 26 KB per token over its 60 layers).  The pages give no format; the reading here:
 * every number is an FP6 E2M3 code (1 sign, 2 exponent bits with bias 1, 3 mantissa bits; magnitudes
 * 0, 1/8 .. 7/8, 1 .. 7.5; no infinity or NaN), rounded to nearest with ties to the even code, and
 * every row carries one scale 2^e, e the smallest integer >= -126 with the row's largest magnitude
 * at most 7.5 * 2^e.  A stored number is code_value * 2^e exactly.
 *   kv_cache6  uint8 [num_pages][MLA_FP6_PAGE_BYTES]: 64 rows of 432 bytes (code i of a row at bits
 *              6i .. 6i+5 of the row's little-endian bit string), then the 64 scales as float32.
 * Rows must hold finite values below 2^127 in magnitude.  436 bytes per token and layer, 37.8 % of
 * the bf16 row.
 */
#define MLA_FP6_PAGE_BYTES 27904

/*
 * mla_cache_append for the ~6-bit cache: row [c_new[b] | kpe_new[b]] is quantized as above and
 * written to logical position positions[b] of sequence b (codes and scale).  Arguments, dtypes and
 * errors as mla_cache_append.
 */
mla_status mla_cache_append_fp6(void* kv_cache6, int num_pages, int page_size, const int32_t* block_table,
                                int max_blocks_per_seq, const int32_t* positions, const void* c_new,
                                const void* kpe_new, int batch, mla_dtype dtype, hipStream_t stream);

/*
 * Quantizes every row of bf16 pages kv_cache [num_pages][64][576] into kv_cache6 [num_pages]
 * [MLA_FP6_PAGE_BYTES] (page i to page i, every slot, used or not).  MLA_ERR_UNSUPPORTED unless
 * page_size is 64; MLA_ERR_SHAPE for num_pages < 0; MLA_ERR_NULL for a null pointer.
 */
mla_status mla_cache_quantize_fp6(const void* kv_cache, void* kv_cache6, int num_pages, int page_size,
                                  hipStream_t stream);

/*
 * mla_decode over the ~6-bit cache: the same attention on the numbers the cache stores (each row
 * code_value * 2^e, converted to bf16 exactly inside the kernel).  Arguments, workspace, results
 * and errors as mla_decode, with two limits: dtype must be MLA_BF16 and num_heads 64 or 128
 * (MLA_ERR_UNSUPPORTED otherwise).
 */
mla_status mla_decode_fp6(const void* q_abs, const void* kv_cache6, int num_pages, int page_size,
                          const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                          int batch, int num_heads, float softmax_scale, void* o_lat, float* lse,
                          void* workspace, size_t workspace_bytes, int num_splits, mla_dtype dtype,
                          hipStream_t stream);

/*
 * Per-head value up-projection after the weighted sum (explainer Step 6: W_UV is applied on the
 * output side instead of to every cached token):
 *   out[b][h][:] = o_lat[b][h][:] @ W_UV[h]      (512 -> 128, fp32 accumulation)
 */
mla_status mla_out_proj(const void* o_lat, const void* w_uv, void* out, int batch, int num_heads,
                        mla_dtype dtype, hipStream_t stream);

/*
 * The attention block's output in the hidden width (explainer Step 6: the heads' outputs are
 * concatenated and mixed by W^O, with W^UV applied before it):
 *   hidden[b][:] = out[b] flattened head-major (num_heads * 128) @ W^O      (5120 wide)
 *   out     [batch][num_heads][128] (mla_out_proj's output), w_o [num_heads * 128][5120] input-major,
 *   hidden  [batch][5120]; bf16 with fp32 accumulation (MLA_BF16) or fp32 throughout (MLA_F32).
 * W^UV is not folded into W^O here: the folded per-head 512 x 5120 matrices would hold 3.6 times
 * the weight bytes of W^UV and W^O together, and decode streams every weight byte per step.
 * workspace: at least mla_out_proj_hidden_workspace_size(batch, num_heads, dtype) bytes (fp32
 * partial sums; none are needed for MLA_F32), contents irrelevant, used only during the call.
 * Errors as mla_out_proj, plus MLA_ERR_WORKSPACE.
 */
size_t mla_out_proj_hidden_workspace_size(int batch, int num_heads, mla_dtype dtype);
mla_status mla_out_proj_hidden(const void* out, const void* w_o, void* hidden, int batch, int num_heads,
                               void* workspace, size_t workspace_bytes, mla_dtype dtype, hipStream_t stream);

/*
 * Attention over the top-k tokens of a cheap index ("DeepSeek (AI)" wiki, "KV cache data movement
 * minimization": each token also carries a cheap index vector; the decode query scores them all,
 * and attention reads only the k best rows).  The pages leave the index format open; here:
 *   index_cache  int8 [num_pages][64][MLA_INDEX_DIM], paged like kv_cache (same block table)
 *   q_index      int8 [batch][MLA_INDEX_DIM]: each sequence's index query
 *   score_t      = q_index[b] . index_cache[token t], an exact integer, for t < seq_lens[b]
 * mla_index_topk keeps the k highest scores of each sequence (ties to the earlier position; all
 * tokens when seq_lens[b] <= k) and writes them to positions [batch][k] in increasing order, with
 * counts[b] = min(k, seq_lens[b]) (entries past counts[b] untouched).  workspace: at least
 * mla_index_topk_workspace_size(batch, max_blocks_per_seq) bytes (int32 scores).
 * mla_gather_rows copies the kept rows of kv_cache into compact pages: sequence b's i-th kept row
 * goes to page b * P + i / 64, slot i % 64 of out_cache [batch * P][64][576] (P = ceil(k / 64)),
 * and out_block_table [batch][P] gets b * P + j; mla_decode over (out_cache, out_block_table,
 * counts) is then the attention over the kept tokens.
 * Errors: MLA_ERR_UNSUPPORTED unless page_size is 64; MLA_ERR_SHAPE for k < 1 or bad sizes;
 * MLA_ERR_NULL, MLA_ERR_WORKSPACE (mla_index_topk); with MLA_DEBUG_CHECKS=1, MLA_ERR_BLOCK_TABLE:
 * for mla_index_topk as mla_decode, for mla_gather_rows a count above k, a position outside the
 * table row or a table entry outside [0, num_pages).
 */
#define MLA_INDEX_DIM 128
size_t mla_index_topk_workspace_size(int batch, int max_blocks_per_seq);
mla_status mla_index_topk(const int8_t* index_cache, int num_pages, int page_size, const int32_t* block_table,
                          int max_blocks_per_seq, const int32_t* seq_lens, const int8_t* q_index, int batch, int k,
                          int32_t* positions, int32_t* counts, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);
mla_status mla_gather_rows(const void* kv_cache, int num_pages, int page_size, const int32_t* block_table,
                           int max_blocks_per_seq, const int32_t* positions, const int32_t* counts, int batch,
                           int k, void* out_cache, int32_t* out_block_table, hipStream_t stream);

/*
 * Attention over the kept tokens read in place (same passage): the result of mla_gather_rows
 * followed by mla_decode over the compact pages, bit for bit, without copying the rows.  Sequence b
 * attends to the tokens at positions[b][0 .. counts[b]) (positions [batch][k] and counts [batch]
 * as mla_index_topk writes them; any token positions in list order are allowed), each row read
 * through block_table as mla_decode reads it.  counts[b] = 0 gives o_lat = 0 and lse = -inf.
 * q_abs, o_lat, lse and scale as for mla_decode; bf16 only; num_heads in {16, 32, 64, 128}.
 * workspace: at least mla_decode_topk_workspace_size(batch, num_heads, k) bytes, contents
 * irrelevant, used only during the call.  Counts and positions are trusted on the fast path; with
 * MLA_DEBUG_CHECKS=1 a count above k, a position outside the table row or a table entry outside
 * [0, num_pages) returns MLA_ERR_BLOCK_TABLE, launching nothing else.
 * Errors: MLA_ERR_UNSUPPORTED (page_size != 64, num_heads not in {16, 32, 64, 128}), MLA_ERR_SHAPE (k < 1,
 * negative sizes, num_pages < 1 with batch > 0, scale not finite and positive), MLA_ERR_NULL,
 * MLA_ERR_WORKSPACE, MLA_ERR_HIP.
 */
size_t mla_decode_topk_workspace_size(int batch, int num_heads, int k);
mla_status mla_decode_topk(const void* q_abs, const void* kv_cache, int num_pages, int page_size,
                           const int32_t* block_table, int max_blocks_per_seq, const int32_t* positions,
                           const int32_t* counts, int batch, int k, int num_heads, float softmax_scale,
                           void* o_lat, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Matrix-core rate calibration (for reading the decode's roofline; not part of the decode path).
 * Launches `blocks` workgroups of four waves on `stream`; every wave issues iters x 4 independent
 * v_mfma_f32_32x32x16_bf16 products (32 x 32 x 16 multiply-adds each) back to back, touching no
 * memory but its one result: out[w] (float, device, blocks * 4 of them, written) for wave w.  The
 * caller times the launch (for example with events on the stream):
 * rate = blocks * 4 * iters * 4 * 32,768 flops / duration.  With blocks a multiple of the compute
 * units every SIMD runs one such wave.  Errors: MLA_ERR_NULL (out), MLA_ERR_SHAPE (blocks < 1 or
 * iters < 1), MLA_ERR_HIP.
 */
mla_status mla_calibrate_mfma(float* out, int blocks, int iters, hipStream_t stream);

/*
 * Read-rate calibration (for reading the decode's roofline; not part of the decode path).
 * Launches `blocks` workgroups of four waves on `stream` that read buf (device, `bytes` of it, a
 * positive multiple of 36,864, not written) in 36,864-byte chunks, chunk c by workgroup c mod blocks,
 * HBM -> LDS with the 16-byte LDS-direct loads the decode uses for its tiles, three chunks in flight
 * per workgroup.  out[g] (int, device, `blocks` of them, written) is the XOR of the first 32-bit word
 * of every chunk workgroup g read.  The caller times the launch: rate = bytes / duration.
 * Errors: MLA_ERR_NULL (buf or out), MLA_ERR_SHAPE (blocks < 1, bytes 0 or not a multiple of
 * 36,864), MLA_ERR_HIP.
 */
mla_status mla_calibrate_read(const void* buf, size_t bytes, int* out, int blocks, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
