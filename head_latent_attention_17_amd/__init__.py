"""MLA decode over a paged latent cache on MI355X (gfx950): a C-ABI HIP library plus this binding.

The entry points carry the C names: mla_cache_append, mla_absorb_q, mla_decode, mla_out_proj,
mla_decode_workspace_size, the producer side mla_cache_append_hidden (with its workspace size), and
the ~6-bit cache: mla_cache_append_fp6, mla_cache_quantize_fp6, mla_decode_fp6 (FP6_PAGE_BYTES per
page), the output projection to the hidden width, mla_out_proj_hidden (with its workspace size), and
the top-k path: mla_index_topk (with its workspace size), mla_gather_rows and mla_decode_topk (with
its workspace size), mla_decode_out_proj (mla_decode and mla_out_proj in one call, with its workspace size), and
mla_decode_noalloc (mla_decode with the library's fixed scratch array in
place of a workspace, for callers that cannot allocate).  Importing the package loads libmla.so and fails if it is not built.
"""
from ._lib import (FP6_PAGE_BYTES, INDEX_DIM, MLA_BF16, MLA_F32, MLAError, mla_abi_version,  # noqa: F401
                   mla_absorb_q, mla_cache_append, mla_cache_append_fp6, mla_cache_append_hidden,
                   mla_cache_append_hidden_workspace_size, mla_cache_quantize_fp6, mla_decode,
                   mla_decode_fp6, mla_decode_workspace_size, mla_out_proj, mla_out_proj_hidden,
                   mla_out_proj_hidden_workspace_size, mla_index_topk, mla_index_topk_workspace_size,
                   mla_gather_rows, mla_decode_topk, mla_decode_topk_workspace_size, mla_status_string,
                   mla_decode_noalloc, mla_decode_noalloc_max_bytes, mla_decode_out_proj,
                   mla_decode_out_proj_workspace_size, mla_calibrate_mfma, mla_calibrate_read,
                   LIB_PATH)
