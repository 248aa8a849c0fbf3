"""MLA decode over a paged latent cache on MI355X (gfx950): a C-ABI HIP library plus this binding.

The entry points carry the C names: mla_cache_append, mla_absorb_q, mla_decode, mla_out_proj,
mla_decode_workspace_size, and the producer side mla_cache_append_hidden (with its workspace size).
Importing the package loads libmla.so and fails if it is not built.
"""
from ._lib import (MLA_BF16, MLA_F32, MLAError, mla_abi_version, mla_absorb_q,  # noqa: F401
                   mla_cache_append, mla_cache_append_hidden, mla_cache_append_hidden_workspace_size,
                   mla_decode, mla_decode_workspace_size, mla_out_proj, mla_status_string, LIB_PATH)
