"""ctypes binding over libmla.so: the C entry points under the same names, taking torch tensors.

Argument marshalling only -- every step of the decode path runs in the HIP kernels of libmla.so.
PyTorch supplies device memory and the current stream.  If the library is missing this module raises
at import: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_BF16, MLA_F32 = 0, 1
STATUS = {0: "MLA_OK", -1: "MLA_ERR_NULL", -2: "MLA_ERR_SHAPE", -3: "MLA_ERR_DTYPE",
          -4: "MLA_ERR_WORKSPACE", -5: "MLA_ERR_UNSUPPORTED", -6: "MLA_ERR_BLOCK_TABLE",
          -7: "MLA_ERR_HIP", -8: "MLA_ERR_SCRATCH"}
EXPORTS = ("mla_status_string", "mla_abi_version", "mla_decode_workspace_size", "mla_cache_append",
           "mla_absorb_q", "mla_decode", "mla_out_proj", "mla_cache_append_hidden_workspace_size",
           "mla_cache_append_hidden", "mla_cache_append_fp6", "mla_cache_quantize_fp6", "mla_decode_fp6",
           "mla_out_proj_hidden_workspace_size", "mla_out_proj_hidden", "mla_index_topk_workspace_size",
           "mla_index_topk", "mla_gather_rows", "mla_decode_topk_workspace_size", "mla_decode_topk", "mla_decode_noalloc_max_bytes", "mla_calibrate_mfma", "mla_calibrate_read",
           "mla_decode_noalloc", "mla_decode_out_proj_workspace_size", "mla_decode_out_proj")
INDEX_DIM = 128          # MLA_INDEX_DIM: int8 numbers in a token's index vector
FP6_PAGE_BYTES = 27904   # MLA_FP6_PAGE_BYTES: 64 rows of 432 code bytes, then 64 float32 scales

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run python head_latent_attention_17_amd/build.py")

lib = ctypes.CDLL(LIB_PATH)

_p, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
lib.mla_status_string.restype = ctypes.c_char_p
lib.mla_status_string.argtypes = [_i]
lib.mla_abi_version.restype = _i
lib.mla_abi_version.argtypes = []
lib.mla_decode_workspace_size.restype = _sz
lib.mla_decode_workspace_size.argtypes = [_i, _i, _i, _i, _i]
lib.mla_cache_append.restype = _i
lib.mla_cache_append.argtypes = [_p, _i, _i, _p, _i, _p, _p, _p, _i, _i, _p]
lib.mla_absorb_q.restype = _i
lib.mla_absorb_q.argtypes = [_p, _p, _p, _i, _i, _i, _p]
lib.mla_decode.restype = _i
lib.mla_decode.argtypes = [_p, _p, _i, _i, _p, _i, _p, _i, _i, _f, _p, _p, _p, _sz, _i, _i, _p]
lib.mla_calibrate_mfma.restype = _i
lib.mla_calibrate_mfma.argtypes = [_p, _i, _i, _p]
lib.mla_calibrate_read.restype = _i
lib.mla_calibrate_read.argtypes = [_p, ctypes.c_size_t, _p, _i, _p]
lib.mla_decode_noalloc_max_bytes.restype = _sz
lib.mla_decode_noalloc_max_bytes.argtypes = []
lib.mla_decode_noalloc.restype = _i
lib.mla_decode_noalloc.argtypes = [_p, _p, _i, _i, _p, _i, _p, _i, _i, _f, _p, _p, _i, _i, _p]
lib.mla_decode_out_proj_workspace_size.restype = _sz
lib.mla_decode_out_proj_workspace_size.argtypes = [_i, _i, _i, _i, _i]
lib.mla_decode_out_proj.restype = _i
lib.mla_decode_out_proj.argtypes = [_p, _p, _i, _i, _p, _i, _p, _i, _i, _f, _p, _p, _p, _p, _p, _sz, _i, _i, _p]
lib.mla_out_proj.restype = _i
lib.mla_out_proj.argtypes = [_p, _p, _p, _i, _i, _i, _p]
lib.mla_cache_append_hidden_workspace_size.restype = _sz
lib.mla_cache_append_hidden_workspace_size.argtypes = [_i, _i]
lib.mla_cache_append_hidden.restype = _i
lib.mla_cache_append_hidden.argtypes = [_p, _i, _i, _p, _i, _p, _p, _p, _p, _f, _i, _p, _sz, _i, _p]
lib.mla_cache_append_fp6.restype = _i
lib.mla_cache_append_fp6.argtypes = [_p, _i, _i, _p, _i, _p, _p, _p, _i, _i, _p]
lib.mla_cache_quantize_fp6.restype = _i
lib.mla_cache_quantize_fp6.argtypes = [_p, _p, _i, _i, _p]
lib.mla_decode_fp6.restype = _i
lib.mla_decode_fp6.argtypes = [_p, _p, _i, _i, _p, _i, _p, _i, _i, _f, _p, _p, _p, _sz, _i, _i, _p]
lib.mla_out_proj_hidden_workspace_size.restype = _sz
lib.mla_out_proj_hidden_workspace_size.argtypes = [_i, _i, _i]
lib.mla_out_proj_hidden.restype = _i
lib.mla_out_proj_hidden.argtypes = [_p, _p, _p, _i, _i, _p, _sz, _i, _p]
lib.mla_index_topk_workspace_size.restype = _sz
lib.mla_index_topk_workspace_size.argtypes = [_i, _i]
lib.mla_index_topk.restype = _i
lib.mla_index_topk.argtypes = [_p, _i, _i, _p, _i, _p, _p, _i, _i, _p, _p, _p, _sz, _p]
lib.mla_gather_rows.restype = _i
lib.mla_gather_rows.argtypes = [_p, _i, _i, _p, _i, _p, _p, _i, _i, _p, _p, _p]
lib.mla_decode_topk_workspace_size.restype = _sz
lib.mla_decode_topk_workspace_size.argtypes = [_i, _i, _i]
lib.mla_decode_topk.restype = _i
lib.mla_decode_topk.argtypes = [_p, _p, _i, _i, _p, _i, _p, _p, _i, _i, _i, _f, _p, _p, _p, _sz, _p]


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {lib.mla_status_string(status).decode()}")
        self.status = status


def _check(status: int, where: str):
    if status != 0:
        raise MLAError(status, where)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.current_stream().cuda_stream


def _dtype_of(t: torch.Tensor) -> int:
    if t.dtype in (torch.bfloat16, torch.int16):
        return MLA_BF16
    if t.dtype == torch.float32:
        return MLA_F32
    raise TypeError(f"unsupported activation dtype {t.dtype}")


def _dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("libmla takes contiguous device tensors")


def mla_status_string(status: int) -> str:
    return lib.mla_status_string(status).decode()


def mla_abi_version() -> int:
    return lib.mla_abi_version()


def mla_decode_workspace_size(batch: int, num_heads: int, max_blocks_per_seq: int,
                              num_splits: int = 0, dtype: int = MLA_BF16) -> int:
    return int(lib.mla_decode_workspace_size(batch, num_heads, max_blocks_per_seq, num_splits, dtype))


def mla_cache_append(kv_cache, block_table, positions, c_new, kpe_new, stream=None):
    """kv_cache bf16 [pages][64][576] (in place); block_table int32 [B][max_blocks];
    positions int32 [B]; c_new [B][512], kpe_new [B][64] (bf16, or fp32 for the debug mode)."""
    _dev(kv_cache, block_table, positions, c_new, kpe_new)
    _check(lib.mla_cache_append(_ptr(kv_cache), kv_cache.shape[0], kv_cache.shape[1],
                                _ptr(block_table), block_table.shape[1], _ptr(positions),
                                _ptr(c_new), _ptr(kpe_new), positions.shape[0], _dtype_of(c_new),
                                _stream(stream)), "mla_cache_append")


def mla_cache_append_hidden_workspace_size(batch: int, dtype: int = MLA_BF16) -> int:
    return int(lib.mla_cache_append_hidden_workspace_size(batch, dtype))


def mla_cache_append_hidden(kv_cache, block_table, positions, hidden, w_dkv, w_kr, rope_base=10000.0,
                            workspace=None, stream=None):
    """Rows [hidden @ w_dkv | RoPE(hidden @ w_kr)] written at positions (the lengths before the
    append).  hidden [B][5120], w_dkv [5120][512], w_kr [5120][64] (bf16, or fp32 for the debug
    mode); workspace: a byte tensor of at least mla_cache_append_hidden_workspace_size(B) bytes."""
    _dev(kv_cache, block_table, positions, hidden, w_dkv, w_kr, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.mla_cache_append_hidden(_ptr(kv_cache), kv_cache.shape[0], kv_cache.shape[1],
                                       _ptr(block_table), block_table.shape[1], _ptr(positions),
                                       _ptr(hidden), _ptr(w_dkv), _ptr(w_kr), float(rope_base),
                                       positions.shape[0], _ptr(workspace), ws_bytes, _dtype_of(hidden),
                                       _stream(stream)), "mla_cache_append_hidden")


def _fp6_pages(kv_cache6) -> int:
    if kv_cache6.dim() != 2 or kv_cache6.shape[1] != FP6_PAGE_BYTES or kv_cache6.element_size() != 1:
        raise ValueError(f"a ~6-bit cache is a byte tensor [num_pages][{FP6_PAGE_BYTES}]")
    return kv_cache6.shape[0]


def mla_cache_append_fp6(kv_cache6, block_table, positions, c_new, kpe_new, stream=None):
    """mla_cache_append into the ~6-bit cache: kv_cache6 uint8 [pages][27904] (in place)."""
    _dev(kv_cache6, block_table, positions, c_new, kpe_new)
    _check(lib.mla_cache_append_fp6(_ptr(kv_cache6), _fp6_pages(kv_cache6), 64, _ptr(block_table),
                                    block_table.shape[1], _ptr(positions), _ptr(c_new), _ptr(kpe_new),
                                    positions.shape[0], _dtype_of(c_new), _stream(stream)),
           "mla_cache_append_fp6")


def mla_cache_quantize_fp6(kv_cache, kv_cache6, stream=None):
    """bf16 pages [pages][64][576] -> ~6-bit pages uint8 [pages][27904], page for page."""
    _dev(kv_cache, kv_cache6)
    if kv_cache.shape[0] != _fp6_pages(kv_cache6):
        raise ValueError("kv_cache and kv_cache6 must hold the same number of pages")
    _check(lib.mla_cache_quantize_fp6(_ptr(kv_cache), _ptr(kv_cache6), kv_cache.shape[0], kv_cache.shape[1],
                                      _stream(stream)), "mla_cache_quantize_fp6")


def mla_decode_fp6(q_abs, kv_cache6, block_table, seq_lens, softmax_scale, o_lat, lse=None,
                   workspace=None, num_splits=0, stream=None):
    """mla_decode over the ~6-bit cache kv_cache6 uint8 [pages][27904]; other arguments as mla_decode."""
    _dev(q_abs, kv_cache6, block_table, seq_lens, o_lat, lse, workspace)
    B, H = q_abs.shape[0], q_abs.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.mla_decode_fp6(_ptr(q_abs), _ptr(kv_cache6), _fp6_pages(kv_cache6), 64, _ptr(block_table),
                              block_table.shape[1], _ptr(seq_lens), B, H, float(softmax_scale), _ptr(o_lat),
                              _ptr(lse), _ptr(workspace), ws_bytes, int(num_splits), _dtype_of(q_abs),
                              _stream(stream)), "mla_decode_fp6")


def mla_absorb_q(q, w_uk, q_abs, stream=None):
    """q [B][H][192] -> q_abs [B][H][576]; w_uk [H][128][512]."""
    _dev(q, w_uk, q_abs)
    _check(lib.mla_absorb_q(_ptr(q), _ptr(w_uk), _ptr(q_abs), q.shape[0], q.shape[1], _dtype_of(q),
                            _stream(stream)), "mla_absorb_q")


def mla_decode(q_abs, kv_cache, block_table, seq_lens, softmax_scale, o_lat, lse=None,
               workspace=None, num_splits=0, stream=None):
    """q_abs [B][H][576]; kv_cache bf16 [pages][64][576]; block_table int32 [B][max_blocks];
    seq_lens int32 [B] -> o_lat [B][H][512] and, if given, lse fp32 [B][H].
    workspace: a byte tensor of at least mla_decode_workspace_size(...) bytes."""
    _dev(q_abs, kv_cache, block_table, seq_lens, o_lat, lse, workspace)
    B, H = q_abs.shape[0], q_abs.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.mla_decode(_ptr(q_abs), _ptr(kv_cache), kv_cache.shape[0], kv_cache.shape[1],
                          _ptr(block_table), block_table.shape[1], _ptr(seq_lens), B, H,
                          float(softmax_scale), _ptr(o_lat), _ptr(lse), _ptr(workspace), ws_bytes,
                          int(num_splits), _dtype_of(q_abs), _stream(stream)), "mla_decode")


def mla_calibrate_mfma(out, blocks: int, iters: int, stream=None):
    """out: float32 device tensor of at least blocks * 4 elements; see the header for the rate."""
    _dev(out)
    if out.dtype != torch.float32 or out.numel() < 4 * blocks:
        raise ValueError("out must be a float32 tensor of at least blocks * 4 elements")
    _check(lib.mla_calibrate_mfma(_ptr(out), int(blocks), int(iters), _stream(stream)), "mla_calibrate_mfma")


def mla_calibrate_read(buf, out, blocks: int, stream=None):
    """buf: device tensor whose byte size is a multiple of 36,864; out: int32 device tensor of at
    least `blocks` elements; see the header for the rate."""
    _dev(buf)
    _dev(out)
    if out.dtype != torch.int32 or out.numel() < blocks:
        raise ValueError("out must be an int32 tensor of at least `blocks` elements")
    nbytes = buf.numel() * buf.element_size()
    _check(lib.mla_calibrate_read(_ptr(buf), nbytes, _ptr(out), int(blocks), _stream(stream)), "mla_calibrate_read")


def mla_decode_noalloc_max_bytes() -> int:
    return int(lib.mla_decode_noalloc_max_bytes())


def mla_decode_noalloc(q_abs, kv_cache, block_table, seq_lens, softmax_scale, o_lat, lse=None, num_splits=0,
                       stream=None):
    """mla_decode with the library's fixed scratch array in place of a workspace (allocates nothing)."""
    _dev(q_abs, kv_cache, block_table, seq_lens, o_lat, lse)
    B, H = q_abs.shape[0], q_abs.shape[1]
    _check(lib.mla_decode_noalloc(_ptr(q_abs), _ptr(kv_cache), kv_cache.shape[0], kv_cache.shape[1],
                                  _ptr(block_table), block_table.shape[1], _ptr(seq_lens), B, H,
                                  float(softmax_scale), _ptr(o_lat), _ptr(lse), int(num_splits),
                                  _dtype_of(q_abs), _stream(stream)), "mla_decode_noalloc")


def mla_decode_out_proj_workspace_size(batch: int, num_heads: int, max_blocks_per_seq: int,
                                       num_splits: int = 0, dtype: int = MLA_BF16) -> int:
    return int(lib.mla_decode_out_proj_workspace_size(batch, num_heads, max_blocks_per_seq, num_splits, dtype))


def mla_decode_out_proj(q_abs, kv_cache, block_table, seq_lens, softmax_scale, w_uv, out, o_lat=None, lse=None,
                        workspace=None, num_splits=0, stream=None):
    """mla_decode then mla_out_proj in one call: out [B][H][128] from q_abs [B][H][576] through
    w_uv [H][512][128]; o_lat and lse written when given."""
    _dev(q_abs, kv_cache, block_table, seq_lens, w_uv, out, o_lat, lse, workspace)
    B, H = q_abs.shape[0], q_abs.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.mla_decode_out_proj(_ptr(q_abs), _ptr(kv_cache), kv_cache.shape[0], kv_cache.shape[1],
                                   _ptr(block_table), block_table.shape[1], _ptr(seq_lens), B, H,
                                   float(softmax_scale), _ptr(w_uv), _ptr(out), _ptr(o_lat), _ptr(lse),
                                   _ptr(workspace), ws_bytes, int(num_splits), _dtype_of(q_abs),
                                   _stream(stream)), "mla_decode_out_proj")


def mla_out_proj(o_lat, w_uv, out, stream=None):
    """o_lat [B][H][512] -> out [B][H][128]; w_uv [H][512][128]."""
    _dev(o_lat, w_uv, out)
    _check(lib.mla_out_proj(_ptr(o_lat), _ptr(w_uv), _ptr(out), o_lat.shape[0], o_lat.shape[1],
                            _dtype_of(o_lat), _stream(stream)), "mla_out_proj")


def mla_out_proj_hidden_workspace_size(batch: int, num_heads: int, dtype: int = MLA_BF16) -> int:
    return int(lib.mla_out_proj_hidden_workspace_size(batch, num_heads, dtype))


def mla_out_proj_hidden(out, w_o, hidden, workspace=None, stream=None):
    """out [B][H][128] -> hidden [B][5120] = out flattened head-major @ w_o [H * 128][5120]."""
    _dev(out, w_o, hidden, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.mla_out_proj_hidden(_ptr(out), _ptr(w_o), _ptr(hidden), out.shape[0], out.shape[1],
                                   _ptr(workspace), ws_bytes, _dtype_of(out), _stream(stream)),
           "mla_out_proj_hidden")


def mla_index_topk_workspace_size(batch: int, max_blocks_per_seq: int) -> int:
    return int(lib.mla_index_topk_workspace_size(batch, max_blocks_per_seq))


def mla_index_topk(index_cache, block_table, seq_lens, q_index, k, positions, counts, workspace, stream=None):
    """index_cache int8 [pages][64][128], q_index int8 [B][128] -> positions int32 [B][k] (increasing)
    and counts int32 [B] of each sequence's k best-scoring tokens."""
    _dev(index_cache, block_table, seq_lens, q_index, positions, counts, workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.mla_index_topk(_ptr(index_cache), index_cache.shape[0], index_cache.shape[1], _ptr(block_table),
                              block_table.shape[1], _ptr(seq_lens), _ptr(q_index), seq_lens.shape[0], int(k),
                              _ptr(positions), _ptr(counts), _ptr(workspace), ws_bytes, _stream(stream)),
           "mla_index_topk")


def mla_gather_rows(kv_cache, block_table, positions, counts, out_cache, out_block_table, stream=None):
    """Kept rows into compact pages out_cache [B * P][64][576] with out_block_table int32 [B][P]."""
    _dev(kv_cache, block_table, positions, counts, out_cache, out_block_table)
    _check(lib.mla_gather_rows(_ptr(kv_cache), kv_cache.shape[0], kv_cache.shape[1], _ptr(block_table),
                               block_table.shape[1], _ptr(positions), _ptr(counts), positions.shape[0],
                               positions.shape[1], _ptr(out_cache), _ptr(out_block_table), _stream(stream)),
           "mla_gather_rows")


def mla_decode_topk_workspace_size(batch: int, num_heads: int, k: int) -> int:
    return int(lib.mla_decode_topk_workspace_size(batch, num_heads, k))


def mla_decode_topk(q_abs, kv_cache, block_table, positions, counts, softmax_scale, o_lat, lse=None,
                    workspace=None, stream=None):
    """Attention over the kept tokens positions [B][k] (first counts[b] of each row) read in place:
    q_abs [B][H][576] -> o_lat [B][H][512] and, if given, lse fp32 [B][H]; bf16 only."""
    _dev(q_abs, kv_cache, block_table, positions, counts, o_lat, lse, workspace)
    B, H = q_abs.shape[0], q_abs.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.mla_decode_topk(_ptr(q_abs), _ptr(kv_cache), kv_cache.shape[0], kv_cache.shape[1],
                               _ptr(block_table), block_table.shape[1], _ptr(positions), _ptr(counts), B,
                               positions.shape[1], H, float(softmax_scale), _ptr(o_lat), _ptr(lse),
                               _ptr(workspace), ws_bytes, _stream(stream)), "mla_decode_topk")
