"""C-ABI checks that need no GPU: the library loads, exports every function include/mla.h declares,
and its host-side validation returns the documented status codes before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


def _lib():
    from head_latent_attention_17_amd import _lib as L
    return L


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_four_path_calls():
    names = declared_functions()
    for n in ("mla_cache_append", "mla_absorb_q", "mla_decode", "mla_out_proj"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib()
    raw = ctypes.CDLL(L.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name
    assert set(declared_functions()) == set(L.EXPORTS)


def test_status_strings_and_version():
    L = _lib()
    assert L.mla_abi_version() == 108
    for code, name in L.STATUS.items():
        assert L.mla_status_string(code).startswith(name)
    assert "unknown" in L.mla_status_string(12345)


def test_workspace_size_formula():
    L = _lib()
    # (units + batch) pieces * heads * (512 partial outputs + max + sum) * 4 bytes
    # one fp32 slot of 512 + 2 values per (piece, head), then 16 bytes per sequence
    assert L.mla_decode_workspace_size(4, 128, 2048, 64) == (64 + 4) * 128 * 514 * 4 + 4 * 16
    assert L.mla_decode_workspace_size(4, 128, 2048, 0) == (256 + 4) * 128 * 514 * 4 + 4 * 16
    assert L.mla_decode_workspace_size(1, 32, 3, 0) == (3 + 1) * 32 * 514 * 4 + 16   # never more units than pages
    assert L.mla_decode_workspace_size(1, 16, 3, 0, 1) == (3 + 1) * 16 * 514 * 4 + 16  # fp32 at 16 heads: pages
    assert L.mla_decode_workspace_size(1, 16, 3, 0) == (6 + 1) * 16 * 514 * 4 + 16   # 16 heads: 32-token tiles
    assert L.mla_decode_topk_workspace_size(1, 16, 130) == (6 + 1) * 16 * 514 * 4 + 16
    assert L.mla_decode_workspace_size(2, 16, 1000, 0) == (256 + 2) * 16 * 514 * 4 + 2 * 16
    assert L.mla_decode_workspace_size(4, 100, 2048, 0) == 0                  # unsupported heads
    assert L.mla_decode_workspace_size(4, 128, 0, 0) == 0
    assert L.mla_decode_workspace_size(4, 128, 8, -1) == 0
    assert L.mla_decode_workspace_size(4, 128, 8, 0, 7) == 0                  # unknown dtype


FAKE = 0x1000   # never dereferenced: every call below fails validation first


def _decode(L, **kw):
    a = dict(q_abs=FAKE, cache=FAKE, num_pages=16, page_size=64, bt=FAKE, max_blocks=16, lens=FAKE,
             batch=1, heads=16, scale=0.07, o_lat=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 30,
             splits=0, dtype=0)
    a.update(kw)
    return L.lib.mla_decode(a["q_abs"], a["cache"], a["num_pages"], a["page_size"], a["bt"],
                            a["max_blocks"], a["lens"], a["batch"], a["heads"], a["scale"],
                            a["o_lat"], a["lse"], a["ws"], a["ws_bytes"], a["splits"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), -3),
    (dict(page_size=32), -5),
    (dict(heads=100), -5),
    (dict(batch=-1), -2),
    (dict(max_blocks=0), -2),
    (dict(splits=-3), -2),
    (dict(scale=0.0), -2),
    (dict(scale=float("nan")), -2),
    (dict(q_abs=None), -1),
    (dict(cache=None), -1),
    (dict(lens=None), -1),
    (dict(o_lat=None), -1),
    (dict(ws=None), -4),
    (dict(ws_bytes=10), -4),
])
def test_decode_validation(kw, status):
    assert _decode(_lib(), **kw) == status


def test_empty_batch_is_a_no_op():
    L = _lib()
    assert _decode(L, batch=0, q_abs=None, cache=None, ws=None) == 0
    assert L.lib.mla_absorb_q(None, None, None, 0, 128, 0, None) == 0
    assert L.lib.mla_out_proj(None, None, None, 0, 128, 0, None) == 0
    assert L.lib.mla_cache_append(None, 0, 64, None, 1, None, None, None, 0, 0, None) == 0


def test_projection_and_append_validation():
    L = _lib()
    assert L.lib.mla_absorb_q(FAKE, FAKE, FAKE, 2, 96, 0, None) == -5
    assert L.lib.mla_absorb_q(FAKE, None, FAKE, 2, 128, 0, None) == -1
    assert L.lib.mla_absorb_q(FAKE, FAKE, FAKE, 2, 128, 9, None) == -3
    assert L.lib.mla_out_proj(FAKE, FAKE, None, 2, 128, 0, None) == -1
    assert L.lib.mla_out_proj(FAKE, FAKE, FAKE, -2, 128, 0, None) == -2
    assert L.lib.mla_cache_append(FAKE, 8, 16, FAKE, 1, FAKE, FAKE, FAKE, 2, 0, None) == -5
    assert L.lib.mla_cache_append(FAKE, 8, 64, FAKE, 1, None, FAKE, FAKE, 2, 0, None) == -1
    assert L.lib.mla_cache_append(FAKE, 0, 64, FAKE, 1, FAKE, FAKE, FAKE, 2, 0, None) == -2


def test_append_hidden_validation_and_workspace():
    """The producer-side append: workspace formula (twenty fp32 partial rows of 576 per sequence) and
    host-side validation, each failing before anything is launched."""
    L = _lib()
    assert L.mla_cache_append_hidden_workspace_size(32) == 32 * 20 * 576 * 4
    assert L.mla_cache_append_hidden_workspace_size(-1) == 0
    assert L.mla_cache_append_hidden_workspace_size(4, 7) == 0
    f = L.lib.mla_cache_append_hidden
    ws = 2 * 20 * 576 * 4
    ok = [FAKE, 8, 64, FAKE, 1, FAKE, FAKE, FAKE, FAKE, 10000.0, 2, FAKE, ws, 0, None]
    def call(**kw):
        args = list(ok)
        names = ["cache", "pages", "page", "bt", "mb", "pos", "h", "wd", "wk", "base", "batch", "ws", "wsb", "dt", "s"]
        for k, v in kw.items():
            args[names.index(k)] = v
        return f(*args)
    assert call(batch=0, cache=None) == 0           # empty batch: nothing to do
    assert call(dt=9) == -3
    assert call(page=16) == -5
    assert call(batch=-1) == -2
    assert call(base=1.0) == -2 and call(base=float("nan")) == -2 and call(base=float("inf")) == -2
    assert call(pages=0) == -2
    assert call(h=None) == -1 and call(wk=None) == -1
    assert call(ws=None) == -4 and call(wsb=ws - 1) == -4


def test_python_binding_rejects_host_tensors():
    import torch
    L = _lib()
    x = torch.zeros(4, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        L.mla_out_proj(x, x, x)


def test_fp6_cache_validation():
    """The ~6-bit cache entry points reject bad arguments before any launch: decode only with bf16
    activations and 64 or 128 heads; quantize and append with the same checks as the bf16 ones."""
    L = _lib()
    assert L.FP6_PAGE_BYTES == 64 * 432 + 64 * 4

    def dec6(**kw):
        a = dict(q_abs=FAKE, cache=FAKE, num_pages=16, page_size=64, bt=FAKE, max_blocks=16, lens=FAKE,
                 batch=1, heads=128, scale=0.07, o_lat=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 30,
                 splits=0, dtype=0)
        a.update(kw)
        return L.lib.mla_decode_fp6(a["q_abs"], a["cache"], a["num_pages"], a["page_size"], a["bt"],
                                    a["max_blocks"], a["lens"], a["batch"], a["heads"], a["scale"],
                                    a["o_lat"], a["lse"], a["ws"], a["ws_bytes"], a["splits"], a["dtype"], None)

    assert dec6(dtype=1) == -5            # fp32 debug mode has no ~6-bit path
    assert dec6(heads=16) == -5
    assert dec6(heads=32) == -5
    assert dec6(heads=100) == -5
    assert dec6(dtype=7) == -3
    assert dec6(page_size=32) == -5
    assert dec6(cache=None) == -1
    assert dec6(ws_bytes=10) == -4
    assert dec6(scale=-1.0) == -2
    assert dec6(batch=0, cache=None, ws=None) == 0
    q = L.lib.mla_cache_quantize_fp6
    assert q(FAKE, FAKE, 4, 32, None) == -5
    assert q(FAKE, FAKE, -1, 64, None) == -2
    assert q(None, FAKE, 4, 64, None) == -1
    assert q(None, None, 0, 64, None) == 0
    a = L.lib.mla_cache_append_fp6
    assert a(FAKE, 8, 16, FAKE, 1, FAKE, FAKE, FAKE, 2, 0, None) == -5
    assert a(FAKE, 8, 64, FAKE, 1, None, FAKE, FAKE, 2, 0, None) == -1
    assert a(FAKE, 0, 64, FAKE, 1, FAKE, FAKE, FAKE, 2, 0, None) == -2
    assert a(FAKE, 8, 64, FAKE, 1, FAKE, FAKE, FAKE, 2, 5, None) == -3
    assert a(None, 0, 64, None, 1, None, None, None, 0, 0, None) == 0


def test_out_proj_hidden_validation_and_workspace():
    """Output projection to the hidden width: workspace = (heads * 128 / 1024) fp32 partial rows of
    5,120 per sequence in bf16 mode, none in fp32 mode; host-side validation before any launch."""
    L = _lib()
    assert L.mla_out_proj_hidden_workspace_size(32, 128) == 16 * 32 * 5120 * 4
    assert L.mla_out_proj_hidden_workspace_size(3, 16) == 2 * 3 * 5120 * 4
    assert L.mla_out_proj_hidden_workspace_size(3, 16, 1) == 0
    assert L.mla_out_proj_hidden_workspace_size(3, 100) == 0
    assert L.mla_out_proj_hidden_workspace_size(-1, 128) == 0
    f = L.lib.mla_out_proj_hidden
    ws = 16 * 2 * 5120 * 4
    assert f(FAKE, FAKE, FAKE, 2, 128, FAKE, ws, 9, None) == -3
    assert f(FAKE, FAKE, FAKE, -1, 128, FAKE, ws, 0, None) == -2
    assert f(FAKE, FAKE, FAKE, 2, 96, FAKE, ws, 0, None) == -5
    assert f(None, FAKE, FAKE, 2, 128, FAKE, ws, 0, None) == -1
    assert f(FAKE, FAKE, FAKE, 2, 128, None, ws, 0, None) == -4
    assert f(FAKE, FAKE, FAKE, 2, 128, FAKE, ws - 1, 0, None) == -4
    assert f(None, None, None, 0, 128, None, 0, 0, None) == 0


def test_index_topk_and_gather_validation():
    """Top-k path: workspace (per sequence: int32 scores for every block, 4,096 + 2,048 histogram
    bins, 4 selection words, 2 words per 1,024-token chunk) and host validation."""
    L = _lib()
    assert L.INDEX_DIM == 128
    assert L.mla_index_topk_workspace_size(4, 2049) == 4 * (2049 * 64 + 4096 + 2048 + 4 + 2 * 129) * 4
    assert L.mla_index_topk_workspace_size(4, 0) == 0
    t = L.lib.mla_index_topk
    ws = 2 * (4 * 64 + 4096 + 2048 + 4 + 2 * 1) * 4
    ok = [FAKE, 8, 64, FAKE, 4, FAKE, FAKE, 2, 16, FAKE, FAKE, FAKE, ws, None]
    def call(i, v):
        a = list(ok)
        a[i] = v
        return t(*a)
    assert t(*ok[:2], 32, *ok[3:]) == -5          # page size
    assert call(8, 0) == -2                        # k
    assert call(7, -1) == -2                       # batch
    assert call(0, None) == -1
    assert call(9, None) == -1
    assert call(11, None) == -4
    assert call(12, ws - 1) == -4
    assert t(None, 0, 64, None, 4, None, None, 0, 16, None, None, None, 0, None) == 0
    g = L.lib.mla_gather_rows
    assert g(FAKE, 8, 64, FAKE, 4, FAKE, FAKE, 2, 0, FAKE, FAKE, None) == -2
    assert g(FAKE, 8, 16, FAKE, 4, FAKE, FAKE, 2, 8, FAKE, FAKE, None) == -5
    assert g(FAKE, 8, 64, FAKE, 4, FAKE, FAKE, 2, 8, None, FAKE, None) == -1
    assert g(None, 0, 64, None, 4, None, None, 0, 8, None, None, None) == 0


def test_decode_topk_validation():
    """In-place top-k decode: its workspace is that of mla_decode over compact pages of the kept
    rows (ceil(k / 64) pages per sequence), and host validation runs before any launch."""
    L = _lib()
    for b, h, k in ((4, 128, 2048), (32, 128, 2048), (3, 64, 100), (1, 32, 1), (2, 16, 300)):
        assert L.mla_decode_topk_workspace_size(b, h, k) == L.mla_decode_workspace_size(b, h, -(-k // 64), 0)
    assert L.mla_decode_topk_workspace_size(4, 128, 0) == 0
    assert L.mla_decode_topk_workspace_size(4, 48, 64) == 0
    f = L.lib.mla_decode_topk
    ws = L.mla_decode_topk_workspace_size(2, 128, 100)
    ok = [FAKE, FAKE, 8, 64, FAKE, 4, FAKE, FAKE, 2, 100, 128, 0.1, FAKE, None, FAKE, ws, None]
    def call(i, v):
        a = list(ok)
        a[i] = v
        return f(*a)
    assert call(3, 32) == -5                       # page size
    assert call(10, 48) == -5
    assert call(9, 0) == -2                        # k
    assert call(8, -1) == -2                       # batch
    assert call(11, 0.0) == -2                     # scale
    assert call(11, float("nan")) == -2
    assert call(2, 0) == -2                        # empty cache with sequences to attend
    assert call(0, None) == -1
    assert call(6, None) == -1                     # positions
    assert call(7, None) == -1                     # counts
    assert call(12, None) == -1
    assert call(14, None) == -4
    assert call(15, ws - 1) == -4
    assert f(None, None, 0, 64, None, 4, None, None, 0, 100, 128, 0.1, None, None, None, 0, None) == 0



def test_decode_noalloc_validation():
    """The no-allocation decode validates like mla_decode and rejects sizes whose workspace would
    exceed its fixed scratch array before any HIP call."""
    L = _lib()
    assert L.mla_decode_noalloc_max_bytes() == 128 << 20

    def call(batch=1, heads=128, max_blocks=16, splits=0, page_size=64, dtype=0, q=FAKE):
        return L.lib.mla_decode_noalloc(q, FAKE, 16, page_size, FAKE, max_blocks, FAKE, batch, heads, 0.07,
                                        FAKE, None, splits, dtype, None)

    assert call(batch=300, max_blocks=64) == -8          # (256 + 300) x 128 x 2,056 B > 128 MiB
    assert call(batch=254, max_blocks=64) == -8
    # the documented limit: 253 sequences at 128 heads and the automatic split (256 ranges)
    assert L.mla_decode_workspace_size(253, 128, 64, 0) <= L.mla_decode_noalloc_max_bytes()
    assert L.mla_decode_workspace_size(254, 128, 64, 0) > L.mla_decode_noalloc_max_bytes()
    assert call(page_size=32) == -5
    assert call(heads=100) == -5
    assert call(dtype=3) == -3
    assert call(batch=-1) == -2
    assert call(q=None) == -1
    assert call(batch=0) == 0


def test_decode_out_proj_validation_and_workspace():
    L = _lib()
    base = L.mla_decode_workspace_size(4, 128, 64, 0)
    # room for an fp32 o_lat behind the decode's workspace, for the paths that keep it
    assert L.mla_decode_out_proj_workspace_size(4, 128, 64, 0) == base + 4 * 128 * 512 * 4
    assert L.mla_decode_out_proj_workspace_size(4, 128, 64, 0, 1) == \
        L.mla_decode_workspace_size(4, 128, 64, 0, 1) + 4 * 128 * 512 * 4
    assert L.mla_decode_out_proj_workspace_size(4, 100, 64, 0) == 0

    def call(batch=1, heads=128, w_uv=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 30, page_size=64, dtype=0):
        return L.lib.mla_decode_out_proj(FAKE, FAKE, 16, page_size, FAKE, 16, FAKE, batch, heads, 0.07, w_uv, out,
                                         None, None, ws, ws_bytes, 0, dtype, None)

    assert call(w_uv=None) == -1
    assert call(out=None) == -1
    assert call(ws=None) == -4
    assert call(ws_bytes=16) == -4
    assert call(page_size=32) == -5
    assert call(heads=100) == -5
    assert call(dtype=5) == -3
    assert call(batch=-2) == -2
    assert call(batch=0) == 0


def test_calibrate_read_validation():
    """The read-rate calibration validates before launching: null pointers, block counts and sizes
    that are not whole 36,864-byte chunks are rejected without touching the GPU."""
    L = _lib()
    f = L.lib.mla_calibrate_read
    assert f(None, 36864, FAKE, 1, None) == -1
    assert f(FAKE, 36864, None, 1, None) == -1
    assert f(FAKE, 36864, FAKE, 0, None) == -2
    assert f(FAKE, 0, FAKE, 1, None) == -2
    assert f(FAKE, 36864 + 4, FAKE, 1, None) == -2
