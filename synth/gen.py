"""Seeded synthetic inputs for MLA decode over a paged latent cache.

This module is shared by both sides of every parity check: the CPU oracle (``oracle/``) and the HIP
library (``head_latent_attention_17_amd``). It holds none of the attention arithmetic. It only

* draws pseudo-random values with a counter-based generator, so that any element (for instance a
  single cache page) can be regenerated on its own, on the CPU or on the GPU, with identical bits;
* rounds each draw to bfloat16 (round-to-nearest-even), which is how the inputs are stored;
* builds per-sequence lengths and a shuffled block table with numpy's PCG64 stream.

Shapes follow DeepSeek-V2 as the explainer "DeepSeek-V2" (aiany.app) gives them: 128 heads of
128 dimensions (Step 2), a 512-number latent note per token (Step 5, eq. 9) and a 64-number decoupled
RoPE key shared by all heads (Step 7), so one cached row holds 512 + 64 = 576 numbers (Step 8).

Generator.  Element ``i`` of stream ``s`` under seed ``k`` is the SplitMix64 output function
(Steele, Lea and Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014) applied to the
state ``key(k, s) + (i + 1) * 0x9E3779B97F4A7C15``.  Its 64 bits are split into four 16-bit uniform
integers whose centred sum (Irwin-Hall with n = 4) is scaled to unit variance: an approximately
normal draw bounded by about 3.46 sigma.  All integer steps are exact, the single float32 multiply is
correctly rounded and the bf16 rounding is done on the integer bits, so the CPU and the GPU produce the
same bits.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

D_C = 512        # latent width d_c (explainer Step 5, eq. 9)
D_R = 64         # decoupled RoPE key / query width (explainer Step 7)
D_NOPE = 128     # per-head content query/key width (explainer Step 2: 128-dim heads)
D_V = 128        # per-head value width (explainer Step 2)
ROW = D_C + D_R  # numbers per cached token per layer (explainer Step 8)
PAGE = 64        # tokens per cache page (the library's fixed page size)
D_MODEL = 5120   # hidden width a token's cache row is projected from
Q_DIM = D_NOPE + D_R

# stream ids (one independent counter stream per kind of input)
S_CACHE, S_Q, S_QABS, S_WUK, S_WUV, S_NEWROW, S_GARBAGE = 1, 2, 3, 4, 5, 6, 7
S_HIDDEN, S_WDKV, S_WKR = 8, 9, 10
S_WO = 11
S_INDEX, S_QINDEX = 12, 13
INDEX_DIM = 128  # int8 numbers in a token's cheap index vector

_U64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_IH_STD = math.sqrt(((1 << 32) - 1) / 3.0)   # std of a sum of four uniform 16-bit integers


def _s64(x: int) -> int:
    """Unsigned 64-bit constant -> the int64 with the same bits."""
    x &= _U64
    return x - (1 << 64) if x >> 63 else x


def splitmix64_py(state: int) -> int:
    """SplitMix64 output function on one Python int (used to pin the tensor version)."""
    z = state & _U64
    z = ((z ^ (z >> 30)) * _M1) & _U64
    z = ((z ^ (z >> 27)) * _M2) & _U64
    return z ^ (z >> 31)


def _lsr(z: torch.Tensor, k: int) -> torch.Tensor:
    return (z >> k) & ((1 << (64 - k)) - 1)


def _mix(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _lsr(z, 30)) * _s64(_M1)
    z = (z ^ _lsr(z, 27)) * _s64(_M2)
    return z ^ _lsr(z, 31)


def stream_key(seed: int, stream: int, layer: int = 0) -> int:
    """Starting state of one stream: SplitMix64 of the packed (seed, layer, stream) triple."""
    return splitmix64_py((seed << 24) ^ (layer << 8) ^ stream)


def raw_u64(key: int, index: torch.Tensor) -> torch.Tensor:
    """64-bit draws (as int64 bits) for integer counters ``index`` (int64 tensor)."""
    state = (index + 1) * _s64(_GAMMA) + _s64(key)
    return _mix(state)


def _f32_to_bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """Round float32 to bfloat16 (nearest, ties to even) on the integer bits; finite inputs only."""
    b = x.contiguous().view(torch.int32).to(torch.int64) & 0xFFFFFFFF
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16) & 0xFFFF
    return r.to(torch.int32).to(torch.int16)   # wraps to the same 16 bits


def normal_bf16(key: int, index: torch.Tensor, std: float) -> torch.Tensor:
    """Approximately N(0, std^2) values for counters ``index``, as bf16 bit patterns (int16)."""
    z = raw_u64(key, index)
    s = (z & 0xFFFF) + (_lsr(z, 16) & 0xFFFF) + (_lsr(z, 32) & 0xFFFF) + _lsr(z, 48)
    s = (s - 2 * 0xFFFF).to(torch.float32)          # |s| < 2^18: exact in float32
    x = s * torch.tensor(std / _IH_STD, dtype=torch.float32, device=s.device)
    return _f32_to_bf16_bits(x)


def garbage_bf16(key: int, index: torch.Tensor) -> torch.Tensor:
    """Finite 'stale memory' values: random sign, magnitude in [2^12, 2^20).  Any cache slot past a
    sequence's length holds these, so a kernel that reads beyond the length fails loudly."""
    z = raw_u64(key, index)
    sign = (z & 1) << 15
    exp = 127 + 12 + (_lsr(z, 1) & 7)                # 2^12 .. 2^19
    mant = _lsr(z, 8) & 0x7F
    return (sign | (exp << 7) | mant).to(torch.int32).to(torch.int16)


# --------------------------------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------------------------------

@dataclass
class Workload:
    """Host-side description of one decode batch: lengths, block table and shapes."""
    name: str
    batch: int
    heads: int
    lens: np.ndarray              # int32 [B], cached tokens before any append
    block_table: np.ndarray       # int32 [B][max_blocks], -1 where unused
    num_pages: int
    seed: int
    layers: int = 1
    append: bool = False          # one new row per sequence is appended before attention
    scale: float = 1.0 / math.sqrt(Q_DIM)
    page_size: int = PAGE
    page_owner: np.ndarray = field(default=None, repr=False)   # int32 [num_pages] sequence id
    page_index: np.ndarray = field(default=None, repr=False)   # int32 [num_pages] block index j

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def attended_lens(self) -> np.ndarray:
        """Tokens attended per sequence (the appended row included)."""
        return self.lens + (1 if self.append else 0)

    @property
    def tokens(self) -> int:
        return int(self.attended_lens.sum())


def _build_table(lens_final: np.ndarray, rng: np.random.Generator | None, page_size: int,
                 max_blocks: int | None = None):
    blocks = (lens_final + page_size - 1) // page_size
    total = int(blocks.sum())
    mb = int(blocks.max()) if max_blocks is None else max_blocks
    table = np.full((len(lens_final), max(mb, 1)), -1, dtype=np.int32)
    phys = np.arange(total, dtype=np.int32) if rng is None else rng.permutation(total).astype(np.int32)
    owner = np.empty(total, dtype=np.int32)
    index = np.empty(total, dtype=np.int32)
    k = 0
    for b, nb in enumerate(blocks):
        table[b, :nb] = phys[k:k + nb]
        owner[phys[k:k + nb]] = b
        index[phys[k:k + nb]] = np.arange(nb, dtype=np.int32)
        k += nb
    return table, total, owner, index


def make_custom(lens, heads: int, seed: int, *, shuffle: bool = True, append: bool = False,
                layers: int = 1, name: str = "custom", max_blocks: int | None = None,
                scale: float | None = None) -> Workload:
    """A workload with explicit lengths (pre-append).  Physical page ids are one random permutation of
    [0, total pages) assigned to (sequence, block) in row-major order, or the identity when
    ``shuffle`` is false."""
    lens = np.asarray(lens, dtype=np.int32)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed))) if shuffle else None
    final = lens + (1 if append else 0)
    table, total, owner, index = _build_table(final, rng, PAGE, max_blocks)
    return Workload(name=name, batch=len(lens), heads=heads, lens=lens, block_table=table,
                    num_pages=total, seed=seed, layers=layers, append=append,
                    scale=(1.0 / math.sqrt(Q_DIM)) if scale is None else scale,
                    page_owner=owner, page_index=index)


CONFIG_NAMES = {
    1: "c1_b1_h16_len1024_contiguous",
    2: "c2_b32_h128_len4096_paged",
    3: "c3_b4_h128_len131072_paged_splitk",
    4: "c4_b128_h128_loguniform256-32768_paged_append",
    5: "c5_60layers_b64_h128_len4096-8192_absorb_outproj",
}


def make_config(config_id: int) -> Workload:
    """The five workloads: seeds 1000 + id; lengths and tables drawn with PCG64 in a fixed order."""
    seed = 1000 + config_id
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    name = CONFIG_NAMES[config_id]
    if config_id == 1:
        return make_custom([1024], 16, seed, shuffle=False, name=name)
    if config_id == 2:
        return make_custom([4096] * 32, 128, seed, name=name)
    if config_id == 3:
        return make_custom([131072] * 4, 128, seed, name=name)
    if config_id == 4:
        u = rng.uniform(math.log(256), math.log(32768), size=128)
        lens = np.clip(np.floor(np.exp(u)), 256, 32768).astype(np.int32)
        return make_custom(lens, 128, seed + 7, append=True, name=name)
    if config_id == 5:
        lens = rng.integers(4096, 8192, size=64, endpoint=True).astype(np.int32)
        return make_custom(lens, 128, seed + 7, layers=60, name=name)
    raise ValueError(f"unknown config {config_id}")


# --------------------------------------------------------------------------------------------------
# Tensors (bf16 bit patterns as int16, on any torch device)
# --------------------------------------------------------------------------------------------------

def _idx(n: int, device, offset: int = 0) -> torch.Tensor:
    return torch.arange(offset, offset + n, dtype=torch.int64, device=device)


def cache_pages(wl: Workload, layer: int = 0, pages=None, device="cpu",
                chunk_pages: int = 256) -> torch.Tensor:
    """Physical cache pages ``pages`` (default: all) as int16 [n][64][576].

    Slots holding a token (position < pre-append length) get N(0,1) draws; every other slot of an
    owned page (the ragged tail, and the slot an append will fill) gets finite garbage."""
    if pages is None:
        pages = np.arange(wl.num_pages, dtype=np.int64)
    pages = np.asarray(pages, dtype=np.int64)
    key_v = stream_key(wl.seed, S_CACHE, layer)
    key_g = stream_key(wl.seed, S_GARBAGE, layer)
    out = torch.empty((len(pages), PAGE, ROW), dtype=torch.int16, device=device)
    per_page = PAGE * ROW
    for s in range(0, len(pages), chunk_pages):
        pg = torch.as_tensor(pages[s:s + chunk_pages], device=device)
        idx = (pg[:, None] * per_page + _idx(per_page, device)[None, :]).reshape(-1)
        vals = normal_bf16(key_v, idx, 1.0).view(len(pg), PAGE, ROW)
        owner = torch.as_tensor(wl.page_owner[pages[s:s + chunk_pages]], device=device).long()
        blk = torch.as_tensor(wl.page_index[pages[s:s + chunk_pages]], device=device).long()
        lens = torch.as_tensor(wl.lens, device=device).long()[owner]
        pos = blk[:, None] * PAGE + _idx(PAGE, device)[None, :]
        stale = pos >= lens[:, None]
        if bool(stale.any()):
            garb = garbage_bf16(key_g, idx).view(len(pg), PAGE, ROW)
            vals = torch.where(stale[:, :, None], garb, vals)
        out[s:s + len(pg)] = vals
    return out


def queries(wl: Workload, layer: int = 0, device="cpu") -> torch.Tensor:
    """q = [q_nope(128) | q_pe(64)] per head, N(0,1), int16 [B][H][192]."""
    n = wl.batch * wl.heads * Q_DIM
    return normal_bf16(stream_key(wl.seed, S_Q, layer), _idx(n, device), 1.0).view(
        wl.batch, wl.heads, Q_DIM)


def latent_queries(wl: Workload, layer: int = 0, device="cpu") -> torch.Tensor:
    """A query already in latent form, [q_lat(512) | q_pe(64)], int16 [B][H][576].  q_lat is drawn
    with std sqrt(128/512) = 0.5, the spread of q_nope (N(0,1), 128 terms) through a 1/sqrt(512)
    weight, so that scaled scores stay near unit variance."""
    n = wl.batch * wl.heads * ROW
    key = stream_key(wl.seed, S_QABS, layer)
    idx = _idx(n, device).view(wl.batch, wl.heads, ROW)
    lat = normal_bf16(key, idx[..., :D_C].reshape(-1), 0.5).view(wl.batch, wl.heads, D_C)
    pe = normal_bf16(key, idx[..., D_C:].reshape(-1), 1.0).view(wl.batch, wl.heads, D_R)
    return torch.cat([lat, pe], dim=-1)


def weights(wl: Workload, layer: int = 0, device="cpu"):
    """W_UK int16 [H][128][512] and W_UV int16 [H][512][128], std 1/sqrt(512) (both read the
    512-wide latent)."""
    std = 1.0 / math.sqrt(D_C)
    n = wl.heads * D_NOPE * D_C
    w_uk = normal_bf16(stream_key(wl.seed, S_WUK, layer), _idx(n, device), std).view(
        wl.heads, D_NOPE, D_C)
    w_uv = normal_bf16(stream_key(wl.seed, S_WUV, layer), _idx(n, device), std).view(
        wl.heads, D_C, D_V)
    return w_uk, w_uv


def new_rows(wl: Workload, layer: int = 0, device="cpu") -> torch.Tensor:
    """Rows to append, [c_new(512) | k_pe_new(64)], N(0,1), int16 [B][576]."""
    n = wl.batch * ROW
    return normal_bf16(stream_key(wl.seed, S_NEWROW, layer), _idx(n, device), 1.0).view(
        wl.batch, ROW)


def hidden_states(wl: Workload, layer: int = 0, device="cpu") -> torch.Tensor:
    """Hidden vectors of the tokens being appended, N(0,1), int16 [B][5120]."""
    n = wl.batch * D_MODEL
    return normal_bf16(stream_key(wl.seed, S_HIDDEN, layer), _idx(n, device), 1.0).view(wl.batch, D_MODEL)


def producer_weights(wl: Workload, layer: int = 0, device="cpu"):
    """W_DKV int16 [5120][512] and W_KR int16 [5120][64], std 1/sqrt(5120) (both read the 5,120-wide
    hidden vector, so the latent and the key come out near unit variance)."""
    std = 1.0 / math.sqrt(D_MODEL)
    w_dkv = normal_bf16(stream_key(wl.seed, S_WDKV, layer), _idx(D_MODEL * D_C, device), std).view(D_MODEL, D_C)
    w_kr = normal_bf16(stream_key(wl.seed, S_WKR, layer), _idx(D_MODEL * D_R, device), std).view(D_MODEL, D_R)
    return w_dkv, w_kr


def output_weights(wl: Workload, layer: int = 0, device="cpu") -> torch.Tensor:
    """W^O int16 [H * 128][5120], std 1/sqrt(H * 128): mixes the heads' outputs into the hidden
    width."""
    k = wl.heads * D_V
    return normal_bf16(stream_key(wl.seed, S_WO, layer), _idx(k * D_MODEL, device), 1.0 / math.sqrt(k)).view(k, D_MODEL)


def uniform_int8(key: int, index: torch.Tensor) -> torch.Tensor:
    """Integers uniform on [-127, 127] for counters ``index`` (int8)."""
    z = raw_u64(key, index)
    return ((_lsr(z, 32) % 255) - 127).to(torch.int8)


def index_cache(wl: Workload, layer: int = 0, device="cpu") -> torch.Tensor:
    """Each token's cheap index vector, int8 [num_pages][64][128], uniform on [-127, 127]; every slot
    of every page is drawn (slots past a length are never scored)."""
    n = wl.num_pages * PAGE * INDEX_DIM
    return uniform_int8(stream_key(wl.seed, S_INDEX, layer), _idx(n, device)).view(wl.num_pages, PAGE, INDEX_DIM)


def index_queries(wl: Workload, layer: int = 0, device="cpu") -> torch.Tensor:
    """Each sequence's index query, int8 [B][128], uniform on [-127, 127]."""
    n = wl.batch * INDEX_DIM
    return uniform_int8(stream_key(wl.seed, S_QINDEX, layer), _idx(n, device)).view(wl.batch, INDEX_DIM)


def as_bf16(t: torch.Tensor) -> torch.Tensor:
    """int16 bit patterns -> torch.bfloat16 view (no copy)."""
    return t.view(torch.bfloat16)


def to_numpy_u16(t: torch.Tensor) -> np.ndarray:
    """int16 bit patterns (any device) -> numpy uint16 on the host."""
    return t.detach().cpu().numpy().view(np.uint16)
