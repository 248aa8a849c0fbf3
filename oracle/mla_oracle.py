"""CPU oracle for Multi-head Latent Attention (MLA) decode over a paged latent cache.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call this module.  The HIP library never does, and this module imports
nothing from it: the two share only the seeded input generator (``synth``), which holds no attention
arithmetic.

Everything here is plain numpy in float64, written for a reader checking it against the pages:

* "DeepSeek-V2" explainer (aiany.app) -- Step 2 (the attention recipe and the MHA cache bill),
  Step 5 (eq. 9: one latent note c per token, re-inflated by W^UK and W^UV), Step 6 (absorption:
  q.k = (W^Q h).(W^UK c), so the key is never built; W^UV folds into the output side), Step 7
  (decoupled RoPE: a per-head 64-dim q^R and one shared 64-dim rotated k^R, whose score adds to the
  content score inside the softmax) and Step 8 (576 cached numbers per token per layer).
* "DeepSeek-V2" paper breakdown (AI360Xpert), "How It Works": only c_t is cached; at generation time
  it is multiplied by up-projection matrices to rebuild K and V; a separate small RoPE key is kept
  beside it.  That is the *decompressed* form, and it is the form ``decode_reference`` computes.
* "DeepSeek (AI)" wiki, "KV cache compression": one key-value vector per (token, layer) instead of a
  key and a value per head, a cut of (d_K + d_V)/d_KV times the head count.

Layouts (the library's, restated so the oracle stands alone):
  cache        uint16 (bf16 bits) [num_pages][page_size][d_c + d_R]; a row is [c | k^R]
  block_table  int32 [B][max_blocks]; token t of sequence b sits in page block_table[b][t // page],
               slot t % page
  q            [B][H][d_nope + d_R] = [q_nope | q^R] (q^R and k^R arrive already rotated)
  W_UK         [H][d_nope][d_c]:  content key of head h is k_h = W_UK[h] @ c
  W_UV         [H][d_c][d_v]:     value of head h is v_h = c @ W_UV[h]
  q_abs        [B][H][d_c + d_R] = [W_UK[h]^T q_nope | q^R], the query in latent form

Readings where the pages are silent (each also listed in the design notes):
  * the softmax scale is an argument (the score formula of Step 7 did not survive extraction);
  * decode has one query that attends to every cached token of its sequence, position 0 .. len-1,
    including the row appended this step -- no mask inside that range;
  * a sequence of length 0 yields o = 0 and lse = -inf;
  * lse is the natural log of the softmax denominator of the *scaled* scores;
  * the ~6-bit cache (the explainer's audit after Step 8 gives only "about six bits" per number) is
    FP6 E2M3 codes with one power-of-two scale per row, rounded to nearest with ties to even.

Every function here is pinned by a test in ``tests/test_oracle_*.py`` against the explainer's worked
2-D example (Step 6), its cache arithmetic (Steps 2 and 8), brute-force loops on tiny shapes, closed
forms and invariants.
"""
from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------------------------------------------
# bf16 storage
# --------------------------------------------------------------------------------------------------


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16/int16) -> float64, exactly (bf16 is the top half of a float32)."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------------------------------
# Paged cache bookkeeping (integer, exact)
# --------------------------------------------------------------------------------------------------


def page_and_slot(block_table: np.ndarray, b: int, t, page_size: int):
    """Physical (page, slot) of logical token t of sequence b."""
    t = np.asarray(t)
    return block_table[b, t // page_size], t % page_size


def gather_rows(cache: np.ndarray, block_table: np.ndarray, b: int, length: int) -> np.ndarray:
    """The ``length`` cached rows of sequence b in logical order (raw stored values, no arithmetic)."""
    page_size = cache.shape[1]
    pages, slots = page_and_slot(block_table, b, np.arange(length), page_size)
    if length and (pages < 0).any():
        raise ValueError("block table has no page for a token inside the sequence")
    return cache[pages, slots]


def append_rows(cache: np.ndarray, block_table: np.ndarray, positions, new_rows) -> np.ndarray:
    """Return a copy of ``cache`` with new_rows[b] stored at logical position positions[b] of
    sequence b (each new token's note is written once and never changes: explainer Step 2)."""
    out = cache.copy()
    page_size = cache.shape[1]
    for b, p in enumerate(np.asarray(positions)):
        page, slot = page_and_slot(block_table, b, int(p), page_size)
        if page < 0:
            raise ValueError("block table has no page for the appended position")
        out[page, slot] = new_rows[b]
    return out


# --------------------------------------------------------------------------------------------------
# The method in decompressed form (breakdown "How It Works"; explainer Steps 5 and 7)
# --------------------------------------------------------------------------------------------------


def softmax_attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    """Textbook attention for one query (explainer Step 2): score every key, softmax, mix values.

    Returns (out, lse, p).  For zero keys: out = 0, lse = -inf, p empty."""
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1]), -math.inf, np.zeros(0)
    s = scale * (keys @ q)
    m = s.max()
    e = np.exp(s - m)
    z = e.sum()
    p = e / z
    return p @ values, m + math.log(z), p


def decompress_head(rows: np.ndarray, w_uk_h: np.ndarray, w_uv_h: np.ndarray, d_c: int):
    """Rebuild one head's content keys and values from the cached notes (explainer Step 5;
    breakdown "How It Works" step 3): K[t] = W_UK[h] @ c_t, V[t] = c_t @ W_UV[h]."""
    c = rows[:, :d_c]
    return c @ w_uk_h.T, c @ w_uv_h


def decode_head(q_h: np.ndarray, rows: np.ndarray, w_uk_h: np.ndarray, w_uv_h: np.ndarray,
                scale: float):
    """One head, one sequence, decompressed form.

    The full key of token t is [W_UK[h] c_t | k^R_t] and the query is [q_nope | q^R]; their dot
    product is the content score plus the position score, the two channels adding inside the
    softmax (explainer Step 7).  k^R is the same for every head (Step 7).  Returns (out, lse, p)."""
    d_nope, d_c = w_uk_h.shape
    k_nope, v = decompress_head(rows, w_uk_h, w_uv_h, d_c)
    keys = np.concatenate([k_nope, rows[:, d_c:]], axis=1)
    assert keys.shape[1] == q_h.shape[0]
    return softmax_attention(q_h, keys, v, scale)


# --------------------------------------------------------------------------------------------------
# Plain definitions of the absorbed pieces (explainer Step 6)
# --------------------------------------------------------------------------------------------------


def absorb_query(q_h: np.ndarray, w_uk_h: np.ndarray) -> np.ndarray:
    """[q_nope | q^R] -> [W_UK[h]^T q_nope | q^R]: the content query moved into latent space, so that
    q_lat . c_t equals q_nope . (W_UK[h] c_t) without building the key (explainer Step 6)."""
    d_nope = w_uk_h.shape[0]
    return np.concatenate([w_uk_h.T @ q_h[:d_nope], q_h[d_nope:]])


def latent_attention(q_abs_h: np.ndarray, rows: np.ndarray, d_c: int, scale: float):
    """Attention of a latent-form query against the cached rows themselves: score = q_abs . row,
    values = the latent notes c_t.  Returns (o_lat, lse, p)."""
    return softmax_attention(q_abs_h, rows, rows[:, :d_c], scale)


def up_project(o_lat_h: np.ndarray, w_uv_h: np.ndarray) -> np.ndarray:
    """Per-head value up-projection applied after the weighted sum: o_lat @ W_UV[h]."""
    return o_lat_h @ w_uv_h


def merge_partials(outs, lses):
    """Combine attention over disjoint token sets: each part carries its normalised output and the
    log of its softmax denominator.  L = log sum_s e^{lse_s}; o = sum_s e^{lse_s - L} o_s."""
    lses = np.asarray(lses, dtype=np.float64)
    outs = np.asarray(outs, dtype=np.float64)
    if np.all(np.isneginf(lses)):
        return np.zeros(outs.shape[1:]), -math.inf
    m = lses.max()
    w = np.exp(lses - m)
    big_l = m + math.log(w.sum())
    return np.tensordot(np.exp(lses - big_l), outs, axes=1), big_l


# --------------------------------------------------------------------------------------------------
# Batched drivers
# --------------------------------------------------------------------------------------------------


def _sel(n, subset):
    return range(n) if subset is None else list(subset)


def absorb_batch(q, w_uk, batch=None, heads=None) -> np.ndarray:
    """q_abs[b][h] for the selected (b, h); other entries NaN.  Inputs are bf16 bits or floats."""
    q = _f64(q)
    w_uk = _f64(w_uk)
    B, H, _ = q.shape
    d_c = w_uk.shape[2]
    out = np.full((B, H, d_c + q.shape[2] - w_uk.shape[1]), np.nan)
    for b in _sel(B, batch):
        for h in _sel(H, heads):
            out[b, h] = absorb_query(q[b, h], w_uk[h])
    return out


def out_proj_batch(o_lat, w_uv, batch=None, heads=None) -> np.ndarray:
    o_lat = _f64(o_lat)
    w_uv = _f64(w_uv)
    B, H, _ = o_lat.shape
    out = np.full((B, H, w_uv.shape[2]), np.nan)
    for b in _sel(B, batch):
        for h in _sel(H, heads):
            out[b, h] = up_project(o_lat[b, h], w_uv[h])
    return out


def latent_decode_batch(q_abs, cache, block_table, seq_lens, scale, d_c=512, batch=None,
                        heads=None):
    """Reference for the latent-space decode step: o_lat [B][H][d_c] and lse [B][H]."""
    q_abs = _f64(q_abs)
    B, H, _ = q_abs.shape
    o = np.full((B, H, d_c), np.nan)
    lse = np.full((B, H), np.nan)
    for b in _sel(B, batch):
        rows = _f64(gather_rows(cache, block_table, b, int(seq_lens[b])))
        for h in _sel(H, heads):
            o[b, h], lse[b, h], _ = latent_attention(q_abs[b, h], rows, d_c, scale)
    return o, lse


def decode_reference(q, cache, block_table, seq_lens, w_uk, w_uv, scale, batch=None, heads=None):
    """End-to-end reference, decompressed form: out [B][H][d_v] and lse [B][H]."""
    q = _f64(q)
    w_uk = _f64(w_uk)
    w_uv = _f64(w_uv)
    B, H, _ = q.shape
    out = np.full((B, H, w_uv.shape[2]), np.nan)
    lse = np.full((B, H), np.nan)
    for b in _sel(B, batch):
        rows = _f64(gather_rows(cache, block_table, b, int(seq_lens[b])))
        for h in _sel(H, heads):
            out[b, h], lse[b, h], _ = decode_head(q[b, h], rows, w_uk[h], w_uv[h], scale)
    return out, lse


def _f64(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype in (np.uint16, np.int16):
        return bf16_to_f64(x)
    return x.astype(np.float64)


# --------------------------------------------------------------------------------------------------
# The producer side of the cache (explainer Step 5, eq. 9; Step 7)
# --------------------------------------------------------------------------------------------------


def rope_rotate(x, position, base: float) -> np.ndarray:
    """Rotary position embedding of one vector (explainer Step 7: each query and key is rotated by an
    angle proportional to its position, so that a score depends only on how far apart the two tokens
    are).  Reading -- the pages give neither the frequencies nor the pairing: consecutive pairs
    (x[2i], x[2i+1]) turn by position * base^(-2i/d) radians, the plain rotary form with no
    context-extension rescaling."""
    x = _f64(x)
    d = x.shape[-1]
    out = np.empty_like(x)
    for i in range(d // 2):
        angle = float(position) * base ** (-2.0 * i / d)
        c, s = math.cos(angle), math.sin(angle)
        out[..., 2 * i] = x[..., 2 * i] * c - x[..., 2 * i + 1] * s
        out[..., 2 * i + 1] = x[..., 2 * i] * s + x[..., 2 * i + 1] * c
    return out


def latent_row(h, w_dkv, w_kr, position, base: float) -> np.ndarray:
    """The cache row one token contributes, [c | k^R] (explainer Step 5, eq. 9: the hidden vector is
    squeezed to the latent note c = W^DKV h, 5,120 -> 512; Step 7: plus one 64-dim rotated key k^R
    shared by all heads).  Reading: k^R = RoPE(W^KR h) with W^KR a 5,120 -> 64 projection; the
    weights are stored [5120][512] and [5120][64], so both products are h @ W."""
    h = _f64(h)
    c = h @ _f64(w_dkv)
    k = rope_rotate(h @ _f64(w_kr), position, base)
    return np.concatenate([c, k])


def latent_rows_batch(h, w_dkv, w_kr, positions, base: float) -> np.ndarray:
    """latent_row for every sequence b: token positions[b] with hidden vector h[b]; [B][576]."""
    return np.stack([latent_row(h[b], w_dkv, w_kr, int(positions[b]), base) for b in range(len(positions))])


# --------------------------------------------------------------------------------------------------
# The output projection to the hidden width (explainer Step 6: the heads' outputs are concatenated
# and mixed by W^O, and W^UV can be folded into it)
# --------------------------------------------------------------------------------------------------


def hidden_out(out_heads, w_o) -> np.ndarray:
    """out_heads [B][H][d_v] concatenated per sequence (head-major) times W^O [H * d_v][d_model]:
    the attention block's output in the hidden width.  Reading: W^O is stored input-major, as the
    other weights here, so the product is out @ W^O."""
    o = _f64(out_heads)
    B = o.shape[0]
    return o.reshape(B, -1) @ _f64(w_o)


def hidden_out_folded(o_lat, w_uv, w_o) -> np.ndarray:
    """The same output with W^UV folded into W^O first (Step 6): per head the 512 x d_model matrix
    W^UV[h] W^O[h], applied to the latent-form output o_lat [B][H][512]."""
    o_lat, w_uv, w_o = _f64(o_lat), _f64(w_uv), _f64(w_o)
    B, H, _ = o_lat.shape
    d_v = w_uv.shape[2]
    out = np.zeros((B, w_o.shape[1]))
    for h in range(H):
        folded = w_uv[h] @ w_o[h * d_v:(h + 1) * d_v]        # [512][d_model]
        out += o_lat[:, h] @ folded
    return out


# --------------------------------------------------------------------------------------------------
# Attention over the top-k tokens of a cheap index (wiki "KV cache data movement minimization":
# score every token's cheap index vector against the query, keep the k best, and run attention
# over those rows only)
# --------------------------------------------------------------------------------------------------

INDEX_DIM = 128   # reading: 128 int8 numbers per token's index vector


def index_scores(index_cache, block_table, b: int, length: int, q_index) -> np.ndarray:
    """Exact integer scores q_index . i_t of sequence b's tokens t < length (int8 vectors, so the
    scores are exact in int64)."""
    pages, slots = page_and_slot(block_table, b, np.arange(length), index_cache.shape[1])
    vecs = np.asarray(index_cache)[pages, slots].astype(np.int64)          # [length][128]
    return vecs @ np.asarray(q_index).astype(np.int64)


def top_k_positions(scores, k: int) -> np.ndarray:
    """The k highest-scoring positions (all of them when there are at most k), ties going to the
    earlier position; returned in increasing position order."""
    scores = np.asarray(scores)
    n = scores.shape[0]
    if n <= k:
        return np.arange(n)
    order = sorted(range(n), key=lambda t: (-int(scores[t]), t))
    return np.sort(np.array(order[:k]))


def sparse_latent_decode(q_abs, cache, block_table, seq_lens, index_cache, q_index, k: int, scale,
                         d_c=512, batch=None, heads=None):
    """Latent decode over each sequence's top-k tokens only: (o_lat [B][H][d_c], lse [B][H],
    positions per sequence)."""
    q_abs = _f64(q_abs)
    B, H, _ = q_abs.shape
    o = np.full((B, H, d_c), np.nan)
    lse = np.full((B, H), np.nan)
    chosen = {}
    for b in _sel(B, batch):
        n = int(seq_lens[b])
        pos = top_k_positions(index_scores(index_cache, block_table, b, n, q_index[b]), k)
        chosen[b] = pos
        pg, sl = page_and_slot(block_table, b, pos, cache.shape[1])
        rows = _f64(np.asarray(cache)[pg, sl]) if len(pos) else np.zeros((0, cache.shape[2]))
        for h in _sel(H, heads):
            o[b, h], lse[b, h], _ = latent_attention(q_abs[b, h], rows, d_c, scale)
    return o, lse, chosen


# --------------------------------------------------------------------------------------------------
# A ~6-bit cache (explainer, the audit after Step 8: deployed V2 stores each cached number in about
# six bits, near 26 KB per token over its 60 layers).  The pages give no format; the reading here:
# each number is an FP6 E2M3 code (1 sign, 2 exponent, 3 mantissa bits, exponent bias 1, no
# infinities or NaN: magnitudes 0, 1/8 .. 7/8, then 1 .. 7.5), and each cached row carries one
# power-of-two scale, so a stored number is code_value * 2^e exactly.
# --------------------------------------------------------------------------------------------------

FP6_ROW_BYTES = 576 * 6 // 8                   # 432: the row's codes, code i at bits 6i .. 6i+5
FP6_PAGE_TOKENS = 64
FP6_PAGE_BYTES = FP6_PAGE_TOKENS * FP6_ROW_BYTES + FP6_PAGE_TOKENS * 4   # rows, then 64 fp32 scales
FP6_MAX = 7.5
FP6_MIN_EXP = -126                             # scales stay normal float32 numbers


def fp6_e2m3_value(code: int) -> float:
    """The number a 6-bit E2M3 code stands for, from the format's fields: exponent field 0 is the
    subnormal range m/8; exponent field e > 0 is (1 + m/8) * 2^(e - 1)."""
    sign = -1.0 if code & 0b100000 else 1.0
    e = (code >> 3) & 0b11
    m = code & 0b111
    mag = m / 8.0 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 1)
    return sign * mag


FP6_VALUES = np.array([fp6_e2m3_value(c) for c in range(64)])


def fp6_e2m3_round(y) -> np.ndarray:
    """Codes of the E2M3 numbers nearest to y (float64 array): ties go to the code with an even
    mantissa, magnitudes beyond 7.5 saturate to 7.5, and the sign is kept (also for zero).  Written
    as a search among the 32 magnitudes (the two neighbours of |y| in the sorted table), not as bit
    arithmetic."""
    y = np.asarray(y, dtype=np.float64)
    mags = FP6_VALUES[:32]                      # codes 0 .. 31, increasing magnitudes
    a = np.minimum(np.abs(y), FP6_MAX)
    hi = np.clip(np.searchsorted(mags, a, side="left"), 1, 31)   # mags[hi - 1] < a <= mags[hi]
    lo = hi - 1
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    code = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    return (code | np.where(np.signbit(y), 32, 0)).astype(np.uint8)


def fp6_row_exponent(amax: float) -> int:
    """The smallest e >= -126 with amax <= 7.5 * 2^e: the row's largest magnitude then maps into
    (3.75, 7.5] and nothing saturates (a row of zeros takes e = -126)."""
    e = FP6_MIN_EXP
    while amax > FP6_MAX * 2.0 ** e:
        e += 1
    return e


def fp6_row_exponents(amax) -> np.ndarray:
    """fp6_row_exponent for many rows at once: a guess from log2, then corrected with the same exact
    comparisons (amax <= 7.5 * 2^e, and not for e - 1)."""
    amax = np.asarray(amax, dtype=np.float64)
    with np.errstate(divide="ignore"):
        e = np.ceil(np.log2(np.maximum(amax, 1e-300) / FP6_MAX))
    e = np.clip(e, FP6_MIN_EXP, 200).astype(np.int64)
    for _ in range(2):
        e = np.where(amax > FP6_MAX * np.exp2(e.astype(np.float64)), e + 1, e)
        e = np.where((e > FP6_MIN_EXP) & (amax <= FP6_MAX * np.exp2(e - 1.0)), e - 1, e)
    return e


def quantize_row_fp6(row) -> tuple[np.ndarray, int]:
    """(codes [576], e) of one cached row: codes round row / 2^e to the nearest E2M3 numbers.  Dividing
    by a power of two is exact, so the only rounding is the code choice."""
    x = _f64(row)
    e = fp6_row_exponent(float(np.max(np.abs(x))) if x.size else 0.0)
    return fp6_e2m3_round(x / 2.0 ** e), e


def pack_fp6(codes) -> np.ndarray:
    """Codes [..., n] (n a multiple of 4) -> bytes [..., 3n/4]: code i occupies bits 6i .. 6i+5 of the
    little-endian bit string (bit k of the string is bit k % 8 of byte k // 8)."""
    codes = np.asarray(codes, dtype=np.uint8)
    bits = (codes[..., :, None] >> np.arange(6)) & 1          # [..., n, 6], least significant first
    bits = bits.reshape(*codes.shape[:-1], -1, 8)             # [..., 3n/4, 8]
    return (bits << np.arange(8)).sum(axis=-1).astype(np.uint8)


def unpack_fp6(data) -> np.ndarray:
    """Inverse of pack_fp6."""
    data = np.asarray(data, dtype=np.uint8)
    bits = (data[..., :, None] >> np.arange(8)) & 1
    bits = bits.reshape(*data.shape[:-1], -1, 6)
    return (bits << np.arange(6)).sum(axis=-1).astype(np.uint8)


def quantize_pages_fp6(pages) -> np.ndarray:
    """bf16 pages [n][64][576] -> fp6 pages [n][27904] bytes: 64 packed rows of 432 bytes, then the
    64 row scales 2^e as little-endian float32.  Each row as quantize_row_fp6, many rows at once."""
    pages = np.asarray(pages)
    n = pages.shape[0]
    out = np.zeros((n, FP6_PAGE_BYTES), np.uint8)
    for i0 in range(0, n, 64):
        x = _f64(pages[i0:i0 + 64])                                  # [k][64][576]
        e = fp6_row_exponents(np.abs(x).max(axis=2))                 # [k][64]
        codes = fp6_e2m3_round(x / np.exp2(e.astype(np.float64))[..., None])
        k = x.shape[0]
        out[i0:i0 + k, :FP6_PAGE_TOKENS * FP6_ROW_BYTES] = pack_fp6(codes).reshape(k, -1)
        out[i0:i0 + k, FP6_PAGE_TOKENS * FP6_ROW_BYTES:] = \
            np.exp2(e.astype(np.float64)).astype(np.float32).view(np.uint8).reshape(k, -1)
    return out


def dequantize_rows_fp6(pages6, page_ids, slots) -> np.ndarray:
    """Stored rows (page_ids[k], slots[k]) of fp6 pages as float64 [k][576]: code value * scale."""
    pages6 = np.asarray(pages6, dtype=np.uint8)
    page_ids = np.asarray(page_ids)
    slots = np.asarray(slots)
    rows = np.stack([pages6[p, s * FP6_ROW_BYTES:(s + 1) * FP6_ROW_BYTES] for p, s in zip(page_ids, slots)]) \
        if len(page_ids) else np.zeros((0, FP6_ROW_BYTES), np.uint8)
    off = FP6_PAGE_TOKENS * FP6_ROW_BYTES
    scales = np.array([pages6[p, off + 4 * s:off + 4 * s + 4].view(np.float32)[0] for p, s in zip(page_ids, slots)],
                      dtype=np.float64)
    return FP6_VALUES[unpack_fp6(rows)] * scales[:, None]


def latent_decode_batch_fp6(q_abs, pages6, block_table, seq_lens, scale, d_c=512, batch=None,
                            heads=None):
    """The latent-space decode over an fp6 cache: the same attention as latent_decode_batch, on the
    numbers the cache stores (each row dequantized exactly)."""
    q_abs = _f64(q_abs)
    B, H, _ = q_abs.shape
    o = np.full((B, H, d_c), np.nan)
    lse = np.full((B, H), np.nan)
    for b in _sel(B, batch):
        n = int(seq_lens[b])
        pg, sl = page_and_slot(block_table, b, np.arange(n), FP6_PAGE_TOKENS)
        if n and (pg < 0).any():
            raise ValueError("block table has no page for a token inside the sequence")
        rows = dequantize_rows_fp6(pages6, pg, sl)
        for h in _sel(H, heads):
            o[b, h], lse[b, h], _ = latent_attention(q_abs[b, h], rows, d_c, scale)
    return o, lse


# --------------------------------------------------------------------------------------------------
# Cache arithmetic (explainer Steps 2 and 8; wiki "KV cache compression")
# --------------------------------------------------------------------------------------------------


def mha_numbers_per_token(heads: int, head_dim: int, layers: int) -> int:
    """Standard multi-head caching: one key and one value per head per layer (explainer Step 2)."""
    return 2 * heads * head_dim * layers


def mla_numbers_per_token(d_c: int, d_r: int, layers: int) -> int:
    """MLA caching: the latent note plus the shared RoPE key, per layer (explainer Step 8)."""
    return (d_c + d_r) * layers


def cache_bytes(numbers: int, bits_per_number: float) -> float:
    return numbers * bits_per_number / 8.0


def gqa_equivalent_groups(d_c: int, d_r: int, head_dim: int) -> float:
    """GQA with g groups caches 2 * g * head_dim numbers per layer; the g that matches MLA's row."""
    return (d_c + d_r) / (2.0 * head_dim)


def gqa_numbers_per_token(groups: int, head_dim: int, layers: int) -> int:
    """Grouped-query caching: one key and one value per group per layer (explainer Step 4)."""
    return 2 * groups * head_dim * layers


def wiki_reduction_factor(d_k: int, d_v: int, d_kv: int, heads: int) -> float:
    """(d_K + d_V) / d_KV x heads (wiki "KV cache compression")."""
    return (d_k + d_v) / d_kv * heads
