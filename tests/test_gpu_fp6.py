"""GPU parity of the ~6-bit cache (FP6 E2M3 codes, one power-of-two scale per row) through the C ABI:
quantization and append byte for byte against the oracle, and decode over the stored numbers
against the oracle's attention on the same numbers, at small sizes (ragged tails, several tiles and
pages, empty sequences, split counts, 64 and 128 heads) and at two full workload sizes."""
import numpy as np
import pytest
import torch

import synth
from oracle import mla_oracle as O
from tests.gpu_cases import BF16_TOL, Gpu, host_inputs, pick, lse_err, rel_err, say, to_host_f64

pytestmark = pytest.mark.gpu

RAGGED = [1, 63, 64, 65, 127, 300, 1000]


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "these tests need the GPU"
    import head_latent_attention_17_amd as L
    return L


def _bits(x) -> np.ndarray:
    """float values exactly representable in bf16 -> their bf16 bit patterns."""
    x = np.asarray(x, np.float32)
    assert np.array_equal(x.view(np.uint32) & 0xFFFF, np.zeros_like(x, np.uint32))
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _crafted_pages() -> np.ndarray:
    """Two pages of rows aimed at the rounding and scale rules."""
    rng = np.random.default_rng(4)
    x = np.zeros((2, 64, 576), np.float32)
    # row 0 stays zero; row 1 plain normal values
    x[0, 1] = rng.normal(0, 1, 576)
    # rows 2-4: exact ties at every grid step with the largest magnitude 7.5 (scale 1)
    for r, (lo, step) in zip((2, 3, 4), ((0.0, 0.125), (2.0, 0.25), (4.0, 0.5))):
        k = rng.integers(0, {0.0: 16, 2.0: 8, 4.0: 7}[lo], 576)
        x[0, r] = (lo + (k + 0.5) * step) * rng.choice([-1.0, 1.0], 576)
        x[0, r, 0] = 7.5
    # row 5: largest magnitude one bf16 step above 7.5 (scale 2)
    x[0, 5] = rng.normal(0, 2, 576)
    x[0, 5, 7] = 7.53125
    # row 6: negative values and negative zeros
    x[0, 6] = -np.abs(rng.normal(0, 1, 576))
    x[0, 6, ::5] = -0.0
    # rows 7-8: very large and very small magnitudes
    x[0, 7] = rng.normal(0, 1, 576) * 2.0 ** 100
    x[0, 8] = rng.normal(0, 1, 576) * 2.0 ** -100
    # row 9: one large value among small ones (the small ones round to zero)
    x[0, 9] = rng.normal(0, 1e-3, 576)
    x[0, 9, 300] = 5000.0
    # the rest, and the second page: normal values at many scales
    x[0, 10:] = rng.normal(0, 1, (54, 576)) * 2.0 ** rng.integers(-20, 20, (54, 1))
    x[1] = rng.normal(0, 1, (64, 576)) * 2.0 ** rng.integers(-8, 8, (64, 1))
    x = (x.view(np.uint32) & 0xFFFF0000).view(np.float32)   # to bf16 (truncation is fine here)
    return _bits(x)


def test_quantize_pages_is_bit_exact(lib):
    """mla_cache_quantize_fp6 against the oracle, byte for byte: crafted rows (ties at every grid
    step, the scale boundary, signed zeros, extreme magnitudes) and a workload's pages with their
    stale slots."""
    wl = synth.make_custom([37, 200, 64], heads=16, seed=81)
    work = synth.to_numpy_u16(synth.cache_pages(wl, 0))
    pages = np.concatenate([_crafted_pages(), work])
    say("quantize", pages.shape[0], "pages")
    src = _to_dev(pages.view(np.int16))
    dst = torch.full((pages.shape[0], lib.FP6_PAGE_BYTES), 0xA5, dtype=torch.uint8, device="cuda")
    lib.mla_cache_quantize_fp6(src.view(torch.bfloat16), dst)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    want = O.quantize_pages_fp6(pages)
    bad = np.argwhere(got != want)
    if bad.size:
        p, b = bad[0]
        say(f"  first mismatch: page {p} byte {b}: got {got[p, b]:#x} want {want[p, b]:#x}")
    assert bad.size == 0


@pytest.mark.parametrize("f32", [False, True])
def test_append_is_bit_exact(lib, f32):
    """mla_cache_append_fp6 writes exactly the oracle's codes and scale at each sequence's position
    and leaves every other byte alone."""
    wl = synth.make_custom([0, 5, 63, 64, 65, 200], heads=16, seed=82, append=True)
    say("append fp6", wl.lens.tolist(), "f32" if f32 else "bf16")
    g = Gpu(wl, f32=f32)
    base = O.quantize_pages_fp6(synth.to_numpy_u16(g.cache.view(torch.int16)))
    cache6 = _to_dev(base)
    lib.mla_cache_append_fp6(cache6, g.bt, g.lens, g.c_new, g.kpe_new)
    torch.cuda.synchronize()
    got = cache6.cpu().numpy()
    rows = synth.to_numpy_u16(synth.new_rows(wl))
    want = base.copy()
    for b, p in enumerate(wl.lens):
        page, slot = wl.block_table[b, p // 64], p % 64
        codes, e = O.quantize_row_fp6(rows[b])
        want[page, slot * 432:(slot + 1) * 432] = O.pack_fp6(codes)
        want[page, 27648 + 4 * slot:27648 + 4 * slot + 4] = np.array([2.0 ** e], np.float32).view(np.uint8)
    assert np.array_equal(got, want)


def _decode_case(lib, wl, splits=0, seqs=None, heads=None):
    """Decode over the oracle-quantized cache; returns the normwise error of o_lat and of lse."""
    g = Gpu(wl)
    seqs = list(range(wl.batch)) if seqs is None else seqs
    hi = host_inputs(wl, 0, seqs)
    # Pages outside the selected sequences are zero; a zero page always quantizes to the same bytes,
    # so only the others go through the quantizer (the same pages as quantizing all of them).
    cache = hi["cache"]
    nz = np.flatnonzero(cache.reshape(cache.shape[0], -1).any(axis=1))
    pages6 = np.repeat(O.quantize_pages_fp6(np.zeros((1,) + cache.shape[1:], cache.dtype)), cache.shape[0], axis=0)
    pages6[nz] = O.quantize_pages_fp6(cache[nz])
    cache6 = _to_dev(pages6)
    lib.mla_decode_fp6(g.q_lat_in, cache6, g.bt, g.attended, wl.scale, g.o_lat, g.lse,
                       g.workspace(lib, splits), splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = O.latent_decode_batch_fp6(hi["q_lat"], pages6, wl.block_table, wl.attended_lens,
                                               wl.scale, batch=seqs, heads=heads)
    hs = list(range(wl.heads)) if heads is None else heads
    sel = np.ix_(seqs, hs)
    o = to_host_f64(g.o_lat)
    e_o = rel_err(o[sel], o_ref[sel])
    lse = g.lse.cpu().numpy()
    e_l = lse_err(lse[sel], lse_ref[sel])
    return e_o, e_l, g


@pytest.mark.parametrize("heads", [64, 128])
def test_decode_matches_oracle(lib, heads):
    wl = synth.make_custom(RAGGED, heads=heads, seed=90 + heads)
    say("decode fp6", heads)
    e_o, e_l, _ = _decode_case(lib, wl)
    say(f"  o_lat err {e_o:.3e}  lse err {e_l:.3e}")
    assert e_o <= BF16_TOL and e_l <= BF16_TOL


@pytest.mark.parametrize("splits", [1, 7, 64, 0])
def test_split_counts(lib, splits):
    """Several segments per work unit and several units per sequence, merged."""
    wl = synth.make_custom(RAGGED + [4096, 2], heads=128, seed=95)
    say("decode fp6 splits", splits)
    e_o, e_l, _ = _decode_case(lib, wl, splits=splits, heads=list(range(0, 128, 9)))
    say(f"  o_lat err {e_o:.3e}  lse err {e_l:.3e}")
    assert e_o <= BF16_TOL and e_l <= BF16_TOL


def test_many_sequences_cost_weighted_cut(lib):
    """300 sequences (every 23rd empty) with at least 8 tiles per unit: the ~6-bit kernel's units
    come from the cost-weighted cut's passes over the lengths, 64 sequences at a time."""
    rng = np.random.default_rng(304)
    lens = [int(x) for x in rng.integers(1, 1200, 300)]
    for i in range(0, len(lens), 23):
        lens[i] = 0
    wl = synth.make_custom(lens, heads=128, seed=304)
    assert sum((n + 31) // 32 for n in lens) >= 8 * min(256, wl.batch * wl.max_blocks)
    say("decode fp6, 300 sequences")
    seqs = [b for b in sorted(set(range(1, wl.batch, 13)) | {wl.batch - 1}) if lens[b] > 0]
    e_o, e_l, g = _decode_case(lib, wl, seqs=seqs, heads=list(range(0, 128, 9)))
    say(f"  o_lat err {e_o:.3e}  lse err {e_l:.3e}")
    assert e_o <= BF16_TOL and e_l <= BF16_TOL
    empty = [b for b in range(wl.batch) if lens[b] == 0]
    assert torch.all(g.o_lat[empty].float() == 0) and torch.all(torch.isneginf(g.lse[empty]))


def test_empty_sequences(lib):
    wl = synth.make_custom([0, 70, 0, 5], heads=128, seed=97)
    say("decode fp6 empty sequences")
    for splits in (0, 3, 8):
        e_o, _, g = _decode_case(lib, wl, splits=splits, seqs=[1, 3])
        o = g.o_lat.float().cpu()
        assert torch.all(o[0] == 0) and torch.all(o[2] == 0)
        assert torch.all(torch.isneginf(g.lse[0])) and torch.all(torch.isneginf(g.lse[2]))
        say(f"  splits {splits}: err {e_o:.3e}")
        assert e_o <= BF16_TOL


def test_lossless_rows_match_the_bf16_path(lib):
    """A cache whose numbers are already code values times a power of two is stored without loss, so
    decode over its ~6-bit form and decode over the bf16 form see the same numbers.  The ~6-bit
    kernel feeds the score product's 576 terms to the matrix cores in another order (32 consecutive
    codes per conversion), so the fp32 sums round differently: the two agree to a few fp32 roundings
    of the scores, far inside the bf16 bound, and any lost or misplaced code or scale would break
    that."""
    wl = synth.make_custom([130, 64, 1000], heads=128, seed=98)
    rng = np.random.default_rng(98)
    n = wl.num_pages
    k = rng.integers(-3, 3, (n, 64, 1)).astype(np.float32)
    vals = O.FP6_VALUES[rng.integers(0, 64, (n, 64, 576))].astype(np.float32) * np.exp2(k)
    vals[:, :, 0] = 7.5 * np.exp2(k[:, :, 0])
    bits = _bits(vals)
    say("lossless rows")
    g = Gpu(wl)
    g.cache.copy_(_to_dev(bits.view(np.int16)).view(torch.bfloat16))
    ws = g.workspace(lib)
    lib.mla_decode(g.q_lat_in, g.cache, g.bt, g.attended, wl.scale, g.o_lat, g.lse, ws)
    torch.cuda.synchronize()
    o16, l16 = g.o_lat.clone(), g.lse.clone()
    cache6 = torch.empty((n, lib.FP6_PAGE_BYTES), dtype=torch.uint8, device="cuda")
    lib.mla_cache_quantize_fp6(g.cache, cache6)
    lib.mla_decode_fp6(g.q_lat_in, cache6, g.bt, g.attended, wl.scale, g.o_lat, g.lse, ws)
    torch.cuda.synchronize()
    e_o = rel_err(g.o_lat.float().cpu(), o16.float().cpu())
    e_l = lse_err(g.lse.cpu(), l16.cpu())
    same = (o16.view(torch.int16) == g.o_lat.view(torch.int16)).float().mean().item()
    say(f"  vs bf16 path: o err {e_o:.3e}  lse err {e_l:.3e}  identical outputs {same:.3f}")
    assert e_o <= 4e-3 and e_l <= 2e-3


@pytest.mark.parametrize("cfg,n_seq,n_heads", [(2, 3, 6), (3, 1, 3)])
def test_full_size(lib, cfg, n_seq, n_heads):
    """The 32 x 4,096-token and 4 x 131,072-token workloads: the GPU quantizes the whole cache with
    mla_cache_quantize_fp6 and decodes it in the launch configuration the benchmark uses; the oracle
    quantizes the sampled sequences' pages itself and checks sampled (sequence, head) pairs."""
    wl = synth.make_config(cfg)
    say(f"fp6 config {cfg}: {wl.name}")
    g = Gpu(wl)
    cache6 = torch.empty((wl.num_pages, lib.FP6_PAGE_BYTES), dtype=torch.uint8, device="cuda")
    lib.mla_cache_quantize_fp6(g.cache, cache6)
    ws = g.workspace(lib)
    del g.cache
    torch.cuda.empty_cache()
    lib.mla_decode_fp6(g.q_lat_in, cache6, g.bt, g.attended, wl.scale, g.o_lat, g.lse, ws, 0)
    torch.cuda.synchronize()
    seqs = pick(wl.batch, n_seq, 300 + cfg)
    heads = pick(wl.heads, n_heads, 400 + cfg)
    o = to_host_f64(g.o_lat)
    lse = g.lse.cpu().numpy()
    del g, cache6, ws
    torch.cuda.empty_cache()
    hi = host_inputs(wl, 0, seqs)
    used = np.unique(np.concatenate([wl.block_table[b][wl.block_table[b] >= 0] for b in seqs]))
    pages6 = np.zeros((wl.num_pages, O.FP6_PAGE_BYTES), np.uint8)
    pages6[used] = O.quantize_pages_fp6(hi["cache"][used])
    o_ref, lse_ref = O.latent_decode_batch_fp6(hi["q_lat"], pages6, wl.block_table, wl.attended_lens,
                                               wl.scale, batch=seqs, heads=heads)
    sel = np.ix_(seqs, heads)
    e_o = rel_err(o[sel], o_ref[sel])
    e_l = lse_err(lse[sel], lse_ref[sel])
    say(f"  o_lat err {e_o:.3e}  lse err {e_l:.3e}")
    assert e_o <= BF16_TOL and e_l <= BF16_TOL
