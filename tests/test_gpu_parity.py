"""GPU parity of the HIP path (through the C ABI) against the CPU oracle, at small sizes that still
span several 32-token tiles, several pages and a ragged tail; plus the exact cases: append bytes,
the needle, page-permutation invariance, empty sequences and determinism."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import mla_oracle as O
from tests.gpu_cases import BF16_TOL, F32_TOL, Gpu, act, host_inputs, lse_err, rel_err, say, to_host_f64

pytestmark = pytest.mark.gpu

RAGGED = [1, 63, 64, 65, 127, 300, 1000]


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "these tests need the GPU"
    import head_latent_attention_17_amd as L
    return L


def _tol(f32):
    return F32_TOL if f32 else BF16_TOL


@pytest.mark.parametrize("f32", [False, True])
def test_append_is_bit_exact(lib, f32):
    wl = synth.make_custom([0, 5, 63, 64, 65, 200], heads=16, seed=21, append=True)
    say("append", wl.lens.tolist(), "f32" if f32 else "bf16")
    g = Gpu(wl, f32=f32)
    before = synth.to_numpy_u16(g.cache.view(torch.int16))
    lib.mla_cache_append(g.cache, g.bt, g.lens, g.c_new, g.kpe_new)
    torch.cuda.synchronize()
    after = synth.to_numpy_u16(g.cache.view(torch.int16))
    rows = synth.to_numpy_u16(synth.new_rows(wl))
    want = O.append_rows(before, wl.block_table, wl.lens, rows)
    assert np.array_equal(after, want)


@pytest.mark.parametrize("heads", [16, 32, 64, 128])
@pytest.mark.parametrize("f32", [False, True])
def test_decode_matches_oracle(lib, heads, f32):
    wl = synth.make_custom(RAGGED, heads=heads, seed=30 + heads)
    say("decode", heads, "f32" if f32 else "bf16")
    g = Gpu(wl, f32=f32)
    g.step(lib, q_abs_from_absorb=False)
    torch.cuda.synchronize()
    hi = host_inputs(wl, 0, range(wl.batch))
    o_ref, lse_ref = O.latent_decode_batch(hi["q_lat"], hi["cache"], wl.block_table, wl.attended_lens, wl.scale)
    e_o = rel_err(to_host_f64(g.o_lat), o_ref)
    e_l = lse_err(g.lse.cpu().numpy(), lse_ref)
    say(f"  o_lat err {e_o:.3e}  lse err {e_l:.3e}")
    assert e_o <= _tol(f32) and e_l <= _tol(f32)


@pytest.mark.parametrize("splits", [1, 2, 7, 64, 0])
def test_split_count_invariance(lib, splits):
    wl = synth.make_custom(RAGGED + [4096, 2], heads=128, seed=41)
    say("splits", splits)
    g = Gpu(wl)
    g.step(lib, splits=splits, q_abs_from_absorb=False)
    torch.cuda.synchronize()
    hi = host_inputs(wl, 0, range(wl.batch))
    o_ref, lse_ref = O.latent_decode_batch(hi["q_lat"], hi["cache"], wl.block_table, wl.attended_lens,
                                           wl.scale, heads=range(0, 128, 9))
    hs = list(range(0, 128, 9))
    e = rel_err(to_host_f64(g.o_lat)[:, hs], o_ref[:, hs])
    say(f"  err {e:.3e}")
    assert e <= BF16_TOL
    assert lse_err(g.lse.cpu().numpy()[:, hs], lse_ref[:, hs]) <= BF16_TOL


@pytest.mark.parametrize("splits", [1, 5, 0, 300])
def test_sixteen_heads_tile_cut(lib, splits):
    """The 16-head kernel cuts the batch's 32-token tiles over min(units, tiles) units: 70 sequences
    (more than one 64-sequence pass over the lengths), every 9th empty, ragged lengths, with one
    unit, a few, the automatic count and more units than tiles.  Sampled sequences against the
    oracle on all 16 heads, the empty ones exactly zero with lse -inf, and the result of every cut
    within rounding of the one-unit cut."""
    rng = np.random.default_rng(316)
    lens = [int(x) for x in rng.integers(1, 200, 70)]
    for i in range(0, len(lens), 9):
        lens[i] = 0
    lens[5] = 1
    lens[6] = 32
    lens[7] = 33
    wl = synth.make_custom(lens, heads=16, seed=316)
    tiles = sum((n + 31) // 32 for n in lens)
    assert splits < tiles or splits == 300 and splits > tiles
    say("16 heads, tile cut", wl.batch, "tiles", tiles, "splits", splits)
    g = Gpu(wl)
    g.step(lib, splits=splits, q_abs_from_absorb=False)
    torch.cuda.synchronize()
    sel = [b for b in sorted(set(range(1, wl.batch, 4)) | {5, 6, 7, wl.batch - 1}) if lens[b] > 0]
    hi = host_inputs(wl, 0, sel)
    o_ref, lse_ref = O.latent_decode_batch(hi["q_lat"], hi["cache"], wl.block_table, wl.attended_lens,
                                           wl.scale, batch=sel)
    o = to_host_f64(g.o_lat)
    e = rel_err(o[sel], o_ref[sel])
    e_l = lse_err(g.lse.cpu().numpy()[sel], lse_ref[sel])
    say(f"  err {e:.3e}  lse err {e_l:.3e}")
    assert e <= BF16_TOL and e_l <= BF16_TOL
    empty = [b for b in range(wl.batch) if lens[b] == 0]
    assert np.all(o[empty] == 0) and torch.all(torch.isneginf(g.lse[empty]))
    g1 = Gpu(wl)
    g1.step(lib, splits=1, q_abs_from_absorb=False)
    torch.cuda.synchronize()
    assert rel_err(to_host_f64(g.o_lat)[sel], to_host_f64(g1.o_lat)[sel]) <= BF16_TOL


@pytest.mark.parametrize("splits", [0, 97])
def test_many_sequences_cost_weighted_cut(lib, splits):
    """300 sequences of mixed lengths, every 23rd empty, with at least 8 tiles per unit: the units
    are cut by cost over 32-token tiles, in passes over the lengths 64 sequences at a time (more
    than 256 sequences).  Every sequence must still be covered exactly once by its pieces: sampled
    sequences against the oracle, the empty ones exactly zero with lse -inf."""
    rng = np.random.default_rng(303)
    lens = [int(x) for x in rng.integers(1, 1200, 300)]
    for i in range(0, len(lens), 23):
        lens[i] = 0
    wl = synth.make_custom(lens, heads=128, seed=303)
    tiles = sum((n + 31) // 32 for n in lens)
    units = splits or min(256, wl.batch * wl.max_blocks)
    assert tiles >= 8 * units, "the workload must take the cost-weighted cut"
    say("many sequences", wl.batch, "tiles", tiles, "units", units)
    g = Gpu(wl)
    g.step(lib, splits=splits, q_abs_from_absorb=False)
    torch.cuda.synchronize()
    sel = [b for b in sorted(set(range(1, wl.batch, 11)) | {wl.batch - 1}) if lens[b] > 0]
    hs = list(range(0, 128, 9))
    hi = host_inputs(wl, 0, sel)
    o_ref, lse_ref = O.latent_decode_batch(hi["q_lat"], hi["cache"], wl.block_table, wl.attended_lens,
                                           wl.scale, batch=sel, heads=hs)
    o = to_host_f64(g.o_lat)
    e = rel_err(o[sel][:, hs], o_ref[sel][:, hs])
    e_l = lse_err(g.lse.cpu().numpy()[sel][:, hs], lse_ref[sel][:, hs])
    say(f"  err {e:.3e}  lse err {e_l:.3e}")
    assert e <= BF16_TOL and e_l <= BF16_TOL
    empty = [b for b in range(wl.batch) if lens[b] == 0]
    assert np.all(o[empty] == 0) and torch.all(torch.isneginf(g.lse[empty]))


@pytest.mark.parametrize("f32", [False, True])
def test_end_to_end_with_append_matches_decompressed_oracle(lib, f32):
    wl = synth.make_custom([1, 64, 200, 777], heads=128, seed=51, append=True)
    say("end-to-end", "f32" if f32 else "bf16")
    g = Gpu(wl, f32=f32)
    g.step(lib)
    torch.cuda.synchronize()
    hi = host_inputs(wl, 0, range(wl.batch))
    out_ref, lse_ref = O.decode_reference(hi["q"], hi["cache"], wl.block_table, wl.attended_lens,
                                          hi["w_uk"], hi["w_uv"], wl.scale)
    q_abs_ref = O.absorb_batch(hi["q"], hi["w_uk"])
    e_q = rel_err(to_host_f64(g.q_abs), q_abs_ref)
    e_out = rel_err(to_host_f64(g.out), out_ref)
    e_l = lse_err(g.lse.cpu().numpy(), lse_ref)
    say(f"  q_abs {e_q:.3e} out {e_out:.3e} lse {e_l:.3e}")
    assert e_q <= _tol(f32) and e_out <= _tol(f32) and e_l <= _tol(f32)


@pytest.mark.parametrize("f32", [False, True])
def test_out_proj_matches_oracle(lib, f32):
    wl = synth.make_custom([5] * 9, heads=64, seed=61)
    say("out_proj", "f32" if f32 else "bf16")
    g = Gpu(wl, f32=f32)
    o_in = g.q_lat_in[..., :synth.D_C].contiguous()   # any seeded bf16 input of the right shape
    lib.mla_out_proj(o_in, g.w_uv, g.out)
    torch.cuda.synchronize()
    _, w_uv = synth.weights(wl)
    ref = O.out_proj_batch(synth.to_numpy_u16(synth.latent_queries(wl))[..., :synth.D_C],
                           synth.to_numpy_u16(w_uv))
    e = rel_err(to_host_f64(g.out), ref)
    say(f"  err {e:.3e}")
    assert e <= _tol(f32)


@pytest.mark.parametrize("heads,batch", [(16, 3), (128, 32), (32, 33), (128, 64), (128, 65), (16, 130),
                                         (128, 130)])
def test_projections_batch_blocks(lib, heads, batch):
    """Absorption and out-projection (bf16) against the oracle with 16, 32 and 128 heads: batch 3 and
    32 (one 32-row block), 33 and 64 (one 64-row pass of the absorption with two blocks), 65 (the
    absorption's second pass holds one row; three blocks in one pass of the out-projection's
    four-block kernel) and 130 (three absorption passes, the last with two rows; five blocks, two
    passes of the out-projection)."""
    wl = synth.make_custom([3] * batch, heads=heads, seed=62 + batch)
    say("projections", heads, batch)
    g = Gpu(wl)
    lib.mla_absorb_q(g.q, g.w_uk, g.q_abs)
    o_in = g.q_lat_in[..., :synth.D_C].contiguous()
    lib.mla_out_proj(o_in, g.w_uv, g.out)
    torch.cuda.synchronize()
    q = synth.to_numpy_u16(synth.queries(wl))
    w_uk, w_uv = (synth.to_numpy_u16(w) for w in synth.weights(wl))
    e_q = rel_err(to_host_f64(g.q_abs), O.absorb_batch(q, w_uk))
    e_o = rel_err(to_host_f64(g.out), O.out_proj_batch(synth.to_numpy_u16(synth.latent_queries(wl))[..., :synth.D_C],
                                                       w_uv))
    say(f"  q_abs {e_q:.3e} out {e_o:.3e}")
    assert e_q <= BF16_TOL and e_o <= BF16_TOL


@pytest.mark.parametrize("heads", [16, 128])
def test_empty_sequences(lib, heads):
    """Empty sequences give zeros and lse = -inf.  With 8 splits of 3 pages most work units hold no
    page (and write nothing) yet sit inside a sequence's unit range; the merges must skip them."""
    wl = synth.make_custom([0, 70, 0, 5], heads=heads, seed=71)
    say("empty sequences", heads)
    g = Gpu(wl)
    hi = host_inputs(wl, 0, range(wl.batch))
    o_ref, lse_ref = O.latent_decode_batch(hi["q_lat"], hi["cache"], wl.block_table, wl.attended_lens,
                                           wl.scale, batch=[1, 3])
    for splits in (0, 3, 8):
        g.o_lat.fill_(7.0)
        g.step(lib, splits=splits, q_abs_from_absorb=False)
        torch.cuda.synchronize()
        o = g.o_lat.float().cpu()
        assert torch.all(o[0] == 0) and torch.all(o[2] == 0)
        assert torch.all(torch.isneginf(g.lse[0])) and torch.all(torch.isneginf(g.lse[2]))
        e = rel_err(to_host_f64(g.o_lat)[[1, 3]], o_ref[[1, 3]])
        say(f"  splits {splits}: err {e:.3e}")
        assert e <= BF16_TOL


@pytest.mark.parametrize("heads", [16, 32, 64, 128])
@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("splits", [0, 1, 7])
def test_needle_is_bit_exact(lib, heads, f32, splits):
    """A RoPE-only query matching one token's k^R: every other weight underflows to exactly zero, so
    o_lat must equal that token's latent note bit for bit, wherever the needle sits.  The scaled
    scores are +-72 (base 2: +-104), so a needle after a unit's first tile raises that unit's running
    maximum by about 208 in base 2: the matrix-core kernel (32 to 128 heads, bf16) must then rescale
    its running sums by exactly 0, and every piece without the needle gets merge weight exactly 0."""
    L = 1000
    wl = synth.make_custom([L, L], heads=heads, seed=81)
    g = Gpu(wl, f32=f32)
    base = g.cache.view(torch.int16).cpu()
    t = np.arange(L)
    for star in (0, 31, 32, 63, 64, 500, L - 1):
        say("needle", heads, star, splits, "f32" if f32 else "bf16")
        cache = base.clone()
        for b in range(wl.batch):
            pages = torch.as_tensor(wl.block_table[b, t // 64]).long()
            slots = torch.as_tensor(t % 64).long()
            vals = torch.full((L,), -16512, dtype=torch.int16)      # -1.0 (0xBF80)
            vals[star] = 0x3F80                                        # +1.0
            cache[pages, slots, synth.D_C] = vals
        g.cache.view(torch.int16).copy_(cache)
        q = torch.zeros(wl.batch, wl.heads, synth.ROW, dtype=torch.float32)
        q[:, :, synth.D_C] = 1000.0
        qa = q.cuda() if f32 else q.to(torch.bfloat16).cuda()
        lib.mla_decode(qa, g.cache, g.bt, g.attended, wl.scale, g.o_lat, g.lse, g.workspace(lib, splits), splits)
        torch.cuda.synchronize()
        got = g.o_lat.float().cpu()
        for b in range(wl.batch):
            page, slot = wl.block_table[b, star // 64], star % 64
            want = (cache[page, slot, :synth.D_C].to(torch.int32) << 16).view(torch.float32)
            assert torch.equal(got[b], want.expand(wl.heads, -1)), (b, star)


def test_page_permutation_invariance_and_determinism(lib):
    wl_s = synth.make_custom([700, 64, 130], heads=128, seed=91)
    wl_c = synth.make_custom([700, 64, 130], heads=128, seed=91, shuffle=False)
    say("permutation invariance")
    gs = Gpu(wl_s)
    gc = Gpu(wl_c)
    # place the same logical rows in the contiguous layout
    src = gs.cache.view(torch.int16)
    dst = gc.cache.view(torch.int16)
    for b in range(wl_s.batch):
        for j in range(int((wl_s.block_table[b] >= 0).sum())):
            dst[wl_c.block_table[b, j]] = src[wl_s.block_table[b, j]]
    gc.q_lat_in.copy_(gs.q_lat_in)
    outs = []
    for g in (gs, gc, gs):
        g.step(lib, q_abs_from_absorb=False)
        torch.cuda.synchronize()
        outs.append((g.o_lat.view(torch.int16).clone(), g.lse.clone()))
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l.view(torch.int32), outs[0][1].view(torch.int32))


def test_debug_checks_reject_bad_tables(lib, monkeypatch):
    """MLA_DEBUG_CHECKS=1: valid tables give the unchecked result bit for bit; a used block-table
    entry outside [0, num_pages), a length past the table row or an append position past it is
    reported as MLA_ERR_BLOCK_TABLE before anything else is launched (the cache is left as it was).
    Bad tables are only ever passed with the check on."""
    wl = synth.make_custom([70, 5, 130], heads=128, seed=81, append=True)
    say("debug checks")
    g = Gpu(wl)
    g.step(lib, q_abs_from_absorb=False)
    torch.cuda.synchronize()
    o_plain = g.o_lat.clone()
    monkeypatch.setenv("MLA_DEBUG_CHECKS", "1")
    g.o_lat.zero_()
    lib.mla_decode(g.q_lat_in, g.cache, g.bt, g.attended, wl.scale, g.o_lat, g.lse, g.workspace(lib), 0)
    torch.cuda.synchronize()
    assert torch.equal(g.o_lat.view(torch.int16), o_plain.view(torch.int16))

    def decode_with(bt, lens):
        lib.mla_decode(g.q_lat_in, g.cache, bt, lens, wl.scale, g.o_lat, g.lse, g.workspace(lib), 0)

    bad = g.bt.clone()
    bad[1, 0] = wl.num_pages + 5          # the only page of sequence 1
    neg = g.bt.clone()
    neg[0, 1] = -1                         # second page of sequence 0 (71 attended tokens)
    long_lens = g.attended.clone()
    long_lens[2] = wl.max_blocks * 64 + 1
    for bt, lens in ((bad, g.attended), (neg, g.attended), (g.bt, long_lens)):
        with pytest.raises(lib.MLAError) as err:
            decode_with(bt, lens)
        assert err.value.status == -6

    before = g.cache.view(torch.int16).clone()
    far = g.lens.clone()
    far[0] = wl.max_blocks * 64            # one past the last slot of the row
    bad_page = g.bt.clone()
    bad_page[2, int(wl.lens[2]) // 64] = -1
    for bt, pos in ((g.bt, far), (bad_page, g.lens)):
        with pytest.raises(lib.MLAError) as err:
            lib.mla_cache_append(g.cache, bt, pos, g.c_new, g.kpe_new)
        assert err.value.status == -6
    torch.cuda.synchronize()
    assert torch.equal(g.cache.view(torch.int16), before)


@pytest.mark.parametrize("f32", [False, True])
def test_append_hidden_matches_oracle(lib, f32):
    """Producer side of the cache (explainer Step 5, eq. 9, and Step 7): the row
    [h W_DKV | RoPE_p(h W_KR)] written at each sequence's next position, against the float64
    oracle, within one bf16 rounding of it (plus fp32 accumulation); positions up to 131,071 give
    large rotation angles.  Every other cache byte is left as it was, and a repeat is bit-identical."""
    lens = [0, 1, 63, 64, 200, 4095, 131071]
    wl = synth.make_custom(lens, heads=16, seed=91, append=True)
    say("append hidden", "f32" if f32 else "bf16")
    dev = "cuda"
    cache = synth.cache_pages(wl, 0, device=dev, chunk_pages=2048).view(torch.bfloat16)
    bt = torch.as_tensor(wl.block_table, device=dev)
    pos = torch.as_tensor(wl.lens, device=dev)
    h_bits = synth.hidden_states(wl, 0, device=dev)
    wd_bits, wk_bits = synth.producer_weights(wl, 0, device=dev)
    h, wd, wk = act(h_bits, f32), act(wd_bits, f32), act(wk_bits, f32)
    ws = torch.empty(lib.mla_cache_append_hidden_workspace_size(wl.batch), dtype=torch.uint8, device=dev)
    before = cache.view(torch.int16).clone()
    lib.mla_cache_append_hidden(cache, bt, pos, h, wd, wk, 10000.0, ws)
    torch.cuda.synchronize()
    after = cache.view(torch.int16).clone()
    pages = [int(wl.block_table[b][lens[b] // 64]) for b in range(wl.batch)]
    slots = [lens[b] % 64 for b in range(wl.batch)]
    keep = torch.ones(cache.shape[:2], dtype=torch.bool, device=dev)
    keep[pages, slots] = False
    assert torch.equal(after[keep], before[keep])
    got = O.bf16_to_f64(after[pages, slots].cpu().numpy())
    ref = O.latent_rows_batch(synth.to_numpy_u16(h_bits), synth.to_numpy_u16(wd_bits),
                              synth.to_numpy_u16(wk_bits), wl.lens, 10000.0)
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max(axis=1, keepdims=True)
    say(f"  max err / bound {float((err / bound).max()):.3f}")
    assert (err <= bound).all()
    lib.mla_cache_append_hidden(cache, bt, pos, h, wd, wk, 10000.0, ws)
    torch.cuda.synchronize()
    assert torch.equal(cache.view(torch.int16), after)


@pytest.mark.parametrize("batch", [32, 33, 100])
def test_append_hidden_batch_blocks(lib, batch):
    """The producer side at the benchmark's batch (32: one full 32-row block) and past it (33 and 100:
    two-block passes with a ragged last block), positions anywhere in their pages: every written row
    against the oracle, every other byte unchanged."""
    rng = np.random.default_rng(batch)
    lens = rng.integers(0, 3000, batch).tolist()
    wl = synth.make_custom(lens, heads=16, seed=92 + batch, append=True)
    say("append hidden, batch", batch)
    dev = "cuda"
    cache = synth.cache_pages(wl, 0, device=dev, chunk_pages=2048).view(torch.bfloat16)
    bt = torch.as_tensor(wl.block_table, device=dev)
    pos = torch.as_tensor(wl.lens, device=dev)
    h_bits = synth.hidden_states(wl, 0, device=dev)
    wd_bits, wk_bits = synth.producer_weights(wl, 0, device=dev)
    ws = torch.empty(lib.mla_cache_append_hidden_workspace_size(batch), dtype=torch.uint8, device=dev)
    before = cache.view(torch.int16).clone()
    lib.mla_cache_append_hidden(cache, bt, pos, act(h_bits, False), act(wd_bits, False), act(wk_bits, False),
                                10000.0, ws)
    torch.cuda.synchronize()
    after = cache.view(torch.int16).clone()
    pages = [int(wl.block_table[b][lens[b] // 64]) for b in range(batch)]
    slots = [lens[b] % 64 for b in range(batch)]
    keep = torch.ones(cache.shape[:2], dtype=torch.bool, device=dev)
    keep[pages, slots] = False
    assert torch.equal(after[keep], before[keep])
    got = O.bf16_to_f64(after[pages, slots].cpu().numpy())
    ref = O.latent_rows_batch(synth.to_numpy_u16(h_bits), synth.to_numpy_u16(wd_bits),
                              synth.to_numpy_u16(wk_bits), wl.lens, 10000.0)
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max(axis=1, keepdims=True)
    say(f"  max err / bound {float((err / bound).max()):.3f}")
    assert (err <= bound).all()


@pytest.mark.parametrize("heads,batch,f32", [(16, 3, False), (128, 32, False), (64, 65, False),
                                             (128, 100, False), (16, 5, True)])
def test_out_proj_hidden_matches_oracle(lib, heads, batch, f32):
    """Output projection to the hidden width (explainer Step 6): out flattened head-major times W^O,
    one batch block, two blocks with a ragged tail, and two groups of 64 rows; bf16 within one
    rounding of the oracle plus fp32 accumulation, fp32 mode within 1e-4."""
    wl = synth.make_custom([5] * batch, heads=heads, seed=120 + heads + batch)
    say("out_proj_hidden", heads, batch, "f32" if f32 else "bf16")
    dev = "cuda"
    o_bits = synth.queries(wl, 0, device=dev)[..., :synth.D_V].contiguous()   # any seeded input of this shape
    w_bits = synth.output_weights(wl, 0, device=dev)
    o_in, w_in = act(o_bits, f32), act(w_bits, f32)
    hidden = torch.empty(batch, synth.D_MODEL, dtype=torch.float32 if f32 else torch.bfloat16, device=dev)
    n = lib.mla_out_proj_hidden_workspace_size(batch, heads, lib.MLA_F32 if f32 else lib.MLA_BF16)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    lib.mla_out_proj_hidden(o_in, w_in, hidden, ws)
    torch.cuda.synchronize()
    got = to_host_f64(hidden)
    ref = O.hidden_out(synth.to_numpy_u16(o_bits), synth.to_numpy_u16(w_bits))
    err = np.abs(got - ref)
    if f32:
        e = rel_err(got, ref)
        say(f"  err {e:.3e}")
        assert e <= F32_TOL
    else:
        bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * np.abs(ref).max(axis=1, keepdims=True)
        say(f"  max err / bound {float((err / bound).max()):.3f}")
        assert (err <= bound).all()
