"""mla_decode_out_proj (the split merge and the W_UV projection in one kernel) through the C ABI:
out, o_lat and lse against the oracle (decompressed form for out, latent attention for o_lat) and
against the two separate calls, at batches below 32, between 32 and 64 and above 64 rows (two row
groups), with empty sequences, every head count, both dtypes and several split counts; then at the
five workloads' full sizes in the launch configuration the benchmark times."""
import numpy as np
import pytest
import torch

import synth
from oracle import mla_oracle as O
from tests.gpu_cases import BF16_TOL, F32_TOL, Gpu, host_inputs, lse_err, pick, rel_err, say, to_host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "these tests need the GPU"
    import head_latent_attention_17_amd as L
    return L


def _run(lib, g, splits=0, with_olat=True):
    wl = g.wl
    dt = lib.MLA_F32 if g.f32 else lib.MLA_BF16
    ws = torch.empty(lib.mla_decode_out_proj_workspace_size(wl.batch, wl.heads, wl.max_blocks, splits, dt),
                     dtype=torch.uint8, device="cuda")
    out = torch.full_like(g.out, 7.0)
    o_lat = torch.full_like(g.o_lat, 7.0) if with_olat else None
    lse = torch.full_like(g.lse, 7.0) if with_olat else None
    if wl.append:
        lib.mla_cache_append(g.cache, g.bt, g.lens, g.c_new, g.kpe_new)
    lib.mla_absorb_q(g.q, g.w_uk, g.q_abs)
    lib.mla_decode_out_proj(g.q_abs, g.cache, g.bt, g.attended, wl.scale, g.w_uv, out, o_lat, lse, ws, splits)
    torch.cuda.synchronize()
    return out, o_lat, lse


def _check(lib, wl, f32=False, splits=0, seqs=None, heads=None):
    g = Gpu(wl, f32=f32)
    out, o_lat, lse = _run(lib, g, splits)
    # the two separate calls on the same inputs (the cache already holds any appended row)
    g.step(lib, splits=splits)
    torch.cuda.synchronize()
    seqs = list(range(wl.batch)) if seqs is None else seqs
    hs = list(range(wl.heads)) if heads is None else heads
    sel = np.ix_(seqs, hs)
    hi = host_inputs(wl, 0, seqs)
    out_ref, lse_ref = O.decode_reference(hi["q"], hi["cache"], wl.block_table, wl.attended_lens, hi["w_uk"],
                                          hi["w_uv"], wl.scale, batch=seqs, heads=hs)
    q_abs = O.absorb_batch(hi["q"], hi["w_uk"], batch=seqs, heads=hs)
    o_ref, _ = O.latent_decode_batch(q_abs, hi["cache"], wl.block_table, wl.attended_lens, wl.scale,
                                     batch=seqs, heads=hs)
    tol = F32_TOL if f32 else BF16_TOL
    e_out = rel_err(to_host_f64(out)[sel], out_ref[sel])
    e_o = rel_err(to_host_f64(o_lat)[sel], o_ref[sel])
    e_l = lse_err(lse.cpu().numpy()[sel], lse_ref[sel])
    e_two = rel_err(to_host_f64(out)[sel], to_host_f64(g.out)[sel])
    say(f"  out {e_out:.2e}  o_lat {e_o:.2e}  lse {e_l:.2e}  vs two calls {e_two:.2e}")
    assert e_out <= tol and e_o <= tol and e_l <= tol and e_two <= tol
    empty = [b for b in seqs if wl.attended_lens[b] == 0]
    for b in empty:
        assert torch.all(out[b] == 0) and torch.all(o_lat[b] == 0) and torch.all(torch.isneginf(lse[b]))
    return out


@pytest.mark.parametrize("heads", [16, 32, 64, 128])
@pytest.mark.parametrize("f32", [False, True], ids=["bf16", "f32"])
def test_small_batches(lib, heads, f32):
    lens = [1, 63, 64, 65, 300, 0, 1000]
    wl = synth.make_custom(lens, heads=heads, seed=400 + heads, append=True)
    say("decode_out_proj", heads, "f32" if f32 else "bf16", wl.lens.tolist())
    _check(lib, wl, f32=f32)


@pytest.mark.parametrize("batch", [31, 33, 64, 65, 130])
def test_row_groups(lib, batch):
    """One and two 32-row blocks, and batches above 64 rows (groups of 64, the slab kept)."""
    rng = np.random.default_rng(batch)
    lens = rng.integers(0, 200, size=batch).tolist()
    wl = synth.make_custom(lens, heads=128, seed=410 + batch)
    say("decode_out_proj rows", batch)
    _check(lib, wl, heads=list(range(0, 128, 11)))


@pytest.mark.parametrize("splits", [1, 2, 7, 64])
def test_split_counts(lib, splits):
    wl = synth.make_custom([4096, 2, 700, 0, 130], heads=128, seed=420)
    say("decode_out_proj splits", splits)
    _check(lib, wl, splits=splits, heads=list(range(0, 128, 9)))


def test_without_o_lat_and_lse(lib):
    wl = synth.make_custom([500, 70, 3], heads=128, seed=430)
    g = Gpu(wl)
    a, _, _ = _run(lib, g)
    b, _, _ = _run(lib, g, with_olat=False)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_repeat_is_bit_identical(lib):
    wl = synth.make_custom([3000, 5, 129], heads=64, seed=440)
    g = Gpu(wl)
    a, oa, la = _run(lib, g)
    b, ob, lb = _run(lib, g)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)) and torch.equal(la, lb)


CASES = [(1, None, None), (2, 6, 6), (3, None, 3), (4, 10, 4), (5, 6, 3)]


@pytest.mark.parametrize("cfg,n_seq,n_heads", CASES, ids=[f"c{c[0]}" for c in CASES])
def test_full_size(lib, cfg, n_seq, n_heads):
    wl = synth.make_config(cfg)
    if not wl.append and wl.layers == 1:
        wl = synth.make_custom(wl.lens, wl.heads, wl.seed, shuffle=cfg != 1, append=True, name=wl.name + "+append")
    say(f"decode_out_proj full size: {wl.name}")
    seqs = None if n_seq is None else pick(wl.batch, n_seq, 500 + cfg)
    heads = None if n_heads is None else pick(wl.heads, n_heads, 600 + cfg)
    _check(lib, wl, seqs=seqs, heads=heads)
    torch.cuda.empty_cache()
