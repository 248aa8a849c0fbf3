"""GPU parity of attention over the top-k tokens of a cheap int8 index, through the C ABI: the kept
positions and counts bit for bit against the oracle (ragged lengths, short sequences, tie-heavy
scores), the gathered rows byte for byte, and the decode over them within the bf16 tolerance, at
small sizes and at 4 x 131,072 tokens with k = 2,048.  The in-place decode over the kept tokens
(mla_decode_topk) must equal gather + decode bit for bit, and the oracle within the tolerance."""
import numpy as np
import pytest
import torch

import synth
from oracle import mla_oracle as O
from tests.gpu_cases import BF16_TOL, Gpu, host_inputs, pick, lse_err, rel_err, say, to_host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "these tests need the GPU"
    import head_latent_attention_17_amd as L
    return L


def _topk(lib, wl, idx, qi, k, lens=None):
    dev = "cuda"
    bt = torch.as_tensor(wl.block_table, device=dev)
    lens = torch.as_tensor(wl.attended_lens.astype(np.int32) if lens is None else lens, device=dev)
    pos = torch.full((wl.batch, k), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((wl.batch,), -7, dtype=torch.int32, device=dev)
    ws = torch.empty(lib.mla_index_topk_workspace_size(wl.batch, wl.max_blocks), dtype=torch.uint8, device=dev)
    lib.mla_index_topk(idx, bt, lens, qi, k, pos, cnt, ws)
    torch.cuda.synchronize()
    return pos.cpu().numpy(), cnt.cpu().numpy()


def _check_positions(wl, idx_np, qi_np, k, pos, cnt, seqs=None):
    for b in (range(wl.batch) if seqs is None else seqs):
        n = int(wl.attended_lens[b])
        want = O.top_k_positions(O.index_scores(idx_np, wl.block_table, b, n, qi_np[b]), k)
        assert cnt[b] == len(want), (b, cnt[b], len(want))
        assert np.array_equal(pos[b, :len(want)], want), b


# block tables of at most 16,384 tokens take the one-launch selection (a workgroup per sequence),
# longer ones the multi-workgroup passes; both must give the oracle's positions bit for bit
SHORT = [0, 1, 5, 64, 100, 1000, 5000]
LONG = [0, 1, 5, 64, 100, 1000, 20000]


@pytest.mark.parametrize("lens", [SHORT, LONG], ids=["one_launch", "multi_pass"])
@pytest.mark.parametrize("k", [1, 7, 64, 256])
def test_topk_matches_oracle(lib, k, lens):
    wl = synth.make_custom(lens, heads=16, seed=140 + k)
    say("index top-k", k, wl.max_blocks * 64)
    idx = synth.index_cache(wl, 0, device="cuda")
    qi = synth.index_queries(wl, 0, device="cuda")
    pos, cnt = _topk(lib, wl, idx, qi, k)
    _check_positions(wl, idx.cpu().numpy(), qi.cpu().numpy(), k, pos, cnt)


def test_topk_many_chunks(lib):
    """64 sequences of about 16,000 tokens: 1,024 selection chunks in all, so scoring runs with its
    full 1,024-token chunks (the smaller workloads above score in 256-token chunks; the full-size
    test below in 1,024-token chunks over 516 workgroups)."""
    k = 300
    wl = synth.make_custom([16500 - 7 * i for i in range(64)], heads=16, seed=145)
    assert wl.max_blocks * 64 > 16384
    say("index top-k, 64 x ~16k tokens", k)
    idx = synth.index_cache(wl, 0, device="cuda")
    qi = synth.index_queries(wl, 0, device="cuda")
    pos, cnt = _topk(lib, wl, idx, qi, k)
    _check_positions(wl, idx.cpu().numpy(), qi.cpu().numpy(), k, pos, cnt)


def test_topk_one_launch_at_capacity(lib):
    """Sequences filling the one-launch path's LDS (16,384 scores) and just below it."""
    k = 2048
    wl = synth.make_custom([16384 - 7 * i for i in range(8)], heads=16, seed=146)
    assert wl.max_blocks * 64 == 16384
    say("index top-k at the one-launch capacity", k)
    idx = synth.index_cache(wl, 0, device="cuda")
    qi = synth.index_queries(wl, 0, device="cuda")
    pos, cnt = _topk(lib, wl, idx, qi, k)
    _check_positions(wl, idx.cpu().numpy(), qi.cpu().numpy(), k, pos, cnt)


@pytest.mark.parametrize("lens", [[300, 2000, 64], [300, 20000, 64]], ids=["one_launch", "multi_pass"])
@pytest.mark.parametrize("levels", [1, 3])
def test_topk_ties(lib, levels, lens):
    """Index vectors with entries in {0} or {-1, 0, 1}: all scores equal, or few distinct values, so
    the tie rule (earlier position first) decides most of the selection."""
    wl = synth.make_custom(lens, heads=16, seed=150 + levels)
    say("index top-k ties", levels)
    rng = np.random.default_rng(levels)
    idx_np = (rng.integers(0, levels, (wl.num_pages, 64, 128)) - (levels // 2)).astype(np.int8)
    qi_np = np.ones((wl.batch, 128), np.int8)
    pos, cnt = _topk(lib, wl, torch.from_numpy(idx_np).cuda(), torch.from_numpy(qi_np).cuda(), 100)
    _check_positions(wl, idx_np, qi_np, 100, pos, cnt)


def _sparse_decode(lib, wl, k, g, cnt_dev, pos_dev):
    dev = "cuda"
    pk = -(-k // 64)
    out_cache = torch.empty((wl.batch * pk, 64, 576), dtype=torch.bfloat16, device=dev)
    out_bt = torch.full((wl.batch, pk), -1, dtype=torch.int32, device=dev)
    lib.mla_gather_rows(g.cache, g.bt, pos_dev, cnt_dev, out_cache, out_bt)
    ws = torch.empty(lib.mla_decode_workspace_size(wl.batch, wl.heads, pk, 0), dtype=torch.uint8, device=dev)
    lib.mla_decode(g.q_lat_in, out_cache, out_bt, cnt_dev, wl.scale, g.o_lat, g.lse, ws)
    torch.cuda.synchronize()
    return out_cache, out_bt


def test_gathered_rows_and_sparse_decode(lib):
    """The gathered compact pages hold exactly the kept rows, and decode over them matches the
    oracle's attention over the top-k tokens; a short sequence keeps all its tokens and an empty one
    gives zeros."""
    k = 256
    wl = synth.make_custom([0, 40, 256, 700, 3000], heads=128, seed=160)
    say("sparse decode", k)
    g = Gpu(wl)
    dev = "cuda"
    idx = synth.index_cache(wl, 0, device=dev)
    qi = synth.index_queries(wl, 0, device=dev)
    bt = torch.as_tensor(wl.block_table, device=dev)
    pos_dev = torch.zeros((wl.batch, k), dtype=torch.int32, device=dev)
    cnt_dev = torch.zeros((wl.batch,), dtype=torch.int32, device=dev)
    ws = torch.empty(lib.mla_index_topk_workspace_size(wl.batch, wl.max_blocks), dtype=torch.uint8, device=dev)
    lib.mla_index_topk(idx, bt, g.attended, qi, k, pos_dev, cnt_dev, ws)
    out_cache, out_bt = _sparse_decode(lib, wl, k, g, cnt_dev, pos_dev)
    hi = host_inputs(wl, 0, range(wl.batch))
    o_ref, lse_ref, chosen = O.sparse_latent_decode(hi["q_lat"], hi["cache"], wl.block_table, wl.attended_lens,
                                                    idx.cpu().numpy(), qi.cpu().numpy(), k, wl.scale)
    pk = -(-k // 64)
    oc = synth.to_numpy_u16(out_cache.view(torch.int16))
    assert np.array_equal(out_bt.cpu().numpy(), np.arange(wl.batch * pk).reshape(wl.batch, pk))
    for b in range(wl.batch):
        rows = hi["cache"][wl.block_table[b][chosen[b] // 64], chosen[b] % 64]
        i = np.arange(len(chosen[b]))
        assert np.array_equal(oc[b * pk + i // 64, i % 64], rows)
    o = to_host_f64(g.o_lat)
    assert torch.all(g.o_lat[0].float() == 0) and torch.all(torch.isneginf(g.lse[0]))
    e_o = rel_err(o[1:], o_ref[1:])
    lse = g.lse.cpu().numpy()
    e_l = lse_err(lse[1:], lse_ref[1:])
    say(f"  o_lat err {e_o:.3e}  lse err {e_l:.3e}")
    assert e_o <= BF16_TOL and e_l <= BF16_TOL


@pytest.mark.parametrize("cfg", [3, 2])
def test_full_size(lib, cfg):
    """4 x 131,072 tokens (+1) (multi-workgroup passes) and 32 x 4,096 (+1) (one launch), k = 2,048:
    every sequence's kept positions bit for bit, and the decode over them on sampled heads."""
    import bench
    wl = bench.bench_workload(cfg)
    k = 2048
    say("sparse full size", wl.name)
    g = Gpu(wl)
    dev = "cuda"
    idx = synth.index_cache(wl, 0, device=dev)
    qi = synth.index_queries(wl, 0, device=dev)
    lib.mla_cache_append(g.cache, g.bt, g.lens, g.c_new, g.kpe_new)
    pos, cnt = _topk(lib, wl, idx, qi, k)
    idx_np, qi_np = idx.cpu().numpy(), qi.cpu().numpy()
    _check_positions(wl, idx_np, qi_np, k, pos, cnt)
    pos_dev = torch.from_numpy(pos).cuda()
    cnt_dev = torch.from_numpy(cnt).cuda()
    _sparse_decode(lib, wl, k, g, cnt_dev, pos_dev)
    heads = pick(wl.heads, 4, 170)
    seqs = [0, 3]
    o = to_host_f64(g.o_lat)
    hi = host_inputs(wl, 0, seqs)
    o_ref, lse_ref, _ = O.sparse_latent_decode(hi["q_lat"], hi["cache"], wl.block_table, wl.attended_lens, idx_np,
                                               qi_np, k, wl.scale, batch=seqs, heads=heads)
    sel = np.ix_(seqs, heads)
    e_o = rel_err(o[sel], o_ref[sel])
    say(f"  o_lat err {e_o:.3e}")
    assert e_o <= BF16_TOL


def _topk_inplace(lib, wl, g, pos_dev, cnt_dev):
    o = torch.empty_like(g.o_lat)
    lse = torch.empty_like(g.lse)
    k = pos_dev.shape[1]
    ws = torch.empty(lib.mla_decode_topk_workspace_size(wl.batch, wl.heads, k), dtype=torch.uint8,
                     device=pos_dev.device)
    lib.mla_decode_topk(g.q_lat_in, g.cache, g.bt, pos_dev, cnt_dev, wl.scale, o, lse, ws)
    torch.cuda.synchronize()
    return o, lse


def _same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16)) if a.dtype == torch.bfloat16 else \
        torch.equal(a.view(torch.int32), b.view(torch.int32))


def _oracle_list_decode(hi, wl, pos, cnt, seqs, heads):
    """The oracle's latent attention over the listed tokens of each chosen sequence."""
    o = np.full((wl.batch, wl.heads, 512), np.nan)
    lse = np.full((wl.batch, wl.heads), np.nan)
    q = O.bf16_to_f64(hi["q_lat"])
    for b in seqs:
        p_b = pos[b, :cnt[b]]
        pg, sl = O.page_and_slot(wl.block_table, b, p_b, 64)
        rows = O.bf16_to_f64(hi["cache"][pg, sl]) if len(p_b) else np.zeros((0, 576))
        for h in heads:
            o[b, h], lse[b, h], _ = O.latent_attention(q[b, h], rows, 512, wl.scale)
    return o, lse


@pytest.mark.parametrize("heads,k", [(128, 100), (128, 256), (64, 7), (64, 100), (32, 256), (16, 100)])
def test_decode_topk_matches_gather(lib, heads, k):
    """mla_decode_topk over mla_index_topk's lists equals mla_gather_rows + mla_decode bit for bit
    (empty, short, ragged and long sequences), and the oracle within the bf16 tolerance."""
    wl = synth.make_custom([0, 1, 40, 256, 700, 3000], heads=heads, seed=180 + heads + k)
    say("in-place top-k decode", heads, k)
    g = Gpu(wl)
    dev = "cuda"
    idx = synth.index_cache(wl, 0, device=dev)
    qi = synth.index_queries(wl, 0, device=dev)
    pos_dev = torch.zeros((wl.batch, k), dtype=torch.int32, device=dev)
    cnt_dev = torch.zeros((wl.batch,), dtype=torch.int32, device=dev)
    ws = torch.empty(lib.mla_index_topk_workspace_size(wl.batch, wl.max_blocks), dtype=torch.uint8, device=dev)
    lib.mla_index_topk(idx, g.bt, g.attended, qi, k, pos_dev, cnt_dev, ws)
    o, lse = _topk_inplace(lib, wl, g, pos_dev, cnt_dev)
    _sparse_decode(lib, wl, k, g, cnt_dev, pos_dev)
    assert _same_bits(o, g.o_lat) and _same_bits(lse, g.lse)
    assert torch.all(o[0].float() == 0) and torch.all(torch.isneginf(lse[0]))
    seqs = range(1, wl.batch)
    hd = pick(heads, 8, 190)
    hi = host_inputs(wl, 0, seqs)
    o_ref, lse_ref = _oracle_list_decode(hi, wl, pos_dev.cpu().numpy(), cnt_dev.cpu().numpy(), seqs, hd)
    sel = np.ix_(list(seqs), hd)
    e_o = rel_err(to_host_f64(o)[sel], o_ref[sel])
    lse_np = lse.cpu().numpy()
    e_l = lse_err(lse_np[sel], lse_ref[sel])
    say(f"  o_lat err {e_o:.3e}  lse err {e_l:.3e}")
    assert e_o <= BF16_TOL and e_l <= BF16_TOL


def test_decode_topk_arbitrary_lists(lib):
    """Any list of positions is attended in list order: unsorted lists with repeats and counts from
    0 to k, against gather + decode bit for bit and the oracle over the same lists."""
    k = 150
    wl = synth.make_custom([5, 90, 600, 2000, 64, 1000, 333], heads=64, seed=200)
    say("in-place top-k decode, arbitrary lists", k)
    g = Gpu(wl)
    rng = np.random.default_rng(201)
    pos = np.full((wl.batch, k), -1, np.int32)            # entries past the count are never read
    cnt = np.array([3, 0, 150, 149, 64, 97, 33], np.int32)
    for b in range(wl.batch):
        pos[b, :cnt[b]] = rng.integers(0, int(wl.attended_lens[b]), cnt[b])
    pos_dev, cnt_dev = torch.from_numpy(pos).cuda(), torch.from_numpy(cnt).cuda()
    o, lse = _topk_inplace(lib, wl, g, pos_dev, cnt_dev)
    _sparse_decode(lib, wl, k, g, cnt_dev, pos_dev)
    assert _same_bits(o, g.o_lat) and _same_bits(lse, g.lse)
    seqs = [b for b in range(wl.batch) if cnt[b] > 0]
    hi = host_inputs(wl, 0, seqs)
    hd = pick(64, 8, 202)
    o_ref, lse_ref = _oracle_list_decode(hi, wl, pos, cnt, seqs, hd)
    sel = np.ix_(seqs, hd)
    e_o = rel_err(to_host_f64(o)[sel], o_ref[sel])
    say(f"  o_lat err {e_o:.3e}")
    assert e_o <= BF16_TOL
    assert torch.all(o[1].float() == 0) and torch.all(torch.isneginf(lse[1]))


def test_decode_topk_debug_checks(lib, monkeypatch):
    """MLA_DEBUG_CHECKS=1: valid lists give the unchecked result bit for bit; a count above k or a
    position outside the table row is reported as MLA_ERR_BLOCK_TABLE before any decode (or gather)
    launch."""
    k = 64
    wl = synth.make_custom([100, 300], heads=128, seed=210)
    say("in-place top-k decode, debug checks")
    g = Gpu(wl)
    # valid lists: every position inside its own sequence (the unchecked call trusts them)
    pos = np.stack([(np.arange(k) * 3) % int(n) for n in wl.attended_lens]).astype(np.int32)
    cnt = np.array([k, 20], np.int32)
    assert all((pos[b, :cnt[b]] < wl.attended_lens[b]).all() for b in range(wl.batch))
    pos_dev, cnt_dev = torch.from_numpy(pos).cuda(), torch.from_numpy(cnt).cuda()
    o0, lse0 = _topk_inplace(lib, wl, g, pos_dev, cnt_dev)
    monkeypatch.setenv("MLA_DEBUG_CHECKS", "1")
    o1, lse1 = _topk_inplace(lib, wl, g, pos_dev, cnt_dev)
    assert _same_bits(o0, o1) and _same_bits(lse0, lse1)
    bad_cnt = torch.tensor([k + 1, 20], dtype=torch.int32, device="cuda")
    with pytest.raises(lib.MLAError) as e:
        _topk_inplace(lib, wl, g, pos_dev, bad_cnt)
    assert e.value.status == -6
    bad_pos = pos.copy()
    bad_pos[1, 5] = wl.max_blocks * 64
    with pytest.raises(lib.MLAError) as e:
        _topk_inplace(lib, wl, g, torch.from_numpy(bad_pos).cuda(), cnt_dev)
    assert e.value.status == -6
    # the gather reads the same lists and is checked the same way
    pk = -(-k // 64)
    out_cache = torch.empty((wl.batch * pk, 64, 576), dtype=torch.bfloat16, device="cuda")
    out_bt = torch.full((wl.batch, pk), -1, dtype=torch.int32, device="cuda")
    lib.mla_gather_rows(g.cache, g.bt, pos_dev, cnt_dev, out_cache, out_bt)
    torch.cuda.synchronize()
    for p_bad, c_bad in ((torch.from_numpy(bad_pos).cuda(), cnt_dev), (pos_dev, bad_cnt)):
        with pytest.raises(lib.MLAError) as e:
            lib.mla_gather_rows(g.cache, g.bt, p_bad, c_bad, out_cache, out_bt)
        assert e.value.status == -6


def test_decode_topk_full_size(lib):
    """4 x 131,072 tokens (+1), k = 2,048: the in-place decode equals gather + decode bit for bit."""
    import bench
    wl = bench.bench_workload(3)
    k = 2048
    say("in-place top-k decode full size", wl.name)
    g = Gpu(wl)
    dev = "cuda"
    idx = synth.index_cache(wl, 0, device=dev)
    qi = synth.index_queries(wl, 0, device=dev)
    lib.mla_cache_append(g.cache, g.bt, g.lens, g.c_new, g.kpe_new)
    pos_dev = torch.zeros((wl.batch, k), dtype=torch.int32, device=dev)
    cnt_dev = torch.zeros((wl.batch,), dtype=torch.int32, device=dev)
    ws = torch.empty(lib.mla_index_topk_workspace_size(wl.batch, wl.max_blocks), dtype=torch.uint8, device=dev)
    lib.mla_index_topk(idx, g.bt, g.attended, qi, k, pos_dev, cnt_dev, ws)
    o, lse = _topk_inplace(lib, wl, g, pos_dev, cnt_dev)
    _sparse_decode(lib, wl, k, g, cnt_dev, pos_dev)
    assert _same_bits(o, g.o_lat) and _same_bits(lse, g.lse)

