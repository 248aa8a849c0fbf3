"""GPU parity at the five workloads' full sizes, in the launch configuration bench.py times (automatic
split count, one call per layer).  The GPU computes every output; the oracle checks a seeded sample
of (sequence, head) pairs one by one:

* latent decode alone (seeded latent-form query) against the oracle's latent attention, and
* the whole path (append when the workload appends, absorb, decode, out-projection) against the
  oracle's decompressed form.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import mla_oracle as O
from tests.gpu_cases import BF16_TOL, F32_TOL, Gpu, host_inputs, pick, lse_err, rel_err, say, to_host_f64

pytestmark = pytest.mark.gpu

# (config, layers checked, sequences sampled, heads sampled)
CASES = [
    (1, [0], None, None),
    (2, [0], 8, 6),
    (3, [0], None, 3),
    (4, [0], 12, 4),
    (5, [0, 59], 6, 3),
]


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "these tests need the GPU"
    import head_latent_attention_17_amd as L
    return L


def _check(lib, cfg, layer, n_seq, n_heads, f32):
    wl = synth.make_config(cfg)
    say(f"config {cfg} layer {layer} {'f32' if f32 else 'bf16'}: {wl.name}, {wl.tokens} tokens")
    g = Gpu(wl, layer=layer, f32=f32)
    seqs = list(range(wl.batch)) if n_seq is None else pick(wl.batch, n_seq, 100 + cfg)
    heads = list(range(wl.heads)) if n_heads is None else pick(wl.heads, n_heads, 200 + cfg + layer)
    # latent decode alone
    g.step(lib, q_abs_from_absorb=False)
    torch.cuda.synchronize()
    o_gpu = to_host_f64(g.o_lat)
    lse_gpu = g.lse.cpu().numpy().astype(np.float64)
    # whole path (the cache already holds the appended row; appending it again is idempotent)
    g.step(lib)
    torch.cuda.synchronize()
    out_gpu = to_host_f64(g.out)
    lse2_gpu = g.lse.cpu().numpy().astype(np.float64)
    del g
    torch.cuda.empty_cache()

    hi = host_inputs(wl, layer, seqs)
    o_ref, lse_ref = O.latent_decode_batch(hi["q_lat"], hi["cache"], wl.block_table, wl.attended_lens,
                                           wl.scale, batch=seqs, heads=heads)
    out_ref, lse2_ref = O.decode_reference(hi["q"], hi["cache"], wl.block_table, wl.attended_lens,
                                           hi["w_uk"], hi["w_uv"], wl.scale, batch=seqs, heads=heads)
    sel = np.ix_(seqs, heads)
    e_o = rel_err(o_gpu[sel], o_ref[sel])
    e_out = rel_err(out_gpu[sel], out_ref[sel])
    e_l = lse_err(lse_gpu[sel], lse_ref[sel])
    e_l2 = lse_err(lse2_gpu[sel], lse2_ref[sel])
    say(f"  o_lat {e_o:.2e}  out {e_out:.2e}  lse {e_l:.2e} / {e_l2:.2e}  ({len(seqs)} seq x {len(heads)} heads)")
    tol = F32_TOL if f32 else BF16_TOL
    assert e_o <= tol and e_out <= tol and e_l <= tol and e_l2 <= tol
    assert np.isfinite(o_gpu).all() and np.isfinite(out_gpu).all()


@pytest.mark.parametrize("cfg,layers,n_seq,n_heads", CASES, ids=[f"c{c[0]}" for c in CASES])
@pytest.mark.parametrize("f32", [False, True], ids=["bf16", "f32"])
def test_full_size_config(lib, cfg, layers, n_seq, n_heads, f32):
    for layer in layers:
        _check(lib, cfg, layer, n_seq, n_heads, f32)
