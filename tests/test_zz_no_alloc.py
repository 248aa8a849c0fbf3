"""mla_decode_noalloc (the decode with the library's fixed scratch array in place of a workspace)
against mla_decode through the C ABI: bit-identical o_lat and lse on two calls in a row, the second
with a smaller input, each also within the bf16 bound of the oracle."""
import numpy as np
import pytest
import torch

import synth
from oracle import mla_oracle as O
from tests.gpu_cases import BF16_TOL, Gpu, host_inputs, lse_err, rel_err, say, to_host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "these tests need the GPU"
    import head_latent_attention_17_amd as L
    return L


def _case(lib, wl, splits):
    g = Gpu(wl)
    qa = g.q_lat_in
    ws = g.workspace(lib, splits)
    o_ref = torch.empty_like(g.o_lat)
    l_ref = torch.empty_like(g.lse)
    lib.mla_decode(qa, g.cache, g.bt, g.attended, wl.scale, o_ref, l_ref, ws, splits)
    g.o_lat.fill_(7.0)
    g.lse.fill_(7.0)
    lib.mla_decode_noalloc(qa, g.cache, g.bt, g.attended, wl.scale, g.o_lat, g.lse, splits)
    torch.cuda.synchronize()
    assert torch.equal(g.o_lat.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(g.lse.view(torch.int32), l_ref.view(torch.int32))
    hi = host_inputs(wl, 0, range(wl.batch))
    o_or, l_or = O.latent_decode_batch(hi["q_lat"], hi["cache"], wl.block_table, wl.attended_lens, wl.scale)
    e_o = rel_err(to_host_f64(g.o_lat), o_or)
    e_l = lse_err(g.lse.cpu().numpy(), l_or)
    say(f"  noalloc: bit-identical to mla_decode; oracle o_lat {e_o:.3e} lse {e_l:.3e}")
    assert e_o <= BF16_TOL and e_l <= BF16_TOL


def test_noalloc_matches_decode_twice(lib):
    assert lib.mla_decode_noalloc_max_bytes() == 128 << 20
    say("noalloc call 1: 128 heads, 5 ragged sequences, automatic split")
    _case(lib, synth.make_custom([1000, 64, 0, 3000, 1], heads=128, seed=301), 0)
    say("noalloc call 2: 32 heads, 2 sequences, 7 splits")
    _case(lib, synth.make_custom([70, 200], heads=32, seed=302), 7)


def test_noalloc_rejects_sizes_past_its_buffer(lib):
    wl = synth.make_custom([64] * 300, heads=128, seed=303)
    g = Gpu(wl)
    with pytest.raises(lib.MLAError) as e:
        lib.mla_decode_noalloc(g.q_lat_in, g.cache, g.bt, g.attended, wl.scale, g.o_lat, g.lse)
    assert e.value.status == -8
