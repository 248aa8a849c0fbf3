"""The decode step captured in a HIP graph and replayed: append, absorption, decode with its merge and
the W_UV projection, as separate calls and with the fused decode + projection call.  Every replay,
with eager calls and synchronisations between the replays, writes the same bits as the eager step
(the library records no memset and no host-side work into the stream, and its reductions run in a
fixed order)."""
import pytest
import torch

import synth
from tests.gpu_cases import Gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "these tests need the GPU"
    import head_latent_attention_17_amd as L
    return L


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.parametrize("heads,fused,splits", [(16, False, 0), (128, False, 0), (128, True, 0),
                                                (64, False, 5), (128, True, 3)])
def test_step_replays_match_eager(lib, heads, fused, splits):
    lens = [300, 1, 2100, 70, 0, 64]
    if fused:  # the merge + projection kernel runs from 16 sequences on (fewer take the two calls)
        lens += list(range(130, 1500, 100))
    wl = synth.make_custom(lens, heads=heads, seed=31 + heads, append=True)
    say(f"graph step: heads {heads}, fused {fused}, splits {splits}")
    g = Gpu(wl)
    B, H = wl.batch, wl.heads
    n = max(lib.mla_decode_workspace_size(B, H, wl.max_blocks, splits),
            lib.mla_decode_out_proj_workspace_size(B, H, wl.max_blocks, splits))
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")

    def step():
        lib.mla_cache_append(g.cache, g.bt, g.lens, g.c_new, g.kpe_new)
        lib.mla_absorb_q(g.q, g.w_uk, g.q_abs)
        if fused:
            lib.mla_decode_out_proj(g.q_abs, g.cache, g.bt, g.attended, wl.scale, g.w_uv, g.out, g.o_lat,
                                    g.lse, ws, splits)
        else:
            lib.mla_decode(g.q_abs, g.cache, g.bt, g.attended, wl.scale, g.o_lat, g.lse, ws, splits)
            lib.mla_out_proj(g.o_lat, g.w_uv, g.out)

    step()
    torch.cuda.synchronize()
    ref = [_bits(t).clone() for t in (g.q_abs, g.o_lat, g.lse, g.out)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        for t in (g.q_abs, g.o_lat, g.lse, g.out):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t, e in zip(("q_abs", "o_lat", "lse", "out"), (g.q_abs, g.o_lat, g.lse, g.out), ref):
            assert torch.equal(_bits(t), e), f"replay {r}: {name} differs from the eager step"
        step()   # eager work between the replays
        torch.cuda.synchronize()
        for name, t, e in zip(("q_abs", "o_lat", "lse", "out"), (g.q_abs, g.o_lat, g.lse, g.out), ref):
            assert torch.equal(_bits(t), e), f"eager step after replay {r}: {name} differs"
    say("  3 replays equal the eager step")
