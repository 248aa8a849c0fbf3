"""mla_calibrate_mfma, the matrix-core rate kernel the benchmark reads its compute ceiling from: it
runs, every wave writes a finite result, and a wave's result depends only on its place in the
workgroup (the operands are built from the thread index alone)."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_calibration_kernel_runs_and_is_uniform_across_workgroups():
    import head_latent_attention_17_amd as L
    blocks, iters = 16, 8
    out = torch.full((blocks * 4,), float("nan"), dtype=torch.float32, device="cuda")
    L.mla_calibrate_mfma(out, blocks, iters)
    torch.cuda.synchronize()
    o = out.view(blocks, 4).cpu()
    assert torch.isfinite(o).all()
    assert torch.equal(o, o[0].expand(blocks, 4))
    with pytest.raises(ValueError):
        L.mla_calibrate_mfma(out, blocks * 2, iters)
