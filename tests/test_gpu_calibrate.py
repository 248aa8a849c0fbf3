"""mla_calibrate_mfma, the matrix-core rate kernel the benchmark reads its compute ceiling from: it
runs, every wave writes a finite result, and a wave's result depends only on its place in the
workgroup (the operands are built from the thread index alone).  mla_calibrate_read, the read-rate
kernel the memory ceiling comes from: every workgroup reports the XOR of the first word of each chunk
it read, which the host recomputes."""
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


def test_read_calibration_reads_every_chunk_once():
    import head_latent_attention_17_amd as L
    chunk = 36 * 1024 // 4                       # int32 words per 36,864-byte chunk
    for nchunks, blocks in ((1, 1), (7, 3), (100, 256), (1000, 7)):
        buf = torch.arange(nchunks * chunk, dtype=torch.int32, device="cuda") * 3 + 11
        out = torch.full((blocks,), -1, dtype=torch.int32, device="cuda")
        L.mla_calibrate_read(buf, out, blocks)
        torch.cuda.synchronize()
        first = (torch.arange(nchunks, dtype=torch.int64) * chunk * 3 + 11).tolist()
        want = [0] * blocks
        for c, v in enumerate(first):
            want[c % blocks] ^= v
        assert out.cpu().tolist() == [w if w < 2 ** 31 else w - 2 ** 32 for w in want]
    with pytest.raises(ValueError):
        L.mla_calibrate_read(buf, out, blocks * 2)
    with pytest.raises(RuntimeError):
        L.mla_calibrate_read(buf[:-1], out, blocks)   # not a multiple of 36,864 bytes
