"""The measurement probes (libattn_probe.so; not attention) launch and leave
the values they promise: one finite sum per thread for each MFMA kind, the XOR
fold of what a bare read touched, nothing for an empty launch."""
import pytest
import torch

import bench

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_probe_mfma_runs(kind):
    blocks = 8
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda:0")
    st = bench.load_probe().attn_probe_mfma(kind, 4, blocks, out.data_ptr(),
                                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert torch.isfinite(out).all()
    assert (out != 0).any()


def test_probe_read_and_empty_run():
    n = (1 << 20) + 48          # a ragged tail past the four-deep stride loop
    x = torch.zeros(n, dtype=torch.uint8, device="cuda:0")
    x[n - 16:n - 12] = torch.tensor([1, 2, 3, 4], dtype=torch.uint8)
    blocks = 4
    out = torch.full((blocks,), -1, dtype=torch.int32, device="cuda:0")
    p = bench.load_probe()
    s = torch.cuda.current_stream().cuda_stream
    assert p.attn_probe_read(x.data_ptr(), n, blocks, out.data_ptr(), s) == 0
    assert p.attn_probe_empty(8, s) == 0
    torch.cuda.synchronize()
    # every chunk is read once: the XOR of the per-workgroup folds is the word 0x04030201
    folded = 0
    for v in out.cpu().tolist():
        folded ^= v & 0xFFFFFFFF
    assert folded == 0x04030201


@pytest.mark.parametrize("kind", range(6))
def test_probe_valu_runs(kind):
    blocks = 8
    out = torch.full((blocks * 256,), 0x7FBADBAD, dtype=torch.int32, device="cuda:0")
    st = bench.load_probe().attn_probe_valu(kind, 4, blocks, out.data_ptr(),
                                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert (out != 0x7FBADBAD).all()     # every thread wrote its chain sum


@pytest.mark.parametrize("nv", [0, 4, 8, 12, 16, 24, 32])
def test_probe_mix_runs(nv):
    blocks = 8
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda:0")
    st = bench.load_probe().attn_probe_mix(nv, 4, blocks, out.data_ptr(),
                                           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert (out.view(torch.int32) != torch.tensor(float("nan")).view(torch.int32).item()).all()


@pytest.mark.parametrize("kind", range(5))
@pytest.mark.parametrize("late", [0, 1])
def test_probe_phase_runs(kind, late):
    blocks = 4
    out = torch.full((blocks * 512,), float("nan"), dtype=torch.float32, device="cuda:0")
    st = bench.load_probe().attn_probe_phase(kind, late, 4, blocks, out.data_ptr(),
                                             torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert (out.view(torch.int32) != torch.tensor(float("nan")).view(torch.int32).item()).all()
