"""The matrix-core rate probe (a measurement helper, not attention) launches
for each MFMA kind and leaves one finite sum per thread."""
import pytest
import torch

import scaled_dot_product_amd as sdpa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_probe_mfma_runs(kind):
    blocks = 8
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda:0")
    sdpa.probe_mfma(kind, 4, blocks, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert (out != 0).any()
