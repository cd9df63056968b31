"""GPU parity of the per-row sliding window (attn_fwd_sliding): query row i
sees keys j >= pos0 + i - W + 1 (and j <= pos0 + i when causal). The HIP path,
called through the C ABI, against the fp64 oracle on the same seeded inputs,
over the prefill kernels (four- and eight-wave grids, quantised mode) and the
split-KV decode."""
import numpy as np
import pytest
import torch

import scaled_dot_product_amd as sdpa
from scaled_dot_product_amd.inputs import WORKLOADS, Workload, make_qkv, sample_rows

from _parity import check_workload, gpu_fwd, masked_rows

pytestmark = pytest.mark.gpu

BF, F16, F32 = torch.bfloat16, torch.float16, torch.float32


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sdpa.load_library()


PREFILL = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, causal, pos0, W
    (1, 4, 2, 1000, 1000, 128, BF, True, 0, 256),
    (1, 2, 2, 777, 900, 64, F16, True, 123, 100),
    (1, 2, 1, 500, 700, 128, BF, False, 100, 64),
    (2, 4, 4, 300, 300, 64, F32, True, 0, 37),
    (1, 8, 8, 300, 5000, 128, BF, True, 4700, 3000),
    (1, 2, 2, 130, 4000, 128, F16, False, 0, 4000),   # the window cuts the last rows only
    (1, 2, 2, 64, 100, 64, BF, True, 200, 10),        # every row past the keys: all zeros
]


@pytest.mark.parametrize("case", PREFILL, ids=[str(i) for i in range(len(PREFILL))])
def test_sliding_prefill(case):
    B, Hq, Hkv, Nq, Nk, D, dt, causal, pos0, W = case
    w = Workload("sliding", B, Hq, Hkv, Nq, Nk, D, dt, causal=causal, pos0=pos0, window_w=W)
    out, _, _, _ = check_workload(w)
    for i in masked_rows(w):
        assert torch.all(out[:, :, i] == 0), i


def test_sliding_window_of_one_is_the_diagonal_value_bitwise():
    w = Workload("sliding_w1", 1, 4, 2, 200, 260, 128, BF, causal=True, pos0=60, window_w=1)
    q, k, v = make_qkv(w)
    out = gpu_fwd(w, q, k, v).cpu()
    G = w.Hq // w.Hkv
    want = v[:, torch.arange(w.Hq) // G, w.pos0:w.pos0 + w.Nq]
    assert torch.equal(out, want)


@pytest.mark.parametrize("window, waves", [(4096, 8), (1024, 4)], ids=["eight-wave", "four-wave"])
def test_sliding_large_grid_sampled(window, waves):
    # D = 128 and >= 2048 workgroups of 256 rows select the eight-wave kernel,
    # unless the per-row window is narrower than 3072 keys
    w = Workload("sliding_grid", 1, 64, 64, 8192, 8192, 128, BF, causal=True, window_w=window)
    p = sdpa.plan(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, causal=True, window=window, dtype=BF)
    assert p.waves == waves
    q, k, v = make_qkv(w)
    rows = sample_rows(w, 192)
    check_workload(w, rows=rows, inputs=(q, k, v))


def test_sliding_video_dit_causal_sampled():
    w = WORKLOADS["video_dit_bf16_32760"].variant(name="video_dit_sliding4096", causal=True,
                                                  window_w=4096)
    rows = sample_rows(w, 160)
    check_workload(w, rows=rows)


DECODE = [
    # Hkv, G, Nq, Nk, pos0, W
    (2, 8, 4, 4096, 4092, 1000),
    (2, 1, 16, 3000, 2984, 700),
    (1, 16, 2, 8260, 8258, 5000),
    (2, 2, 8, 2000, 1992, 3),       # three keys per row: few tiles
]


@pytest.mark.parametrize("case", DECODE, ids=[str(c) for c in DECODE])
def test_sliding_decode(case):
    Hkv, G, Nq, Nk, pos0, W = case
    w = Workload("sliding_decode", 1, Hkv * G, Hkv, Nq, Nk, 128, F16, causal=True, pos0=pos0,
                 window_w=W)
    check_workload(w)


def test_sliding_quant_mode():
    w = Workload("sliding_quant", 1, 2, 2, 600, 600, 128, BF, causal=True, window_w=200, mode=1)
    out, _, _, _ = check_workload(w)
