"""GPU parity on score distributions that drive the online softmax through its
rare paths, against the fp64 oracle.

The kernels take each tile's weights against the running maximum as it stands
and raise it only when a weight could pass a bound (or the row has no maximum
yet). These inputs make that happen often and in every way:

* rising   — key norms grow along the sequence, so later tiles keep beating the
             running maximum by many powers of two (repeated rescales);
* huge     — scores of several hundred in log2 units: the weights of a row's
             first tile, taken before any maximum exists, overflow to inf;
* sunken   — every score of a row lies far below zero, so those first weights
             underflow to 0 (only the missing maximum triggers the rescale).

The inputs are seeded normals reshaped by fixed factors (no method arithmetic).
"""
import numpy as np
import pytest
import torch

from _parity import check_workload, masked_rows
from scaled_dot_product_amd.inputs import Workload, normal

pytestmark = pytest.mark.gpu


def shaped_inputs(kind, w):
    q = normal(w.q_shape, 71, torch.float32)
    k = normal(w.kv_shape, 72, torch.float32)
    v = normal(w.kv_shape, 73, torch.float32)
    if kind in ("rising", "rising_mild"):
        # key j scaled by 0.2 + 40 j / Nk: the largest score of a row grows by
        # tens of powers of two from the first tile to the last (by a few, for
        # the INT8 mode, whose score rounding grows with the key norms)
        top = 40.0 if kind == "rising" else 4.0
        f = 0.2 + top * torch.arange(w.Nk, dtype=torch.float32) / w.Nk
        k = k * f[None, None, :, None]
    elif kind == "huge":
        q, k = 10.0 * q, 10.0 * k
    elif kind == "sunken":
        # all keys near one direction u, queries near -10 u: scores about
        # -10 |u|^2 = -10 D, plus the spread of the small noise terms
        u = normal((1, 1, 1, w.D), 74, torch.float32)
        k = u + 0.05 * k
        q = -10.0 * u + 0.05 * q
    else:
        raise ValueError(kind)
    return tuple(t.to(w.dtype) for t in (q, k, v))


CASES = [
    # (kind, Nq, Nk, D, dtype, causal, pos0)
    ("rising", 300, 700, 128, torch.bfloat16, False, 0),
    ("rising", 300, 700, 64, torch.float16, True, 400),
    ("huge", 200, 700, 128, torch.bfloat16, False, 0),
    ("huge", 130, 700, 64, torch.bfloat16, True, 570),
    ("sunken", 200, 700, 128, torch.bfloat16, False, 0),
    ("sunken", 200, 700, 64, torch.float16, True, 500),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{i}" for i, c in enumerate(CASES)])
def test_prefill_softmax_paths(case):
    kind, Nq, Nk, D, dt, causal, pos0 = case
    w = Workload(kind, 1, 4, 2, Nq, Nk, D, dt, causal=causal, pos0=pos0)
    out, _, _, _ = check_workload(w, inputs=shaped_inputs(kind, w))
    for i in masked_rows(w):
        assert torch.all(out[:, :, i] == 0), i


@pytest.mark.parametrize("kind", ["rising", "huge", "sunken"])
def test_decode_softmax_paths(kind):
    # four packed rows per KV head at the end of a 4 100-key cache (split-KV)
    w = Workload(kind, 1, 8, 2, 4, 4100, 128, torch.float16, causal=True, pos0=4096)
    check_workload(w, inputs=shaped_inputs(kind, w))


def test_quant_softmax_paths():
    # INT8 Q K^T / FP8 P V against exact attention, the quantised mode's bar;
    # its running maximum may trail by only 2 powers of two, so mildly rising
    # scores already rescale often
    w = Workload("rising_mild", 1, 2, 2, 256, 700, 128, torch.bfloat16, mode=1)
    check_workload(w, inputs=shaped_inputs("rising_mild", w))
