"""GPU parity of rotary position embedding (attn_fwd_rope), called through the
C ABI, against the fp64 oracle (which turns Q and K in double precision and
then takes exact attention). The exact mode is held to the exact-mode bar; the
rotated Q and K are rounded to the operand type once more than in the oracle,
well inside it. The quantised and MX modes are held to their 6e-2."""
import pytest
import torch

import scaled_dot_product_amd as sdpa
from scaled_dot_product_amd.inputs import WORKLOADS, Workload, sample_rows

from _parity import check_rope

pytestmark = pytest.mark.gpu

BF, F16, F32 = torch.bfloat16, torch.float16, torch.float32
PLAIN = dict(style=0, scaling=0, base=10000.0)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sdpa.load_library()


def _check(w, rope, rows=None):
    check_rope(w, rope, rows)


ROPES = [
    PLAIN,
    dict(style=1, scaling=0, base=10000.0),
    dict(style=0, scaling=1, base=10000.0, factor=8.0),
    dict(style=1, scaling=2, base=500000.0, factor=4.0, orig_ctx=256, beta_fast=32.0, beta_slow=1.0),
]


@pytest.mark.parametrize("rope", ROPES, ids=["plain", "interleaved", "ntk", "yarn"])
def test_rope_prefill_bf16(rope):
    _check(Workload("rope", 1, 4, 2, 300, 300, 128, BF, causal=True), rope)


@pytest.mark.parametrize("case", [(64, F16, False, 0, 0), (128, F32, True, 40, 100), (64, BF, True, 0, 900)])
def test_rope_prefill_shapes(case):
    D, dt, causal, wlo, pos0 = case
    _check(Workload("rope_shapes", 2, 2, 1, 200, 260 + pos0 // 4, D, dt, causal=causal, window_lo=wlo,
                    pos0=pos0 if causal else 0), ROPES[3] if dt == F32 else PLAIN)


def test_rope_large_positions_sampled():
    # positions up to 32 759: the angle reduction must keep its precision
    w = WORKLOADS["video_dit_bf16_32760"].variant(name="rope_video_4heads", Hq=4, Hkv=4)
    _check(w, ROPES[0], rows=sample_rows(w, 128))


@pytest.mark.parametrize("rope", [ROPES[0], ROPES[3]], ids=["plain", "yarn"])
def test_rope_decode(rope):
    _check(WORKLOADS["gqa_decode_f16_4096"], rope)


@pytest.mark.parametrize("mode", [1, 2], ids=["quant", "mx"])
def test_rope_low_precision_modes(mode):
    _check(Workload("rope_lp", 1, 2, 2, 600, 600, 128, BF, causal=True, mode=mode), ROPES[2])
