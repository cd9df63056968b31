"""GPU parity of the MX mode (OCP MX FP8 blocks on the scaled FP8 matrix
cores), called through the C ABI, against the fp64 oracle.

The MX quantiser (attn_quantize_mx) must match the oracle's codes and scale
bytes bit for bit. The attention is compared with two references: exact
attention on the MX-dequantised Q, K, V (what remains is the E4M3 rounding of
the softmax weights, at most 2^-4 relative per weight and about 2^-4/sqrt(3)
in RMS over many keys, so MX_P_REL = 4e-2 leaves a margin), and exact
attention on the original inputs, held to the quantised modes' 6e-2.
"""
import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_amd as sdpa
from scaled_dot_product_amd.inputs import WORKLOADS, Workload, make_qkv, normal, sample_rows

from _parity import QUANT_REL, announce, gpu_fwd, masked_rows, metrics

pytestmark = pytest.mark.gpu

MX_P_REL = 4e-2
BF, F16 = torch.bfloat16, torch.float16


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sdpa.load_library()


@pytest.mark.parametrize("dtype", [BF, F16])
@pytest.mark.parametrize("shape", [(1, 2, 64, 64), (2, 3, 130, 128), (1, 1, 333, 64), (1, 2, 31, 128)])
def test_mx_quantiser_bit_exact(dtype, shape):
    announce(f"mx quantiser {shape} {dtype}")
    x = normal(shape, 51, dtype)
    x[..., 5, :] *= 1000.0        # blocks with large and small maxima
    x[..., 7, 3:40] = 0.0
    for axis in (0, 1):
        c, s = sdpa.quantize_mx(x.cuda(), axis=axis)
        torch.cuda.synchronize()
        rc, rs = oracle.quant_mx(x, axis=axis)
        assert np.array_equal(c.cpu().numpy(), rc), axis
        assert np.array_equal(s.cpu().numpy(), rs), axis


def _check(w, rows=None, inputs=None, mx_ref=True):
    announce(f"mx {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} D={w.D} {w.dtype} "
             f"causal={w.causal} window_lo={w.window_lo} pos0={w.pos0} window_w={w.window_w}")
    q, k, v = inputs if inputs is not None else make_qkv(w)
    out = gpu_fwd(w, q, k, v).double().cpu()
    assert torch.isfinite(out).all()
    kw = dict(scale=w.scale, causal=w.causal, window_lo=w.window_lo, pos0=w.pos0)
    if rows is None:
        got = out.numpy()
        ref = oracle.attn(q, k, v, window_w=w.window_w, **kw)
        ref_mx = oracle.attn_mx(q, k, v, **kw) if w.window_w == 0 and mx_ref else None
    else:
        got = out.reshape(-1, w.D)[torch.from_numpy(rows)].numpy()
        ref = oracle.attn(q, k, v, window_w=w.window_w, rows=rows, **kw)
        ref_mx = oracle.attn_mx(q, k, v, rows=rows, **kw) if w.window_w == 0 and mx_ref else None
    rel, _ = metrics(got, ref)
    line = f"    rel(vs exact)={rel:.3e}"
    if ref_mx is not None:
        rel_mx, _ = metrics(got, ref_mx)
        line += f" rel(vs MX-dequantised inputs)={rel_mx:.3e}"
        assert rel_mx <= MX_P_REL, rel_mx
    print(line, flush=True)
    assert rel <= QUANT_REL, rel
    for i in masked_rows(w):
        assert torch.all(out[:, :, i] == 0), i
    return out


SMALL = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, causal, window_lo, pos0
    (1, 2, 2, 256, 256, 128, BF, False, 0, 0),
    (1, 4, 2, 300, 333, 64, F16, False, 0, 0),
    (2, 2, 1, 200, 260, 128, BF, True, 0, 60),
    (1, 2, 2, 130, 500, 128, F16, True, 100, 370),
    (1, 2, 2, 64, 100, 64, BF, True, 120, 0),      # every row masked: zeros
]


@pytest.mark.parametrize("case", SMALL, ids=[str(i) for i in range(len(SMALL))])
def test_mx_mode_small(case):
    B, Hq, Hkv, Nq, Nk, D, dt, causal, wlo, pos0 = case
    _check(Workload("mx", B, Hq, Hkv, Nq, Nk, D, dt, causal=causal, window_lo=wlo, pos0=pos0, mode=2))


def test_mx_mode_sliding_window():
    _check(Workload("mx_sliding", 1, 2, 2, 600, 600, 128, BF, causal=True, window_w=200, mode=2))


def test_mx_mode_video_dit_sampled():
    # against exact attention on 128 sampled rows of every head, and against
    # the MX reference on two whole heads' samples: MX blocks never cross a
    # head, so the oracle's MX dequantisation of one head's K and V (a
    # brute-force E4M3 encode per element) is that head's slice of the full one
    w = WORKLOADS["video_dit_bf16_32760"].variant(name="video_dit_mx_32760", mode=2)
    q, k, v = make_qkv(w)
    out = _check(w, rows=sample_rows(w, 128), inputs=(q, k, v), mx_ref=False)
    kw = dict(scale=w.scale, causal=w.causal, window_lo=w.window_lo, pos0=w.pos0)
    rng = np.random.default_rng(5)
    for h in (0, 39):
        announce(f"mx video head {h} against the MX reference")
        rows = np.unique(np.concatenate([rng.choice(w.Nq, 62, replace=False),
                                         np.array([0, w.Nq - 1])])).astype(np.int64)
        sl = (slice(None), slice(h, h + 1))
        ref_mx = oracle.attn_mx(q[sl].contiguous(), k[sl].contiguous(), v[sl].contiguous(),
                                rows=rows, **kw)
        got = out[0, h].numpy()[rows]
        rel_mx, _ = metrics(got, ref_mx)
        print(f"    head {h}: rel(vs MX-dequantised inputs)={rel_mx:.3e}", flush=True)
        assert rel_mx <= MX_P_REL, rel_mx


def test_mx_mode_sdxl_1024px_against_mx_reference():
    # a mid-size shape where the MX-dequantised reference is cheap: 64 sampled rows
    w = WORKLOADS["sdxl_1024px_bf16"].variant(name="sdxl_mx", mode=2)
    _check(w, rows=sample_rows(w, 64))


def test_mx_mode_zero_q_closed_form():
    # Q = 0: every score is 0 and every weight 1, which the kernel scales by
    # 2^7 (exact in E4M3): each row is the plain mean of the MX-dequantised V
    w = Workload("mx_qzero", 1, 2, 2, 64, 300, 128, BF, mode=2)
    _, k, v = make_qkv(w)
    q = torch.zeros(w.q_shape, dtype=BF)
    out = gpu_fwd(w, q, k, v).double().cpu().numpy()
    c, s = oracle.quant_mx(v, axis=1)
    vals = np.array([oracle.e4m3_decode(x) for x in range(256)])[c]
    vhat = vals * np.ldexp(1.0, np.repeat(s.astype(np.int64) - 127, 32, axis=2)[:, :, :300, :])
    want = vhat.mean(axis=2)
    for h in range(2):
        np.testing.assert_allclose(out[0, h], np.broadcast_to(want[0, h], (64, 128)),
                                   rtol=8e-3, atol=1e-3)
