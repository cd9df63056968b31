"""Pins for the oracle's FP4 pieces (CPU only): the OCP E2M1 codec, MX FP4
blocks, and the diagonal-tiled mixed MXFP8 / MXFP4 attention emulation.

Checked against the E2M1 definition (every code's value, round trips,
midpoints, saturation, and a nearest-value rounding done here on the step grid
of each binade with numpy's half-to-even rint: another method than the
oracle's search over the codes), the OCP block rule (scale from the block
maximum, the maximum element landing in [4, 8) before clamping, zero and
ragged blocks, the two block axes agreeing on a transposed tensor), a
hand-worked row (tests/golden/mxd_worked_example.txt), exact closed forms (one
visible key gives its dequantised V, power-of-two scaling of V), and a second
implementation of the emulation written here from the stated rules with
torch's float8_e4m3fn cast for the E4M3 weights.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from scaled_dot_product_amd.inputs import normal

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


E2M1 = [(int(c, 16), float(v)) for c, v in _golden("e2m1_ocp_values.txt")]


@pytest.mark.parametrize("code,val", E2M1)
def test_e2m1_every_code(code, val):
    dec = oracle.e2m1_decode(code)
    assert dec == val and math.copysign(1.0, dec) == math.copysign(1.0, val)
    assert oracle.e2m1_encode(val) == code


def _e2m1_round_grid(x):
    """E2M1 rounding of x (clamped to +-6) on each binade's step grid with
    half-to-even rint: steps 0.5 below 2, 1 in [2, 4), 2 in [4, 6]."""
    a = np.minimum(np.abs(x), 6.0)
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    return np.sign(x) * np.rint(a / step) * step


def test_e2m1_encode_is_nearest_even_on_a_dense_grid():
    xs = np.concatenate([np.arange(-8.0, 8.0 + 1e-9, 1.0 / 64.0),
                         normal((4000,), 3, torch.float32).double().numpy() * 3.0])
    got = np.array([oracle.e2m1_decode(oracle.e2m1_encode(float(np.float32(x)))) for x in xs])
    want = _e2m1_round_grid(xs.astype(np.float32).astype(np.float64))
    np.testing.assert_array_equal(np.abs(got), np.abs(want))


def test_e2m1_midpoints_and_saturation():
    # each midpoint goes to the neighbour with the even code
    for mid, want in ((0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0), (2.5, 2.0),
                      (3.5, 4.0), (5.0, 4.0)):
        assert oracle.e2m1_decode(oracle.e2m1_encode(mid)) == want
        assert oracle.e2m1_decode(oracle.e2m1_encode(-mid)) == -want
    for big in (6.0, 6.5, 7.99, 100.0, 1e30):
        assert oracle.e2m1_encode(big) == 0x7 and oracle.e2m1_encode(-big) == 0xF


def _dq4(codes, scales, axis):
    vals = np.array([oracle.e2m1_decode(c) for c in range(16)])[codes]
    e = scales.astype(np.int64) - 127
    if axis == 0:
        e = np.repeat(e, 32, axis=-1)
    else:
        e = np.repeat(e, 32, axis=-2)[..., : codes.shape[-2], :]
    return vals * np.exp2(e.astype(np.float64))


@pytest.mark.parametrize("axis", [0, 1])
def test_quant_mx4_block_rule(axis):
    x = (normal((2, 3, 70, 64), 11 + axis, torch.float32) * 2.0).to(torch.bfloat16)
    x[0, 0, :32, 0] = 0.0          # an all-zero block along the tokens
    x[0, 0, 5, :32] = 0.0          # and along the channels
    codes, scales = oracle.quant_mx4(x, axis=axis)
    xf = x.double().numpy()
    assert codes.max() <= 0xF
    # the block scale: floor(log2 amax) - 2, or byte 0 for an all-zero block
    if axis == 0:
        blocks = xf.reshape(2, 3, 70, 2, 32)
        amax = np.abs(blocks).max(-1)
    else:
        pad = np.zeros((2, 3, 96, 64))
        pad[:, :, :70] = xf
        amax = np.abs(pad.reshape(2, 3, 3, 32, 64)).max(-2)
    want = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2 + 127, 0)
    np.testing.assert_array_equal(scales, want.astype(np.uint8))
    # the elements: the grid rounding of x * 2^-e, clamped to +-6
    e = scales.astype(np.int64) - 127
    e = np.repeat(e, 32, axis=-1) if axis == 0 else np.repeat(e, 32, axis=-2)[..., :70, :]
    y = xf * np.exp2(-e.astype(np.float64))
    np.testing.assert_array_equal(_dq4(codes, scales, axis), _e2m1_round_grid(y) * np.exp2(e))
    # every non-zero block's largest element maps into [4, 8) before the clamp
    nz = scales > 0
    assert np.all((amax * np.exp2(-(scales.astype(np.int64) - 127)))[nz] >= 4.0)
    assert np.all((amax * np.exp2(-(scales.astype(np.int64) - 127)))[nz] < 8.0)


def test_quant_mx4_axes_agree_on_the_transpose():
    x = normal((1, 2, 64, 96), 5, torch.float16)
    c1, s1 = oracle.quant_mx4(x, axis=1)
    c0, s0 = oracle.quant_mx4(x.transpose(-1, -2).contiguous(), axis=0)
    np.testing.assert_array_equal(c1, np.swapaxes(c0, -1, -2))
    np.testing.assert_array_equal(s1, np.swapaxes(s0, -1, -2))


def _worked_inputs():
    step = np.float32(np.float32(2.1) / np.float32(127.0))
    q = torch.zeros(1, 1, 1, 32, dtype=torch.float32)
    q[0, 0, 0, 0] = 1.0
    k = torch.zeros(1, 1, 3, 32, dtype=torch.float32)
    for j, n in enumerate((18, -36, -127)):
        k[0, 0, j, 0] = float(np.float32(n * step))
    v = torch.zeros(1, 1, 3, 32, dtype=torch.float32)
    v[0, 0, :, 0] = torch.tensor([4.0, -2.0, 1.0])
    return q, k, v


@pytest.mark.parametrize("pos0,want", [(int(p), float(w)) for p, w in
                                       _golden("mxd_worked_example.txt")])
def test_mxd_worked_row(pos0, want):
    q, k, v = _worked_inputs()
    o = oracle.attn_mxd(q, k, v, scale=math.log(2.0), pos0=pos0)
    assert abs(o[0, 0, 0, 0] - want) < 1e-6
    assert np.all(o[0, 0, 0, 1:] == 0.0)


def test_mxd_single_visible_key_gives_its_dequantised_value():
    # causal row 0 at pos0 = 0 sees key 0 only (diagonal: MXFP8 V); with the
    # shared lower bound 150 and 151 keys, key 150 alone is visible, in tile 2,
    # off the diagonal of rows 0..31 at positions 200..231: MXFP4 V
    q = normal((1, 1, 4, 64), 21, torch.bfloat16)
    k = normal((1, 1, 151, 64), 22, torch.bfloat16)
    v = normal((1, 1, 151, 64), 23, torch.bfloat16)
    c8, s8 = oracle.quant_mx(v, axis=1)
    v8 = np.array([oracle.e4m3_decode(c) for c in range(256)])[c8] * np.exp2(
        np.repeat(s8.astype(np.int64) - 127, 32, axis=-2)[..., :151, :].astype(np.float64))
    c4, s4 = oracle.quant_mx4(v, axis=1)
    v4 = _dq4(c4, s4, 1)
    o = oracle.attn_mxd(q, k, v, scale=0.125, causal=True, pos0=0, rows=[0])
    np.testing.assert_array_equal(o[0], v8[0, 0, 0])
    o = oracle.attn_mxd(q, k, v, scale=0.125, window_lo=150, pos0=200, rows=[0])
    np.testing.assert_array_equal(o[0], v4[0, 0, 150])


def test_mxd_power_of_two_scaling_of_v_is_exact():
    q = normal((1, 2, 40, 64), 41, torch.bfloat16)
    k = normal((1, 1, 200, 64), 42, torch.bfloat16)
    v = normal((1, 1, 200, 64), 43, torch.bfloat16)
    a = oracle.attn_mxd(q, k, v, scale=0.125, causal=True, pos0=160)
    b = oracle.attn_mxd(q, k, v * 8, scale=0.125, causal=True, pos0=160)
    np.testing.assert_array_equal(b, a * 8)


def _mxd_here(q, k, v, scale, pos0, causal):
    """The emulation again, from the stated rules: INT8 Q, K and MX V from the
    oracle's (separately pinned) quantisers; the weights rounded here."""
    qc, qs = oracle.quant_int8(q)
    kc, ks = oracle.quant_int8(k)
    qh = qc.astype(np.float64) * np.repeat(qs.astype(np.float64), 64, -1)[..., : q.shape[2], None]
    kh = kc.astype(np.float64) * np.repeat(ks.astype(np.float64), 64, -1)[..., : k.shape[2], None]
    c8, s8 = oracle.quant_mx(v, axis=1)
    N = v.shape[2]
    v8 = np.array([oracle.e4m3_decode(c) for c in range(256)])[c8] * np.exp2(
        np.repeat(s8.astype(np.int64) - 127, 32, axis=-2)[..., :N, :].astype(np.float64))
    c4, s4 = oracle.quant_mx4(v, axis=1)
    v4 = _dq4(c4, s4, 1)
    B, Hq, Nq, D = q.shape
    G = Hq // k.shape[1]
    out = np.zeros((B, Hq, Nq, D))
    for b in range(B):
        for h in range(Hq):
            t = (qh[b, h] @ kh[b, h // G].T) * scale / math.log(2.0)
            for i in range(Nq):
                vis = np.arange(N) <= pos0 + i if causal else np.ones(N, bool)
                if not vis.any():
                    continue
                M = math.floor(t[i][vis].max())
                num, den = np.zeros(D), 0.0
                for b0 in range(0, N, 32):
                    js = [j for j in range(b0, min(b0 + 32, N)) if vis[j]]
                    if not js:
                        continue
                    r0, k0 = pos0 + 32 * (i // 32), 64 * (b0 // 64)
                    diag = k0 <= r0 + 31 and k0 + 63 >= r0
                    x = t[i][js] - M
                    E = math.floor(x.max()) - (7 if diag else 2)
                    w = np.exp2(x - E)
                    if diag:
                        pw = torch.from_numpy(w).float().to(torch.float8_e4m3fn).double().numpy()
                    else:
                        pw = _e2m1_round_grid(np.minimum(w, 6.0))
                    pw = pw * 2.0 ** E
                    vv = (v8 if diag else v4)[b, h // G, js]
                    num += pw @ vv
                    den += pw.sum()
                out[b, h, i] = num / den
    return out


@pytest.mark.parametrize("pos0,causal", [(0, True), (37, True), (0, False), (90, False)])
def test_mxd_matches_a_second_implementation(pos0, causal):
    q = normal((1, 2, 70, 64), 100 + pos0, torch.bfloat16)
    k = normal((1, 1, 150, 64), 200 + pos0, torch.bfloat16)
    v = normal((1, 1, 150, 64), 300 + pos0, torch.bfloat16)
    got = oracle.attn_mxd(q, k, v, scale=0.3, causal=causal, pos0=pos0)
    want = _mxd_here(q, k, v, 0.3, pos0, causal)
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-12)


def test_mxd_error_against_exact_attention():
    # FP4 weights and values cost far more than the MXFP8-only variant; rows
    # whose keys all sit in diagonal tiles keep the MXFP8 precision
    q = normal((1, 2, 128, 64), 91, torch.bfloat16)
    k = normal((1, 2, 1024, 64), 92, torch.bfloat16)
    v = normal((1, 2, 1024, 64), 93, torch.bfloat16)
    ex = oracle.attn(q, k, v, scale=0.125)
    md = oracle.attn_mxd(q, k, v, scale=0.125, pos0=0)
    rel = np.linalg.norm(md - ex) / np.linalg.norm(ex)
    assert 0.05 < rel < 0.4, rel
    kk, vv = k[:, :, :64], v[:, :, :64]
    ex = oracle.attn(q[:, :, :32], kk, vv, scale=0.125)
    md = oracle.attn_mxd(q[:, :, :32], kk, vv, scale=0.125, pos0=0)
    rel = np.linalg.norm(md - ex) / np.linalg.norm(ex)
    assert rel < 0.06, rel
