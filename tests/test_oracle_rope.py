"""Pins for the oracle's rotary position embedding (CPU only): frequencies in
closed form for the plain, NTK and YaRN rules, the rotation's invariants (norm,
identity at position 0, the pair layouts as permutations of each other, the
relative-position property of the scores) and attention on rotated inputs."""
import math

import numpy as np
import pytest
import torch

import oracle
from scaled_dot_product_amd.inputs import normal


def test_plain_frequencies_closed_form():
    th, mult = oracle.rope_freqs(8, oracle.ROPE_PLAIN, base=10000.0)
    np.testing.assert_allclose(th, [1.0, 0.1, 0.01, 0.001], rtol=1e-15)
    assert mult == 1.0
    th, _ = oracle.rope_freqs(4, oracle.ROPE_PLAIN, base=16.0)
    np.testing.assert_allclose(th, [1.0, 0.25], rtol=1e-15)


def test_ntk_frequencies_closed_form():
    th1, _ = oracle.rope_freqs(8, oracle.ROPE_NTK, base=10000.0, factor=1.0)
    np.testing.assert_allclose(th1, [1.0, 0.1, 0.01, 0.001], rtol=1e-15)
    # base' = 10000 * 8^(8/6) = 10000 * 16: theta_i = (160000)^(-i/4)
    th, _ = oracle.rope_freqs(8, oracle.ROPE_NTK, base=10000.0, factor=8.0)
    np.testing.assert_allclose(th, [160000.0 ** (-i / 4) for i in range(4)], rtol=1e-13)


def test_yarn_regimes():
    # s = 1 is the plain rule with no logit factor
    th, mult = oracle.rope_freqs(8, oracle.ROPE_YARN, base=10000.0, factor=1.0, orig_ctx=64)
    np.testing.assert_allclose(th, [1.0, 0.1, 0.01, 0.001], rtol=1e-15)
    assert mult == 1.0
    # s = 4, L = 64: wavelengths 2 pi / theta_i; L / wavelength = 10.19, 1.02,
    # 0.10, 0.01: the last two (below beta_slow = 1) are pure interpolation
    # theta / 4; with beta_fast = 10 the first is pure extrapolation theta
    th, mult = oracle.rope_freqs(8, oracle.ROPE_YARN, base=10000.0, factor=4.0, orig_ctx=64,
                                 beta_fast=10.0, beta_slow=1.0)
    assert th[0] == 1.0
    np.testing.assert_allclose(th[2:], [0.0025, 0.00025], rtol=1e-14)
    r1 = 64 * 0.1 / (2 * math.pi)
    g = (r1 - 1.0) / 9.0
    np.testing.assert_allclose(th[1], (1 - g) * 0.025 + g * 0.1, rtol=1e-13)
    np.testing.assert_allclose(mult, (0.1 * math.log(4.0) + 1.0) ** 2, rtol=1e-15)


@pytest.mark.parametrize("style", [oracle.ROPE_HALF, oracle.ROPE_INTERLEAVED])
def test_rotation_invariants(style):
    x = normal((2, 3, 40, 64), 61, torch.float32)
    th, _ = oracle.rope_freqs(64)
    y = oracle.rope_apply(x, 0, th, style)
    # position 0 is the identity (row 0 of every head)
    np.testing.assert_allclose(y[:, :, 0], x[:, :, 0].double().numpy(), rtol=0, atol=0)
    # each pair keeps its length
    xd = x.double().numpy()
    if style == oracle.ROPE_HALF:
        nx = xd[..., :32] ** 2 + xd[..., 32:] ** 2
        ny = y[..., :32] ** 2 + y[..., 32:] ** 2
    else:
        nx = xd[..., 0::2] ** 2 + xd[..., 1::2] ** 2
        ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-12, atol=1e-14)


def test_pair_layouts_are_permutations_of_each_other():
    x = normal((1, 2, 17, 32), 62, torch.float32)
    th, _ = oracle.rope_freqs(32, base=500.0)
    # z = x[perm] puts x's interleaved pair (2i, 2i+1) at half-split places (i, i+16)
    perm = np.array([2 * i for i in range(16)] + [2 * i + 1 for i in range(16)])
    y_int = oracle.rope_apply(x, 5, th, oracle.ROPE_INTERLEAVED)
    y_half = oracle.rope_apply(x[..., perm].contiguous(), 5, th, oracle.ROPE_HALF)
    np.testing.assert_allclose(y_half, y_int[..., perm], rtol=1e-13, atol=1e-14)


def test_rotated_scores_depend_on_relative_position_only():
    # q at position m, k at position n: (R_m q) . (R_n k) = (R_{m-n} q) . k
    x = normal((1, 1, 2, 64), 63, torch.float32)
    th, _ = oracle.rope_freqs(64)
    q, k = x[:, :, :1], x[:, :, 1:]
    for m, n in ((7, 3), (100, 96), (4, 0)):
        s1 = (oracle.rope_apply(q, m, th) * oracle.rope_apply(k, n, th)).sum()
        s2 = (oracle.rope_apply(q, m - n, th) * k.double().numpy()).sum()
        np.testing.assert_allclose(s1, s2, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("style,scaling", [(0, 0), (1, 1), (0, 2)])
def test_attention_on_rotated_inputs(style, scaling):
    # attn_rope = attn on Q, K rotated by rope_apply (values rounded to fp32
    # for the second call), scale times the logit multiplier
    B, Hq, Hkv, Nq, Nk, D, pos0 = 1, 4, 2, 12, 40, 64, 28
    q, k, v = (normal(s, sd, torch.bfloat16) for s, sd in
               (((B, Hq, Nq, D), 64), ((B, Hkv, Nk, D), 65), ((B, Hkv, Nk, D), 66)))
    kw = dict(scaling=scaling, base=10000.0, factor=4.0 if scaling else 1.0, orig_ctx=16)
    th, mult = oracle.rope_freqs(D, **kw)
    qr = torch.from_numpy(oracle.rope_apply(q, pos0, th, style).astype(np.float32))
    kr = torch.from_numpy(oracle.rope_apply(k, 0, th, style).astype(np.float32))
    want = oracle.attn(qr, kr, v.float(), scale=0.125 * mult, causal=True, pos0=pos0)
    got = oracle.attn_rope(q, k, v, scale=0.125, causal=True, pos0=pos0, style=style, **kw)
    np.testing.assert_allclose(got, want, rtol=2e-6, atol=2e-6)
    # and the rotation is really applied
    plain = oracle.attn(q, k, v, scale=0.125, causal=True, pos0=pos0)
    assert np.abs(got - plain).max() > 1e-2
