"""Pins for the exact-attention oracle (oracle.attn), CPU only.

Each test checks the oracle against something other than itself: a closed
form, an invariant of softmax attention, brute force on a tiny input, or a
library routine (torch's float64 scaled_dot_product_attention on the CPU).
Together they are chosen so that a dropped term (scale, max shift), a wrong
sign, a wrong index (GQA head, causal offset, window edge) or a transposed
operand fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from scaled_dot_product_amd.inputs import Workload, make_qkv, normal


def _dyadic(shape, seed, lo=-48, hi=48, den=16.0):
    """Small dyadic rationals: exact in fp32 and closed under +, * by dyadics."""
    g = torch.Generator().manual_seed(seed)
    return (torch.randint(lo, hi + 1, shape, generator=g).to(torch.float32) / den)


def test_single_key_returns_v():
    q = normal((1, 2, 5, 16), 1, torch.float32)
    k = normal((1, 2, 1, 16), 2, torch.float32)
    v = normal((1, 2, 1, 16), 3, torch.float32)
    o = oracle.attn(q, k, v, scale=0.7)
    for h in range(2):
        for i in range(5):
            np.testing.assert_array_equal(o[0, h, i], v[0, h, 0].double().numpy())


def test_two_keys_logistic_closed_form():
    D = 4
    q = torch.zeros(1, 1, 1, D)
    q[0, 0, 0, 0] = 1.0
    k = torch.zeros(1, 1, 2, D)
    k[0, 0, 0, 0] = 1.5
    k[0, 0, 1, 0] = -0.25
    v = torch.tensor([[[[1.0, 2.0, -3.0, 0.5], [-1.0, 4.0, 0.25, 8.0]]]])
    scale = 0.8
    s0, s1 = scale * 1.5, scale * -0.25
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    w1 = 1.0 / (1.0 + math.exp(s0 - s1))
    want = w0 * v[0, 0, 0].double().numpy() + w1 * v[0, 0, 1].double().numpy()
    o, lse = oracle.attn(q, k, v, scale=scale, want_lse=True)
    np.testing.assert_allclose(o[0, 0, 0], want, rtol=0, atol=1e-14)
    assert abs(lse[0] - math.log(math.exp(s0) + math.exp(s1))) < 1e-14


def test_hand_example_three_keys():
    # scores 0, ln2-ish and -inf (masked by the window) worked by hand:
    # with q = e0 and keys k_j = a_j e0, scale 1: weights are exp(a_j)/sum.
    q = torch.tensor([[[[1.0, 0.0]]]])
    k = torch.tensor([[[[5.0, 9.0], [0.0, 1.0], [1.0, -1.0]]]])
    v = torch.tensor([[[[100.0, 100.0], [2.0, 0.0], [0.0, 2.0]]]])
    o, w = oracle.attn(q, k, v, scale=1.0, window_lo=1, want_weights=True)
    e = math.e
    np.testing.assert_allclose(w[0], [0.0, 1 / (1 + e), e / (1 + e)], atol=1e-15)
    np.testing.assert_allclose(o[0, 0, 0], [2 / (1 + e), 2 * e / (1 + e)], atol=1e-14)


def test_weights_rows_sum_to_one_and_masked_zero():
    w = Workload("t", 1, 2, 1, 24, 40, 8, torch.float32, causal=True, pos0=5, window_lo=3)
    q, k, v = make_qkv(w)
    _, wts = oracle.attn(q, k, v, scale=w.scale, causal=True, pos0=5, window_lo=3,
                         want_weights=True)
    for r in range(wts.shape[0]):
        i = r % w.Nq
        vis = np.array([(j >= 3 and j <= 5 + i) for j in range(w.Nk)])
        assert np.all(wts[r][~vis] == 0.0)
        assert np.all(wts[r][vis] > 0.0)
        assert abs(wts[r].sum() - 1.0) < 1e-12


def test_constant_v_gives_constant_output():
    q = normal((1, 2, 16, 8), 5, torch.float32)
    k = normal((1, 2, 33, 8), 6, torch.float32)
    v = torch.full((1, 2, 33, 8), 0.375)
    o = oracle.attn(q, k, v, scale=0.35, causal=True, pos0=3)
    np.testing.assert_allclose(o, 0.375, rtol=0, atol=1e-15)


def test_key_permutation_invariance_noncausal():
    q = normal((1, 1, 8, 16), 7, torch.float32)
    k = normal((1, 1, 50, 16), 8, torch.float32)
    v = normal((1, 1, 50, 16), 9, torch.float32)
    perm = torch.randperm(50, generator=torch.Generator().manual_seed(3))
    o1 = oracle.attn(q, k, v, scale=0.25)
    o2 = oracle.attn(q, k[:, :, perm], v[:, :, perm], scale=0.25)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)


def test_single_visible_key_returns_its_row():
    q = normal((1, 1, 4, 8), 10, torch.float32)
    k = normal((1, 1, 20, 8), 11, torch.float32)
    v = normal((1, 1, 20, 8), 12, torch.float32)
    # window lower bound at the last key: one visible key for every row
    o = oracle.attn(q, k, v, scale=1.0, window_lo=19)
    for i in range(4):
        np.testing.assert_array_equal(o[0, 0, i], v[0, 0, 19].double().numpy())
    # causal, pos0 = 0: row 0 sees key 0 only
    o = oracle.attn(q, k, v, scale=1.0, causal=True)
    np.testing.assert_array_equal(o[0, 0, 0], v[0, 0, 0].double().numpy())


def test_fully_masked_rows_are_zero():
    q = normal((1, 1, 6, 8), 13, torch.float32)
    k = normal((1, 1, 20, 8), 14, torch.float32)
    v = normal((1, 1, 20, 8), 15, torch.float32)
    # rows i with pos0 + i < window_lo see nothing
    o, lse = oracle.attn(q, k, v, scale=1.0, causal=True, pos0=2, window_lo=5,
                         want_lse=True)
    for i in range(6):
        if 2 + i < 5:
            assert np.all(o[0, 0, i] == 0.0) and lse[i] == -np.inf
        else:
            assert np.any(o[0, 0, i] != 0.0) and np.isfinite(lse[i])


def test_key_shift_invariance():
    # adding one vector c to every key adds q.c to a whole score row
    q = _dyadic((1, 2, 12, 8), 1)
    k = _dyadic((1, 2, 30, 8), 2)
    v = _dyadic((1, 2, 30, 8), 3)
    c = _dyadic((8,), 4)
    o1 = oracle.attn(q, k, v, scale=0.5, causal=True, pos0=10)
    o2 = oracle.attn(q, k + c, v, scale=0.5, causal=True, pos0=10)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)


def test_linearity_in_v():
    q = _dyadic((1, 1, 10, 8), 5)
    k = _dyadic((1, 1, 25, 8), 6)
    v1 = _dyadic((1, 1, 25, 8), 7)
    v2 = _dyadic((1, 1, 25, 8), 8)
    a, b = 0.75, -2.5
    o1 = oracle.attn(q, k, v1, scale=0.3)
    o2 = oracle.attn(q, k, v2, scale=0.3)
    o12 = oracle.attn(q, k, a * v1 + b * v2, scale=0.3)
    np.testing.assert_allclose(o12, a * o1 + b * o2, rtol=0, atol=1e-12)


def test_zero_scale_gives_mean_of_visible_v():
    q = normal((1, 1, 5, 8), 16, torch.float32)
    k = normal((1, 1, 30, 8), 17, torch.float32)
    v = normal((1, 1, 30, 8), 18, torch.float32)
    o = oracle.attn(q, k, v, scale=0.0, causal=True, pos0=20, window_lo=4)
    vv = v[0, 0].double().numpy()
    for i in range(5):
        np.testing.assert_allclose(o[0, 0, i], vv[4:21 + i].mean(axis=0), atol=1e-14)


def test_gqa_head_mapping_closed_form():
    # V of kv-head g is the constant g, so every output of query head h is h // G
    B, Hq, Hkv = 2, 6, 3
    q = normal((B, Hq, 7, 8), 19, torch.float32)
    k = normal((B, Hkv, 11, 8), 20, torch.float32)
    v = torch.arange(Hkv, dtype=torch.float32).view(1, Hkv, 1, 1).expand(B, Hkv, 11, 8).contiguous()
    o = oracle.attn(q, k, v, scale=0.4)
    for h in range(Hq):
        np.testing.assert_allclose(o[:, h], h // (Hq // Hkv), atol=1e-14)


def test_causal_row_equals_truncated_noncausal():
    q = normal((1, 1, 6, 8), 21, torch.float32)
    k = normal((1, 1, 40, 8), 22, torch.float32)
    v = normal((1, 1, 40, 8), 23, torch.float32)
    pos0 = 30
    o = oracle.attn(q, k, v, scale=0.6, causal=True, pos0=pos0)
    for i in range(6):
        n = min(40, pos0 + i + 1)
        oi = oracle.attn(q[:, :, i:i + 1], k[:, :, :n].contiguous(), v[:, :, :n].contiguous(),
                         scale=0.6)
        np.testing.assert_allclose(o[0, 0, i], oi[0, 0, 0], rtol=0, atol=1e-14)


def test_window_equals_sliced_keys():
    q = normal((1, 2, 9, 8), 24, torch.float32)
    k = normal((1, 2, 64, 8), 25, torch.float32)
    v = normal((1, 2, 64, 8), 26, torch.float32)
    o = oracle.attn(q, k, v, scale=0.6, window_lo=17)
    o2 = oracle.attn(q, k[:, :, 17:].contiguous(), v[:, :, 17:].contiguous(), scale=0.6)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-14)


def test_large_logits_are_stable():
    q = normal((1, 1, 8, 16), 27, torch.float32) * 100
    k = normal((1, 1, 32, 16), 28, torch.float32) * 1000
    v = normal((1, 1, 32, 16), 29, torch.float32)
    o, w = oracle.attn(q, k, v, scale=1.0, want_weights=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(w))
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-12)


def _sdpa_reference(q, k, v, scale, causal, window_lo, pos0):
    """torch float64 SDPA on the CPU with an explicit boolean mask."""
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    i = torch.arange(Nq).view(-1, 1)
    j = torch.arange(Nk).view(1, -1)
    mask = (j >= window_lo) & (i >= 0)
    if causal:
        mask = mask & (j <= pos0 + i)
    G = Hq // Hkv
    kk = k.double().repeat_interleave(G, dim=1)
    vv = v.double().repeat_interleave(G, dim=1)
    out = torch.nn.functional.scaled_dot_product_attention(
        q.double(), kk, vv, attn_mask=mask, scale=scale)
    return out.numpy(), mask.any(dim=1).numpy()


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("causal,window_lo,pos0", [(False, 0, 0), (True, 0, 0),
                                                   (True, 0, 37), (True, 23, 40),
                                                   (False, 9, 0), (True, 60, 0)])
def test_matches_torch_sdpa_float64(dtype, causal, window_lo, pos0):
    w = Workload("x", 2, 4, 2, 19, 77, 16, dtype)
    q, k, v = make_qkv(w)
    o = oracle.attn(q, k, v, scale=0.3, causal=causal, window_lo=window_lo, pos0=pos0)
    ref, has_key = _sdpa_reference(q, k, v, 0.3, causal, window_lo, pos0)
    rows_ok = has_key
    np.testing.assert_allclose(o[:, :, rows_ok], ref[:, :, rows_ok], rtol=0, atol=1e-12)
    assert np.all(o[:, :, ~rows_ok] == 0.0)


def test_causal_pos0_zero_matches_sdpa_is_causal():
    w = Workload("x", 1, 3, 3, 48, 48, 32, torch.bfloat16)
    q, k, v = make_qkv(w)
    o = oracle.attn(q, k, v, scale=1 / math.sqrt(32), causal=True)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.double(), k.double(), v.double(), is_causal=True, scale=1 / math.sqrt(32))
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)


def test_lse_matches_logsumexp():
    w = Workload("x", 1, 2, 1, 10, 45, 16, torch.float16)
    q, k, v = make_qkv(w)
    _, lse = oracle.attn(q, k, v, scale=0.25, causal=True, pos0=30, want_lse=True)
    s = 0.25 * torch.matmul(q.double(), k.double().transpose(-1, -2).repeat_interleave(2, dim=1))
    i = torch.arange(10).view(-1, 1)
    j = torch.arange(45).view(1, -1)
    s = s.masked_fill(~(j <= 30 + i), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).reshape(-1).numpy(), atol=1e-12)


def test_row_subset_equals_full():
    w = Workload("x", 2, 4, 2, 33, 70, 16, torch.bfloat16, causal=True, pos0=20)
    q, k, v = make_qkv(w)
    full = oracle.attn(q, k, v, scale=0.2, causal=True, pos0=20).reshape(-1, 16)
    rows = np.array([0, 5, 32, 33, 100, 263], dtype=np.int64)
    sub = oracle.attn(q, k, v, scale=0.2, causal=True, pos0=20, rows=rows)
    np.testing.assert_array_equal(sub, full[rows])
    # a row list may only name rows that exist (2 x 4 x 33 = 264 of them)
    for bad in (264, -1):
        with pytest.raises(ValueError):
            oracle.attn(q, k, v, scale=0.2, causal=True, pos0=20,
                        rows=np.array([0, bad], dtype=np.int64))


def test_input_widening_is_exact_for_every_f16_and_bf16_code():
    # one key: the output row is V itself, so it exposes the decoder exactly
    for dt in (torch.float16, torch.bfloat16):
        bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
        vals = bits.view(dt)
        finite = torch.isfinite(vals.float())
        vals = vals[finite]
        D = vals.numel()
        v = vals.view(1, 1, 1, D).contiguous()
        q = torch.zeros(1, 1, 1, D, dtype=dt)
        k = torch.zeros(1, 1, 1, D, dtype=dt)
        o = oracle.attn(q, k, v, scale=1.0)
        np.testing.assert_array_equal(o.reshape(-1), vals.double().numpy())


# ---- per-row sliding window ---------------------------------------------------

@pytest.mark.parametrize("causal", [True, False])
def test_sliding_window_rows_equal_unmasked_attention_on_their_keys(causal):
    # row i sees keys [max(0, pos0 + i - W + 1), pos0 + i] (causal) or
    # [max(0, pos0 + i - W + 1), Nk) (not causal): the same as plain attention of
    # that one row over exactly those keys
    B, Hq, Hkv, Nq, Nk, D, W, pos0 = 1, 4, 2, 20, 90, 32, 13, 60
    q = normal((B, Hq, Nq, D), 1, torch.float32)
    k = normal((B, Hkv, Nk, D), 2, torch.float32)
    v = normal((B, Hkv, Nk, D), 3, torch.float32)
    got = oracle.attn(q, k, v, scale=0.2, causal=causal, pos0=pos0, window_w=W)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        for i in range(Nq):
            lo = max(0, pos0 + i - W + 1)
            hi = min(Nk, pos0 + i + 1) if causal else Nk
            if hi <= lo:
                assert np.all(got[0, h, i] == 0)
                continue
            want = oracle.attn(q[:, h:h + 1, i:i + 1], k[:, g:g + 1, lo:hi].contiguous(),
                               v[:, g:g + 1, lo:hi].contiguous(), scale=0.2)
            np.testing.assert_allclose(got[0, h, i], want[0, 0, 0], rtol=1e-13, atol=1e-14)


def test_sliding_window_wider_than_the_history_is_no_window():
    B, Hq, Hkv, Nq, Nk, D, pos0 = 1, 2, 1, 16, 40, 16, 24
    q, k, v = (normal(s, sd, torch.float16) for s, sd in
               (((B, Hq, Nq, D), 4), ((B, Hkv, Nk, D), 5), ((B, Hkv, Nk, D), 6)))
    a = oracle.attn(q, k, v, scale=0.25, causal=True, pos0=pos0)
    b = oracle.attn(q, k, v, scale=0.25, causal=True, pos0=pos0, window_w=pos0 + Nq)
    assert np.array_equal(a, b)
    c = oracle.attn(q, k, v, scale=0.25, causal=True, pos0=pos0, window_w=pos0 + Nq - 1)
    assert not np.array_equal(a[0, :, Nq - 1], c[0, :, Nq - 1])   # the last row loses key 0


def test_sliding_window_of_one_is_the_diagonal_value():
    # causal, W = 1: row i sees only key pos0 + i, with weight 1
    B, Hq, Hkv, Nq, Nk, D, pos0 = 1, 3, 3, 10, 30, 8, 17
    q, k, v = (normal(s, sd, torch.bfloat16) for s, sd in
               (((B, Hq, Nq, D), 7), ((B, Hkv, Nk, D), 8), ((B, Hkv, Nk, D), 9)))
    got = oracle.attn(q, k, v, scale=1.0, causal=True, pos0=pos0, window_w=1)
    want = v[0, :, pos0:pos0 + Nq].double().numpy()
    assert np.array_equal(got[0], want)


def test_sliding_window_single_row_equals_shared_lower_bound():
    B, Hq, Hkv, Nk, D, W, pos0 = 2, 2, 2, 70, 16, 25, 66
    q, k, v = (normal(s, sd, torch.float32) for s, sd in
               (((B, Hq, 1, D), 10), ((B, Hkv, Nk, D), 11), ((B, Hkv, Nk, D), 12)))
    a = oracle.attn(q, k, v, scale=0.3, causal=True, pos0=pos0, window_w=W)
    b = oracle.attn(q, k, v, scale=0.3, causal=True, pos0=pos0, window_lo=pos0 - W + 1)
    assert np.array_equal(a, b)
