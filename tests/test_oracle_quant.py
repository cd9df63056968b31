"""Pins for the oracle's quantisers and E4M3 codec (CPU only).

Checked against the OCP E4M3 definition (named values, exhaustive round
trips, tie rules), torch's own float8_e4m3fn cast (a library routine), closed
forms of the symmetric INT8 quantiser (integer and half-integer blocks,
power-of-two scaling, sign symmetry, the amax element mapping to +-127), and
the page's printed error of the INT8-QK / FP8-PV recipe.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from scaled_dot_product_amd.inputs import Workload, make_qkv, normal, sample_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e4m3_named():
    out = []
    with open(os.path.join(GOLDEN, "e4m3_ocp_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                val, code = line.split()
                out.append((float(val), int(code, 16)))
    return out


@pytest.mark.parametrize("val,code", _e4m3_named())
def test_e4m3_named_values(val, code):
    assert oracle.e4m3_encode(val) == code
    dec = oracle.e4m3_decode(code)
    assert dec == val and math.copysign(1.0, dec) == math.copysign(1.0, val)


def test_e4m3_nan_codes():
    assert math.isnan(oracle.e4m3_decode(0x7F))
    assert math.isnan(oracle.e4m3_decode(0xFF))


def test_e4m3_round_trip_every_code():
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        assert oracle.e4m3_encode(oracle.e4m3_decode(c)) == c


def test_e4m3_midpoints_tie_to_even():
    mags = sorted({abs(oracle.e4m3_decode(c)) for c in range(0x7F)})
    for a, b in zip(mags[:-1], mags[1:]):
        mid = (a + b) / 2.0  # exact in fp32 (one more mantissa bit)
        ca, cb = oracle.e4m3_encode(a), oracle.e4m3_encode(b)
        want = ca if ca % 2 == 0 else cb
        assert oracle.e4m3_encode(mid) == want
        assert oracle.e4m3_encode(-mid) == want | 0x80
        # just off the midpoint goes to the nearer side
        assert oracle.e4m3_encode(np.nextafter(np.float32(mid), np.float32(0))) == ca
        assert oracle.e4m3_encode(np.nextafter(np.float32(mid), np.float32(1e9))) == cb


def test_e4m3_matches_torch_float8_cast():
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch has no float8_e4m3fn")
    g = np.random.default_rng(5)
    vals = np.concatenate([
        np.arange(-448 * 64, 448 * 64 + 1) / 64.0,
        g.uniform(-448, 448, 4000),
        g.standard_normal(4000) * 0.01,
        np.ldexp(g.uniform(-1, 1, 2000), -8),
    ]).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([oracle.e4m3_encode(float(x)) for x in vals], dtype=np.uint8)
    np.testing.assert_array_equal(ours, ref)


def test_int8_integer_block_is_identity():
    # amax 127 gives scale = inv = 1, so integer inputs are their own codes
    x = torch.arange(-127, 129, dtype=torch.float32)[:256].clamp(-127, 127)
    x = x.reshape(1, 64, 4)
    codes, scales = oracle.quant_int8(x)
    assert scales.tolist() == [[1.0]]
    np.testing.assert_array_equal(codes.astype(np.float32), x.numpy())


def test_int8_half_integers_round_to_even():
    half = torch.tensor([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 127.0])
    x = torch.zeros(1, 64, 8)
    x[0, 0] = half
    codes, scales = oracle.quant_int8(x)
    assert scales[0, 0] == 1.0
    assert codes[0, 0].tolist() == [0, 2, 2, 0, -2, -2, 126, 127]


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_int8_properties_on_random_blocks(dtype):
    x = normal((3, 200, 32), 11, dtype)      # 4 blocks per head, last holds 8 tokens
    codes, scales = oracle.quant_int8(x)
    assert codes.shape == (3, 200, 32) and scales.shape == (3, 4)
    xf = x.float().numpy()
    for h in range(3):
        for t in range(4):
            blk = xf[h, 64 * t:64 * t + 64]
            cb = codes[h, 64 * t:64 * t + 64].astype(np.int32)
            amax = np.float32(np.abs(blk).max())
            assert scales[h, t] == np.float32(amax / np.float32(127))
            assert np.abs(cb).max() == 127 and np.all(np.abs(cb) <= 127)
            # the amax element maps to +-127 with its sign
            idx = np.unravel_index(np.abs(blk).argmax(), blk.shape)
            assert cb[idx] == (127 if blk[idx] > 0 else -127)
            err = np.abs(blk.astype(np.float64) - cb * np.float64(scales[h, t]))
            # half a step, plus the fp32 rounding of x*inv (|x*inv| <= 127)
            assert err.max() <= scales[h, t] * (0.5 + 2 ** -12)


def test_int8_sign_symmetry_and_power_of_two_scaling():
    x = normal((2, 130, 16), 12, torch.float32)
    c0, s0 = oracle.quant_int8(x)
    c1, s1 = oracle.quant_int8(-x)
    np.testing.assert_array_equal(c1, -c0)
    np.testing.assert_array_equal(s1, s0)
    c2, s2 = oracle.quant_int8(x * 8.0)
    np.testing.assert_array_equal(c2, c0)
    np.testing.assert_array_equal(s2, s0 * 8.0)


def test_blocks_are_independent_and_zero_block():
    x = normal((1, 192, 8), 13, torch.float32)
    x[0, 64:128] = 0.0
    c0, s0 = oracle.quant_int8(x)
    assert s0[0, 1] == 0.0 and np.all(c0[0, 64:128] == 0)
    e0, es0 = oracle.quant_e4m3(x)
    assert es0[0, 1] == 0.0 and np.all(e0[0, 64:128] == 0)
    y = x.clone()
    y[0, 150] *= 3.0
    c1, s1 = oracle.quant_int8(y)
    np.testing.assert_array_equal(c1[0, :128], c0[0, :128])
    np.testing.assert_array_equal(s1[0, :2], s0[0, :2])


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_e4m3_quantiser_properties(dtype):
    x = normal((2, 100, 64), 14, dtype)
    codes, scales = oracle.quant_e4m3(x)
    xf = x.float().numpy()
    for h in range(2):
        for t in range(2):
            blk = xf[h, 64 * t:64 * t + 64]
            amax = np.float32(np.abs(blk).max())
            assert scales[h, t] == np.float32(amax / np.float32(448))
            inv = np.float32(np.float32(448) / amax)
            y = np.clip((blk * inv).astype(np.float32), -448, 448)
            # codes equal torch's float8 cast of the clamped scaled block
            ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            np.testing.assert_array_equal(codes[h, 64 * t:64 * t + 64], ref)
            # the amax element saturates to the largest finite magnitude
            idx = np.unravel_index(np.abs(blk).argmax(), blk.shape)
            assert codes[h, 64 * t + idx[0], idx[1]] & 0x7F == 0x7E


def test_quant_emulation_uniform_scores_closed_form():
    # Q = 0: Q's block amax is 0, so every score is 0 and every weight is 1,
    # which E4M3 holds exactly at scale 448: the output is the mean of V^.
    w = Workload("x", 1, 1, 1, 8, 70, 32, torch.bfloat16, causal=True, pos0=40, window_lo=5)
    _, k, v = make_qkv(w)
    q = torch.zeros(w.q_shape, dtype=torch.bfloat16)
    o = oracle.attn_quant(q, k, v, scale=w.scale, causal=True, pos0=40, window_lo=5)
    vc, vs = oracle.quant_e4m3(v)
    dec = np.array([oracle.e4m3_decode(c) for c in range(256)])
    vhat = dec[vc[0, 0]] * np.repeat(vs[0, 0].astype(np.float64), 64)[:70, None]
    for i in range(8):
        np.testing.assert_allclose(o[0, 0, i], vhat[5:41 + i].mean(axis=0), atol=1e-13)


def test_quant_emulation_exact_inputs_closed_form():
    # integer Q, K with amax 127 and V of E4M3 values with amax 448 are their own
    # codes; scores differ by multiples of ln 2 (to fp32 rounding of the scale),
    # so every 448 * p_j is 448 * 2^-n up to rounding and E4M3 keeps it exactly.
    D, Nk = 4, 6
    q = torch.zeros(1, 1, 1, D)
    q[0, 0, 0, 0] = 127.0
    k = torch.zeros(1, 1, Nk, D)
    k[0, 0, :, 0] = torch.tensor([1.0, 0.0, -1.0, -2.0, 1.0, 0.0])
    k[0, 0, 0, 1] = 127.0   # make K's amax 127 without touching the scores
    v = torch.zeros(1, 1, Nk, D)
    v[0, 0, :, 0] = torch.tensor([448.0, 2.0, -3.0, 0.5, 1.0, -8.0])
    scale = math.log(2.0) / 127.0
    o = oracle.attn_quant(q, k, v, scale=scale)
    p = np.array([2.0 ** n for n in (0, -1, -2, -3, 0, -1)])
    s = np.array([1.0, 0.0, -1.0, -2.0, 1.0, 0.0]) * 127 * scale
    l = np.exp(s - s.max()).sum()
    want = (p * v[0, 0, :, 0].double().numpy()).sum() / l
    assert abs(o[0, 0, 0, 0] - want) < 1e-6 * abs(want)


def test_quant_emulation_error_matches_page_figure():
    with open(os.path.join(GOLDEN, "page_error_figures.json")) as f:
        fig = json.load(f)
    lo, hi = fig["band_used_in_tests"]
    w = Workload("x", 1, 1, 1, 4096, 4096, 128, torch.bfloat16)
    q, k, v = make_qkv(w)
    rows = sample_rows(w, 128)
    ex = oracle.attn(q, k, v, scale=w.scale, rows=rows)
    qe = oracle.attn_quant(q, k, v, scale=w.scale, rows=rows)
    err = np.linalg.norm(qe - ex) / np.linalg.norm(ex)
    assert lo <= err <= hi, err


# ---- attention over a quantised KV cache --------------------------------------

def _f8_values(codes):
    """E4M3 code bytes -> values through torch's float8_e4m3fn (a library cast)."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(codes, dtype=np.uint8)))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _random_cache(rng, B, Hkv, Nk, D):
    nblk = (Nk + 63) // 64
    kc = rng.integers(-127, 128, size=(B, Hkv, Nk, D)).astype(np.int8)
    mag = rng.integers(0, 0x7F, size=(B, Hkv, Nk, D))           # 0x7F (NaN) excluded
    vc = (mag | (rng.integers(0, 2, size=mag.shape) << 7)).astype(np.uint8)
    # power-of-two block scales keep every dequantised value exact in fp32
    ks = np.ldexp(1.0, rng.integers(-9, -4, size=(B, Hkv, nblk))).astype(np.float32)
    vs = np.ldexp(1.0, rng.integers(-6, 0, size=(B, Hkv, nblk))).astype(np.float32)
    return kc, ks, vc, vs


def _per_key(scales, Nk):
    return np.repeat(scales.astype(np.float64), 64, axis=2)[:, :, :Nk, None]


@pytest.mark.parametrize("causal,window_lo,pos0", [(False, 0, 0), (True, 0, 147), (True, 40, 100),
                                                    (False, 130, 0)])
def test_kvq_exact_cache_matches_attention(causal, window_lo, pos0):
    # codes * power-of-two scales are exact fp32 values: attention over the cache
    # must equal exact attention over those values (V decoded by torch's cast)
    B, Hq, Hkv, Nq, Nk, D = 2, 6, 3, 3, 150, 64
    rng = np.random.default_rng(5)
    kc, ks, vc, vs = _random_cache(rng, B, Hkv, Nk, D)
    kf = torch.from_numpy((kc.astype(np.float64) * _per_key(ks, Nk)).astype(np.float32))
    vf = torch.from_numpy((_f8_values(vc) * _per_key(vs, Nk)).astype(np.float32))
    q = normal((B, Hq, Nq, D), 11, torch.float32)
    sc = 0.125
    want = oracle.attn(q, kf, vf, scale=sc, causal=causal, window_lo=window_lo, pos0=pos0)
    got = oracle.attn_kvq(q, kc, ks, vc, vs, scale=sc, causal=causal, window_lo=window_lo,
                          pos0=pos0)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_kvq_zero_keys_give_the_mean_of_visible_values():
    # all K codes 0: every score is 0, so each row is the plain mean of the
    # values of its visible keys
    B, Hq, Hkv, Nq, Nk, D = 1, 4, 2, 5, 200, 64
    rng = np.random.default_rng(9)
    _, ks, vc, vs = _random_cache(rng, B, Hkv, Nk, D)
    kc = np.zeros((B, Hkv, Nk, D), dtype=np.int8)
    q = normal((B, Hq, Nq, D), 3, torch.float16)
    vals = _f8_values(vc) * _per_key(vs, Nk)
    pos0, wlo = 150, 20
    got = oracle.attn_kvq(q, kc, ks, vc, vs, scale=0.3, causal=True, window_lo=wlo, pos0=pos0)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        for i in range(Nq):
            want = vals[0, g, wlo:pos0 + i + 1].mean(axis=0)
            np.testing.assert_allclose(got[0, h, i], want, rtol=1e-12, atol=1e-15)


def test_kvq_quantised_q_on_the_grid_is_exact():
    # Q entries on the INT8 grid of its own block (integer codes times 2^-5,
    # with a 127 in every head's block): scale 2^-5 and inverse 2^5 are exact,
    # so the quantised Q reproduces Q and both variants agree bit for bit
    B, Hq, Hkv, Nq, Nk, D = 1, 4, 2, 3, 130, 128
    rng = np.random.default_rng(4)
    kc, ks, vc, vs = _random_cache(rng, B, Hkv, Nk, D)
    qi = rng.integers(-126, 127, size=(B, Hq, Nq, D)).astype(np.float32)
    qi[:, :, 0, 0] = 127.0
    q = torch.from_numpy(np.ldexp(qi, -5).astype(np.float32))
    a = oracle.attn_kvq(q, kc, ks, vc, vs, scale=0.09, quant_q=False)
    b = oracle.attn_kvq(q, kc, ks, vc, vs, scale=0.09, quant_q=True)
    assert np.array_equal(a, b)


def test_kvq_quantised_q_uses_per_head_blocks():
    # off the grid, quant_q uses the dequantised per-(head, 64-row block) codes:
    # the same as passing those values in as Q (70 rows: two blocks per head)
    B, Hq, Hkv, Nq, Nk, D = 1, 2, 1, 70, 100, 64
    rng = np.random.default_rng(8)
    kc, ks, vc, vs = _random_cache(rng, B, Hkv, Nk, D)
    q = normal((B, Hq, Nq, D), 21, torch.bfloat16)
    qc, qs = oracle.quant_int8(q)
    qd = torch.from_numpy((qc.astype(np.float64) *
                           np.repeat(qs.astype(np.float64), 64, axis=2)[:, :, :Nq, None])
                          .astype(np.float32))
    a = oracle.attn_kvq(q, kc, ks, vc, vs, scale=0.125, quant_q=True)
    b = oracle.attn_kvq(qd, kc, ks, vc, vs, scale=0.125, quant_q=False)
    # (Q's dequantised values are rounded to fp32 for the second call)
    np.testing.assert_allclose(a, b, rtol=1e-5, atol=1e-5)
    c = oracle.attn_kvq(q, kc, ks, vc, vs, scale=0.125, quant_q=False)
    assert np.abs(a - c).max() > 1e-3   # the quantisation is really applied


# ---- OCP MX FP8 blocks (the MX variant) ---------------------------------------

def _mx_deq(codes, scales, axis, N):
    vals = _f8_values(codes)
    s = np.ldexp(1.0, scales.astype(np.int64) - 127)
    if axis == 0:
        return vals * np.repeat(s, 32, axis=-1)
    return vals * np.repeat(s, 32, axis=-2)[..., :N, :]


def test_mx_named_blocks():
    x = torch.zeros(1, 4, 64)
    x[0, 0, :32] = 1.0                      # amax 1: e = -8, 1 -> 256 (0x78)
    x[0, 0, 32:] = 3.0                      # amax 3: e = -7, 3 -> 384 (0x7C)
    x[0, 1, :32] = 1.0
    x[0, 1, 0] = 3.875                      # e = -7; 3.875 -> 496 saturates to 448 (0x7E); 1 -> 128 (0x70)
    x[0, 1, 1] = 2.0 ** -20                 # 2^-12 after scaling: below half the smallest subnormal -> 0
    x[0, 1, 2] = -0.5                       # -64 -> 0xE8
    # row 2, first block stays zero: scale byte 0, zero codes
    x[0, 2, 32:] = 2.0 ** -130              # below any scale: e clamps to -127
    c, s = oracle.quant_mx(x, axis=0)
    assert c[0, 0, 0] == 0x78 and s[0, 0, 0] == 119
    assert c[0, 0, 40] == 0x7C and s[0, 0, 1] == 120
    assert c[0, 1, 0] == 0x7E and c[0, 1, 5] == 0x70 and s[0, 1, 0] == 120
    assert c[0, 1, 1] == 0x00 and c[0, 1, 2] == 0xE8
    assert s[0, 2, 0] == 0 and np.all(c[0, 2, :32] == 0)
    assert s[0, 2, 1] == 0   # clamped exponent -127


def test_mx_power_of_two_scaling_moves_only_the_scale():
    x = normal((2, 40, 64), 31, torch.float32)
    c0, s0 = oracle.quant_mx(x, axis=0)
    for j in (-5, 3, 11):
        c1, s1 = oracle.quant_mx(x * 2.0 ** j, axis=0)
        assert np.array_equal(c0, c1)
        assert np.array_equal(s1.astype(int) - s0.astype(int), np.full(s0.shape, j))


def test_mx_axes_agree_under_transpose():
    x = normal((3, 64, 96), 32, torch.bfloat16)
    c1, s1 = oracle.quant_mx(x, axis=1)                         # blocks along N
    c0, s0 = oracle.quant_mx(x.transpose(1, 2).contiguous(), axis=0)   # the same blocks along D
    assert np.array_equal(c1, c0.transpose(0, 2, 1))
    assert np.array_equal(s1, s0.transpose(0, 2, 1))


def test_mx_partial_last_block_along_n():
    x = torch.full((1, 70, 32), 0.25, dtype=torch.float16)
    x[0, 64:, :] = 5.0                       # the last block (tokens 64..69) alone has amax 5
    x[0, 10, 3] = -1.0
    c, s = oracle.quant_mx(x, axis=1)
    assert s.shape == (1, 3, 32)
    assert s[0, 0, 3] == 127 - 8             # channel 3 of block 0: amax 1, e = -8
    assert np.all(np.delete(s[0, 0], 3) == 127 - 10)   # amax 0.25: e = -10
    assert np.all(s[0, 1] == 127 - 10)
    assert np.all(s[0, 2] == 127 - 6)        # tokens 64..69 only: amax 5, e = -6


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_mx_elements_match_torch_cast_and_error_bound(dtype):
    x = normal((2, 50, 128), 33, dtype)
    for axis in (0, 1):
        c, s = oracle.quant_mx(x, axis=axis)
        xf = x.double().numpy()
        if axis == 0:
            e = np.repeat(s.astype(np.int64) - 127, 32, axis=-1)
        else:
            e = np.repeat(s.astype(np.int64) - 127, 32, axis=-2)[..., :50, :]
        y = np.clip(np.ldexp(xf, -e), -448, 448).astype(np.float32)
        want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(c, want)
        deq = _mx_deq(c, s, axis, 50)
        a = np.abs(xf)
        normal_range = (np.ldexp(a, -e) >= 2.0 ** -6) & (np.ldexp(a, -e) <= 448)
        assert np.all(np.abs(deq - xf)[normal_range] <= 2.0 ** -4 * a[normal_range])
        assert np.all(np.abs(deq - xf)[~normal_range & (np.ldexp(a, -e) < 1)]
                      <= np.ldexp(2.0 ** -10, e)[~normal_range & (np.ldexp(a, -e) < 1)])


def _mx_grid(rng, shape):
    """Values exactly on the MX grid along N: E4M3 values times 2^e per block
    of 32 tokens of a channel, each block holding one +-256 * 2^e element so
    that its scale is exactly 2^e."""
    mags = np.array([oracle.e4m3_decode(c) for c in range(0x7F)])
    vals = rng.choice(mags[mags <= 240], size=shape) * rng.choice([-1.0, 1.0], size=shape)
    *lead, N, D = shape
    e = rng.integers(-12, -6, size=tuple(lead) + ((N + 31) // 32, D))
    vals[..., ::32, :] = 256.0 * rng.choice([-1.0, 1.0], size=vals[..., ::32, :].shape)
    return vals * np.ldexp(1.0, np.repeat(e, 32, axis=-2)[..., :N, :])


def _int8_grid(rng, shape):
    """Integer codes times 2^-5 with a 127 in every 64-token block: the INT8
    rule reproduces them exactly (scale 2^-5, inverse 2^5)."""
    x = rng.integers(-126, 127, size=shape).astype(np.float64)
    x[..., ::64, 0] = 127.0
    return np.ldexp(x, -5)


@pytest.mark.parametrize("causal,window_lo,pos0", [(False, 0, 0), (True, 0, 40), (True, 17, 10)])
def test_mx_attention_on_grid_inputs_is_exact_attention(causal, window_lo, pos0):
    rng = np.random.default_rng(12)
    B, Hq, Hkv, Nq, Nk, D = 1, 4, 2, 24, 70, 64
    q = torch.from_numpy(_int8_grid(rng, (B, Hq, Nq, D)).astype(np.float32))
    k = torch.from_numpy(_int8_grid(rng, (B, Hkv, Nk, D)).astype(np.float32))
    v = torch.from_numpy(_mx_grid(rng, (B, Hkv, Nk, D)).astype(np.float32))
    c, s_ = oracle.quant_mx(v, axis=1)
    assert np.array_equal(_mx_deq(c, s_, 1, Nk), v.double().numpy())
    a = oracle.attn_mx(q, k, v, scale=0.1, causal=causal, window_lo=window_lo, pos0=pos0)
    b = oracle.attn(q, k, v, scale=0.1, causal=causal, window_lo=window_lo, pos0=pos0)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_mx_attention_quantises_all_three_inputs():
    # off the grid each of Q, K (INT8) and V (MX) changes the result; feeding
    # the dequantised values back in changes nothing (the grids are fixed points)
    B, Hq, Hkv, Nq, Nk, D = 1, 2, 2, 16, 96, 64
    q, k, v = (normal(s_, sd, torch.float32) for s_, sd in
               (((B, Hq, Nq, D), 41), ((B, Hkv, Nk, D), 42), ((B, Hkv, Nk, D), 43)))
    base = oracle.attn_mx(q, k, v, scale=0.125)
    exact = oracle.attn(q, k, v, scale=0.125)
    rel = np.linalg.norm(base - exact) / np.linalg.norm(exact)
    assert 1e-3 < rel < 6e-2
    t = [q, k, v]
    for which in (0, 1):
        c, s_ = oracle.quant_int8(t[which])
        n = t[which].shape[2]
        t[which] = torch.from_numpy((c.astype(np.float64) *
                                     np.repeat(s_.astype(np.float64), 64, axis=-1)[..., :n, None])
                                    .astype(np.float32))
    c, s_ = oracle.quant_mx(t[2], axis=1)
    t[2] = torch.from_numpy(_mx_deq(c, s_, 1, Nk).astype(np.float32))
    np.testing.assert_allclose(oracle.attn_mx(*t, scale=0.125), base, rtol=1e-5, atol=1e-6)
    # and the same values as plain inputs give the same attention
    np.testing.assert_allclose(oracle.attn(*t, scale=0.125), base, rtol=1e-5, atol=1e-6)
