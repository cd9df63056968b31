"""GPU parity of the diagonal-tiled mixed MX mode (MXFP8 on each row block's
diagonal key tiles, MXFP4 elsewhere), called through the C ABI, against the
fp64 oracle.

The FP4 quantiser (attn_quantize_mx4) must match the oracle's codes and scale
bytes bit for bit, midpoints and saturation included (this also pins the
rounding of the conversion instruction the kernel uses for its weights). The
attention is compared with the oracle's emulation of the mode, which rounds
every weight as the mode defines: what remains is fp32 arithmetic and two
bf16/f16 roundings (2^-9 relative each: the first pass's partial rows and the
output), so MXD_REL = 1e-2 leaves a margin of about four, for the whole output
and for every single row (a weight whose
exact value sat within an fp32 rounding of an E2M1 midpoint could round the
other way and move its row by up to a third of that weight; the kernel forms
each exponent exactly up to one fp32 rounding so that this stays out of
reach). Against exact attention the mode is far less precise (FP4 weights and
values); that error is reported and bounded loosely.
"""
import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_amd as sdpa
from scaled_dot_product_amd.inputs import WORKLOADS, Workload, make_qkv, normal, sample_rows

from _parity import announce, gpu_fwd, masked_rows, metrics

pytestmark = pytest.mark.gpu

MXD_REL, MXD_ROW, MXD_EXACT = 1e-2, 1e-2, 0.3
BF, F16 = torch.bfloat16, torch.float16


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sdpa.load_library()


def _pack(codes):
    """Oracle codes (one nibble per element) to the library's bytes."""
    c = codes.astype(np.uint8)
    return c[..., 0::2] | (c[..., 1::2] << 4)


@pytest.mark.parametrize("dtype", [BF, F16])
@pytest.mark.parametrize("shape", [(1, 2, 64, 64), (2, 3, 130, 128), (1, 1, 333, 64), (1, 2, 31, 128)])
def test_mx4_quantiser_bit_exact(dtype, shape):
    announce(f"mx4 quantiser {shape} {dtype}")
    x = normal(shape, 61, dtype)
    x[..., 5, :] *= 1000.0
    x[..., 7, 3:40] = 0.0
    # every E2M1 midpoint and the saturation band, in a block of scale 2^0
    # (amax 7: floor(log2 7) - 2 = 0) along both axes
    mids = torch.tensor([7.0, 6.5, 5.0, 3.5, 2.5, 1.75, 1.25, 0.75, 0.25, -0.25, -0.75, -1.25,
                         -1.75, -2.5, -3.5, -5.0, 6.0, -6.0, 4.0, 0.5])
    x[0, 0, 9, :20] = mids.to(dtype)
    x[0, 0, 10:30, 1] = mids.to(dtype)
    for axis in (0, 1):
        c, s = sdpa.quantize_mx4(x.cuda(), axis=axis)
        torch.cuda.synchronize()
        rc, rs = oracle.quant_mx4(x, axis=axis)
        assert np.array_equal(c.cpu().numpy(), _pack(rc)), axis
        assert np.array_equal(s.cpu().numpy(), rs), axis


def _check(w, rows=None, inputs=None):
    announce(f"mxd {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} D={w.D} {w.dtype} "
             f"causal={w.causal} window_lo={w.window_lo} pos0={w.pos0} window_w={w.window_w}")
    q, k, v = inputs if inputs is not None else make_qkv(w)
    out = gpu_fwd(w, q, k, v).double().cpu()
    assert torch.isfinite(out).all()
    kw = dict(scale=w.scale, causal=w.causal, window_lo=w.window_lo, pos0=w.pos0,
              window_w=w.window_w)
    if rows is None:
        got = out.numpy().reshape(-1, w.D)
        ref = oracle.attn_mxd(q, k, v, **kw).reshape(-1, w.D)
        ex = oracle.attn(q, k, v, **kw).reshape(-1, w.D)
    else:
        got = out.reshape(-1, w.D)[torch.from_numpy(rows)].numpy()
        ref = oracle.attn_mxd(q, k, v, rows=rows, **kw)
        ex = oracle.attn(q, k, v, rows=rows, **kw)
    rel, _ = metrics(got, ref)
    nr = np.linalg.norm(ref, axis=1)
    row = np.where(nr > 0, np.linalg.norm(got - ref, axis=1) / np.where(nr > 0, nr, 1.0), 0.0)
    rel_ex, _ = metrics(got, ex)
    print(f"    rel(vs emulation)={rel:.3e} worst row={row.max():.3e} rows above 1e-2: "
          f"{int((row > 1e-2).sum())} of {row.size} rel(vs exact)={rel_ex:.3e}", flush=True)
    assert rel <= MXD_REL, rel
    assert row.max() <= MXD_ROW, row.max()
    assert rel_ex <= MXD_EXACT, rel_ex
    for i in masked_rows(w):
        assert torch.all(out[:, :, i] == 0), i
    return out


SMALL = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, causal, window_lo, pos0, window_w
    (1, 2, 2, 256, 256, 128, BF, False, 0, 0, 0),
    (1, 4, 2, 300, 333, 64, F16, False, 0, 0, 0),
    (2, 2, 1, 200, 260, 128, BF, True, 0, 60, 0),
    (1, 2, 2, 130, 500, 128, F16, True, 100, 370, 0),
    (1, 2, 2, 64, 100, 64, BF, True, 120, 0, 0),      # every row masked: zeros
    (1, 2, 1, 97, 700, 128, BF, False, 0, 37, 0),     # row blocks straddle two key tiles
    (1, 1, 1, 5, 64, 64, BF, True, 0, 59, 0),         # every visible tile diagonal
    (1, 2, 2, 40, 2000, 128, F16, False, 0, 1900, 0), # diagonal tiles at the far end
    (1, 2, 2, 600, 600, 128, BF, True, 0, 0, 200),    # per-row window
]


@pytest.mark.parametrize("case", SMALL, ids=[str(i) for i in range(len(SMALL))])
def test_mxd_mode_small(case):
    B, Hq, Hkv, Nq, Nk, D, dt, causal, wlo, pos0, ww = case
    _check(Workload("mxd", B, Hq, Hkv, Nq, Nk, D, dt, causal=causal, window_lo=wlo, pos0=pos0,
                    mode=sdpa.MODE_MXD, window_w=ww))


def test_mxd_mode_is_deterministic():
    w = Workload("mxd_det", 1, 2, 1, 300, 700, 128, BF, causal=True, pos0=400, mode=sdpa.MODE_MXD)
    q, k, v = make_qkv(w)
    a = gpu_fwd(w, q, k, v).cpu()
    b = gpu_fwd(w, q, k, v).cpu()
    assert torch.equal(a, b)


def test_mxd_mode_zero_q_closed_form():
    # Q = 0: every score is 0, so every weight of a block is 1 (2^2 in E2M1 off
    # the diagonal, 2^7 in E4M3 on it, both exact): each row is the plain mean
    # of V, dequantised from MXFP8 on the row block's diagonal tiles and from
    # MXFP4 elsewhere
    w = Workload("mxd_qzero", 1, 2, 2, 100, 300, 128, BF, pos0=50, mode=sdpa.MODE_MXD)
    _, k, v = make_qkv(w)
    q = torch.zeros(w.q_shape, dtype=BF)
    out = gpu_fwd(w, q, k, v).double().cpu().numpy()
    c8, s8 = oracle.quant_mx(v, axis=1)
    v8 = np.array([oracle.e4m3_decode(x) for x in range(256)])[c8] * np.ldexp(
        1.0, np.repeat(s8.astype(np.int64) - 127, 32, axis=2)[:, :, :300, :])
    c4, s4 = oracle.quant_mx4(v, axis=1)
    v4 = np.array([oracle.e2m1_decode(x) for x in range(16)])[c4] * np.ldexp(
        1.0, np.repeat(s4.astype(np.int64) - 127, 32, axis=2)[:, :, :300, :])
    for i in range(w.Nq):
        r0 = w.pos0 + 32 * (i // 32)
        diag = np.array([64 * (j // 64) <= r0 + 31 and 64 * (j // 64) + 63 >= r0
                         for j in range(300)])
        want = np.where(diag[None, :, None], v8[0], v4[0]).mean(axis=1)
        np.testing.assert_allclose(out[0, :, i], want, rtol=8e-3, atol=1e-3)


def test_mxd_mode_video_dit_sampled():
    # the video shape, 1 x 40 x 32760 x 128 bf16: 64 sampled rows of heads 0
    # and 39 against the emulation (blocks never cross a head, so the oracle
    # runs on each head's slice) and against exact attention
    w = WORKLOADS["video_dit_bf16_32760"].variant(name="video_dit_mxd_32760", mode=sdpa.MODE_MXD)
    q, k, v = make_qkv(w)
    out = gpu_fwd(w, q, k, v).double().cpu()
    assert torch.isfinite(out).all()
    kw = dict(scale=w.scale, causal=w.causal, window_lo=w.window_lo, pos0=w.pos0)
    rng = np.random.default_rng(7)
    for h in (0, 39):
        announce(f"mxd video head {h}")
        rows = np.unique(np.concatenate([rng.choice(w.Nq, 62, replace=False),
                                         np.array([0, w.Nq - 1])])).astype(np.int64)
        sl = (slice(None), slice(h, h + 1))
        qs, ks, vs = q[sl].contiguous(), k[sl].contiguous(), v[sl].contiguous()
        ref = oracle.attn_mxd(qs, ks, vs, rows=rows, **kw)
        ex = oracle.attn(qs, ks, vs, rows=rows, **kw)
        got = out[0, h].numpy()[rows]
        rel, _ = metrics(got, ref)
        rel_ex, _ = metrics(got, ex)
        print(f"    head {h}: rel(vs emulation)={rel:.3e} rel(vs exact)={rel_ex:.3e}", flush=True)
        assert rel <= MXD_REL, rel
        assert rel_ex <= MXD_EXACT, rel_ex


def test_mxd_mode_with_rope():
    # attn_fwd_rope in the diagonal-tiled mode: Q and K are turned inside the
    # INT8 quantiser. Against exact attention on the rotated inputs (the mode's
    # own error), and against the mode's emulation on the oracle's rotation
    # rounded to fp32: the two rotations differ in their last bits, which may
    # move an INT8 code by one step, so this comparison gets twice the bar
    w = Workload("mxd_rope", 1, 2, 2, 300, 300, 128, BF, causal=True, mode=sdpa.MODE_MXD)
    q, k, v = make_qkv(w)
    plain = dict(style=0, scaling=0, base=10000.0)
    announce(f"mxd rope {plain}")
    dev = torch.device("cuda:0")
    out = sdpa.fwd_rope(q.to(dev), k.to(dev), v.to(dev), sdpa.Rope(**plain), causal=True,
                        scale=w.scale, mode=sdpa.MODE_MXD)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    ex = oracle.attn_rope(q, k, v, scale=w.scale, causal=True, **plain)
    theta, _ = oracle.rope_freqs(w.D, base=10000.0)
    qr = torch.from_numpy(oracle.rope_apply(q, 0, theta)).float()
    kr = torch.from_numpy(oracle.rope_apply(k, 0, theta)).float()
    ref = oracle.attn_mxd(qr, kr, v.float(), scale=w.scale, causal=True)
    rel, _ = metrics(got, ref)
    rel_ex, _ = metrics(got, ex)
    print(f"    rel(vs emulation on rotated inputs)={rel:.3e} rel(vs exact)={rel_ex:.3e}", flush=True)
    assert rel <= 2 * MXD_REL, rel
    assert rel_ex <= MXD_EXACT, rel_ex


def test_mxd_mode_sdxl_1024px_sampled():
    # head dim 64 at scale: 2 x 10 x 4096 x 64 bf16, 64 sampled rows
    w = WORKLOADS["sdxl_1024px_bf16"].variant(name="sdxl_mxd", mode=sdpa.MODE_MXD)
    _check(w, rows=sample_rows(w, 64))
