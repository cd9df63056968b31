"""GPU checks of the split-KV decode beyond parity with the oracle: it must
agree with the prefill kernel on the same rows (cross-kernel), its result must
not depend on how the keys are split across workgroups, every element type and
head dimension it is built for must take it, and shapes it cannot take must
land on the prefill. The partial-buffer comparison across variants follows the
"measured results" of "round 21 track b — qsa2"."""
import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_amd as sdpa
from scaled_dot_product_amd.inputs import WORKLOADS, Workload, make_qkv

from _parity import EXACT_ABS, EXACT_REL, announce, masked_rows, metrics

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sdpa.load_library()


def _oracle_check(out, q, k, v, **kw):
    ref = oracle.attn(q, k, v, **kw)
    rel, mabs = metrics(out.double().cpu().numpy(), ref)
    print(f"    rel={rel:.3e} max_abs={mabs:.3e}", flush=True)
    assert rel <= EXACT_REL and mabs <= EXACT_ABS, (rel, mabs)


@pytest.mark.parametrize("window_lo", [0, 1000])
def test_decode_rows_equal_last_rows_of_causal_prefill(window_lo):
    # decode rows 4092..4095 (pos0 4092) against rows 4092..4095 of a pos0 = 0
    # causal prefill over the same 4096 keys
    w = WORKLOADS["gqa_decode_f16_4096"]
    announce(f"cross-kernel decode vs prefill, window_lo={window_lo}")
    full = Workload("full", 1, w.Hq, w.Hkv, w.Nk, w.Nk, w.D, w.dtype, causal=True)
    qf, k, v = make_qkv(full)
    qf, k, v = qf.to(DEV), k.to(DEV), v.to(DEV)
    pre = sdpa.plan(1, w.Hq, w.Hkv, w.Nk, w.Nk, w.D, causal=True, window_lo=window_lo,
                    dtype=w.dtype)
    assert pre.kernel == sdpa.KERNEL_PREFILL
    dec = sdpa.plan(1, w.Hq, w.Hkv, 4, w.Nk, w.D, causal=True, window_lo=window_lo, pos0=4092,
                    dtype=w.dtype)
    assert dec.kernel == sdpa.KERNEL_DECODE
    o_pre = sdpa.fwd(qf, k, v, causal=True, window_lo=window_lo, scale=w.scale)
    qd = qf[:, :, 4092:].contiguous()
    o_dec = sdpa.fwd(qd, k, v, causal=True, window_lo=window_lo, pos0=4092, scale=w.scale)
    torch.cuda.synchronize()
    a = o_pre[:, :, 4092:].double().cpu().numpy()
    b = o_dec.double().cpu().numpy()
    rel, mabs = metrics(b, a)
    print(f"    decode vs prefill rows: rel={rel:.3e} max_abs={mabs:.3e}", flush=True)
    # both round the same fp32 results to f16 once; they differ in summation order
    assert rel <= 2e-3 and mabs <= 2.0 ** -9, (rel, mabs)
    _oracle_check(o_dec, qd.cpu(), k.cpu(), v.cpu(), scale=w.scale, causal=True,
                  window_lo=window_lo, pos0=4092)


@pytest.mark.parametrize("window_lo", [0, 1000])
def test_decode_split_count_invariance(window_lo):
    w = WORKLOADS["gqa_decode_f16_4096"].variant(window_lo=window_lo)
    q, k, v = make_qkv(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    outs = {}
    for s in (0, 1, 2, 8, 32):
        announce(f"decode splits={s} window_lo={window_lo}")
        outs[s] = sdpa.fwd_decode(qd, kd, vd, causal=True, window_lo=window_lo, pos0=w.pos0,
                                  scale=w.scale, splits=s)
    ref_lib = sdpa.fwd(qd, kd, vd, causal=True, window_lo=window_lo, pos0=w.pos0, scale=w.scale)
    torch.cuda.synchronize()
    # splits = 0 is the library's own plan: what attn_fwd runs, bit for bit
    assert torch.equal(outs[0], ref_lib)
    base = outs[1].double().cpu().numpy()
    for s, o in outs.items():
        got = o.double().cpu().numpy()
        rel, mabs = metrics(got, base)
        print(f"    splits {s} vs 1: rel={rel:.3e} max_abs={mabs:.3e}", flush=True)
        # fp32 partials merged in another order, rounded once to f16
        assert mabs <= 2.0 ** -10, (s, mabs)
    _oracle_check(outs[32], q, k, v, scale=w.scale, causal=True, window_lo=window_lo,
                  pos0=w.pos0)


DTYPE_CASES = [
    # (Hq, Hkv, Nq, Nk, D, dtype, pos0)
    (16, 8, 4, 4096, 64, torch.float16, 4092),
    (16, 8, 4, 4096, 128, torch.bfloat16, 4092),
    (8, 2, 8, 2000, 64, torch.bfloat16, 1992),
    (16, 8, 4, 4096, 128, torch.float32, 4092),
    (4, 4, 1, 1500, 64, torch.float32, 1499),
]


@pytest.mark.parametrize("case", DTYPE_CASES, ids=[str(i) for i in range(len(DTYPE_CASES))])
def test_decode_every_dtype_and_head_dim(case):
    Hq, Hkv, Nq, Nk, D, dt, pos0 = case
    w = Workload("dec_dt", 1, Hq, Hkv, Nq, Nk, D, dt, causal=True, pos0=pos0)
    announce(f"decode dtype case {case}")
    p = sdpa.plan(1, Hq, Hkv, Nq, Nk, D, causal=True, pos0=pos0, dtype=dt)
    assert p.kernel == sdpa.KERNEL_DECODE
    q, k, v = make_qkv(w)
    out = sdpa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, pos0=pos0, scale=w.scale)
    torch.cuda.synchronize()
    assert out.dtype == dt
    _oracle_check(out, q, k, v, scale=w.scale, causal=True, pos0=pos0)


@pytest.mark.parametrize("case", [
    # (Nq, Nk, causal, window_lo, pos0, splits): short ranges, a ragged tail,
    # more splits than tiles, and rows that see no key at all
    (4, 100, True, 0, 96, 4),
    (1, 65, False, 0, 0, 64),
    (3, 700, True, 650, 600, 8),
    (2, 300, True, 299, 100, 2),
])
def test_forced_decode_short_ranges(case):
    Nq, Nk, causal, wlo, pos0, splits = case
    w = Workload("dec_short", 1, 8, 2, Nq, Nk, 128, torch.float16, causal=causal,
                 window_lo=wlo, pos0=pos0)
    announce(f"forced decode {case}")
    q, k, v = make_qkv(w)
    out = sdpa.fwd_decode(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window_lo=wlo,
                          pos0=pos0, scale=w.scale, splits=splits)
    torch.cuda.synchronize()
    for i in masked_rows(w):
        assert torch.all(out[:, :, i] == 0), i
    _oracle_check(out, q, k, v, scale=w.scale, causal=causal, window_lo=wlo, pos0=pos0)


def test_more_kv_heads_than_the_decode_grid_takes():
    # B * Hkv = 65 537 rows of the decode grid's y axis: attn_fwd takes the
    # prefill (the decode entry point refuses the shape)
    B, Nk, D = 65537, 512, 64
    announce(f"B={B} single-row heads over {Nk} keys")
    p = sdpa.plan(B, 1, 1, 1, Nk, D, causal=True, pos0=Nk - 1, dtype=torch.float16)
    assert p.kernel == sdpa.KERNEL_PREFILL
    g = torch.Generator(device=DEV)
    g.manual_seed(44)
    q = torch.randn((B, 1, 1, D), generator=g, device=DEV).to(torch.float16)
    k = torch.randn((B, 1, Nk, D), generator=g, device=DEV).to(torch.float16)
    v = torch.randn((B, 1, Nk, D), generator=g, device=DEV).to(torch.float16)
    out = sdpa.fwd(q, k, v, causal=True, pos0=Nk - 1, scale=0.125)
    torch.cuda.synchronize()
    with pytest.raises(sdpa.AttnError):
        sdpa.fwd_decode(q, k, v, causal=True, pos0=Nk - 1, scale=0.125)
    for b in (0, 1, 40000, B - 1):
        sl = slice(b, b + 1)
        _oracle_check(out[sl], q[sl].cpu(), k[sl].cpu(), v[sl].cpu(), scale=0.125, causal=True,
                      pos0=Nk - 1)
    del q, k, v, out
    torch.cuda.empty_cache()
