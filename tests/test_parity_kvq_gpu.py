"""GPU parity of the decode over a quantised KV cache (INT8 K codes, E4M3 V
codes, fp32 scales per 64-key block), called through the C ABI, against the
fp64 oracle on the same seeded caches.

Two references: the oracle with Q through its own per-block INT8 codes (the
kernel's recipe up to the E4M3 rounding of the softmax weights), and exact
attention over the dequantised cache with Q as given. The bound for the first
follows from the weight rounding: E4M3 keeps 3 mantissa bits, so each weight
is off by at most 2^-4 relative and, over many keys, by about 2^-4/sqrt(3) in
RMS; KVQ_REL = 4e-2 (in the shared helpers) leaves a margin over that. The
second adds the INT8 rounding of Q and is held to the quantised mode's 6e-2.
"""
import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_amd as sdpa
from scaled_dot_product_amd.inputs import WORKLOADS, Workload, make_kv_codes, make_qkv, normal

from _parity import QUANT_REL, check_kvq, metrics

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sdpa.load_library()


def _run(w, q, cache, **kw):
    dev = torch.device("cuda:0")
    kc, ks, vc, vs = (t.to(dev) for t in cache)
    out = sdpa.decode_kvq(q.to(dev), kc, ks, vc, vs, causal=w.causal, window_lo=w.window_lo,
                          pos0=w.pos0, scale=w.scale, **kw)
    torch.cuda.synchronize()
    return out


_check = check_kvq


def test_gqa_decode_kvq_workload():
    # the decode configuration the benchmark times, every row compared
    _check(WORKLOADS["gqa_decode_kvq_f16_4096"])


KVQ = []
for rows_, G in [(1, 1), (4, 2), (8, 4), (1, 16), (2, 16)]:
    for pos0, Nk, wlo in [(4092, 4096, 0), (600, 640, 17), (2047, 2051, 64), (50, 70, 0),
                          (8192, 8260, 0), (1000, 1040, 1100), (5, 1, 0)]:
        KVQ.append((rows_, G, pos0, Nk, wlo))


@pytest.mark.parametrize("case", KVQ, ids=[str(c) for c in KVQ])
def test_kvq_decode_edges(case):
    nq, G, pos0, Nk, wlo = case
    Hkv = 2
    w = Workload("kvq", 1, Hkv * G, Hkv, nq, Nk, 128, torch.float16, causal=True,
                 window_lo=wlo, pos0=pos0, mode=2)
    _check(w)


@pytest.mark.parametrize("D,dtype,causal", [(64, torch.bfloat16, True), (64, torch.float16, False),
                                            (128, torch.bfloat16, False)])
def test_kvq_head_dims_and_dtypes(D, dtype, causal):
    w = Workload("kvq_dims", 2, 8, 2, 3, 3000, D, dtype, causal=causal, pos0=2997, mode=2)
    _check(w)


def test_kvq_long_cache_many_tiles_per_wave():
    # 65 536 keys: 1024 tiles over 32 splits of 4 waves, eight tiles per wave,
    # V block scales changing from tile to tile
    w = Workload("kvq_long", 1, 8, 1, 1, 65536, 128, torch.bfloat16, mode=2)
    _check(w)


def test_kvq_zero_keys_closed_form():
    # K codes 0: every weight is exp(0) = 1 and, with one V scale per head,
    # is passed to the FP8 product as 448 * 2^-margin, which rounds to 448 in
    # E4M3 (the denominator keeps the unrounded value): the output is the plain
    # mean of the visible values times 2^(2^-12), exactly.
    w = Workload("kvq_zero_k", 1, 8, 2, 2, 1500, 128, torch.float16, causal=True,
                 window_lo=30, pos0=1400, mode=2)
    kc, ks, vc, vs = make_kv_codes(w)
    kc = torch.zeros_like(kc)
    vs = torch.empty_like(vs)
    vs[0, 0] = 0.01
    vs[0, 1] = 0.25
    q = normal(w.q_shape, 41, w.dtype)
    out = _run(w, q, (kc, ks, vc, vs)).double().cpu().numpy()
    vals = vc.view(torch.float8_e4m3fn).double().numpy() * vs.double().numpy()[0, :, :1, None]
    G = w.Hq // w.Hkv
    f = 2.0 ** (2.0 ** -12)
    for h in range(w.Hq):
        for i in range(w.Nq):
            want = vals[0, h // G, w.window_lo:w.pos0 + i + 1].mean(axis=0) * f
            np.testing.assert_allclose(out[0, h, i], want, rtol=2e-3, atol=2e-3 * np.abs(want).max())


def test_kvq_from_the_library_quantisers_matches_exact_attention():
    # the product pipeline: a 16-bit cache through attn_quantize_qk (K half) and
    # attn_quantize_v, then the quantised decode, against exact fp64 attention on
    # the original 16-bit inputs
    w = WORKLOADS["gqa_decode_kvq_f16_4096"]
    q, k, v = make_qkv(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    _, _, kc, ks = sdpa.quantize_qk(qd, kd)
    vc, vs = sdpa.quantize_v(vd)
    out = sdpa.decode_kvq(qd, kc, ks, vc, vs, causal=True, pos0=w.pos0, scale=w.scale)
    torch.cuda.synchronize()
    ref = oracle.attn(q, k, v, scale=w.scale, causal=True, pos0=w.pos0)
    rel, _ = metrics(out.double().cpu().numpy(), ref)
    print(f"    rel(vs exact attention on the 16-bit inputs)={rel:.3e}", flush=True)
    assert rel <= QUANT_REL, rel


def test_kvq_garbage_workspace_and_reuse():
    # arrival counters live in the workspace: any prior content must work, and
    # a workspace reused by the next call must give the same bits
    w = WORKLOADS["gqa_decode_kvq_f16_4096"]
    dev = torch.device("cuda:0")
    q = normal(w.q_shape, 41, w.dtype).to(dev)
    kc, ks, vc, vs = (t.to(dev) for t in make_kv_codes(w))
    n = sdpa.decode_kvq_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, causal=True,
                                        pos0=w.pos0, dtype=w.dtype)
    ref = None
    for fill in (0x00, 0xFF, 0xA5):
        ws = torch.full((n,), fill, dtype=torch.uint8, device=dev)
        for _ in range(2):
            out = sdpa.decode_kvq(q, kc, ks, vc, vs, causal=True, pos0=w.pos0, scale=w.scale,
                                  workspace=ws)
            torch.cuda.synchronize()
            if ref is None:
                ref = out.clone()
            assert torch.equal(out, ref), fill


def test_kvq_graph_replays_match_eager():
    w = WORKLOADS["gqa_decode_kvq_f16_4096"]
    dev = torch.device("cuda:0")
    q = normal(w.q_shape, 41, w.dtype).to(dev)
    kc, ks, vc, vs = (t.to(dev) for t in make_kv_codes(w))
    n = sdpa.decode_kvq_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, causal=True,
                                        pos0=w.pos0, dtype=w.dtype)
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    call = lambda **kw: sdpa.decode_kvq(q, kc, ks, vc, vs, causal=True, pos0=w.pos0,
                                        scale=w.scale, workspace=ws, **kw)
    eager = call()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out=out)
    for r in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), r
        e2 = call()
        torch.cuda.synchronize()
        assert torch.equal(e2, eager)
