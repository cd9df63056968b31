"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle
on the same seeded inputs. Full-size workloads check sampled rows (the oracle
computes them one by one); smaller cases check every row."""
import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_amd as sdpa
from scaled_dot_product_amd.inputs import WORKLOADS, Workload, make_qkv, sample_rows

from _parity import announce, check_workload, gpu_fwd, masked_rows, metrics

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sdpa.load_library()


# ---- the five workloads -----------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_tiny_fp32(causal):
    w = WORKLOADS["tiny_fp32_256"].variant(causal=causal)
    check_workload(w)


@pytest.mark.parametrize("window_lo", [0, 1000])
def test_gqa_decode(window_lo):
    w = WORKLOADS["gqa_decode_f16_4096"].variant(window_lo=window_lo)
    check_workload(w)


def test_sdxl_1024px_sampled():
    w = WORKLOADS["sdxl_1024px_bf16"]
    check_workload(w, rows=sample_rows(w, 512))


def test_video_dit_sampled():
    w = WORKLOADS["video_dit_bf16_32760"]
    check_workload(w, rows=sample_rows(w, 256))


def test_video_dit_causal_sampled():
    # causal prefill at video scale (heaviest q-tiles dispatched first)
    w = WORKLOADS["video_dit_bf16_32760"].variant(name="video_dit_causal", causal=True)
    check_workload(w, rows=sample_rows(w, 256))


def test_video_dit_quant_sampled():
    w = WORKLOADS["video_dit_quant_32760"]
    _, _, rel, _ = check_workload(w, rows=sample_rows(w, 256))
    print(f"    quantised-mode error vs fp64: {rel:.4f}")


# ---- edge matrix --------------------------------------------------------------

EDGE = [
    # (B, Hq, Hkv, Nq, Nk, D, dtype, causal, window_lo, pos0)
    (1, 2, 2, 1, 1, 64, torch.bfloat16, False, 0, 0),          # one key
    (1, 2, 1, 37, 200, 128, torch.bfloat16, False, 0, 0),      # ragged second tile
    (2, 4, 2, 130, 130, 64, torch.float16, True, 0, 0),        # causal square, GQA
    (1, 3, 3, 77, 300, 128, torch.bfloat16, True, 0, 223),     # bottom-right causal
    (1, 2, 2, 64, 400, 64, torch.bfloat16, True, 17, 300),     # window inside first tile
    (1, 2, 2, 50, 300, 128, torch.float16, False, 129, 0),     # window, non-causal
    (1, 8, 2, 300, 513, 64, torch.bfloat16, True, 0, 213),     # G=4 prefill
    (1, 2, 2, 20, 90, 64, torch.float32, True, 60, 30),        # rows fully masked
    (1, 1, 1, 260, 1000, 128, torch.bfloat16, True, 200, 740), # several tiles, window
    (2, 2, 2, 129, 129, 128, torch.float32, False, 0, 0),      # fp32, ragged
]


@pytest.mark.parametrize("case", EDGE, ids=[str(i) for i in range(len(EDGE))])
def test_prefill_edges(case):
    B, Hq, Hkv, Nq, Nk, D, dt, causal, wlo, pos0 = case
    w = Workload("edge", B, Hq, Hkv, Nq, Nk, D, dt, causal=causal, window_lo=wlo, pos0=pos0)
    out, ref, _, _ = check_workload(w)
    for i in masked_rows(w):
        assert torch.all(out[:, :, i] == 0), i


# Grids of at least eight rounds of 256-row workgroups (head dim 128) take the
# eight-wave prefill; these shapes reach it with ragged query and key ends.
EIGHT_WAVE = [
    # (B, Hq, Hkv, Nq, Nk, dtype, causal, window_lo, pos0)
    (1, 16, 4, 32760, 1000, torch.bfloat16, True, 100, 0),
    (1, 16, 16, 32760, 777, torch.float16, False, 0, 0),
]


@pytest.mark.parametrize("case", EIGHT_WAVE, ids=[str(i) for i in range(len(EIGHT_WAVE))])
def test_prefill_eight_wave_grid(case):
    B, Hq, Hkv, Nq, Nk, dt, causal, wlo, pos0 = case
    w = Workload("eightwave", B, Hq, Hkv, Nq, Nk, 128, dt, causal=causal, window_lo=wlo,
                 pos0=pos0)
    # sampled rows plus the ends of the first and last query tiles of a few heads
    edge = [h * Nq + i for h in (0, 5, Hq - 1) for i in (0, 1, 99, 100, 255, 256, Nq - 2, Nq - 1)]
    rows = np.unique(np.concatenate([sample_rows(w, 256), np.array(edge, dtype=np.int64)]))
    out, _, _, _ = check_workload(w, rows=rows)
    for i in masked_rows(w):
        assert torch.all(out[:, :, i] == 0), i


DECODE = []
for rows_, G in [(1, 1), (2, 2), (4, 2), (8, 4), (4, 8), (1, 16)]:
    for pos0, Nk, wlo in [(4092, 4096, 0), (4092, 4096, 17), (600, 640, 0), (2047, 2051, 64),
                          (2050, 2070, 1000), (8192, 8260, 0), (1000, 1040, 1100)]:
        DECODE.append((rows_, G, pos0, Nk, wlo))


@pytest.mark.parametrize("case", DECODE, ids=[str(c) for c in DECODE])
def test_decode_edges(case):
    nq, G, pos0, Nk, wlo = case
    Hkv = 2
    w = Workload("decode", 1, Hkv * G, Hkv, nq, Nk, 128, torch.float16, causal=True,
                 window_lo=wlo, pos0=pos0)
    out, ref, _, _ = check_workload(w)
    for i in masked_rows(w):
        assert torch.all(out[:, :, i] == 0), i


def test_single_key_output_is_v_bitwise():
    w = Workload("one", 1, 2, 2, 70, 1, 128, torch.bfloat16)
    q, k, v = make_qkv(w)
    out = gpu_fwd(w, q, k, v).cpu()
    assert torch.equal(out, v.expand(1, 2, 70, 128))


def test_causal_row0_is_v0_bitwise():
    w = Workload("row0", 1, 2, 2, 300, 300, 64, torch.bfloat16, causal=True)
    q, k, v = make_qkv(w)
    out = gpu_fwd(w, q, k, v).cpu()
    assert torch.equal(out[:, :, 0], v[:, :, 0])


def test_gqa_head_mapping_closed_form():
    # V of kv head g is the constant g: every output of query head h is h // G exactly
    B, Hq, Hkv, N = 1, 8, 2, 200
    w = Workload("gqa", B, Hq, Hkv, N, N, 64, torch.bfloat16)
    q, k, _ = make_qkv(w)
    v = torch.arange(Hkv, dtype=torch.bfloat16).view(1, Hkv, 1, 1).expand(B, Hkv, N, 64).contiguous()
    out = gpu_fwd(w, q, k, v).float().cpu()
    for h in range(Hq):
        assert torch.all(out[:, h] == h // (Hq // Hkv))


def test_run_to_run_bitwise_determinism():
    for name in ("sdxl_1024px_bf16", "gqa_decode_f16_4096"):
        w = WORKLOADS[name]
        q, k, v = make_qkv(w)
        a = gpu_fwd(w, q, k, v).cpu()
        b = gpu_fwd(w, q, k, v).cpu()
        assert torch.equal(a, b), name


def test_output_guard_bands_untouched():
    w = Workload("guard", 1, 2, 2, 100, 300, 64, torch.bfloat16, causal=True, pos0=200)
    q, k, v = make_qkv(w)
    dev = torch.device("cuda:0")
    n = q.numel()
    buf = torch.full((n + 2048,), 7.0, dtype=torch.bfloat16, device=dev)
    out = buf[1024:1024 + n].view(q.shape)
    sdpa.fwd(q.to(dev), k.to(dev), v.to(dev), causal=True, pos0=200, scale=w.scale, out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[:1024] == 7.0) and torch.all(buf[1024 + n:] == 7.0)


# ---- quantisers: bit-exact against the oracle ---------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("shape", [(1, 2, 1, 130, 64), (2, 4, 2, 64, 128), (1, 3, 3, 333, 128),
                                   (1, 1, 1, 1, 64)])
def test_quantizers_bit_exact(dtype, shape):
    B, Hq, Hkv, N, D = shape
    announce(f"quantisers {shape} {dtype}")
    w = Workload("quant", B, Hq, Hkv, N, N + 17, D, dtype)
    q, k, v = make_qkv(w)
    q = q * 3.0
    q[:, :, :64] = 0 if N > 64 else q[:, :, :64]   # an all-zero block
    q = q.contiguous()
    dev = torch.device("cuda:0")
    qc, qs, kc, ks = sdpa.quantize_qk(q.to(dev), k.to(dev))
    vc, vs = sdpa.quantize_v(v.to(dev))
    torch.cuda.synchronize()
    for got_c, got_s, x, fn in ((qc, qs, q, oracle.quant_int8), (kc, ks, k, oracle.quant_int8),
                                (vc, vs, v, oracle.quant_e4m3)):
        want_c, want_s = fn(x)
        assert np.array_equal(got_c.cpu().numpy(), want_c)
        assert np.array_equal(got_s.cpu().numpy().view(np.uint32), want_s.view(np.uint32))


def test_quant_full_video_codes_bit_exact():
    w = WORKLOADS["video_dit_quant_32760"]
    announce("quantiser codes at 1x40x32760x128")
    q, k, v = make_qkv(w)
    dev = torch.device("cuda:0")
    qc, qs, kc, ks = sdpa.quantize_qk(q.to(dev), k.to(dev))
    vc, vs = sdpa.quantize_v(v.to(dev))
    torch.cuda.synchronize()
    # heads 0 and 39 in full (the oracle quantises them in a few seconds)
    for h in (0, 39):
        wc, ws = oracle.quant_int8(q[:, h:h + 1].contiguous())
        assert np.array_equal(qc[:, h:h + 1].cpu().numpy(), wc)
        assert np.array_equal(qs[:, h:h + 1].cpu().numpy(), ws)
        wc, ws = oracle.quant_e4m3(v[:, h:h + 1].contiguous())
        assert np.array_equal(vc[:, h:h + 1].cpu().numpy(), wc)
        assert np.array_equal(vs[:, h:h + 1].cpu().numpy(), ws)


# ---- quantised mode: smaller shapes, also against the oracle's emulation ------

@pytest.mark.parametrize("case", [
    (1, 2, 2, 256, 256, 64, torch.bfloat16, False, 0, 0),
    (1, 4, 2, 200, 700, 128, torch.float16, True, 0, 500),
    (1, 2, 2, 300, 300, 128, torch.bfloat16, True, 70, 0),
    (2, 2, 1, 130, 1000, 128, torch.bfloat16, False, 0, 0),
])
def test_quant_mode_small(case):
    B, Hq, Hkv, Nq, Nk, D, dt, causal, wlo, pos0 = case
    w = Workload("qsmall", B, Hq, Hkv, Nq, Nk, D, dt, causal=causal, window_lo=wlo, pos0=pos0,
                 mode=1)
    out, ref, rel, _ = check_workload(w)
    q, k, v = make_qkv(w)
    emu = oracle.attn_quant(q, k, v, scale=w.scale, causal=causal, window_lo=wlo, pos0=pos0)
    rel_emu, _ = metrics(out.double().numpy(), emu)
    print(f"    vs quantised emulation: {rel_emu:.4f} (vs exact {rel:.4f})")
    # the GPU rounds P at the running maximum and per key block at a scale
    # that carries V's block scale, the emulation at the final maximum and a
    # static scale: both are quantisations of the same weights, so they agree
    # far better than either agrees with exact attention.
    assert rel_emu <= rel
    for i in masked_rows(w):
        assert torch.all(out[:, :, i] == 0), i


@pytest.mark.parametrize("H, Nk", [(2, 300), (1, 65600)], ids=["short", "1025-blocks"])
def test_quant_mode_zero_q_closed_form(H, Nk):
    # Q = 0: every score is 0 and every weight 1. Key block t's weights are
    # rounded once, to E4M3(448 s_v,t / s_ref) / (448 s_v,t / s_ref) = w_t with
    # s_ref the largest V block scale the query tile sees; numerator and
    # denominator both use the rounded weights, so the output is the w_t-weighted
    # mean of V^ over the keys (plain mean where s_v,t = s_ref). The kernel
    # keeps the per-block factors of the first 1024 blocks in LDS and computes
    # the rest as it goes: 65 600 keys take both paths.
    w = Workload("qzero", 1, H, H, 64, Nk, 128, torch.bfloat16, mode=1)
    _, k, v = make_qkv(w)
    q = torch.zeros(w.q_shape, dtype=torch.bfloat16)
    out = gpu_fwd(w, q, k, v).double().cpu().numpy()
    vc, vs = oracle.quant_e4m3(v)
    dec = np.array([oracle.e4m3_decode(c) for c in range(256)])
    gap = 0.0
    for h in range(H):
        s_v = vs[0, h].astype(np.float64)
        vhat = dec[vc[0, h]] * np.repeat(s_v, 64)[:Nk, None]
        ratio = s_v / s_v.max()
        wt = np.array([oracle.e4m3_decode(oracle.e4m3_encode(np.float32(448.0 * r))) / (448.0 * r)
                       for r in ratio])
        wk = np.repeat(wt, 64)[:Nk, None]
        want = (wk * vhat).sum(axis=0) / wk.sum()
        np.testing.assert_allclose(out[0, h], np.broadcast_to(want, (64, 128)), rtol=0, atol=1e-3)
        gap = max(gap, np.abs(want - vhat.mean(axis=0)).max())
    # the per-block factors are not all 1 here, so this also checks they are applied
    if Nk == 300:
        assert gap > 3e-3


# ---- fused decode: workspace state and graph replay --------------------------

def _decode_case():
    w = WORKLOADS["gqa_decode_f16_4096"]
    q, k, v = make_qkv(w)
    dev = torch.device("cuda:0")
    return w, q.to(dev), k.to(dev), v.to(dev)


def test_decode_garbage_workspace():
    # the arrival counters live in the workspace; any prior content must work
    w, q, k, v = _decode_case()
    n = sdpa.fwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, causal=True,
                                 pos0=w.pos0, dtype=w.dtype)
    ref = None
    for fill in (0x00, 0xFF, 0xA5):
        ws = torch.full((n,), fill, dtype=torch.uint8, device=q.device)
        out = sdpa.fwd(q, k, v, causal=True, pos0=w.pos0, scale=w.scale, workspace=ws)
        torch.cuda.synchronize()
        if ref is None:
            qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
            r = oracle.attn(qc, kc, vc, scale=w.scale, causal=True, pos0=w.pos0)
            rel, _ = metrics(out.double().cpu().numpy(), r)
            assert rel < 1e-2
            ref = out.clone()
        assert torch.equal(out, ref), fill
        # the same workspace again: counters were left reset
        out2 = sdpa.fwd(q, k, v, causal=True, pos0=w.pos0, scale=w.scale, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out2, ref)


def test_decode_graph_replays_match_eager():
    w, q, k, v = _decode_case()
    n = sdpa.fwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, causal=True,
                                 pos0=w.pos0, dtype=w.dtype)
    ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q)
    eager = sdpa.fwd(q, k, v, causal=True, pos0=w.pos0, scale=w.scale, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sdpa.fwd(q, k, v, causal=True, pos0=w.pos0, scale=w.scale, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        sdpa.fwd(q, k, v, causal=True, pos0=w.pos0, scale=w.scale, out=out, workspace=ws)
    for r in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), r
        # eager work on the same workspace between replays
        e2 = sdpa.fwd(q, k, v, causal=True, pos0=w.pos0, scale=w.scale, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(e2, eager)


def test_binding_rejects_host_workspace_and_outputs():
    # a workspace or output in host memory would be written by the kernels
    # through a host address: the binding refuses it before any launch
    w = Workload("bind", 1, 2, 2, 64, 600, 128, torch.float16)
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in make_qkv(w))
    host_ws = torch.empty(1 << 20, dtype=torch.uint8)
    for call in (lambda: sdpa.fwd(q, k, v, workspace=host_ws),
                 lambda: sdpa.fwd_sliding(q, k, v, window=100, workspace=host_ws),
                 lambda: sdpa.fwd_decode(q[:, :, :4].contiguous(), k, v, workspace=host_ws),
                 lambda: sdpa.fwd(q, k, v, out=torch.empty(q.shape, dtype=q.dtype)),
                 lambda: sdpa.fwd(q, k.cpu(), v)):
        with pytest.raises(sdpa.AttnError):
            call()
    kc, ks = sdpa.quantize_qk(q, k)[2:]
    vc, vs = sdpa.quantize_v(v)
    with pytest.raises(sdpa.AttnError):
        sdpa.decode_kvq(q[:, :, :4].contiguous(), kc, ks, vc, vs, workspace=host_ws)
    with pytest.raises(sdpa.AttnError):
        sdpa.decode_kvq(q[:, :, :4].contiguous(), kc, ks.cpu(), vc, vs)
    # and a device workspace still works
    ws = torch.empty(sdpa.fwd_workspace_bytes(1, 2, 2, 64, 600, 128, dtype=torch.float16) + 1,
                     dtype=torch.uint8, device=dev)
    out = sdpa.fwd(q, k, v, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
