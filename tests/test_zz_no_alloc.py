"""attn_fwd_noalloc, the entry point for callers that cannot allocate, called
through the C ABI: its results must equal attn_fwd's (same kernels, same
plan; only the workspace differs) bit for bit, call after call on the same
fixed device array, including a second, smaller call, inside a captured graph,
and within the parity bar against the fp64 oracle (for the diagonal-tiled MX
mode, against the oracle's emulation of that mode)."""
import pytest
import torch

import oracle
import scaled_dot_product_amd as sdpa
from scaled_dot_product_amd.inputs import WORKLOADS, Workload, make_qkv

from _parity import EXACT_ABS, EXACT_REL, announce, metrics

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sdpa.load_library()


def _pair(w, **kw):
    q, k, v = (t.to(DEV) for t in make_qkv(w))
    args = dict(causal=w.causal, window_lo=w.window_lo, pos0=w.pos0, scale=w.scale, mode=w.mode)
    args.update(kw)
    a = sdpa.fwd_noalloc(q, k, v, **args)
    b = sdpa.fwd(q, k, v, **args)
    torch.cuda.synchronize()
    return q, k, v, a, b


def _oracle(out, q, k, v, w):
    ref = oracle.attn(q.cpu(), k.cpu(), v.cpu(), scale=w.scale, causal=w.causal,
                      window_lo=w.window_lo, pos0=w.pos0)
    rel, mabs = metrics(out.double().cpu().numpy(), ref)
    print(f"    rel={rel:.3e} max_abs={mabs:.3e}", flush=True)
    assert rel <= EXACT_REL and mabs <= EXACT_ABS


def test_noalloc_decode_two_calls_second_smaller():
    # the decode keeps its partials and arrival counters in the fixed array
    big = WORKLOADS["gqa_decode_f16_4096"]
    small = Workload("dec_small", 1, 8, 4, 2, 1500, 64, torch.float16, causal=True, pos0=1498,
                     window_lo=100)
    for w in (big, small, big):
        announce(f"noalloc {w.name} Nk={w.Nk} D={w.D}")
        p = sdpa.plan(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, causal=w.causal, window_lo=w.window_lo,
                      pos0=w.pos0, dtype=w.dtype)
        assert p.kernel == sdpa.KERNEL_DECODE and 0 < p.workspace_bytes <= sdpa.NOALLOC_SCRATCH_BYTES
        q, k, v, a, b = _pair(w)
        assert torch.equal(a, b)
        _oracle(a, q, k, v, w)


def test_noalloc_fp32_staging_then_bf16_prefill():
    # fp32 inputs are staged as bf16 copies in the array; a bf16 prefill needs none
    for w in (WORKLOADS["tiny_fp32_256"].variant(causal=True),
              Workload("pre_small", 1, 2, 2, 100, 130, 64, torch.bfloat16, causal=True, pos0=30)):
        announce(f"noalloc {w.name}")
        q, k, v, a, b = _pair(w)
        assert torch.equal(a, b)
        _oracle(a, q, k, v, w)


def test_noalloc_diagonal_tiled_mx_two_calls_second_smaller():
    # the diagonal-tiled mode keeps its codes, scales and row partials in the
    # array; two launches per call, the second merging the first's partials
    for w in (Workload("mxd_big", 1, 4, 2, 300, 700, 128, torch.bfloat16, causal=True, pos0=400,
                       mode=sdpa.MODE_MXD),
              Workload("mxd_small", 1, 2, 1, 97, 200, 64, torch.float16, pos0=37,
                       mode=sdpa.MODE_MXD)):
        announce(f"noalloc {w.name}")
        q, k, v, a, b = _pair(w)
        assert torch.equal(a, b)
        ref = oracle.attn_mxd(q.cpu(), k.cpu(), v.cpu(), scale=w.scale, causal=w.causal,
                              pos0=w.pos0)
        rel, _ = metrics(a.double().cpu().numpy(), ref)
        print(f"    rel(vs emulation)={rel:.3e}", flush=True)
        assert rel <= 1e-2, rel


def test_noalloc_too_large_is_refused():
    w = Workload("q_big", 1, 8, 8, 8192, 8192, 128, torch.bfloat16, mode=1)
    assert sdpa.fwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, mode=1) > \
        sdpa.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(w.q_shape, dtype=w.dtype, device=DEV)
    out = torch.full_like(q, 3.0)
    with pytest.raises(sdpa.AttnError, match="status -5"):
        sdpa.fwd_noalloc(q, q, q, mode=1, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)        # nothing was enqueued


def test_noalloc_decode_in_a_captured_graph():
    w = WORKLOADS["gqa_decode_f16_4096"]
    q, k, v = (t.to(DEV) for t in make_qkv(w))
    kw = dict(causal=True, pos0=w.pos0, scale=w.scale)
    eager = sdpa.fwd(q, k, v, **kw)
    out = torch.empty_like(q)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sdpa.fwd_noalloc(q, k, v, out=out, **kw)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sdpa.fwd_noalloc(q, k, v, out=out, **kw)
    for r in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), r
        # eager use of the same array between replays
        e2 = sdpa.fwd_noalloc(q, k, v, **kw)
        torch.cuda.synchronize()
        assert torch.equal(e2, eager), r
    del g
