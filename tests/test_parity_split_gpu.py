"""The split prefill. A grid of at most 128 query tiles runs each query
tile's key range as 2-4 workgroups; each publishes its normalised partial
(O / l in the output type, m and l in fp32) and the last one of the tile to
arrive merges them with log-sum-exp weights. A grid between half a round and
one round of workgroups runs enough tiles in two halves that the jobs fill
the slots, and a second launch merges the halves. Checked against the
oracle, against the unsplit schedule of the same call (a workspace too small
for the split runs it unsplit), with garbage left in the workspace, and under
graph replay."""
import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_amd as sdpa
from scaled_dot_product_amd.inputs import Workload, make_qkv, sample_rows

from _parity import announce, check_workload, masked_rows, metrics

pytestmark = pytest.mark.gpu

bf16, f16, f32 = torch.bfloat16, torch.float16, torch.float32

SPLIT = [
    # (B, Hq, Hkv, Nq, Nk, D, dtype, causal, window_lo, pos0, parts)
    (1, 8, 8, 1024, 4096, 64, bf16, False, 0, 0, 4),       # 64 tiles
    (1, 8, 2, 700, 1000, 128, f16, True, 0, 300, 4),       # causal GQA: uneven and empty parts
    (1, 4, 4, 333, 555, 64, bf16, True, 100, 200, 4),      # window + causal, ragged tiles
    (1, 2, 2, 256, 260, 64, f32, False, 0, 0, 2),          # fp32 staging, fp32 partials
    (1, 4, 4, 512, 8192, 128, bf16, False, 0, 0, 4),       # head dim 128, long keys
    (2, 2, 2, 2048, 2048, 128, f16, True, 0, 0, 4),        # causal square, 64 tiles
    (1, 85, 85, 128, 1000, 64, bf16, False, 0, 0, 3),      # 85 tiles -> 3 parts
    # the balanced schedule (between half a round and one round of workgroups):
    # slots - tiles tiles in two halves, merged by a second launch
    (2, 10, 10, 4096, 4096, 64, bf16, False, 0, 0, 2),     # SDXL: 640 tiles, 128 in halves
    (1, 20, 5, 2560, 2560, 64, f16, True, 0, 0, 2),        # causal, 400 tiles, 368 in halves
    (1, 300, 3, 128, 1000, 128, bf16, False, 0, 0, 2),     # head dim 128: 300 tiles on 512 slots
    (1, 50, 50, 1000, 700, 64, f32, True, 200, 100, 2),    # fp32, window, ragged q and k tiles
]


def _workload(case):
    B, Hq, Hkv, Nq, Nk, D, dt, causal, wlo, pos0, _ = case
    return Workload("split", B, Hq, Hkv, Nq, Nk, D, dt, causal=causal, window_lo=wlo, pos0=pos0)


def _rows(w):
    n = w.B * w.Hq * w.Nq
    if n <= 4096:
        return None
    edge = [h * w.Nq + i for h in (0, w.Hq - 1) for i in {0, 1, 127, 128, w.Nq - 1} if i < w.Nq]
    return np.unique(np.concatenate([sample_rows(w, 384), np.array(edge, dtype=np.int64)]))


def _unsplit(w, q, k, v):
    """The same call with the least workspace attn_fwd accepts: unsplit."""
    dev = torch.device("cuda:0")
    staging = 3 * 2 * (w.B * w.Hq * w.Nq * w.D) if w.dtype == f32 else 0
    # fp32 inputs need their bf16 copies (three 256-aligned areas)
    n = 0 if staging == 0 else sum((2 * s + 255) // 256 * 256 for s in
                                   (w.B * w.Hq * w.Nq * w.D, w.B * w.Hkv * w.Nk * w.D,
                                    w.B * w.Hkv * w.Nk * w.D))
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    out = sdpa.fwd(q.to(dev), k.to(dev), v.to(dev), causal=w.causal, window_lo=w.window_lo,
                   pos0=w.pos0, scale=w.scale, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu()


@pytest.mark.parametrize("case", SPLIT, ids=[str(i) for i in range(len(SPLIT))])
def test_split_prefill_matches_oracle_and_unsplit(case):
    w = _workload(case)
    p = sdpa.plan(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, causal=w.causal, window_lo=w.window_lo,
                  pos0=w.pos0, dtype=w.dtype)
    assert p.kernel == sdpa.KERNEL_PREFILL and p.splits == case[-1], p.splits
    q, k, v = make_qkv(w)
    rows = _rows(w)
    out, ref, rel, _ = check_workload(w, rows=rows, inputs=(q, k, v))
    for i in masked_rows(w):
        assert torch.all(out[:, :, i] == 0), i
    announce(f"unsplit schedule of the same call")
    un = _unsplit(w, q, k, v).float()
    got_un = un.double().numpy() if rows is None else \
        un.reshape(-1, w.D)[torch.from_numpy(rows)].double().numpy()
    rel_un, _ = metrics(got_un, ref)
    print(f"    unsplit rel={rel_un:.3e}", flush=True)
    assert rel_un <= 1e-2
    # the two schedules differ only in rounding (the partials' output type)
    d, _ = metrics(out.double().numpy(), un.double().numpy())
    assert d <= 8e-3, d
    for i in masked_rows(w):
        assert torch.all(un[:, :, i] == 0), i


def _case_dev(case):
    w = _workload(case)
    q, k, v = make_qkv(w)
    dev = torch.device("cuda:0")
    return w, q.to(dev), k.to(dev), v.to(dev)


def test_split_prefill_garbage_workspace_and_reuse():
    # the arrival counters live in the workspace; any prior content must work,
    # and the merge order is fixed, so every run is bitwise the same
    w, q, k, v = _case_dev(SPLIT[1])
    n = sdpa.fwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, causal=w.causal,
                                 pos0=w.pos0, dtype=w.dtype)
    ref = None
    for fill in (0x00, 0xFF, 0xA5):
        announce(f"split prefill, workspace filled with {fill:#x}")
        ws = torch.full((n,), fill, dtype=torch.uint8, device=q.device)
        for rep in range(2):
            out = sdpa.fwd(q, k, v, causal=w.causal, pos0=w.pos0, scale=w.scale, workspace=ws)
            torch.cuda.synchronize()
            if ref is None:
                r = oracle.attn(q.cpu(), k.cpu(), v.cpu(), scale=w.scale, causal=w.causal,
                                pos0=w.pos0)
                rel, _ = metrics(out.double().cpu().numpy(), r)
                assert rel < 1e-2
                ref = out.clone()
            assert torch.equal(out, ref), (fill, rep)


@pytest.mark.parametrize("which", [0, 7], ids=["fused-merge", "balanced"])
def test_split_prefill_graph_replays_match_eager(which):
    w, q, k, v = _case_dev(SPLIT[which])
    n = sdpa.fwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, dtype=w.dtype)
    ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q)
    eager = sdpa.fwd(q, k, v, scale=w.scale, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sdpa.fwd(q, k, v, scale=w.scale, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    announce("split prefill captured in a graph, 4 replays with eager calls between")
    with torch.cuda.graph(g):
        sdpa.fwd(q, k, v, scale=w.scale, out=out, workspace=ws)
    for r in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), r
        e2 = sdpa.fwd(q, k, v, scale=w.scale, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(e2, eager)
