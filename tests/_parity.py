"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the oracle on the same seeded inputs, and measure the difference."""
import math
import sys

import numpy as np
import torch

import oracle
import scaled_dot_product_amd as sdpa
from scaled_dot_product_amd.inputs import make_kv_codes, make_qkv, normal, sample_rows

# Tolerances stated for the path: exact mode rel-RMS <= 1e-2 and max-abs <= 2e-2,
# quantised mode rel-L2 <= 6e-2, both against the fp64 oracle.
EXACT_REL, EXACT_ABS, QUANT_REL = 1e-2, 2e-2, 6e-2


def announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def metrics(o, r):
    o = np.asarray(o, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    diff = o - r
    den = np.linalg.norm(r)
    rel = np.linalg.norm(diff) / den if den > 0 else np.linalg.norm(diff)
    return rel, float(np.abs(diff).max()) if diff.size else 0.0


def gpu_fwd(w, q, k, v, **kw):
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    if w.window_w > 0:
        assert w.window_lo == 0
        out = sdpa.fwd_sliding(qd, kd, vd, window=w.window_w, causal=w.causal, pos0=w.pos0,
                               scale=w.scale, mode=w.mode, **kw)
    else:
        out = sdpa.fwd(qd, kd, vd, causal=w.causal, window_lo=w.window_lo, pos0=w.pos0,
                       scale=w.scale, mode=w.mode, **kw)
    torch.cuda.synchronize()
    return out


def check_workload(w, rows=None, tol=None, inputs=None):
    """Run w on the GPU and compare (all rows, or a sample) with the oracle."""
    announce(f"{w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} D={w.D} "
             f"{w.dtype} causal={w.causal} window_lo={w.window_lo} pos0={w.pos0} mode={w.mode} "
             f"window_w={w.window_w}")
    q, k, v = inputs if inputs is not None else make_qkv(w)
    out = gpu_fwd(w, q, k, v).float().cpu()
    assert torch.isfinite(out).all()
    if rows is None:
        ref = oracle.attn(q, k, v, scale=w.scale, causal=w.causal, window_lo=w.window_lo,
                          pos0=w.pos0, window_w=w.window_w)
        got = out.double().numpy()
    else:
        ref = oracle.attn(q, k, v, scale=w.scale, causal=w.causal, window_lo=w.window_lo,
                          pos0=w.pos0, window_w=w.window_w, rows=rows)
        got = out.reshape(-1, w.D)[torch.from_numpy(rows)].double().numpy()
    rel, mabs = metrics(got, ref)
    print(f"    rel={rel:.3e} max_abs={mabs:.3e}", flush=True)
    if w.mode == 0:
        assert rel <= (tol or EXACT_REL), rel
        assert mabs <= EXACT_ABS, mabs
    else:
        assert rel <= (tol or QUANT_REL), rel
    # rows with no visible key are exact zeros
    return out, ref, rel, mabs


def masked_rows(w):
    """Query rows (per head) that see no key."""
    out = []
    for i in range(w.Nq):
        hi = min(w.Nk - 1, w.pos0 + i) if w.causal else w.Nk - 1
        lo = w.window_lo
        if w.window_w > 0:
            lo = max(lo, w.pos0 + i - w.window_w + 1)
        if hi < lo:
            out.append(i)
    return out


def check_rope(w, rope, rows=None):
    """Run w through attn_fwd_rope with the rotary embedding rope (keyword
    arguments of sdpa.Rope) and compare with the oracle, which turns Q and K
    in double precision and then takes exact attention."""
    announce(f"rope {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} D={w.D} {w.dtype} "
             f"causal={w.causal} window_lo={w.window_lo} pos0={w.pos0} mode={w.mode} rope={rope}")
    q, k, v = make_qkv(w)
    dev = torch.device("cuda:0")
    out = sdpa.fwd_rope(q.to(dev), k.to(dev), v.to(dev), sdpa.Rope(**rope), causal=w.causal,
                        window_lo=w.window_lo, pos0=w.pos0, scale=w.scale, mode=w.mode)
    torch.cuda.synchronize()
    out = out.double().cpu()
    assert torch.isfinite(out).all()
    kw = dict(scale=w.scale, causal=w.causal, window_lo=w.window_lo, pos0=w.pos0, **rope)
    if rows is None:
        ref = oracle.attn_rope(q, k, v, **kw)
        got = out.numpy()
    else:
        ref = oracle.attn_rope(q, k, v, rows=rows, **kw)
        got = out.reshape(-1, w.D)[torch.from_numpy(rows)].numpy()
    rel, mabs = metrics(got, ref)
    print(f"    rel={rel:.3e} max_abs={mabs:.3e}", flush=True)
    if w.mode == 0:
        assert rel <= EXACT_REL, rel
        assert mabs <= EXACT_ABS, mabs
    else:
        assert rel <= QUANT_REL, rel
    for i in masked_rows(w):
        assert torch.all(out[:, :, i] == 0), i
    return out, ref, rel, mabs


# Quantised-cache decode: against the oracle with Q through its own INT8
# codes the only difference is the E4M3 rounding of the weights (each off by
# at most 2^-4 relative, about 2^-4/sqrt(3) in RMS over many keys); KVQ_REL
# leaves a margin over that. Against exact attention on the dequantised cache
# the INT8 rounding of Q is added, held to QUANT_REL.
KVQ_REL = 4e-2


def check_kvq(w, q=None, cache=None, **kw_run):
    """attn_decode_kvq on w's seeded quantised cache against both oracles."""
    announce(f"kvq {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} D={w.D} "
             f"{w.dtype} causal={w.causal} window_lo={w.window_lo} pos0={w.pos0}")
    q = q if q is not None else normal(w.q_shape, 41, w.dtype)
    cache = cache if cache is not None else make_kv_codes(w)
    dev = torch.device("cuda:0")
    kc, ks, vc, vs = (t.to(dev) for t in cache)
    out = sdpa.decode_kvq(q.to(dev), kc, ks, vc, vs, causal=w.causal, window_lo=w.window_lo,
                          pos0=w.pos0, scale=w.scale, **kw_run)
    torch.cuda.synchronize()
    out = out.double().cpu()
    assert torch.isfinite(out).all()
    kw = dict(scale=w.scale, causal=w.causal, window_lo=w.window_lo, pos0=w.pos0)
    ref_q = oracle.attn_kvq(q, *cache, quant_q=True, **kw)
    ref = oracle.attn_kvq(q, *cache, quant_q=False, **kw)
    rel_q, _ = metrics(out.numpy(), ref_q)
    rel, _ = metrics(out.numpy(), ref)
    print(f"    rel(vs quantised-Q oracle)={rel_q:.3e} rel(vs exact on the cache)={rel:.3e}",
          flush=True)
    assert rel_q <= KVQ_REL, rel_q
    assert rel <= QUANT_REL, rel
    for i in masked_rows(w):
        assert torch.all(out[:, :, i] == 0), i
    return out
