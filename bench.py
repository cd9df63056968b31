"""Benchmark of the fused attention forward on one MI355X.

One step is one attention forward of the video-DiT workload (B=1, 40 heads,
32760 tokens, head dim 128, bf16, non-causal) — the shape on which the table
in section 1 of "Attention kernels on a home RTX 5080" times its kernels. The
same run also measures the other shapes of the hot path: the few-row GQA
decode (cold K/V, rotated over 48 caches so the 256 MB Infinity Cache cannot
hold them), the quantised INT8-QK / FP8-PV mode and the MX mode (MX FP8
blocks on the P V product) and rotary position embedding on the video
shape, the
SDXL 1024px shape, the causal video shape with a per-row sliding window of
4096 keys, and the decode over a quantised (INT8 K / E4M3 V) KV cache. It
prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Timing: HIP events on the stream the kernels are launched on (torch's current
stream, which the binding hands to the library), around K back-to-back steps
after W untimed ones. Decode calls are a few microseconds each, so they are
captured in a HIP graph and the graph replay is timed. The CPU baseline times
the fp64 oracle on a bounded sample of rows of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 / int8 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
METRIC = "attention fwd TFLOPS (%bf16 MFMA peak) at 40×32760×128; decode µs + HBM GB/s"
# The pages' number for this workload and metric: PyTorch SDPA, 511 ms on an
# RTX 5080 for 1 x 40 x 32760 x 128 bf16 (4*B*H*N*N*D flops -> 43.0 TFLOP/s).
PAGE_SDPA_TFLOPS = 4 * 40 * 32760 * 32760 * 128 / 0.511 / 1e12


_INPUTS = {}


def inputs(w):
    """Seeded CPU inputs of w, generated once per shape and dtype in this run."""
    from scaled_dot_product_amd.inputs import make_qkv
    key = (w.q_shape, w.kv_shape, w.dtype)
    if key not in _INPUTS:
        _INPUTS[key] = make_qkv(w)
    return _INPUTS[key]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_events(fn, iters, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters  # ms


def bench_prefill(w, steps, warmup):
    import torch
    import scaled_dot_product_amd as sdpa
    from scaled_dot_product_amd.inputs import make_qkv
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in inputs(w))
    out = torch.empty_like(q)
    if w.window_w > 0:
        ws_n = sdpa.fwd_sliding_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D,
                                                window=w.window_w, causal=w.causal, pos0=w.pos0,
                                                mode=w.mode, dtype=w.dtype)
    else:
        ws_n = sdpa.fwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, causal=w.causal,
                                        window_lo=w.window_lo, pos0=w.pos0, mode=w.mode,
                                        dtype=w.dtype)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)

    def step():
        if w.window_w > 0:
            sdpa.fwd_sliding(q, k, v, window=w.window_w, causal=w.causal, pos0=w.pos0,
                             scale=w.scale, mode=w.mode, out=out, workspace=ws)
        else:
            sdpa.fwd(q, k, v, causal=w.causal, window_lo=w.window_lo, pos0=w.pos0,
                     scale=w.scale, mode=w.mode, out=out, workspace=ws)

    ms = time_events(step, steps, warmup)
    del q, k, v, out, ws
    return ms


def bench_quant_prep(w, iters=5):
    """Time of the standalone quantisers on the same inputs (preparation share)."""
    import torch
    import scaled_dot_product_amd as sdpa
    from scaled_dot_product_amd.inputs import make_qkv
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in inputs(w))

    def prep():
        sdpa.quantize_qk(q, k)
        sdpa.quantize_v(v)

    return time_events(prep, iters, 2)


def bench_decode(w, nbuf=48, reps=20):
    """Cold-cache decode: nbuf independent KV caches, one call per cache, captured
    in a HIP graph; returns (us per call cold, us per call hot, bytes per call).
    w.mode 2: the cache is INT8 K / E4M3 V codes with per-64-key scales."""
    import torch
    import scaled_dot_product_amd as sdpa
    from scaled_dot_product_amd.inputs import SEED_Q, make_kv_codes, make_qkv, normal
    dev = torch.device("cuda:0")
    kvq = w.mode == 2
    if kvq:
        q0 = normal(w.q_shape, SEED_Q, w.dtype).to(dev)
        kv0 = [t.to(dev) for t in make_kv_codes(w)]
        ws_n = sdpa.decode_kvq_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D,
                                               causal=w.causal, window_lo=w.window_lo,
                                               pos0=w.pos0, dtype=w.dtype)
    else:
        q0, k0, v0 = (t.to(dev) for t in make_qkv(w))
        kv0 = [k0, v0]
        ws_n = sdpa.fwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, causal=w.causal,
                                        window_lo=w.window_lo, pos0=w.pos0, dtype=w.dtype)
    # nbuf copies at distinct addresses: together larger than every cache level
    sets = [(q0.clone(), [t.clone() for t in kv0], torch.empty_like(q0)) for _ in range(nbuf)]
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)

    def call(i):
        q, kv, o = sets[i]
        if kvq:
            sdpa.decode_kvq(q, *kv, causal=w.causal, window_lo=w.window_lo, pos0=w.pos0,
                            scale=w.scale, out=o, workspace=ws)
        else:
            sdpa.fwd(q, *kv, causal=w.causal, window_lo=w.window_lo, pos0=w.pos0,
                     scale=w.scale, out=o, workspace=ws)

    for i in range(nbuf):
        call(i)
    torch.cuda.synchronize()
    results = {}
    for label, order in (("cold", list(range(nbuf))), ("hot", [0] * nbuf)):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            call(order[0])
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in order:
                call(i)
        torch.cuda.synchronize()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        results[label] = e0.elapsed_time(e1) * 1e3 / (reps * len(order))
        del g
    return results["cold"], results["hot"], decode_bytes(w)


def decode_bytes(w):
    """Algorithmic bytes of one decode call: K and V rows of the visible keys (2
    bytes per element, or 1 per code plus one fp32 scale per 64-key block and
    tensor for a quantised cache), Q in, O out."""
    lo = w.window_lo
    hi = min(w.Nk, w.pos0 + w.Nq) if w.causal else w.Nk
    if w.mode == 2:
        tiles = (hi + 63) // 64 - lo // 64 if hi > lo else 0
        kv = 2 * w.B * w.Hkv * ((hi - lo) * w.D + tiles * 4)
    else:
        kv = 2 * w.B * w.Hkv * (hi - lo) * w.D * 2
    return kv + 2 * w.B * w.Hq * w.Nq * w.D * 2


# Ops per MFMA of the rate probe's kinds: bf16 32x32x16, int8 32x32x32, fp8 32x32x64.
PROBE_OPS = {0: 32768.0, 1: 65536.0, 2: 131072.0}


def measured_peaks():
    """What this part sustains on the box: the MFMA rate probe (register
    operands, 2 waves per SIMD, no memory traffic) per dtype, and a 1 GiB device
    copy for HBM (bytes read + written)."""
    import torch
    import scaled_dot_product_amd as sdpa
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 2 * cus, 512
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    res = {}
    for kind, key in ((0, "bf16_tflops"), (1, "int8_tops"), (2, "fp8_tops")):
        ms = time_events(lambda: sdpa.probe_mfma(kind, iters, blocks, out), 5, 2)
        res[key] = round(blocks * 4 * iters * 16 * PROBE_OPS[kind] / (ms * 1e-3) / 1e12, 1)
    n = 1 << 30
    x = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    y = torch.empty_like(x)
    ms = time_events(lambda: y.copy_(x), 5, 2)
    res["copy_gbs"] = round(2 * n / (ms * 1e-3) / 1e9, 1)
    del x, y
    log(f"measured peaks: {res}")
    return res


def cpu_baseline(w, budget_s=12.0):
    """The oracle as it stands, on a bounded sample of rows of w (host cores)."""
    import numpy as np
    import oracle
    from scaled_dot_product_amd.inputs import make_qkv, sample_rows
    q, k, v = inputs(w)
    threads = oracle.default_threads()
    rows_all = sample_rows(w, 32768, seed=11)
    done, t_used, n = 0, 0.0, threads
    while t_used < budget_s and done < rows_all.size:
        chunk = rows_all[done:done + n]
        t0 = time.perf_counter()
        oracle.attn(q, k, v, scale=w.scale, causal=w.causal, window_lo=w.window_lo,
                    pos0=w.pos0, rows=chunk, nthreads=threads)
        dt = time.perf_counter() - t0
        t_used += dt
        done += chunk.size
        n = min(4 * n, max(threads, int(chunk.size * (budget_s - t_used) / max(dt, 1e-3))))
    flops = done * 4.0 * w.Nk * w.D   # non-causal rows: every key visible
    return {"value": round(flops / t_used / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} sampled query rows of {w.name} (exact fp64 attention, "
                      f"{t_used:.1f} s; full problem extrapolates to "
                      f"{t_used * w.B * w.Hq * w.Nq / done / 3600:.1f} h)"}


def run_extra(part):
    from scaled_dot_product_amd.inputs import WORKLOADS
    extra = {}
    if part == "copy":
        import torch
        n = 1 << 30
        x = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        y = torch.empty_like(x)
        ms = time_events(lambda: y.copy_(x), 5, 2)
        extra["copy"] = {"bytes_read": n, "bytes_written": n, "ms": round(ms, 4),
                         "gbs": round(2 * n / (ms * 1e-3) / 1e9, 1)}
        log(f"copy: 1 GiB in {ms:.3f} ms")
    elif part == "quant":
        wq = WORKLOADS["video_dit_quant_32760"]
        ms_q = bench_prefill(wq, 10, 2)
        ms_prep = bench_quant_prep(wq)
        extra["quant"] = {"workload": wq.name, "ms_per_call": round(ms_q, 4),
                          "tops": round(wq.flops() / (ms_q * 1e-3) / 1e12, 2),
                          "prep_ms": round(ms_prep, 4),
                          "kernel_tops_est": round(wq.flops() / ((ms_q - ms_prep) * 1e-3) / 1e12, 2),
                          "frac_of_fp8_peak": round(wq.flops() / (ms_q * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)}
        log(f"quant: {ms_q:.3f} ms/call incl. {ms_prep:.3f} ms preparation")
    elif part == "mx":
        wm = WORKLOADS["video_dit_bf16_32760"].variant(name="video_dit_mx_32760", mode=2)
        ms_m = bench_prefill(wm, 10, 2)
        extra["mx"] = {"workload": wm.name, "ms_per_call": round(ms_m, 4),
                       "tops": round(wm.flops() / (ms_m * 1e-3) / 1e12, 2),
                       "frac_of_fp8_peak": round(wm.flops() / (ms_m * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)}
        log(f"mx: {ms_m:.3f} ms/call incl. preparation")
    elif part == "rope":
        import torch
        import scaled_dot_product_amd as sdpa
        wr = WORKLOADS["video_dit_bf16_32760"]
        dev = torch.device("cuda:0")
        q, k, v = (t.to(dev) for t in inputs(wr))
        out = torch.empty_like(q)
        rope = sdpa.Rope(style=sdpa.ROPE_HALF, scaling=sdpa.ROPE_PLAIN, base=10000.0)
        ws = torch.empty(max(sdpa.fwd_rope_workspace_bytes(wr.B, wr.Hq, wr.Hkv, wr.Nq, wr.Nk, wr.D,
                                                            dtype=wr.dtype), 1),
                         dtype=torch.uint8, device=dev)
        ms_r = time_events(lambda: sdpa.fwd_rope(q, k, v, rope, scale=wr.scale, out=out,
                                                 workspace=ws), 10, 2)
        extra["rope"] = {"workload": "video_dit_rope_bf16_32760", "ms_per_call": round(ms_r, 4),
                         "tflops": round(wr.flops() / (ms_r * 1e-3) / 1e12, 2),
                         "frac_of_bf16_peak": round(wr.flops() / (ms_r * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        log(f"rope: {ms_r:.3f} ms/call (K turned in one pass, Q in the kernel)")
        del q, k, v, out, ws
    elif part == "causal":
        wc = WORKLOADS["video_dit_bf16_32760"].variant(name="video_dit_causal_bf16_32760", causal=True)
        ms_c = bench_prefill(wc, 10, 2)
        extra["causal"] = {"workload": wc.name, "ms_per_call": round(ms_c, 4),
                           "tflops": round(wc.flops() / (ms_c * 1e-3) / 1e12, 2),
                           "frac_of_bf16_peak": round(wc.flops() / (ms_c * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        log(f"causal: {ms_c:.3f} ms/call")
    elif part == "sliding":
        wsl = WORKLOADS["video_dit_bf16_32760"].variant(name="video_dit_sliding4096_bf16_32760",
                                                        causal=True, window_w=4096)
        ms_w = bench_prefill(wsl, 10, 2)
        extra["sliding"] = {"workload": wsl.name, "window": wsl.window_w,
                            "ms_per_call": round(ms_w, 4),
                            "tflops": round(wsl.flops() / (ms_w * 1e-3) / 1e12, 2),
                            "frac_of_bf16_peak": round(wsl.flops() / (ms_w * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        log(f"sliding: {ms_w:.3f} ms/call")
    elif part == "sdxl":
        ws_ = WORKLOADS["sdxl_1024px_bf16"]
        ms_s = bench_prefill(ws_, 50, 10)
        extra["sdxl"] = {"workload": ws_.name, "us_per_call": round(ms_s * 1e3, 2),
                         "tflops": round(ws_.flops() / (ms_s * 1e-3) / 1e12, 2),
                         "frac_of_bf16_peak": round(ws_.flops() / (ms_s * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        log(f"sdxl: {ms_s * 1e3:.1f} us/call")
    elif part == "decode":
        for wlo in (0, 1000):
            wd = WORKLOADS["gqa_decode_f16_4096"].variant(window_lo=wlo)
            cold_us, hot_us, nbytes = bench_decode(wd)
            key = "decode" if wlo == 0 else "decode_window1000"
            extra[key] = {"workload": wd.name + ("" if wlo == 0 else "_window_lo1000"),
                          "us_per_call_cold": round(cold_us, 3),
                          "gbs_cold": round(nbytes / (cold_us * 1e-6) / 1e9, 1),
                          "us_per_call_hot": round(hot_us, 3),
                          "bytes_per_call": nbytes,
                          "frac_of_hbm_peak_cold": round(nbytes / (cold_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
            log(f"{key}: cold {cold_us:.2f} us ({extra[key]['gbs_cold']} GB/s), hot {hot_us:.2f} us")
        extra["decode"]["sync_us_median"] = round(decode_sync_latency(WORKLOADS["gqa_decode_f16_4096"]), 2)
        log(f"decode: one synchronous call {extra['decode']['sync_us_median']} us (host wall clock)")
        sweep = {}
        for nk in (4096, 8192, 16384, 32768, 65536):
            wd = WORKLOADS["gqa_decode_f16_4096"].variant(Nk=nk, pos0=nk - 4)
            per = 2 * wd.B * wd.Hkv * nk * wd.D * 2
            nbuf = max(3, min(48, -(-640_000_000 // per)))   # > 600 MB of caches: cold
            cold_us, _, nbytes = bench_decode(wd, nbuf=nbuf, reps=10)
            sweep[str(nk)] = {"us_cold": round(cold_us, 2),
                              "gbs_cold": round(nbytes / (cold_us * 1e-6) / 1e9, 1)}
            log(f"decode sweep Nk={nk}: {cold_us:.2f} us, {sweep[str(nk)]['gbs_cold']} GB/s")
        extra["decode_kv_sweep"] = sweep
    elif part == "decode_kvq":
        wk = WORKLOADS["gqa_decode_kvq_f16_4096"]
        cold_us, hot_us, nbytes = bench_decode(wk)
        extra["decode_kvq"] = {"workload": wk.name, "us_per_call_cold": round(cold_us, 3),
                               "gbs_cold": round(nbytes / (cold_us * 1e-6) / 1e9, 1),
                               "us_per_call_hot": round(hot_us, 3), "bytes_per_call": nbytes,
                               "frac_of_hbm_peak_cold": round(nbytes / (cold_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        log(f"decode_kvq: cold {cold_us:.2f} us ({extra['decode_kvq']['gbs_cold']} GB/s), hot {hot_us:.2f} us")
        sweep = {}
        for nk in (4096, 8192, 16384, 32768, 65536):
            wd = wk.variant(Nk=nk, pos0=nk - 4)
            per = 2 * wd.B * wd.Hkv * nk * wd.D
            nbuf = max(3, min(48, -(-640_000_000 // per)))   # > 600 MB of caches: cold
            cold_us, _, nbytes = bench_decode(wd, nbuf=nbuf, reps=10)
            sweep[str(nk)] = {"us_cold": round(cold_us, 2),
                              "gbs_cold": round(nbytes / (cold_us * 1e-6) / 1e9, 1)}
            log(f"decode_kvq sweep Nk={nk}: {cold_us:.2f} us, {sweep[str(nk)]['gbs_cold']} GB/s")
        extra["decode_kvq_kv_sweep"] = sweep
    return extra


def decode_sync_latency(w, calls=50):
    """Median host wall time of one decode call followed by a device synchronize."""
    import torch
    import scaled_dot_product_amd as sdpa
    from scaled_dot_product_amd.inputs import make_qkv
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in make_qkv(w))
    out = torch.empty_like(q)
    ws_n = sdpa.fwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, causal=w.causal,
                                    window_lo=w.window_lo, pos0=w.pos0, dtype=w.dtype)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
    ts = []
    for i in range(calls + 5):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        sdpa.fwd(q, k, v, causal=w.causal, window_lo=w.window_lo, pos0=w.pos0, scale=w.scale,
                 out=out, workspace=ws)
        torch.cuda.synchronize()
        if i >= 5:
            ts.append((time.perf_counter() - t0) * 1e6)
    ts.sort()
    return ts[len(ts) // 2]


def recorded_traffic(record: str):
    """HBM bytes per launch measured by rocprofv3 counters (FETCH_SIZE and
    WRITE_SIZE, scaled by the same counters on a plain copy), as recorded in
    profiles/; None unless the record was taken on the current kernel sources
    (the SHA-256 of the listed source files, concatenated in order)."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", record)) as f:
            rec = json.load(f)
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
    except (OSError, ValueError, KeyError, TypeError):
        return None
    if rec.get("source_sha256") != h.hexdigest():
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--skip-cpu", action="store_true", help="omit the CPU oracle baseline")
    ap.add_argument("--only-headline", action="store_true", help="time the headline step only")
    ap.add_argument("--only", choices=["decode", "decode_kvq", "quant", "mx", "rope", "causal",
                                       "sliding", "sdxl", "copy"],
                    help="time one secondary workload only (for kernel profiles); "
                         "'copy' runs a plain 1 GiB device copy, the reference for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(each GPU would run independent heads, or key ranges merged by log-sum-exp).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import scaled_dot_product_amd as sdpa
    from scaled_dot_product_amd.inputs import WORKLOADS
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sdpa.load_library()
    free, total = torch.cuda.mem_get_info()
    log(f"device {torch.cuda.get_device_name(0)}; free HBM {free / 2**30:.1f} of {total / 2**30:.1f} GiB")

    if args.only:
        extra = run_extra(args.only)
        print(json.dumps({"only": args.only, "extra": extra}), flush=True)
        return

    w = WORKLOADS["video_dit_bf16_32760"]
    log(f"headline: {w.name}, {args.warmup} warmup + {args.steps} timed steps")
    ms = bench_prefill(w, args.steps, args.warmup)
    tflops = w.flops() / (ms * 1e-3) / 1e12
    log(f"headline: {ms:.3f} ms/step, {tflops:.1f} TFLOP/s")

    extra = {}
    if not args.only_headline:
        for part in ("quant", "mx", "rope", "causal", "sliding", "sdxl", "decode", "decode_kvq"):
            extra.update(run_extra(part))

    peaks = measured_peaks()
    if "quant" in extra:
        extra["quant"]["frac_of_measured_int8_fp8"] = round(
            extra["quant"]["tops"] / (0.5 * (peaks["int8_tops"] + peaks["fp8_tops"])), 4)
    if "mx" in extra:
        extra["mx"]["frac_of_measured_int8_fp8"] = round(
            extra["mx"]["tops"] / (0.5 * (peaks["int8_tops"] + peaks["fp8_tops"])), 4)
    for key in ("decode", "decode_kvq"):
        if key in extra:
            extra[key]["frac_of_measured_copy_cold"] = round(extra[key]["gbs_cold"] / peaks["copy_gbs"], 4)
    extra["measured_peaks"] = peaks

    cpu = None if args.skip_cpu else cpu_baseline(w)
    if cpu:
        log(f"cpu baseline: {cpu['value']} TFLOP/s on {cpu['cores']} threads")

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(tflops / PAGE_SDPA_TFLOPS, 3),
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q/K/V rounded to bf16",
        "config": {"workload": w.name, "B": w.B, "H": w.Hq, "N": w.Nq, "D": w.D,
                   "causal": w.causal, "global_batch": w.B, "seq_len": w.Nq,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic("prefill_video_dit_traffic.json"),
                     "kernel": "prefill_kernel<bf16,bf16,128>",
                     "measured_peak": peaks["bf16_tflops"],
                     "frac_of_measured": round(tflops / peaks["bf16_tflops"], 4),
                     "per_launch": "21.979 TFLOP (4*B*H*N*N*D)"},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
