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
after W untimed ones, and around each step (per-launch durations). Decode
calls are a few microseconds each, so they are captured in a HIP graph and
the graph replay is timed. The CPU baseline times the fp64 oracle on a
bounded sample of rows of the same workload.

    python bench.py --ab LIB_A LIB_B --part decode [--pairs 10]

compares two builds of the library on one workload with a paired protocol:
blocks alternate A B, B A, A B, ...; the first pair is discarded; the ratio
B / A of each later pair is resampled (bootstrap) for a 95 % interval, and a
change counts only when the whole interval lies on one side of 1.
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
PEAK_FP4_TFLOPS = 10100.0    # MI355X dense fp4 MFMA
# half INT8 (Q K^T), half FP4 (P V): 1 / (0.5 / 5000 + 0.5 / 10100)
PEAK_INT8_FP4_TOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_FP4_TFLOPS)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
METRIC = "attention fwd TFLOPS (%bf16 MFMA peak) at 40×32760×128; decode µs + HBM GB/s"
# Context only (another machine, not a baseline): PyTorch SDPA takes 511 ms on
# an RTX 5080 for 1 x 40 x 32760 x 128 bf16 in the table of section 1 of
# "Attention kernels on a home RTX 5080" (4*B*H*N*N*D flops -> 43.0 TFLOP/s).
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


# Seconds of back-to-back work before any timed region: from idle the part
# needs tens of milliseconds of load before its clocks settle (a 110 us kernel
# measured 128 us per call over its first 60 launches and 112 us after 200),
# so warm-up is counted in time as well as in launches.
WARM_S = 0.2


def _warm(fn, warmup):
    """Run fn warmup times, then until WARM_S seconds of them have passed."""
    import torch
    t0 = time.perf_counter()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < WARM_S:
        for _ in range(max(warmup, 1)):
            fn()
        torch.cuda.synchronize()


def time_events(fn, iters, warmup, per_launch=None):
    """ms per call over iters back-to-back calls (HIP events on the current
    stream), after the warm-up of _warm. per_launch: a list that receives each
    call's own duration (ms)."""
    import torch
    _warm(fn, warmup)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)] \
        if per_launch is not None else None
    e0.record()
    for i in range(iters):
        if marks:
            marks[i].record()
        fn()
    if marks:
        marks[iters].record()
    e1.record()
    torch.cuda.synchronize()
    if marks:
        per_launch.extend(marks[i].elapsed_time(marks[i + 1]) for i in range(iters))
    return e0.elapsed_time(e1) / iters  # ms


def bench_prefill(w, steps, warmup, per_launch=None):
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

    ms = time_events(step, steps, warmup, per_launch)
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


def bench_decode(w, nbuf=48, reps=20, hot=True):
    """Cold-cache decode: nbuf independent KV caches, one call per cache, captured
    in a HIP graph; returns (us per call cold, us per call hot or None, bytes per
    call).
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
    cold = graph_us_per_call([lambda i=i: call(i) for i in range(nbuf)], reps)
    hot_us = graph_us_per_call([lambda: call(0)] * nbuf, reps) if hot else None
    del sets, ws
    return cold, hot_us, decode_bytes(w)


def decode_chunk_sweep(splits_list=(64, 32, 16, 8, 4), rounds=9, reps=20, nbuf=48, seed=1):
    """Cold decode at gqa_decode_f16_4096 with each split count (keys per
    partial = 4096 / splits): one graph of nbuf calls over rotated caches per
    split count, timed in rounds that visit the counts in alternating order
    (round 0 discarded); per count the median us per call and the bootstrap
    95 % interval of the mean ratio to the library's own plan (16 splits)."""
    import numpy as np
    import torch
    import scaled_dot_product_amd as sdpa
    from scaled_dot_product_amd.inputs import WORKLOADS, make_qkv
    w = WORKLOADS["gqa_decode_f16_4096"]
    dev = torch.device("cuda:0")
    q0, k0, v0 = (t.to(dev) for t in make_qkv(w))
    sets = [(q0.clone(), k0.clone(), v0.clone(), torch.empty_like(q0)) for _ in range(nbuf)]
    graphs = {}
    for sp in splits_list:
        need = sdpa.fwd_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, causal=w.causal,
                                               window_lo=w.window_lo, pos0=w.pos0, dtype=w.dtype,
                                               splits=sp)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

        def call(i, sp=sp, ws=ws):
            q, k, v, o = sets[i]
            sdpa.fwd_decode(q, k, v, causal=w.causal, window_lo=w.window_lo, pos0=w.pos0,
                            scale=w.scale, splits=sp, out=o, workspace=ws)
        for i in range(nbuf):
            call(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(nbuf):
                call(i)
        torch.cuda.synchronize()
        graphs[sp] = (g, ws)
    first = splits_list[0]
    _warm(graphs[first][0].replay, 3)
    times = {sp: [] for sp in splits_list}
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    for r in range(rounds + 1):
        order = list(splits_list) if r % 2 == 0 else list(reversed(splits_list))
        for sp in order:
            g = graphs[sp][0]
            g.replay()
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            times[sp].append(e0.elapsed_time(e1) * 1e3 / (reps * nbuf))
    ref = np.array(times[16][1:]) if 16 in times else np.array(times[first][1:])
    rng = np.random.default_rng(seed)
    out = {}
    for sp in splits_list:
        t = np.array(times[sp][1:])
        ratio = t / ref
        boots = np.array([ratio[rng.integers(0, ratio.size, ratio.size)].mean() for _ in range(4000)])
        lo, hi = np.percentile(boots, [2.5, 97.5])
        p = sdpa.plan(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, causal=w.causal, pos0=w.pos0, dtype=w.dtype)
        out[str(sp)] = {"keys_per_partial": -(-w.Nk // sp), "us_cold_median": round(float(np.median(t)), 3),
                        "ratio_to_16": round(float(ratio.mean()), 4),
                        "ci95": [round(float(lo), 4), round(float(hi), 4)]}
        log(f"decode splits {sp}: {out[str(sp)]}")
    del sets, graphs
    return {"workload": w.name, "rounds": rounds, "plan_splits": int(p.splits), "by_splits": out}


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

_PROBE = None


def load_probe():
    """libattn_probe.so (include/attn_probe.h): measurement probes, not attention."""
    global _PROBE
    if _PROBE is None:
        import ctypes
        from scaled_dot_product_amd.build import PROBE_LIB
        lib = ctypes.CDLL(PROBE_LIB)
        i, vp, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        lib.attn_probe_mfma.argtypes = [i, i, i, vp, vp]
        lib.attn_probe_read.argtypes = [vp, sz, i, vp, vp]
        lib.attn_probe_empty.argtypes = [i, vp]
        lib.attn_probe_valu.argtypes = [i, i, i, vp, vp]
        lib.attn_probe_mix.argtypes = [i, i, i, vp, vp]
        lib.attn_probe_phase.argtypes = [i, i, i, i, vp, vp]
        for f in (lib.attn_probe_mfma, lib.attn_probe_read, lib.attn_probe_empty,
                  lib.attn_probe_valu, lib.attn_probe_mix, lib.attn_probe_phase):
            f.restype = i
        _PROBE = lib
    return _PROBE


def _probe_call(status, what):
    if status != 0:
        raise RuntimeError(f"{what}: status {status}")


def measured_peaks():
    """What this part sustains on the box: the MFMA rate probe (register
    operands, 2 waves per SIMD, no memory traffic) per dtype, and a 1 GiB device
    copy for HBM (bytes read + written)."""
    import torch
    probe = load_probe()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 2 * cus, 512
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    for kind, key in ((0, "bf16_tflops"), (1, "int8_tops"), (2, "fp8_tops")):
        ms = time_events(lambda: _probe_call(probe.attn_probe_mfma(kind, iters, blocks, out.data_ptr(),
                                                                   stream), "attn_probe_mfma"), 5, 2)
        res[key] = round(blocks * 4 * iters * 16 * PROBE_OPS[kind] / (ms * 1e-3) / 1e12, 1)
    n = 1 << 30
    x = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    y = torch.empty_like(x)
    ms = time_events(lambda: y.copy_(x), 5, 2)
    res["copy_gbs"] = round(2 * n / (ms * 1e-3) / 1e9, 1)
    del x, y
    log(f"measured peaks: {res}")
    return res


VALU_KINDS = ("v_exp_f32", "v_fma_f32", "v_cvt_pk_bf16_f32", "v_cvt_pk_fp8_f32", "v_max3_f32",
              "v_dot2c_f32_bf16")
PHASE_KINDS = ("96 vector + 16 MFMA", "96 vector only", "16 MFMA only", "48 vector + 16 MFMA",
               "144 vector + 16 MFMA")


def valu_costs():
    """Issue cost of the softmax's vector instructions (attn_probe_valu, 8
    waves per SIMD: ns per wave instruction per SIMD, and relative to the FMA),
    and the bf16 MFMA rate with vector work beside it (attn_probe_mix, 2 waves
    per SIMD: percent of the MFMA-only rate per vector instructions per MFMA)."""
    import torch
    probe = load_probe()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream().cuda_stream
    out = torch.empty(8 * cus * 256, dtype=torch.float32, device="cuda:0")
    iters = 2000
    ns = {}
    for kind, name in enumerate(VALU_KINDS):
        blocks = 8 * cus
        ms = time_events(lambda: _probe_call(probe.attn_probe_valu(kind, iters, blocks, out.data_ptr(),
                                                                   stream), "attn_probe_valu"), 3, 1)
        ns[name] = ms * 1e6 / (8 * iters * 16)
    costs = {k: {"ns_per_wave_instruction_per_simd": round(v, 3),
                 "relative_to_fma": round(v / ns["v_fma_f32"], 2)} for k, v in ns.items()}
    mix = {}
    base = None
    for nv in (0, 4, 8, 12, 16, 24, 32):
        blocks = 2 * cus
        ms = time_events(lambda: _probe_call(probe.attn_probe_mix(nv, iters, blocks, out.data_ptr(),
                                                                  stream), "attn_probe_mix"), 3, 1)
        per = ms * 1e6 / (2 * iters * 4)   # ns per MFMA per SIMD
        base = per if nv == 0 else base
        mix[str(nv / 4)] = {"ns_per_mfma_per_simd": round(per, 3),
                            "mfma_rate_pct": round(100 * base / per, 1)}
    # two waves per SIMD alternating vector and matrix blocks between barriers:
    # every wave in the same order, or the SIMD's second wave matrix-first
    phase = {}
    out8 = torch.empty(cus * 512, dtype=torch.float32, device="cuda:0")
    for kind, name in enumerate(PHASE_KINDS):
        for late in (0, 1):
            if late and kind in (1, 2):
                continue
            ms = time_events(lambda: _probe_call(probe.attn_probe_phase(kind, late, iters, cus,
                                                                        out8.data_ptr(), stream),
                                                 "attn_probe_phase"), 3, 1)
            phase[name + (", second wave matrix-first" if late else "")] = round(ms * 1e6 / iters, 1)
    log(f"vector instruction costs: {costs}")
    log(f"MFMA rate beside vector work (vector instructions per MFMA -> % of MFMA-only): "
        f"{ {k: v['mfma_rate_pct'] for k, v in mix.items()} }")
    log(f"vector/matrix blocks, ns per round (two waves per SIMD): {phase}")
    return {"valu_costs": costs, "mfma_beside_valu": mix, "phase_ns_per_round": phase}


def graph_us_per_call(calls, reps=20):
    """Capture calls (a list of thunks) in one HIP graph and time its replays:
    microseconds per call."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls[0]()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    torch.cuda.synchronize()
    _warm(g.replay, 3)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / (reps * len(calls))


def decode_floor(nbytes, nbuf=48):
    """The floors under a decode call of nbytes: a launch that does nothing,
    and a bare read of nbytes from caches rotated over nbuf buffers (cold) or
    from one buffer (hot), each timed as replays of a captured graph."""
    import torch
    probe = load_probe()
    n = (nbytes + 15) // 16 * 16
    bufs = [torch.ones(n, dtype=torch.uint8, device="cuda:0") for _ in range(nbuf)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    # enough lanes that each issues its four loads once: one memory round trip
    blocks = min(65535, max(2 * cus, -(-n // (16 * 4 * 256))))
    out = torch.empty(blocks, dtype=torch.int32, device="cuda:0")

    def rd(b):
        return lambda: _probe_call(probe.attn_probe_read(
            b.data_ptr(), n, blocks, out.data_ptr(), torch.cuda.current_stream().cuda_stream),
            "attn_probe_read")

    empty = lambda: _probe_call(probe.attn_probe_empty(
        cus, torch.cuda.current_stream().cuda_stream), "attn_probe_empty")
    res = {"bytes": n, "read_blocks": blocks,
           "empty_launch_us": round(graph_us_per_call([empty] * nbuf), 3),
           "read_cold_us": round(graph_us_per_call([rd(b) for b in bufs]), 3),
           "read_hot_us": round(graph_us_per_call([rd(bufs[0])] * nbuf), 3)}
    res["read_cold_gbs"] = round(n / (res["read_cold_us"] * 1e-6) / 1e9, 1)
    del bufs
    log(f"decode floor: {res}")
    return res


def host_cpu():
    """CPU model, host CPU count and the threads this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS")
    threads = min(affinity, int(share)) if share and share.isdigit() and int(share) > 0 else affinity
    return {"cpu_model": model, "host_cpus": os.cpu_count(), "affinity_cpus": affinity,
            "threads": threads}


def cpu_baseline(w, budget_s=12.0):
    """The oracle as it stands, on a bounded sample of rows of w, on every CPU
    thread this process may use (the box's share for one GPU, OMP_NUM_THREADS,
    when that is set below the affinity mask)."""
    import oracle
    from scaled_dot_product_amd.inputs import sample_rows
    q, k, v = inputs(w)
    cpu = host_cpu()
    threads = cpu["threads"]
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
            "kind": "oracle", "cpu_model": cpu["cpu_model"], "host_cpus": cpu["host_cpus"],
            "affinity_cpus": cpu["affinity_cpus"],
            "sample": f"{done} sampled query rows of {w.name} (exact fp64 attention on "
                      f"{threads} threads, {t_used:.1f} s; full problem extrapolates to "
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
    elif part == "floor":
        extra["decode_floor"] = decode_floor(decode_bytes(WORKLOADS["gqa_decode_f16_4096"]))
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
    elif part == "mxd":
        # the diagonal-tiled mode: half of the work (Q K^T) on the INT8 matrix
        # cores (5.0 POP/s), the other half (P V) almost all on FP4 ones (10.1
        # PFLOP/s): a combined peak of 1 / (0.5 / 5.0 + 0.5 / 10.1) = 6.69 POP/s
        wd = WORKLOADS["video_dit_bf16_32760"].variant(name="video_dit_mxd_32760", mode=3)
        ms_d = bench_prefill(wd, 10, 2)
        tops = wd.flops() / (ms_d * 1e-3) / 1e12
        extra["mxd"] = {"workload": wd.name, "ms_per_call": round(ms_d, 4), "tops": round(tops, 2),
                        "frac_of_int8_fp4_peak": round(tops / PEAK_INT8_FP4_TOPS, 4)}
        log(f"mxd: {ms_d:.3f} ms/call incl. preparation")
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
    elif part == "valu":
        extra.update(valu_costs())
    elif part == "decode_chunks":
        extra["decode_chunks"] = decode_chunk_sweep()
    elif part in ("decode_cold", "decode_kvq_cold"):
        # the cold Nk = 4096 case alone (for profiler runs)
        wd = WORKLOADS["gqa_decode_f16_4096" if part == "decode_cold" else "gqa_decode_kvq_f16_4096"]
        cold_us, _, nbytes = bench_decode(wd, hot=False)
        extra[part] = {"workload": wd.name, "us_per_call_cold": round(cold_us, 3),
                       "gbs_cold": round(nbytes / (cold_us * 1e-6) / 1e9, 1), "bytes_per_call": nbytes}
        log(f"{part}: {cold_us:.2f} us ({extra[part]['gbs_cold']} GB/s)")
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


# Workloads the A/B mode can time, one number per block (lower is better).
def ab_part(part):
    from scaled_dot_product_amd.inputs import WORKLOADS
    if part == "headline":
        w = WORKLOADS["video_dit_bf16_32760"]
        return "ms", lambda: bench_prefill(w, 5, 1)
    if part == "causal":
        w = WORKLOADS["video_dit_bf16_32760"].variant(name="video_dit_causal_bf16_32760", causal=True)
        return "ms", lambda: bench_prefill(w, 8, 1)
    if part == "sliding":
        w = WORKLOADS["video_dit_bf16_32760"].variant(name="video_dit_sliding4096_bf16_32760",
                                                      causal=True, window_w=4096)
        return "ms", lambda: bench_prefill(w, 10, 1)
    if part == "sdxl":
        w = WORKLOADS["sdxl_1024px_bf16"]
        return "us", lambda: bench_prefill(w, 200, 10) * 1e3
    if part == "quant":
        w = WORKLOADS["video_dit_quant_32760"]
        return "ms", lambda: bench_prefill(w, 6, 1)
    if part == "mx":
        w = WORKLOADS["video_dit_bf16_32760"].variant(name="video_dit_mx_32760", mode=2)
        return "ms", lambda: bench_prefill(w, 6, 1)
    if part == "mxd":
        w = WORKLOADS["video_dit_bf16_32760"].variant(name="video_dit_mxd_32760", mode=3)
        return "ms", lambda: bench_prefill(w, 6, 1)
    if part in ("decode", "decode_window1000"):
        w = WORKLOADS["gqa_decode_f16_4096"].variant(window_lo=0 if part == "decode" else 1000)
        return "us", lambda: bench_decode(w, reps=20)[0]
    if part == "decode_kvq":
        w = WORKLOADS["gqa_decode_kvq_f16_4096"]
        return "us", lambda: bench_decode(w, reps=20)[0]
    if part == "decode_65536":
        w = WORKLOADS["gqa_decode_f16_4096"].variant(Nk=65536, pos0=65532)
        return "us", lambda: bench_decode(w, nbuf=3, reps=10)[0]
    raise SystemExit(f"unknown --part {part}")


def run_ab(lib_a, lib_b, part, pairs, seed=1):
    """Paired A/B of two library builds: blocks in the order A B, B A, A B, ...
    (pair 0 discarded), bootstrap 95 % interval of the mean ratio B / A."""
    import scaled_dot_product_amd as sdpa
    handles = {"A": sdpa.open_library(lib_a), "B": sdpa.open_library(lib_b)}
    unit, fn = ab_part(part)
    times = {"A": [], "B": []}
    for i in range(pairs + 1):
        order = ("A", "B") if i % 2 == 0 else ("B", "A")
        for key in order:
            with sdpa.using(handles[key]):
                t = fn()
            times[key].append(t)
        log(f"ab {part} pair {i}: A {times['A'][-1]:.4f} {unit}, B {times['B'][-1]:.4f} {unit}"
            + (" (discarded)" if i == 0 else ""))
    rec = ab_stats(times["A"][1:], times["B"][1:], seed)
    return {"ab": part, "unit": unit, "lib_a": lib_a, "lib_b": lib_b, **rec}


def ab_stats(a, b, seed=1, boots=4000):
    """Paired times of A and B (one entry per block pair) -> mean ratio B / A,
    its bootstrap 95 % interval (pairs resampled with replacement) and the
    verdict: a change only when the whole interval lies on one side of 1."""
    import numpy as np
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0 or a.shape != b.shape:
        raise ValueError("need the same positive number of A and B times")
    ratio = b / a
    rng = np.random.default_rng(seed)
    means = np.array([ratio[rng.integers(0, ratio.size, ratio.size)].mean() for _ in range(boots)])
    lo, hi = np.percentile(means, [2.5, 97.5])
    verdict = "B faster" if hi < 1.0 else ("B slower" if lo > 1.0 else "no difference")
    return {"pairs": int(ratio.size),
            "a_median": round(float(np.median(a)), 4), "b_median": round(float(np.median(b)), 4),
            "ratio_b_over_a": round(float(ratio.mean()), 4),
            "ci95": [round(float(lo), 4), round(float(hi), 4)], "verdict": verdict}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--skip-cpu", action="store_true", help="omit the CPU oracle baseline")
    ap.add_argument("--only-headline", action="store_true", help="time the headline step only")
    ap.add_argument("--only", choices=["decode", "decode_kvq", "decode_cold", "decode_kvq_cold",
                                       "decode_chunks", "valu",
                                       "quant", "mx", "mxd", "rope", "causal", "sliding", "sdxl",
                                       "copy",
                                       "floor"],
                    help="time one secondary workload only (for kernel profiles); "
                         "'copy' runs a plain 1 GiB device copy, the reference for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters; 'floor' the "
                         "empty-launch and bare-read floors under the decode; "
                         "'decode_cold' / 'decode_kvq_cold' the cold Nk = 4096 decode alone; "
                         "'decode_chunks' that decode at 64 ... 1024 keys per partial; "
                         "'valu' the vector-instruction and MFMA-beside-vector probes")
    ap.add_argument("--ab", nargs=2, metavar=("LIB_A", "LIB_B"),
                    help="paired A/B of two builds of libattn.so on --part")
    ap.add_argument("--part", default="headline", help="workload of --ab")
    ap.add_argument("--pairs", type=int, default=10, help="block pairs of --ab (after pair 0)")
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

    if args.ab:
        print(json.dumps(run_ab(args.ab[0], args.ab[1], args.part, args.pairs)), flush=True)
        return
    if args.only:
        extra = run_extra(args.only)
        print(json.dumps({"only": args.only, "extra": extra}), flush=True)
        return

    w = WORKLOADS["video_dit_bf16_32760"]
    log(f"headline: {w.name}, {args.warmup} warmup + {args.steps} timed steps")
    per = []
    ms = bench_prefill(w, args.steps, args.warmup, per)
    per.sort()
    ms_med = per[len(per) // 2]
    tflops = w.flops() / (ms * 1e-3) / 1e12
    log(f"headline: {ms:.3f} ms/step (median launch {ms_med:.3f} ms), {tflops:.1f} TFLOP/s")

    extra = {}
    if not args.only_headline:
        for part in ("quant", "mx", "mxd", "rope", "causal", "sliding", "sdxl", "decode",
                     "decode_kvq", "floor"):
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
    extra["page_context"] = {
        "note": "another machine's number, context only: PyTorch SDPA on an RTX 5080, same shape",
        "rtx5080_sdpa_tflops": round(PAGE_SDPA_TFLOPS, 2),
        "ratio": round(tflops / PAGE_SDPA_TFLOPS, 2)}

    cpu = None if args.skip_cpu else cpu_baseline(w)
    if cpu:
        log(f"cpu baseline: {cpu['value']} TFLOP/s on {cpu['cores']} threads ({cpu['cpu_model']}, "
            f"{cpu['host_cpus']} host CPUs)")

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "none (one GPU)",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q/K/V rounded to bf16",
        "config": {"workload": w.name, "B": w.B, "H": w.Hq, "N": w.Nq, "D": w.D,
                   "causal": w.causal, "global_batch": w.B, "seq_len": w.Nq,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic("prefill_video_dit_traffic.json"),
                     "kernel": "prefill_kernel<bf16,bf16,128,8>",
                     "launch_ms_mean": round(ms, 4), "launch_ms_median": round(ms_med, 4),
                     "measured_peak": peaks["bf16_tflops"],
                     "frac_of_measured": round(tflops / peaks["bf16_tflops"], 4),
                     "per_launch": "21.979 TFLOP (4*B*H*N*N*D), one launch per step"},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
