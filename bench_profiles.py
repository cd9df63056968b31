"""Summaries of rocprofv3 output for profiles/ (runs on the CPU, after the GPU run).

The raw rocprofv3 output (CSV files) stays out of the repository; this script
turns it into the short text summaries committed under profiles/, so every
figure there can be regenerated from a profiler run of committed files.

    python bench_profiles.py trace    --dir OUT --kernel NAME_PART --skip W --title T \\
                                      --cmd "rocprofv3 ..." [--flops F | --bytes N] \\
                                      [--bench BENCH_JSON_LINE_FILE] --out profiles/x.md
    python bench_profiles.py counters --dir OUT1 [OUT2 ...] --kernel NAME_PART --title T \\
                                      --cmd "..." [--cmd "..."] [--skip W] [--trace OUT] \\
                                      --out profiles/x.md
    python bench_profiles.py traffic  --fetch OUT --write OUT --copy-fetch OUT --copy-write OUT \\
                                      --kernel NAME_PART --skip W --algorithmic BYTES \\
                                      --sources FILE ... --title T --cmd "..." \\
                                      --out profiles/x.md [--json profiles/x.json]

`--skip W` drops the first W dispatches of the kernel (warm-up launches), so
the figures are those of the timed launches only; `--first N` keeps the N
dispatches after them (one case of a command that runs several). Timestamps are nanoseconds.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys


def _find(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        sys.exit(f"no *{suffix} under {d}")
    return hits


def kernel_trace(d):
    """[(name, start_ns, end_ns)] of every dispatch in dispatch order."""
    rows = []
    for path in _find(d, "kernel_trace.csv"):
        with open(path) as f:
            for r in csv.DictReader(f):
                rows.append((int(r.get("Dispatch_Id", 0) or 0), r["Kernel_Name"],
                             int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    rows.sort()
    return [(n, s, e) for _, n, s, e in rows]


def counter_rows(d):
    """{dispatch_id: (kernel name, {counter: value})}."""
    out = {}
    for path in _find(d, "counter_collection.csv"):
        with open(path) as f:
            for r in csv.DictReader(f):
                did = int(r["Dispatch_Id"])
                name, vals = out.setdefault(did, (r["Kernel_Name"], {}))
                vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _short(name, n=110):
    return name if len(name) <= n else name[:n] + "..."


def _pick(items, part, what):
    sel = [x for x in items if part in x[0]]
    if not sel:
        sys.exit(f"no {what} dispatch of a kernel whose name contains {part!r}")
    return sel


def cmd_trace(a):
    tr = kernel_trace(a.dir)
    lines = [f"# {a.title} (kernel trace)", "",
             "Command (from the repository root on one MI355X, `export TMPDIR=/tmp` first):", "",
             "```"] + a.cmd + ["```", ""]
    stats = {}
    for n, s, e in tr:
        stats.setdefault(n, []).append((e - s) / 1e3)
    lines += ["| kernel | calls | mean (us) | median (us) | min (us) | max (us) |",
              "|---|---|---|---|---|---|"]
    for n, v in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{_short(n)}` | {len(v)} | {statistics.mean(v):.2f} | "
                     f"{statistics.median(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    sel = _pick(tr, a.kernel, "traced")
    seg_note = ""
    if a.segment is not None:
        # runs of dispatches separated by more than gap_ms of idle time
        segs = [[sel[0]]]
        for prev, cur in zip(sel, sel[1:]):
            if cur[1] - prev[2] > a.gap_ms * 1e6:
                segs.append([])
            segs[-1].append(cur)
        seg_note = (f" Split at idle gaps over {a.gap_ms} ms the dispatches form runs of "
                    f"{', '.join(str(len(x)) for x in segs)}; run {a.segment} is kept"
                    + (f", its last {a.tail}" if a.tail else "") + ".")
        sel = segs[a.segment][-a.tail:] if a.tail else segs[a.segment]
    durs = [(e - s) / 1e3 for _, s, e in sel]
    timed = durs[a.skip:a.skip + a.first] if a.first else durs[a.skip:]
    if not timed:
        sys.exit("nothing left after --skip")
    mean, med = statistics.mean(timed), statistics.median(timed)
    lines += ["", f"Kernel `{_short(sel[0][0])}`: {len(durs)} dispatches; the first {a.skip} "
                  f"(warm-up) are dropped" + (f", the {len(timed)} after them are the timed "
                                              f"launches" if a.first else "") + "." + seg_note, ""]
    if len(durs) <= 64:
        lines += ["Per-dispatch durations (us): " + ", ".join(f"{x:.1f}" for x in durs) + ".", ""]
    lines += ["| timed launches | value |", "|---|---|",
              f"| count | {len(timed)} |", f"| mean (us) | {mean:.2f} |",
              f"| median (us) | {med:.2f} |"]
    if a.flops:
        lines += [f"| work per launch | {a.flops / 1e12:.4f} TFLOP |",
                  f"| rate at the mean | {a.flops / (mean * 1e-6) / 1e12:.1f} TFLOP/s |",
                  f"| rate at the median | {a.flops / (med * 1e-6) / 1e12:.1f} TFLOP/s |"]
    if a.bytes:
        lines += [f"| bytes per launch | {a.bytes} |",
                  f"| rate at the median | {a.bytes / (med * 1e-6) / 1e9:.1f} GB/s |"]
    if a.bench:
        with open(a.bench) as f:
            b = json.loads([l for l in f if l.strip().startswith("{")][-1])
        ms = b.get("ms_per_step")
        lines += [f"| bench.py ms_per_step, same session (HIP events) | {ms} ms |",
                  f"| trace mean / bench ms_per_step | {mean / 1e3 / ms:.4f} |"]
        if "roofline" in b:
            lines += [f"| bench.py roofline.frac | {b['roofline']['frac']} |"]
            if a.flops:
                lines += [f"| roofline frac from the trace mean | "
                          f"{a.flops / (mean * 1e-6) / 1e12 / b['roofline']['peak']:.4f} |"]
    if a.note:
        lines += ["", a.note]
    _write(a.out, lines)


# SQ/GRBM counters are summed over the device; GRBM_GUI_ACTIVE over 8 XCDs.
XCDS, SIMDS = 8, 1024


def cmd_counters(a):
    per = {}
    for d in a.dir:
        for did, (name, vals) in counter_rows(d).items():
            if a.kernel in name:
                per.setdefault(d, []).append((did, vals))
    if not per:
        sys.exit(f"no counted dispatch of {a.kernel!r}")
    merged = {}
    for d, lst in per.items():
        lst.sort()
        lst = lst[a.skip:] or lst
        for c in lst[0][1]:
            if c not in merged:   # a counter repeated in a later pass keeps the first pass's value
                merged[c] = statistics.median(v[c] for _, v in lst if c in v)
    lines = [f"# {a.title} (counters)", "",
             "Commands (from the repository root on one MI355X, `export TMPDIR=/tmp` first):", "",
             "```"] + a.cmd + ["```", "", "| counter | value (median over the counted dispatches) |",
                                "|---|---|"]
    for c in sorted(merged):
        lines.append(f"| `{c}` | {merged[c]:.4g} |")
    der = []
    cyc = merged.get("GRBM_GUI_ACTIVE")
    if cyc:
        cyc_x = cyc / XCDS
        der.append(("GPU cycles per XCD (`GRBM_GUI_ACTIVE` / 8)", f"{cyc_x:.4g}"))
        if a.trace:
            tr = _pick(kernel_trace(a.trace), a.kernel, "traced")
            durs = sorted((e - s) / 1e3 for _, s, e in tr)
            med = statistics.median(durs[a.skip:] if len(durs) > a.skip else durs)
            der.append(("clock (cycles per XCD / median kernel time of the trace)",
                        f"{cyc_x / (med * 1e-6) / 1e9:.3f} GHz"))
        if "SQ_VALU_MFMA_BUSY_CYCLES" in merged:
            der.append(("MFMA busy / SIMD cycles (`SQ_VALU_MFMA_BUSY_CYCLES` / (1024 x cycles))",
                        f"{100 * merged['SQ_VALU_MFMA_BUSY_CYCLES'] / (SIMDS * cyc_x):.1f}%"))
        if "SQ_BUSY_CU_CYCLES" in merged:
            der.append(("CU busy (`SQ_BUSY_CU_CYCLES` / (256 x cycles))",
                        f"{100 * merged['SQ_BUSY_CU_CYCLES'] / (SIMDS // 4 * cyc_x):.1f}%"))
    if "SQ_WAVE_CYCLES" in merged and "SQ_ACTIVE_INST_VALU" in merged:
        der.append(("VALU active per wave (`SQ_ACTIVE_INST_VALU` / `SQ_WAVE_CYCLES`)",
                    f"{100 * merged['SQ_ACTIVE_INST_VALU'] / merged['SQ_WAVE_CYCLES']:.1f}%"))
    if "SQ_WAVE_CYCLES" in merged and "SQ_ACTIVE_INST_LDS" in merged:
        der.append(("LDS instructions active per wave (`SQ_ACTIVE_INST_LDS` / `SQ_WAVE_CYCLES`)",
                    f"{100 * merged['SQ_ACTIVE_INST_LDS'] / merged['SQ_WAVE_CYCLES']:.1f}%"))
    if "SQ_WAVES" in merged:
        for c, lab in (("SQ_INSTS_VALU", "VALU instructions per wave (MFMAs included)"),
                       ("SQ_INSTS_MFMA", "MFMA instructions per wave"),
                       ("SQ_INSTS_LDS", "LDS instructions per wave"),
                       ("SQ_INSTS_SALU", "SALU instructions per wave")):
            if c in merged:
                der.append((lab, f"{merged[c] / merged['SQ_WAVES']:.0f}"))
    if "TCC_HIT_sum" in merged and "TCC_MISS_sum" in merged:
        tot = merged["TCC_HIT_sum"] + merged["TCC_MISS_sum"]
        der.append(("L2 hit rate (`TCC_HIT_sum` / (hit + miss))", f"{100 * merged['TCC_HIT_sum'] / tot:.1f}%"))
    if "SQ_LDS_BANK_CONFLICT" in merged:
        der.append(("LDS bank conflicts", f"{merged['SQ_LDS_BANK_CONFLICT']:.0f}"))
    if der:
        lines += ["", "| derived | value |", "|---|---|"] + [f"| {k} | {v} |" for k, v in der]
    if a.note:
        lines += ["", a.note]
    _write(a.out, lines)


def _median_counter(d, part, counter, skip, first=0):
    vals = sorted((did, v[counter]) for did, (n, v) in counter_rows(d).items()
                  if part in n and counter in v)
    vals = [x for _, x in vals[skip:]] or [x for _, x in vals]
    if first:
        vals = vals[:first]
    if not vals:
        sys.exit(f"no {counter} for {part!r} under {d}")
    return statistics.median(vals), len(vals)


def cmd_traffic(a):
    copy_part = "copyBuffer"
    fk, nf = _median_counter(a.fetch, a.kernel, "FETCH_SIZE", a.skip, a.first)
    wk, nw = _median_counter(a.write, a.kernel, "WRITE_SIZE", a.skip, a.first)
    cf, _ = _median_counter(a.copy_fetch, copy_part, "FETCH_SIZE", 0)
    cw, _ = _median_counter(a.copy_write, copy_part, "WRITE_SIZE", 0)
    gib_kib = (1 << 30) / 1024
    fs, ws = gib_kib / cf, gib_kib / cw
    hbm = fk * 1024 * fs + wk * 1024 * ws
    rec = {"kernel": a.kernel, "sources": a.sources,
           "source_sha256": _sha(a.sources),
           "fetch_size_kib_per_dispatch": fk, "write_size_kib_per_dispatch": wk,
           "copy_1gib_fetch_size_kib": cf, "copy_1gib_write_size_kib": cw,
           "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
           "hbm_bytes_per_launch": int(round(hbm)),
           "algorithmic_bytes_per_launch": a.algorithmic}
    lines = [f"# {a.title} (HBM traffic counters)", "",
             "Commands (from the repository root on one MI355X, `export TMPDIR=/tmp` first):", "",
             "```"] + a.cmd + ["```", "", "| quantity | value |", "|---|---|",
                                f"| FETCH_SIZE per dispatch (KiB, median of {nf}) | {fk:.0f} |",
                                f"| WRITE_SIZE per dispatch (KiB, median of {nw}) | {wk:.0f} |",
                                f"| FETCH_SIZE for a 1 GiB copy (KiB) | {cf:.0f} |",
                                f"| WRITE_SIZE for a 1 GiB copy (KiB) | {cw:.0f} |",
                                f"| fetch scale (1 GiB / copy FETCH_SIZE) | {fs:.4f} |",
                                f"| write scale (1 GiB / copy WRITE_SIZE) | {ws:.4f} |",
                                f"| HBM bytes per launch (scaled fetch + scaled write) | {hbm / 1e9:.4f} GB |",
                                f"| algorithmic bytes per launch | {a.algorithmic / 1e9:.4f} GB |",
                                f"| ratio | {hbm / a.algorithmic:.2f} |"]
    if a.note:
        lines += ["", a.note]
    _write(a.out, lines)
    if a.json:
        with open(a.json, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(f"wrote {a.json}")


def _sha(files):
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for src in files:
        with open(os.path.join(root, src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _write(path, lines):
    with open(path, "w") as f:
        f.write("\n".join(lines).rstrip() + "\n")
    print(f"wrote {path}")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--dir", required=True)
    t.add_argument("--flops", type=float)
    t.add_argument("--bytes", type=float)
    t.add_argument("--bench")
    t.add_argument("--segment", type=int, help="keep one run of dispatches (split at idle gaps)")
    t.add_argument("--tail", type=int, default=0, help="of that run, keep the last N")
    t.add_argument("--gap-ms", type=float, default=1.0)
    c = sub.add_parser("counters")
    c.add_argument("--dir", nargs="+", required=True)
    c.add_argument("--trace")
    r = sub.add_parser("traffic")
    for k in ("--fetch", "--write", "--copy-fetch", "--copy-write"):
        r.add_argument(k, required=True)
    r.add_argument("--algorithmic", type=float, required=True)
    r.add_argument("--sources", nargs="+", required=True)
    r.add_argument("--json")
    for p in (t, c, r):
        p.add_argument("--kernel", required=True)
        p.add_argument("--skip", type=int, default=0)
        p.add_argument("--first", type=int, default=0,
                       help="keep only the first N dispatches after --skip")
        p.add_argument("--title", required=True)
        p.add_argument("--cmd", action="append", required=True)
        p.add_argument("--note")
        p.add_argument("--out", required=True)
    a = ap.parse_args()
    {"trace": cmd_trace, "counters": cmd_counters, "traffic": cmd_traffic}[a.what](a)


if __name__ == "__main__":
    main()
