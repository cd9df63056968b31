"""Build the gfx950 libraries in-tree.

* ``scaled_dot_product_amd/libattn.so`` — the attention library: the HIP
  kernels and the C ABI of ``include/attn.h``.
* ``scaled_dot_product_amd/libattn_probe.so`` — measurement probes of
  ``include/attn_probe.h`` (matrix-core rate, bare HBM read, empty launch);
  not attention, kept out of the product library.

Every translation unit is compiled by its own ``hipcc -c`` for gfx950 only
(in parallel), then linked. Packed fp32 instructions are disabled
(-packed-fp32-ops) and fp32 division is correctly rounded (the quantisers'
scale = amax / 127 must be bit-exact).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn.so")
PROBE_LIB = os.path.join(HERE, "libattn_probe.so")
SOURCES = ["attn_api.cpp", "attn_noalloc.hip", "attn_prefill.hip", "attn_decode.hip",
           "attn_quant.hip", "attn_mx.hip"]
PROBE_SOURCES = ["attn_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
OBJDIR = os.path.join(HERE, "_build")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-rdc", "-Wno-unused-variable"]
NOISE = "is not a recognized feature for this target"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if NOISE not in l)
    return res.returncode, err


def _compile(src: str, defines=()) -> tuple[str, int, str]:
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJDIR, src + ".o")
    cmd = [HIPCC] + FLAGS + [f"-D{d}" for d in defines] + ["-c", "-o", obj]
    cmd += (["-x", "hip", path] if src.endswith(".cpp") else [path])
    rc, err = _run(cmd)
    return obj, rc, err


def _link(objs, out: str, verbose: bool):
    tmp = out + ".tmp%d" % os.getpid()
    rc, err = _run([HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", "-o", tmp] + objs)
    if rc != 0:
        raise RuntimeError("link failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False, jobs: int | None = None, defines=()) -> str:
    """Compile both libraries; returns the attention library's path."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 1)))
    if verbose:
        print(f"{HIPCC} {' '.join(FLAGS)} -c <each of {', '.join(srcs)}>", flush=True)
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, defines), srcs))
    objs = {}
    for src, (obj, rc, err) in zip(srcs, results):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
        objs[src] = obj
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
