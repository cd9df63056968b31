"""Build the gfx950 attention library in-tree: scaled_dot_product_amd/libattn.so.

One hipcc invocation compiles the HIP kernels and the C ABI for gfx950 only.
Packed fp32 instructions are disabled (-packed-fp32-ops) and fp32 division is
correctly rounded (the quantisers' scale = amax / 127 must be bit-exact).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn.so")
SOURCES = ["attn_api.cpp", "attn_prefill.hip", "attn_decode.hip", "attn_quant.hip", "attn_mx.hip",
           "attn_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def command(out: str) -> list[str]:
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-rdc",
           "-Wno-unused-variable", "-o", out]
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        if src.endswith(".cpp"):
            cmd += ["-x", "hip", path]
        else:
            cmd += [path]
    return cmd


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
