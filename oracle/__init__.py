"""CPU oracle for the fused attention forward — TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product library never does, and the oracle shares no
code with it: ``oracle.c`` is plain C compiled by gcc, this module is argument
marshalling through ctypes.

Functions (each wraps the C function of the same name; see ``oracle.c`` for
the definitions and the passages they follow):

* :func:`attn` — exact attention in fp64 over all rows or a row sample.
* :func:`quant_int8`, :func:`quant_e4m3` — per-64-token-block codes + scales.
* :func:`e4m3_encode`, :func:`e4m3_decode` — the OCP E4M3 format.
* :func:`attn_quant` — quantised-mode emulation (diagnostic).
* :func:`attn_kvq` — exact attention over a quantised KV cache (codes + scales).
* :func:`quant_mx` — OCP MX FP8 blocks (32 E4M3 elements, one E8M0 scale).
* :func:`attn_mx` — exact attention on the MX variant's inputs (INT8 Q, K; MX V).
* :func:`quant_mx4`, :func:`e2m1_encode`, :func:`e2m1_decode` — OCP MX FP4 blocks.
* :func:`attn_mxd` — the diagonal-tiled mixed MXFP8 / MXFP4 variant, weights rounded.
* :func:`rope_freqs`, :func:`rope_apply`, :func:`attn_rope` — rotary position
  embedding (plain, NTK, YaRN) and attention on rotated Q, K.

Pins: every function is checked in ``tests/test_oracle_*.py`` against closed
forms, invariants, brute force and library special cases. ``attn_quant`` is
pinned only through closed-form special cases (uniform scores; exactly
representable inputs) — its general output has no independent reference. ``attn_kvq`` is pinned
against :func:`attn` on exactly representable caches (values decoded by
torch's float8 cast), a uniform-weight closed form and the grid case of Q.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
            "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        i, i64, d = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        vp = ctypes.c_void_p
        lib.oracle_attn.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, i, i, i, i, d,
                                    vp, i64, vp, vp, vp, i]
        lib.oracle_attn.restype = i
        lib.oracle_attn_quant.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, i, i, i,
                                          d, vp, i64, vp, i]
        lib.oracle_attn_quant.restype = i
        lib.oracle_attn_kvq.argtypes = [vp, i, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i,
                                        d, i, vp, i64, vp, i]
        lib.oracle_attn_kvq.restype = i
        lib.oracle_quant_mx.argtypes = [vp, i, i64, i, i, i, vp, vp]
        lib.oracle_quant_mx.restype = i
        lib.oracle_attn_mx.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, i, i, i, d, vp, i64, vp, i]
        lib.oracle_attn_mx.restype = i
        lib.oracle_quant_mx4.argtypes = [vp, i, i64, i, i, i, vp, vp]
        lib.oracle_quant_mx4.restype = i
        lib.oracle_attn_mxd.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, i, i, i, i, d, vp, i64,
                                        vp, i]
        lib.oracle_attn_mxd.restype = i
        lib.oracle_e2m1_encode.argtypes = [ctypes.c_float]
        lib.oracle_e2m1_encode.restype = ctypes.c_uint8
        lib.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e2m1_decode.restype = ctypes.c_float
        lib.oracle_rope_freqs.argtypes = [i, i, d, d, i, d, d, vp, vp]
        lib.oracle_rope_freqs.restype = i
        lib.oracle_rope_apply.argtypes = [vp, i, i64, i, i, i, i, vp, vp]
        lib.oracle_rope_apply.restype = i
        lib.oracle_attn_rope.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, i, i, i, d,
                                         i, i, d, d, i, d, d, vp, i64, vp, i]
        lib.oracle_attn_rope.restype = i
        lib.oracle_quant_int8.argtypes = [vp, i, i64, i, i, vp, vp]
        lib.oracle_quant_int8.restype = i
        lib.oracle_quant_e4m3.argtypes = [vp, i, i64, i, i, vp, vp]
        lib.oracle_quant_e4m3.restype = i
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_decode.restype = ctypes.c_float
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(os.cpu_count() or 1, 16))


def _cpu(t: torch.Tensor) -> torch.Tensor:
    if t.dtype not in DTYPE_CODE:
        raise TypeError("oracle inputs must be float32, float16 or bfloat16")
    return t.detach().to("cpu").contiguous()


def attn(q, k, v, *, scale, causal=False, window_lo=0, pos0=0, window_w=0, rows=None,
         want_lse=False, want_weights=False, nthreads=None):
    """Exact fp64 attention. q: [B,Hq,Nq,D]; k, v: [B,Hkv,Nk,D] (same dtype).

    ``window_w`` > 0: per-row sliding window, row i also needs key
    j >= pos0 + i - window_w + 1.

    ``rows``: optional int64 flat indices (b*Hq + h)*Nq + i. Returns out
    [nrows, D] (or [B,Hq,Nq,D] when rows is None) as float64 numpy, plus lse
    and weights if asked.
    """
    q, k, v = _cpu(q), _cpu(k), _cpu(v)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    B, Hq, Nq, D = q.shape
    _, Hkv, Nk, _ = k.shape
    if rows is None:
        nrows = B * Hq * Nq
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
    out = np.zeros((nrows, D), dtype=np.float64)
    lse = np.zeros(nrows, dtype=np.float64) if want_lse else None
    w = np.zeros((nrows, Nk), dtype=np.float64) if want_weights else None
    rc = _load().oracle_attn(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), DTYPE_CODE[q.dtype],
        B, Hq, Hkv, Nq, Nk, D, int(causal), int(window_lo), int(pos0), int(window_w),
        float(scale), None if rows_arr is None else rows_arr.ctypes.data, nrows,
        out.ctypes.data, None if lse is None else lse.ctypes.data,
        None if w is None else w.ctypes.data, nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_attn rejected the arguments")
    if rows is None:
        out = out.reshape(B, Hq, Nq, D)
    res = [out]
    if want_lse:
        res.append(lse)
    if want_weights:
        res.append(w)
    return res[0] if len(res) == 1 else tuple(res)


def attn_quant(q, k, v, *, scale, causal=False, window_lo=0, pos0=0, rows=None,
               nthreads=None):
    """Quantised-mode emulation (see oracle.c). Same conventions as attn()."""
    q, k, v = _cpu(q), _cpu(k), _cpu(v)
    B, Hq, Nq, D = q.shape
    _, Hkv, Nk, _ = k.shape
    if rows is None:
        nrows, rows_arr = B * Hq * Nq, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
    out = np.zeros((nrows, D), dtype=np.float64)
    rc = _load().oracle_attn_quant(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), DTYPE_CODE[q.dtype],
        B, Hq, Hkv, Nq, Nk, D, int(causal), int(window_lo), int(pos0), float(scale),
        None if rows_arr is None else rows_arr.ctypes.data, nrows,
        out.ctypes.data, nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_attn_quant failed")
    return out.reshape(B, Hq, Nq, D) if rows is None else out


def attn_kvq(q, k_codes, k_scales, v_codes, v_scales, *, scale, causal=False, window_lo=0,
             pos0=0, quant_q=False, rows=None, nthreads=None):
    """Exact fp64 attention over a quantised KV cache (see oracle.c).

    q: [B,Hq,Nq,D] torch (fp32/f16/bf16); k_codes int8 and v_codes uint8 (E4M3)
    [B,Hkv,Nk,D]; k_scales, v_scales float32 [B,Hkv,ceil(Nk/64)] (numpy or torch).
    quant_q: use Q's per-block INT8 dequantisation instead of Q. Same return
    conventions as attn().
    """
    q = _cpu(q)
    kc = np.ascontiguousarray(np.asarray(k_codes.cpu() if hasattr(k_codes, "cpu") else k_codes, dtype=np.int8))
    vc = np.ascontiguousarray(np.asarray(v_codes.cpu() if hasattr(v_codes, "cpu") else v_codes, dtype=np.uint8))
    ks = np.ascontiguousarray(np.asarray(k_scales.cpu() if hasattr(k_scales, "cpu") else k_scales, dtype=np.float32))
    vs = np.ascontiguousarray(np.asarray(v_scales.cpu() if hasattr(v_scales, "cpu") else v_scales, dtype=np.float32))
    B, Hq, Nq, D = q.shape
    _, Hkv, Nk, _ = kc.shape
    nblk = (Nk + 63) // 64
    if vc.shape != kc.shape or ks.shape != (B, Hkv, nblk) or vs.shape != (B, Hkv, nblk):
        raise ValueError("codes [B,Hkv,Nk,D] and scales [B,Hkv,ceil(Nk/64)] expected")
    if rows is None:
        nrows, rows_arr = B * Hq * Nq, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
    out = np.zeros((nrows, D), dtype=np.float64)
    rc = _load().oracle_attn_kvq(
        q.data_ptr(), DTYPE_CODE[q.dtype], kc.ctypes.data, ks.ctypes.data, vc.ctypes.data,
        vs.ctypes.data, B, Hq, Hkv, Nq, Nk, D, int(causal), int(window_lo), int(pos0),
        float(scale), int(bool(quant_q)),
        None if rows_arr is None else rows_arr.ctypes.data, nrows, out.ctypes.data,
        nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_attn_kvq rejected the arguments")
    return out.reshape(B, Hq, Nq, D) if rows is None else out


def quant_mx(x, axis=0):
    """MX FP8 codes (uint8 E4M3, x's layout) and E8M0 scale bytes (uint8):
    axis 0 -> scales [..., N, D/32]; axis 1 -> scales [..., ceil(N/32), D]."""
    x = _cpu(x)
    *lead, N, D = x.shape
    BH = int(np.prod(lead)) if lead else 1
    codes = np.zeros(x.shape, dtype=np.uint8)
    sshape = tuple(lead) + ((N, D // 32) if axis == 0 else ((N + 31) // 32, D))
    scales = np.zeros(sshape, dtype=np.uint8)
    rc = _load().oracle_quant_mx(x.data_ptr(), DTYPE_CODE[x.dtype], BH, N, D, int(axis),
                                 codes.ctypes.data, scales.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_quant_mx rejected the arguments")
    return codes, scales


def attn_mx(q, k, v, *, scale, causal=False, window_lo=0, pos0=0, rows=None, nthreads=None):
    """Exact fp64 attention on the MX variant's inputs: Q and K through their
    per-64-token INT8 blocks, V through MX blocks of 32 keys. Same conventions
    as attn()."""
    q, k, v = _cpu(q), _cpu(k), _cpu(v)
    B, Hq, Nq, D = q.shape
    _, Hkv, Nk, _ = k.shape
    if rows is None:
        nrows, rows_arr = B * Hq * Nq, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
    out = np.zeros((nrows, D), dtype=np.float64)
    rc = _load().oracle_attn_mx(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), DTYPE_CODE[q.dtype],
        B, Hq, Hkv, Nq, Nk, D, int(causal), int(window_lo), int(pos0), float(scale),
        None if rows_arr is None else rows_arr.ctypes.data, nrows, out.ctypes.data,
        nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_attn_mx rejected the arguments")
    return out.reshape(B, Hq, Nq, D) if rows is None else out


def quant_mx4(x, axis=0):
    """MX FP4 codes (one uint8 per element holding the 4-bit E2M1 code, x's
    layout) and E8M0 scale bytes, laid out as quant_mx's."""
    x = _cpu(x)
    *lead, N, D = x.shape
    BH = int(np.prod(lead)) if lead else 1
    codes = np.zeros(x.shape, dtype=np.uint8)
    sshape = tuple(lead) + ((N, D // 32) if axis == 0 else ((N + 31) // 32, D))
    scales = np.zeros(sshape, dtype=np.uint8)
    rc = _load().oracle_quant_mx4(x.data_ptr(), DTYPE_CODE[x.dtype], BH, N, D, int(axis),
                                  codes.ctypes.data, scales.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_quant_mx4 rejected the arguments")
    return codes, scales


def attn_mxd(q, k, v, *, scale, causal=False, window_lo=0, pos0=0, window_w=0, rows=None,
             nthreads=None):
    """The diagonal-tiled mixed MX variant in fp64: Q and K through their
    per-64-token INT8 blocks; per row, the weights of each 32-key block and V
    in MXFP8 on the row's diagonal key tiles and in MXFP4 elsewhere, rounded as
    the variant rounds them. Same conventions as attn()."""
    q, k, v = _cpu(q), _cpu(k), _cpu(v)
    B, Hq, Nq, D = q.shape
    _, Hkv, Nk, _ = k.shape
    if rows is None:
        nrows, rows_arr = B * Hq * Nq, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
    out = np.zeros((nrows, D), dtype=np.float64)
    rc = _load().oracle_attn_mxd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), DTYPE_CODE[q.dtype],
        B, Hq, Hkv, Nq, Nk, D, int(causal), int(window_lo), int(pos0), int(window_w),
        float(scale), None if rows_arr is None else rows_arr.ctypes.data, nrows,
        out.ctypes.data, nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_attn_mxd rejected the arguments")
    return out.reshape(B, Hq, Nq, D) if rows is None else out


def e2m1_encode(y: float) -> int:
    return int(_load().oracle_e2m1_encode(float(y)))


def e2m1_decode(code: int) -> float:
    return float(_load().oracle_e2m1_decode(int(code)))


ROPE_PLAIN, ROPE_NTK, ROPE_YARN = 0, 1, 2
ROPE_HALF, ROPE_INTERLEAVED = 0, 1


def rope_freqs(D, scaling=ROPE_PLAIN, base=10000.0, factor=1.0, orig_ctx=4096,
               beta_fast=32.0, beta_slow=1.0):
    """Rotary frequencies theta [D/2] (float64) and the logit multiplier."""
    theta = np.zeros(D // 2, dtype=np.float64)
    mult = np.zeros(1, dtype=np.float64)
    rc = _load().oracle_rope_freqs(D, scaling, float(base), float(factor), int(orig_ctx),
                                   float(beta_fast), float(beta_slow), theta.ctypes.data,
                                   mult.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_rope_freqs rejected the arguments")
    return theta, float(mult[0])


def rope_apply(x, pos_base, theta, style=ROPE_HALF):
    """x [..., N, D] rotated at positions pos_base + n: float64 numpy."""
    x = _cpu(x)
    *lead, N, D = x.shape
    BH = int(np.prod(lead)) if lead else 1
    out = np.zeros(x.shape, dtype=np.float64)
    th = np.ascontiguousarray(np.asarray(theta, dtype=np.float64))
    rc = _load().oracle_rope_apply(x.data_ptr(), DTYPE_CODE[x.dtype], BH, N, D, int(pos_base),
                                   int(style), th.ctypes.data, out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_rope_apply rejected the arguments")
    return out


def attn_rope(q, k, v, *, scale, causal=False, window_lo=0, pos0=0, style=ROPE_HALF,
              scaling=ROPE_PLAIN, base=10000.0, factor=1.0, orig_ctx=4096, beta_fast=32.0,
              beta_slow=1.0, rows=None, nthreads=None):
    """Exact fp64 attention on Q rotated at positions pos0 + i and K at j."""
    q, k, v = _cpu(q), _cpu(k), _cpu(v)
    B, Hq, Nq, D = q.shape
    _, Hkv, Nk, _ = k.shape
    if rows is None:
        nrows, rows_arr = B * Hq * Nq, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
    out = np.zeros((nrows, D), dtype=np.float64)
    rc = _load().oracle_attn_rope(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), DTYPE_CODE[q.dtype],
        B, Hq, Hkv, Nq, Nk, D, int(causal), int(window_lo), int(pos0), float(scale),
        int(style), int(scaling), float(base), float(factor), int(orig_ctx), float(beta_fast),
        float(beta_slow), None if rows_arr is None else rows_arr.ctypes.data, nrows,
        out.ctypes.data, nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_attn_rope rejected the arguments")
    return out.reshape(B, Hq, Nq, D) if rows is None else out


def _quant(fn, x, code_dtype):
    x = _cpu(x)
    *lead, N, D = x.shape
    BH = int(np.prod(lead)) if lead else 1
    nblk = (N + 63) // 64
    codes = np.zeros(x.shape, dtype=code_dtype)
    scales = np.zeros(tuple(lead) + (nblk,), dtype=np.float32)
    rc = fn(x.data_ptr(), DTYPE_CODE[x.dtype], BH, N, D, codes.ctypes.data,
            scales.ctypes.data)
    if rc != 0:
        raise ValueError("quantiser rejected the arguments")
    return codes, scales


def quant_int8(x):
    """INT8 codes [..., N, D] (int8) and scales [..., ceil(N/64)] (float32)."""
    return _quant(_load().oracle_quant_int8, x, np.int8)


def quant_e4m3(x):
    """E4M3 codes [..., N, D] (uint8) and scales [..., ceil(N/64)] (float32)."""
    return _quant(_load().oracle_quant_e4m3, x, np.uint8)


def e4m3_encode(y: float) -> int:
    return int(_load().oracle_e4m3_encode(float(y)))


def e4m3_decode(code: int) -> float:
    return float(_load().oracle_e4m3_decode(int(code)))
