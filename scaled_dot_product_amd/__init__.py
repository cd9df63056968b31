"""Fused attention forward for MI355X (gfx950) — thin Python binding.

This module only marshals arguments into the C ABI of ``libattn.so``
(declared in ``include/attn.h``): it takes device pointers from torch tensors,
allocates the output and the workspace with torch (device memory is the only
thing torch is used for here, besides streams), and raises on any non-zero
status. Every step of the computation runs in the HIP kernels; there is no
fallback: if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os

import torch

__all__ = ["fwd", "fwd_workspace_bytes", "fwd_sliding", "fwd_sliding_workspace_bytes",
           "fwd_rope", "fwd_rope_workspace_bytes", "Rope", "ROPE_HALF", "ROPE_INTERLEAVED",
           "ROPE_PLAIN", "ROPE_NTK", "ROPE_YARN",
           "quantize_qk", "quantize_v", "quantize_mx", "quantize_mx4", "decode_kvq",
           "decode_kvq_workspace_bytes", "fwd_decode", "fwd_decode_workspace_bytes", "plan",
           "Plan", "KERNEL_PREFILL", "KERNEL_DECODE", "KERNEL_PREFILL_QUANT", "KERNEL_PREFILL_MX",
           "KERNEL_PREFILL_MXD",
           "fwd_noalloc", "NOALLOC_SCRATCH_BYTES", "load_library", "open_library", "using",
           "MODE_EXACT", "MODE_QUANT", "MODE_MX", "MODE_MXD", "AttnError", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

MODE_EXACT = 0
MODE_QUANT = 1
MODE_MX = 2
MODE_MXD = 3      # diagonal-tiled mixed MXFP8 / MXFP4 (ATTN_MODE_MXD)
_DTYPE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
ROPE_HALF, ROPE_INTERLEAVED = 0, 1
ROPE_PLAIN, ROPE_NTK, ROPE_YARN = 0, 1, 2
KERNEL_PREFILL, KERNEL_DECODE, KERNEL_PREFILL_QUANT, KERNEL_PREFILL_MX = 1, 2, 3, 4
KERNEL_PREFILL_MXD = 5
NOALLOC_SCRATCH_BYTES = 16 << 20      # ATTN_NOALLOC_SCRATCH_BYTES of include/attn.h


class Rope(ctypes.Structure):
    """attn_rope of include/attn.h: rotary position embedding of Q and K."""
    _fields_ = [("style", ctypes.c_int), ("scaling", ctypes.c_int), ("base", ctypes.c_float),
                ("factor", ctypes.c_float), ("orig_ctx", ctypes.c_int),
                ("beta_fast", ctypes.c_float), ("beta_slow", ctypes.c_float)]

    def __init__(self, style=ROPE_HALF, scaling=ROPE_PLAIN, base=10000.0, factor=1.0,
                 orig_ctx=4096, beta_fast=32.0, beta_slow=1.0):
        super().__init__(style, scaling, base, factor, orig_ctx, beta_fast, beta_slow)

class Plan(ctypes.Structure):
    """attn_plan of include/attn.h: the kernels a call would launch."""
    _fields_ = [("kernel", ctypes.c_int), ("waves", ctypes.c_int), ("rows", ctypes.c_int),
                ("splits", ctypes.c_int), ("workgroups", ctypes.c_longlong),
                ("pre_launches", ctypes.c_int), ("workspace_bytes", ctypes.c_size_t)]


_lib = None


class AttnError(RuntimeError):
    pass


def load_library():
    """Load libattn.so (build it with ``scaled_dot_product_amd/build.py``)."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = open_library(LIB_PATH)
    return _lib


def open_library(path: str):
    """A separate handle on a build of the library at ``path`` with every entry
    point declared (``using`` routes this module's calls through it)."""
    if not os.path.exists(path):
        raise AttnError(f"{path} is not built; run python scaled_dot_product_amd/build.py")
    lib = ctypes.CDLL(path)
    i, f, vp, sz = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.attn_fwd.restype = i
    lib.attn_fwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, i, i, i]
    lib.attn_fwd_workspace_bytes.restype = sz
    lib.attn_fwd_sliding.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.attn_fwd_sliding.restype = i
    lib.attn_fwd_sliding_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, i, i, i]
    lib.attn_fwd_sliding_workspace_bytes.restype = sz
    lib.attn_fwd_rope.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i, i,
                                  ctypes.POINTER(Rope), vp, sz, vp]
    lib.attn_fwd_rope.restype = i
    lib.attn_fwd_rope_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, i, i, i]
    lib.attn_fwd_rope_workspace_bytes.restype = sz
    lib.attn_quantize_qk.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
    lib.attn_quantize_qk.restype = i
    lib.attn_quantize_v.argtypes = [vp, vp, vp, i, i, i, i, i, vp]
    lib.attn_quantize_v.restype = i
    lib.attn_quantize_mx.argtypes = [vp, vp, vp, i, i, i, i, i, i, vp]
    lib.attn_quantize_mx.restype = i
    lib.attn_quantize_mx4.argtypes = [vp, vp, vp, i, i, i, i, i, i, vp]
    lib.attn_quantize_mx4.restype = i
    lib.attn_decode_kvq.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i,
                                     vp, sz, vp]
    lib.attn_decode_kvq.restype = i
    lib.attn_decode_kvq_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, i, i]
    lib.attn_decode_kvq_workspace_bytes.restype = sz
    lib.attn_fwd_decode.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.attn_fwd_decode.restype = i
    lib.attn_fwd_decode_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, i, i, i]
    lib.attn_fwd_decode_workspace_bytes.restype = sz
    lib.attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i, i, vp]
    lib.attn_fwd_noalloc.restype = i
    lib.attn_fwd_plan.argtypes = [i, i, i, i, i, i, i, i, i, i, i, i, i, ctypes.POINTER(Plan)]
    lib.attn_fwd_plan.restype = i
    lib.attn_status_string.argtypes = [i]
    lib.attn_status_string.restype = ctypes.c_char_p
    return lib


@contextlib.contextmanager
def using(lib):
    """Route this module's calls through ``lib`` (a handle from open_library)
    inside the block: two builds can be timed in one process."""
    global _lib
    saved = load_library()
    _lib = lib
    try:
        yield lib
    finally:
        _lib = saved


def _check(status: int, what: str):
    if status != 0:
        msg = load_library().attn_status_string(status).decode()
        raise AttnError(f"{what}: status {status} ({msg})")


def _stream_handle(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise AttnError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise AttnError(f"{name} must be contiguous")
    return t


def fwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, *, causal=False, window_lo=0, pos0=0,
                        mode=MODE_EXACT, dtype=torch.bfloat16) -> int:
    return int(load_library().attn_fwd_workspace_bytes(
        B, Hq, Hkv, Nq, Nk, D, int(causal), int(window_lo), int(pos0), int(mode),
        _DTYPE[dtype]))


def _same_device(ref: torch.Tensor, *named):
    for t, name in named:
        if t.device != ref.device:
            raise AttnError(f"{name} must be on {ref.device}, like q")


def _check_qkv(q, k, v):
    _dev(q, "q"), _dev(k, "k"), _dev(v, "v")
    _same_device(q, (k, "k"), (v, "v"))
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or k.shape != v.shape:
        raise AttnError("expected q [B,Hq,Nq,D] and k, v [B,Hkv,Nk,D]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPE:
        raise AttnError("q, k, v must share one dtype among float32, float16, bfloat16")
    B, Hq, Nq, D = q.shape
    _, Hkv, Nk, Dk = k.shape
    if Dk != D or k.shape[0] != B:
        raise AttnError("q and k disagree on B or D")
    return B, Hq, Hkv, Nq, Nk, D


def _workspace(q, workspace, need):
    """Device pointer and byte length of the workspace (allocated when not
    given): a given one must be a contiguous device tensor on q's device."""
    if workspace is None:
        if need <= 0:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    _same_device(q, (workspace, "workspace"))
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _out_and_workspace(q, out, workspace, need):
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, "out")
        _same_device(q, (out, "out"))
        if out.shape != q.shape or out.dtype != q.dtype:
            raise AttnError("out must match q's shape and dtype")
    ws_ptr, ws_len = _workspace(q, workspace, need)
    return out, ws_ptr, ws_len


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal=False, window_lo=0,
        pos0=0, scale=None, mode=MODE_EXACT, out=None, workspace=None) -> torch.Tensor:
    """O = softmax(scale * Q K^T + mask) V on the current stream.

    q: [B, Hq, Nq, D]; k, v: [B, Hkv, Nk, D]; one dtype (fp32, f16, bf16).
    Returns O [B, Hq, Nq, D] in q's dtype (written into ``out`` if given).
    """
    lib = load_library()
    B, Hq, Hkv, Nq, Nk, D = _check_qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = fwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, causal=causal, window_lo=window_lo,
                               pos0=pos0, mode=mode, dtype=q.dtype)
    out, ws_ptr, ws_len = _out_and_workspace(q, out, workspace, need)
    st = lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                      B, Hq, Hkv, Nq, Nk, D, int(bool(causal)), int(window_lo), int(pos0),
                      float(scale), int(mode), _DTYPE[q.dtype], ws_ptr, ws_len,
                      _stream_handle(q))
    _check(st, "attn_fwd")
    return out


def fwd_sliding_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, *, window, causal=True, pos0=0,
                                mode=MODE_EXACT, dtype=torch.bfloat16) -> int:
    return int(load_library().attn_fwd_sliding_workspace_bytes(
        B, Hq, Hkv, Nq, Nk, D, int(causal), int(window), int(pos0), int(mode), _DTYPE[dtype]))


def fwd_sliding(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, window, causal=True,
                pos0=0, scale=None, mode=MODE_EXACT, out=None, workspace=None) -> torch.Tensor:
    """Attention with a per-row sliding window: row i sees keys
    j >= pos0 + i - window + 1 (and j <= pos0 + i when causal)."""
    lib = load_library()
    B, Hq, Hkv, Nq, Nk, D = _check_qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = fwd_sliding_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, window=window, causal=causal,
                                       pos0=pos0, mode=mode, dtype=q.dtype)
    out, ws_ptr, ws_len = _out_and_workspace(q, out, workspace, need)
    st = lib.attn_fwd_sliding(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              B, Hq, Hkv, Nq, Nk, D, int(bool(causal)), int(window), int(pos0),
                              float(scale), int(mode), _DTYPE[q.dtype], ws_ptr, ws_len,
                              _stream_handle(q))
    _check(st, "attn_fwd_sliding")
    return out


def fwd_rope_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, *, causal=False, window_lo=0, pos0=0,
                             mode=MODE_EXACT, dtype=torch.bfloat16) -> int:
    return int(load_library().attn_fwd_rope_workspace_bytes(
        B, Hq, Hkv, Nq, Nk, D, int(causal), int(window_lo), int(pos0), int(mode), _DTYPE[dtype]))


def fwd_rope(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rope: Rope, *, causal=False,
             window_lo=0, pos0=0, scale=None, mode=MODE_EXACT, out=None,
             workspace=None) -> torch.Tensor:
    """Attention on rotary-embedded Q (row i at position pos0 + i) and K (key j at j)."""
    lib = load_library()
    B, Hq, Hkv, Nq, Nk, D = _check_qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = fwd_rope_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, causal=causal, window_lo=window_lo,
                                    pos0=pos0, mode=mode, dtype=q.dtype)
    out, ws_ptr, ws_len = _out_and_workspace(q, out, workspace, need)
    st = lib.attn_fwd_rope(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           B, Hq, Hkv, Nq, Nk, D, int(bool(causal)), int(window_lo), int(pos0),
                           float(scale), int(mode), _DTYPE[q.dtype],
                           None if rope is None else ctypes.byref(rope), ws_ptr, ws_len,
                           _stream_handle(q))
    _check(st, "attn_fwd_rope")
    return out


def quantize_qk(q: torch.Tensor, k: torch.Tensor):
    """Per-64-token-block INT8 codes + fp32 scales of Q and K (bf16/f16 input)."""
    lib = load_library()
    if q.dim() != 4 or k.dim() != 4:
        raise AttnError("expected q [B,Hq,Nq,D] and k [B,Hkv,Nk,D]")
    if q.dtype != k.dtype or q.dtype not in (torch.float16, torch.bfloat16):
        raise AttnError("q and k must share one dtype, float16 or bfloat16")
    B, Hq, Nq, D = q.shape
    Bk, Hkv, Nk, Dk = k.shape
    if Bk != B or Dk != D:
        raise AttnError("q and k disagree on B or D")
    if Hq % Hkv != 0:
        raise AttnError("Hq must be a multiple of Hkv")
    _dev(q, "q"), _dev(k, "k")
    _same_device(q, (k, "k"))
    qc = torch.empty(q.shape, dtype=torch.int8, device=q.device)
    kc = torch.empty(k.shape, dtype=torch.int8, device=k.device)
    qs = torch.empty((B, Hq, (Nq + 63) // 64), dtype=torch.float32, device=q.device)
    ks = torch.empty((B, Hkv, (Nk + 63) // 64), dtype=torch.float32, device=k.device)
    st = lib.attn_quantize_qk(q.data_ptr(), k.data_ptr(), qc.data_ptr(), qs.data_ptr(),
                              kc.data_ptr(), ks.data_ptr(), B, Hq, Hkv, Nq, Nk, D,
                              _DTYPE.get(q.dtype, -1), _stream_handle(q))
    _check(st, "attn_quantize_qk")
    return qc, qs, kc, ks


def quantize_v(v: torch.Tensor):
    """Per-64-token-block E4M3 codes (uint8) + fp32 scales of V (bf16/f16 input)."""
    lib = load_library()
    _dev(v, "v")
    if v.dim() != 4:
        raise AttnError("expected v [B,Hkv,Nk,D]")
    B, Hkv, Nk, D = v.shape
    vc = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    vs = torch.empty((B, Hkv, (Nk + 63) // 64), dtype=torch.float32, device=v.device)
    st = lib.attn_quantize_v(v.data_ptr(), vc.data_ptr(), vs.data_ptr(), B, Hkv, Nk, D,
                             _DTYPE.get(v.dtype, -1), _stream_handle(v))
    _check(st, "attn_quantize_v")
    return vc, vs


def quantize_mx(x: torch.Tensor, axis: int = 0):
    """OCP MX FP8 codes (uint8 E4M3, x's layout) and E8M0 scale bytes (uint8) of
    x [B, H, N, D] (bf16/f16): axis 0 -> scales [B, H, N, D/32] (blocks of 32
    channels), axis 1 -> scales [B, H, ceil(N/32), D] (blocks of 32 tokens)."""
    lib = load_library()
    _dev(x, "x")
    if x.dim() != 4:
        raise AttnError("expected x [B,H,N,D]")
    B, H, N, D = x.shape
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    sshape = (B, H, N, D // 32) if axis == 0 else (B, H, (N + 31) // 32, D)
    scales = torch.empty(sshape, dtype=torch.uint8, device=x.device)
    st = lib.attn_quantize_mx(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), B, H, N, D,
                              int(axis), _DTYPE.get(x.dtype, -1), _stream_handle(x))
    _check(st, "attn_quantize_mx")
    return codes, scales


def quantize_mx4(x: torch.Tensor, axis: int = 0):
    """OCP MX FP4 codes (uint8 [B, H, N, D/2]: channel 2c in bits 0..3 of byte
    c, 2c + 1 in bits 4..7) and E8M0 scale bytes (uint8, laid out as
    quantize_mx's) of x [B, H, N, D] (bf16/f16)."""
    lib = load_library()
    _dev(x, "x")
    if x.dim() != 4:
        raise AttnError("expected x [B,H,N,D]")
    B, H, N, D = x.shape
    codes = torch.empty((B, H, N, D // 2), dtype=torch.uint8, device=x.device)
    sshape = (B, H, N, D // 32) if axis == 0 else (B, H, (N + 31) // 32, D)
    scales = torch.empty(sshape, dtype=torch.uint8, device=x.device)
    st = lib.attn_quantize_mx4(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), B, H, N, D,
                               int(axis), _DTYPE.get(x.dtype, -1), _stream_handle(x))
    _check(st, "attn_quantize_mx4")
    return codes, scales


def decode_kvq_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, *, causal=False, window_lo=0, pos0=0,
                               dtype=torch.float16) -> int:
    return int(load_library().attn_decode_kvq_workspace_bytes(
        B, Hq, Hkv, Nq, Nk, D, int(causal), int(window_lo), int(pos0), _DTYPE[dtype]))


def decode_kvq(q: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor,
               v_codes: torch.Tensor, v_scales: torch.Tensor, *, causal=False, window_lo=0,
               pos0=0, scale=None, out=None, workspace=None) -> torch.Tensor:
    """Decode over a quantised KV cache on the current stream.

    q: [B, Hq, Nq, D] f16/bf16; k_codes int8 and v_codes uint8 (E4M3) [B, Hkv, Nk, D];
    k_scales, v_scales fp32 [B, Hkv, ceil(Nk/64)] (the outputs of quantize_qk's K half
    and quantize_v). (Hq / Hkv) * Nq must be <= 32. Returns O [B, Hq, Nq, D] in q's dtype.
    """
    lib = load_library()
    for t, name in ((q, "q"), (k_codes, "k_codes"), (k_scales, "k_scales"),
                    (v_codes, "v_codes"), (v_scales, "v_scales")):
        _dev(t, name)
    _same_device(q, (k_codes, "k_codes"), (k_scales, "k_scales"), (v_codes, "v_codes"),
                 (v_scales, "v_scales"))
    if q.dim() != 4 or k_codes.dim() != 4 or v_codes.shape != k_codes.shape:
        raise AttnError("expected q [B,Hq,Nq,D] and k_codes, v_codes [B,Hkv,Nk,D]")
    if k_codes.dtype != torch.int8 or v_codes.dtype != torch.uint8:
        raise AttnError("k_codes must be int8 and v_codes uint8")
    B, Hq, Nq, D = q.shape
    _, Hkv, Nk, Dk = k_codes.shape
    if Dk != D or k_codes.shape[0] != B:
        raise AttnError("q and the codes disagree on B or D")
    sshape = (B, Hkv, (Nk + 63) // 64)
    for t, name in ((k_scales, "k_scales"), (v_scales, "v_scales")):
        if t.dtype != torch.float32 or tuple(t.shape) != sshape:
            raise AttnError(f"{name} must be float32 of shape {sshape}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dt = _DTYPE.get(q.dtype, -1)
    need = int(lib.attn_decode_kvq_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, int(bool(causal)),
                                                   int(window_lo), int(pos0), dt))
    out, ws_ptr, ws_len = _out_and_workspace(q, out, workspace, need)
    st = lib.attn_decode_kvq(q.data_ptr(), k_codes.data_ptr(), k_scales.data_ptr(),
                             v_codes.data_ptr(), v_scales.data_ptr(), out.data_ptr(),
                             B, Hq, Hkv, Nq, Nk, D, int(bool(causal)), int(window_lo),
                             int(pos0), float(scale), dt, ws_ptr, ws_len, _stream_handle(q))
    _check(st, "attn_decode_kvq")
    return out


def fwd_decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, *, causal=False, window_lo=0, pos0=0,
                               dtype=torch.float16, splits=0) -> int:
    return int(load_library().attn_fwd_decode_workspace_bytes(
        B, Hq, Hkv, Nq, Nk, D, int(causal), int(window_lo), int(pos0), _DTYPE[dtype],
        int(splits)))


def fwd_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal=False, window_lo=0,
               pos0=0, scale=None, splits=0, out=None, workspace=None) -> torch.Tensor:
    """The split-KV decode kernel with at most ``splits`` workgroups per KV head
    (0 = the library's plan), for (Hq / Hkv) * Nq <= 32 whatever the key count."""
    lib = load_library()
    B, Hq, Hkv, Nq, Nk, D = _check_qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = fwd_decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, causal=causal, window_lo=window_lo,
                                      pos0=pos0, dtype=q.dtype, splits=splits)
    out, ws_ptr, ws_len = _out_and_workspace(q, out, workspace, need)
    st = lib.attn_fwd_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             B, Hq, Hkv, Nq, Nk, D, int(bool(causal)), int(window_lo), int(pos0),
                             float(scale), _DTYPE[q.dtype], int(splits), ws_ptr, ws_len,
                             _stream_handle(q))
    _check(st, "attn_fwd_decode")
    return out


def plan(B, Hq, Hkv, Nq, Nk, D, *, causal=False, window_lo=0, window=0, pos0=0,
         mode=MODE_EXACT, dtype=torch.bfloat16, rope=False) -> Plan:
    """The kernels attn_fwd (window > 0: attn_fwd_sliding; rope: attn_fwd_rope)
    would launch for these sizes (host only)."""
    p = Plan()
    st = load_library().attn_fwd_plan(B, Hq, Hkv, Nq, Nk, D, int(bool(causal)), int(window_lo),
                                      int(window), int(pos0), int(mode), _DTYPE[dtype],
                                      int(bool(rope)), ctypes.byref(p))
    _check(st, "attn_fwd_plan")
    return p


def fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal=False, window_lo=0,
                pos0=0, scale=None, mode=MODE_EXACT, out=None) -> torch.Tensor:
    """attn_fwd_noalloc: fwd whose workspace is the library's fixed device array
    (no device allocation by the library; calls that overlap on one GPU race)."""
    lib = load_library()
    B, Hq, Hkv, Nq, Nk, D = _check_qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, "out")
        _same_device(q, (out, "out"))
        if out.shape != q.shape or out.dtype != q.dtype:
            raise AttnError("out must match q's shape and dtype")
    st = lib.attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              B, Hq, Hkv, Nq, Nk, D, int(bool(causal)), int(window_lo), int(pos0),
                              float(scale), int(mode), _DTYPE[q.dtype], _stream_handle(q))
    _check(st, "attn_fwd_noalloc")
    return out
