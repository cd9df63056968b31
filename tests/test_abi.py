"""The C-ABI libraries load and export every entry point include/attn.h and
include/attn_probe.h declare; argument checks reject bad calls before touching
the GPU; the dispatch policy (which kernel each workload takes) is fixed (CPU
only: no compute call is made)."""
import ctypes
import os
import re

import pytest

import scaled_dot_product_amd as sdpa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")
PROBE_HEADER = os.path.join(ROOT, "include", "attn_probe.h")

OK, E_INVALID, E_UNSUPPORTED, E_WORKSPACE = 0, -1, -2, -3


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(attn_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    from scaled_dot_product_amd import build
    if not os.path.exists(sdpa.LIB_PATH) or not os.path.exists(build.PROBE_LIB):
        build.build()
    return sdpa.load_library()


@pytest.fixture(scope="module")
def probe(lib):
    from scaled_dot_product_amd import build
    p = ctypes.CDLL(build.PROBE_LIB)
    p.attn_probe_mfma.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p] * 2
    p.attn_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_void_p]
    p.attn_probe_empty.argtypes = [ctypes.c_int, ctypes.c_void_p]
    p.attn_probe_valu.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p] * 2
    p.attn_probe_mix.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p] * 2
    p.attn_probe_phase.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 2
    return p


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("attn_fwd", "attn_fwd_workspace_bytes", "attn_quantize_qk",
              "attn_quantize_v", "attn_decode_kvq", "attn_decode_kvq_workspace_bytes",
              "attn_fwd_sliding", "attn_fwd_sliding_workspace_bytes", "attn_quantize_mx",
              "attn_quantize_mx4",
              "attn_fwd_rope", "attn_fwd_rope_workspace_bytes", "attn_fwd_decode",
              "attn_fwd_decode_workspace_bytes", "attn_fwd_plan", "attn_fwd_noalloc",
              "attn_status_string"):
        assert n in names
    assert "attn_probe_mfma" not in names     # measurement probes live in their own library
    assert _declared_functions(PROBE_HEADER) == ["attn_probe_empty", "attn_probe_mfma",
                                                 "attn_probe_mix", "attn_probe_phase",
                                                 "attn_probe_read", "attn_probe_valu"]


def test_library_exports_every_declared_symbol(lib, probe):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    for name in _declared_functions(PROBE_HEADER):
        assert hasattr(probe, name), name
    assert not hasattr(lib, "attn_probe_mfma")


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(lib.attn_status_string(st), bytes)


# A fake, 256-aligned address: the checks below fail before any dereference.
FAKE = 1 << 20


def _fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, Hq=2, Hkv=2, Nq=8, Nk=8, D=64,
             causal=0, window_lo=0, pos0=0, scale=0.125, mode=0, dtype=2,
             ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["B"], a["Hq"], a["Hkv"], a["Nq"],
                        a["Nk"], a["D"], a["causal"], a["window_lo"], a["pos0"], a["scale"],
                        a["mode"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), E_INVALID),
    (dict(o=None), E_INVALID),
    (dict(k=FAKE + 8), E_INVALID),            # misaligned
    (dict(B=0), E_INVALID),
    (dict(Nq=0), E_INVALID),
    (dict(Nk=-3), E_INVALID),
    (dict(Hq=3, Hkv=2), E_INVALID),           # Hq % Hkv != 0
    (dict(window_lo=-1), E_INVALID),
    (dict(pos0=-5, causal=1), E_INVALID),
    (dict(scale=0.0), E_INVALID),
    (dict(scale=-0.1), E_INVALID),
    (dict(scale=float("nan")), E_INVALID),
    (dict(scale=float("inf")), E_INVALID),
    (dict(D=96), E_UNSUPPORTED),
    (dict(D=256), E_UNSUPPORTED),
    (dict(dtype=7), E_UNSUPPORTED),
    (dict(mode=5), E_UNSUPPORTED),
    (dict(mode=4), E_UNSUPPORTED),
    (dict(mode=3, dtype=0), E_UNSUPPORTED),   # the diagonal-tiled MX mode needs 16-bit inputs
    (dict(mode=3), E_WORKSPACE),
    (dict(mode=1, dtype=0), E_UNSUPPORTED),   # quantised mode needs 16-bit inputs
    (dict(dtype=0), E_WORKSPACE),             # fp32 inputs need a bf16 staging workspace
    (dict(mode=1), E_WORKSPACE),
])
def test_fwd_rejects_before_enqueue(lib, kw, want):
    assert _fwd(lib, **kw) == want


def test_workspace_misaligned_rejected(lib):
    need = lib.attn_fwd_workspace_bytes(1, 2, 2, 8, 8, 64, 0, 0, 0, 0, 0)
    assert need > 0
    assert _fwd(lib, dtype=0, ws=FAKE + 16, ws_bytes=need) == E_INVALID


def test_workspace_bytes(lib):
    ws = lib.attn_fwd_workspace_bytes
    # exact bf16 prefill needs none; decode, fp32 staging and quant mode do
    assert ws(1, 40, 40, 32760, 32760, 128, 0, 0, 0, 0, 2) == 0
    assert ws(1, 16, 8, 4, 4096, 128, 1, 0, 4092, 0, 1) > 0
    assert ws(1, 2, 2, 256, 256, 64, 0, 0, 0, 0, 0) >= 3 * 2 * 256 * 64 * 2
    q = ws(1, 40, 40, 32760, 32760, 128, 0, 0, 0, 1, 2)
    assert q >= 3 * 40 * 32760 * 128
    # rejected arguments report 0
    assert ws(1, 3, 2, 8, 8, 64, 0, 0, 0, 0, 2) == 0
    assert ws(1, 2, 2, 8, 8, 96, 0, 0, 0, 0, 2) == 0


def test_quantizers_reject_before_enqueue(lib):
    assert lib.attn_quantize_qk(None, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 2, 8, 8, 64, 2, None) == E_INVALID
    assert lib.attn_quantize_qk(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 2, 8, 8, 64, 0, None) == E_UNSUPPORTED
    assert lib.attn_quantize_qk(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 3, 2, 8, 8, 64, 2, None) == E_INVALID
    assert lib.attn_quantize_v(FAKE, FAKE, None, 1, 2, 8, 64, 2, None) == E_INVALID
    assert lib.attn_quantize_v(FAKE, FAKE, FAKE, 1, 2, 8, 80, 2, None) == E_UNSUPPORTED
    assert lib.attn_quantize_v(FAKE, FAKE, FAKE, 1, 2, 0, 64, 2, None) == E_INVALID


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(sdpa.AttnError):
        sdpa.fwd(q, q, q)


def _kvq(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, ks=FAKE, vc=FAKE, vs=FAKE, o=FAKE, B=1, Hq=16, Hkv=8, Nq=4,
             Nk=4096, D=128, causal=1, window_lo=0, pos0=4092, scale=0.088, dtype=1,
             ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.attn_decode_kvq(a["q"], a["kc"], a["ks"], a["vc"], a["vs"], a["o"], a["B"],
                               a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["D"], a["causal"],
                               a["window_lo"], a["pos0"], a["scale"], a["dtype"], a["ws"],
                               a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), E_INVALID),
    (dict(kc=None), E_INVALID),
    (dict(vs=None), E_INVALID),
    (dict(o=None), E_INVALID),
    (dict(vc=FAKE + 8), E_INVALID),            # codes need 16-byte alignment
    (dict(ks=FAKE + 2), E_INVALID),            # scales need 4-byte alignment
    (dict(ws=FAKE + 16), E_INVALID),           # workspace needs 256-byte alignment
    (dict(ws=None), E_INVALID),
    (dict(ws_bytes=64), E_WORKSPACE),
    (dict(Hq=12, Hkv=8), E_INVALID),
    (dict(Nk=0), E_INVALID),
    (dict(window_lo=-1), E_INVALID),
    (dict(scale=float("nan")), E_INVALID),
    (dict(D=96), E_UNSUPPORTED),
    (dict(dtype=0), E_UNSUPPORTED),            # fp32 Q is not supported here
    (dict(Nq=17), E_UNSUPPORTED),              # 2 x 17 = 34 rows per KV head
    (dict(B=8192, Hq=16, Hkv=16, Nq=1), E_UNSUPPORTED),   # more than 65535 KV heads
])
def test_decode_kvq_rejects_before_enqueue(lib, kw, want):
    assert _kvq(lib, **kw) == want


def test_decode_kvq_workspace_bytes(lib):
    ws = lib.attn_decode_kvq_workspace_bytes
    need = ws(1, 16, 8, 4, 4096, 128, 1, 0, 4092, 1)
    # arrival counters plus fp32 partials (O, max, sum) of every split and row
    assert need >= 8 * 8 * (128 + 2) * 4
    assert need % 256 == 0
    assert ws(1, 16, 8, 4, 4096, 128, 1, 0, 4092, 0) == 0     # fp32 rejected
    assert ws(1, 64, 1, 1, 4096, 128, 0, 0, 0, 2) == 0        # 64 rows per KV head
    assert ws(1, 32, 1, 1, 4096, 64, 0, 0, 0, 2) > 0          # 32 rows fit
    assert _kvq(lib, ws_bytes=need - 1) == E_WORKSPACE


def _sliding(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, Hq=2, Hkv=2, Nq=8, Nk=8, D=64,
             causal=1, window=4, pos0=0, scale=0.125, mode=0, dtype=2,
             ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.attn_fwd_sliding(a["q"], a["k"], a["v"], a["o"], a["B"], a["Hq"], a["Hkv"],
                                a["Nq"], a["Nk"], a["D"], a["causal"], a["window"], a["pos0"],
                                a["scale"], a["mode"], a["dtype"], a["ws"], a["ws_bytes"],
                                a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(window=0), E_INVALID),
    (dict(window=-3), E_INVALID),
    (dict(q=None), E_INVALID),
    (dict(v=FAKE + 4), E_INVALID),
    (dict(pos0=-1), E_INVALID),
    (dict(scale=0.0), E_INVALID),
    (dict(D=80), E_UNSUPPORTED),
    (dict(mode=1, dtype=0), E_UNSUPPORTED),
    (dict(dtype=0), E_WORKSPACE),
])
def test_sliding_rejects_before_enqueue(lib, kw, want):
    assert _sliding(lib, **kw) == want


def test_sliding_workspace_bytes(lib):
    ws = lib.attn_fwd_sliding_workspace_bytes
    assert ws(1, 40, 40, 32760, 32760, 128, 1, 4096, 0, 0, 2) == 0      # bf16 prefill: none
    assert ws(1, 16, 8, 4, 4096, 128, 1, 1000, 4092, 0, 1) > 0          # decode partials
    assert ws(1, 16, 8, 4, 4096, 128, 1, 0, 4092, 0, 1) == 0            # window 0 rejected



def test_probe_rejects_before_enqueue(probe):
    p = probe.attn_probe_mfma
    assert p(0, 4, 2, None, None) == E_INVALID          # no output buffer
    assert p(0, 4, 2, FAKE + 4, None) == E_INVALID      # misaligned
    assert p(3, 4, 2, FAKE, None) == E_INVALID          # unknown kind
    assert p(0, 0, 2, FAKE, None) == E_INVALID          # no iterations
    assert p(1, 4, 0, FAKE, None) == E_INVALID          # no workgroups
    assert p(2, 4, 65536, FAKE, None) == E_INVALID      # grid too large
    r = probe.attn_probe_read
    assert r(None, 1024, 4, FAKE, None) == E_INVALID
    assert r(FAKE + 8, 1024, 4, FAKE, None) == E_INVALID    # misaligned source
    assert r(FAKE, 1000, 4, FAKE, None) == E_INVALID        # not whole 16-byte chunks
    assert r(FAKE, 0, 4, FAKE, None) == E_INVALID
    assert r(FAKE, 1024, 0, FAKE, None) == E_INVALID
    assert probe.attn_probe_empty(0, None) == E_INVALID
    assert probe.attn_probe_empty(70000, None) == E_INVALID
    v = probe.attn_probe_valu
    assert v(0, 4, 2, None, None) == E_INVALID          # no output buffer
    assert v(0, 4, 2, FAKE + 2, None) == E_INVALID      # misaligned
    assert v(6, 4, 2, FAKE, None) == E_INVALID          # unknown kind
    assert v(-1, 4, 2, FAKE, None) == E_INVALID
    assert v(1, 0, 2, FAKE, None) == E_INVALID          # no iterations
    assert v(1, 4, 65536, FAKE, None) == E_INVALID      # grid too large
    m = probe.attn_probe_mix
    assert m(0, 4, 2, None, None) == E_INVALID
    assert m(5, 4, 2, FAKE, None) == E_INVALID          # not a built vector count
    assert m(8, 0, 2, FAKE, None) == E_INVALID
    assert m(8, 4, 0, FAKE, None) == E_INVALID
    ph = probe.attn_probe_phase
    assert ph(0, 0, 4, 2, None, None) == E_INVALID
    assert ph(0, 0, 4, 2, FAKE + 2, None) == E_INVALID   # misaligned
    assert ph(5, 0, 4, 2, FAKE, None) == E_INVALID       # unknown kind
    assert ph(0, 2, 4, 2, FAKE, None) == E_INVALID       # late is 0 or 1
    assert ph(0, 1, 0, 2, FAKE, None) == E_INVALID
    assert ph(0, 1, 4, 65536, FAKE, None) == E_INVALID


def test_mx_entry_points_reject_before_enqueue(lib):
    q = lib.attn_quantize_mx
    assert q(None, FAKE, FAKE, 1, 2, 64, 128, 0, 2, None) == E_INVALID
    assert q(FAKE, FAKE, FAKE, 1, 2, 64, 96, 0, 2, None) == E_UNSUPPORTED     # D 96
    assert q(FAKE, FAKE, FAKE, 1, 2, 64, 128, 0, 0, None) == E_UNSUPPORTED    # fp32
    assert q(FAKE, FAKE, FAKE, 1, 2, 64, 128, 2, 2, None) == E_INVALID        # axis 2
    assert q(FAKE + 4, FAKE, FAKE, 1, 2, 64, 128, 1, 2, None) == E_INVALID    # misaligned
    # the MX mode of attn_fwd: 16-bit inputs only, and a workspace
    assert _fwd(lib, mode=2, dtype=0) == E_UNSUPPORTED
    assert _fwd(lib, mode=2) == E_WORKSPACE
    ws = lib.attn_fwd_workspace_bytes
    need = ws(1, 40, 40, 32760, 32760, 128, 0, 0, 0, 2, 2)
    # INT8 codes of Q and K, E4M3 codes of V (1 byte each), V's scale bytes (one
    # per 32 keys of a channel) and the fp32 scales of Q's and K's 64-token blocks
    assert need >= 3 * 40 * 32760 * 128 + 40 * 32760 * 128 // 32 + 2 * 40 * 512 * 4
    # the FP4 quantiser: the same checks
    q4 = lib.attn_quantize_mx4
    assert q4(None, FAKE, FAKE, 1, 2, 64, 128, 0, 2, None) == E_INVALID
    assert q4(FAKE, FAKE, FAKE, 1, 2, 64, 96, 0, 2, None) == E_UNSUPPORTED
    assert q4(FAKE, FAKE, FAKE, 1, 2, 64, 128, 0, 0, None) == E_UNSUPPORTED
    assert q4(FAKE, FAKE, FAKE, 1, 2, 64, 128, 2, 2, None) == E_INVALID
    assert q4(FAKE, FAKE + 4, FAKE, 1, 2, 64, 128, 1, 2, None) == E_INVALID   # misaligned codes
    # the diagonal-tiled mode also holds V's MXFP4 codes (half a byte per element)
    # and scale bytes, and the row partials (D 16-bit values and 4 floats per query row)
    need3 = ws(1, 40, 40, 32760, 32760, 128, 0, 0, 0, 3, 2)
    assert need3 >= need + 40 * 32760 * 128 // 2 + 40 * 32760 * 128 // 32 + 40 * 32760 * (256 + 16)



@pytest.mark.parametrize("rope,want", [
    (dict(style=2), E_INVALID),
    (dict(scaling=3), E_INVALID),
    (dict(base=0.0), E_INVALID),
    (dict(base=float("inf")), E_INVALID),
    (dict(scaling=1, factor=0.5), E_INVALID),
    (dict(scaling=2, factor=2.0, orig_ctx=0), E_INVALID),
    (dict(scaling=2, factor=2.0, beta_fast=1.0, beta_slow=1.0), E_INVALID),
    (dict(), E_WORKSPACE),          # valid: fp32 inputs still need their staging workspace
])
def test_rope_rejects_before_enqueue(lib, rope, want):
    r = sdpa.Rope(**rope)
    st = lib.attn_fwd_rope(FAKE, FAKE, FAKE, FAKE, 1, 2, 2, 8, 8, 64, 0, 0, 0, 0.125, 0, 0,
                           ctypes.byref(r), None, 0, None)
    assert st == want


def test_rope_workspace_bytes(lib):
    ws = lib.attn_fwd_rope_workspace_bytes
    # exact bf16 prefill: room for the rotated K only
    assert ws(1, 40, 40, 32760, 32760, 128, 0, 0, 0, 0, 2) >= 40 * 32760 * 128 * 2
    assert ws(1, 40, 40, 32760, 32760, 128, 0, 0, 0, 0, 2) < 2 * 40 * 32760 * 128 * 2
    assert ws(1, 3, 2, 8, 8, 64, 0, 0, 0, 0, 2) == 0    # rejected shape


# ---- split-count decode entry point ----------------------------------------

def _dec(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, Hq=16, Hkv=8, Nq=4, Nk=4096, D=128,
             causal=1, window_lo=0, pos0=4092, scale=0.088, dtype=1, splits=0,
             ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.attn_fwd_decode(a["q"], a["k"], a["v"], a["o"], a["B"], a["Hq"], a["Hkv"],
                               a["Nq"], a["Nk"], a["D"], a["causal"], a["window_lo"], a["pos0"],
                               a["scale"], a["dtype"], a["splits"], a["ws"], a["ws_bytes"],
                               a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(splits=-1), E_INVALID),
    (dict(q=None), E_INVALID),
    (dict(v=FAKE + 2), E_INVALID),
    (dict(ws=FAKE + 16), E_INVALID),
    (dict(ws_bytes=100), E_WORKSPACE),
    (dict(Nq=5), E_UNSUPPORTED),                         # 2 x 5 = 10 rows: fine ...
    (dict(Nq=17), E_UNSUPPORTED),                        # ... 34 rows per KV head are not
    (dict(B=70000, Hq=2, Hkv=1, Nq=1), E_UNSUPPORTED),   # more than 65535 KV heads
    (dict(D=96), E_UNSUPPORTED),
    (dict(scale=0.0), E_INVALID),
])
def test_decode_entry_rejects_before_enqueue(lib, kw, want):
    if kw == dict(Nq=5):
        # 10 rows fit: this call only fails on the fake workspace size check
        assert _dec(lib, Nq=5, ws_bytes=64) == E_WORKSPACE
        return
    assert _dec(lib, **kw) == want


def test_decode_entry_workspace_grows_with_splits(lib):
    ws = lib.attn_fwd_decode_workspace_bytes
    args = (1, 16, 8, 4, 4096, 128, 1, 0, 4092, 1)
    one, lib_plan, many = ws(*args, 1), ws(*args, 0), ws(*args, 32)
    # counters + per split and packed row: D + 2 fp32 values
    assert one >= 8 * 8 * 130 * 4
    assert one < lib_plan < many
    assert many >= 32 * 8 * 8 * 130 * 4
    assert ws(*args, 1000) == ws(*args, 64)              # at most one split per 64-key tile ...
    assert ws(1, 16, 8, 4, 100, 128, 1, 0, 96, 1, 64) == ws(1, 16, 8, 4, 100, 128, 1, 0, 96, 1, 2)
    assert ws(*args, -1) == 0
    assert ws(1, 16, 8, 17, 4096, 128, 1, 0, 4092, 1, 0) == 0


# ---- dispatch policy -----------------------------------------------------------

def _plan(**kw):
    import torch
    dt = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}[kw.pop("dtype", 2)]
    args = [kw.pop(k) for k in ("B", "Hq", "Hkv", "Nq", "Nk", "D")]
    return sdpa.plan(*args, dtype=dt, **kw)


def test_dispatch_of_the_five_workloads(lib):
    from scaled_dot_product_amd.inputs import WORKLOADS
    import torch
    want = {
        # name: (kernel, waves, rows, splits, workgroups, pre_launches)
        "tiny_fp32_256": (sdpa.KERNEL_PREFILL, 4, 128, 2, 8, 3),
        "gqa_decode_f16_4096": (sdpa.KERNEL_DECODE, 4, 8, 16, 128, 0),
        "sdxl_1024px_bf16": (sdpa.KERNEL_PREFILL, 4, 128, 2, 768, 0),
        "video_dit_bf16_32760": (sdpa.KERNEL_PREFILL, 8, 256, 1, 5120, 0),
        "video_dit_quant_32760": (sdpa.KERNEL_PREFILL_QUANT, 4, 128, 1, 10240, 3),
    }
    for name, exp in want.items():
        w = WORKLOADS[name]
        p = sdpa.plan(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, causal=w.causal, window_lo=w.window_lo,
                      pos0=w.pos0, mode=w.mode, dtype=w.dtype)
        got = (p.kernel, p.waves, p.rows, p.splits, p.workgroups, p.pre_launches)
        assert got == exp, (name, got)
        assert p.workspace_bytes == sdpa.fwd_workspace_bytes(
            w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, causal=w.causal, window_lo=w.window_lo,
            pos0=w.pos0, mode=w.mode, dtype=w.dtype)
    # the window variant of the decode shape still decodes, over fewer tiles
    p = sdpa.plan(1, 16, 8, 4, 4096, 128, causal=True, window_lo=1000, pos0=4092,
                  dtype=torch.float16)
    assert p.kernel == sdpa.KERNEL_DECODE and p.splits == 13


def test_prefill_split_policy(lib):
    """Grids of at most 128 query tiles split each tile's key range into 2-4
    parts of >= 2 key tiles, as many as keep the split grid within 256
    workgroups; the workspace holds one counter per tile and a partial (O / l
    in the output type, m and l in fp32) per part and row."""
    import torch
    # 64 tiles -> 4 parts; counters + 256 x 128 x (64 x 2 + 8) bytes
    p = _plan(B=1, Hq=8, Hkv=8, Nq=1024, Nk=4096, D=64)
    assert (p.splits, p.workgroups) == (4, 256)
    assert p.workspace_bytes == 512 + 256 * 128 * 64 * 2 + 256 * 128 * 8
    # 128 tiles -> 2 parts; 129 tiles -> none, no workspace
    p = _plan(B=1, Hq=128, Hkv=1, Nq=128, Nk=4096, D=64)
    assert (p.splits, p.workgroups) == (2, 256)
    p = _plan(B=1, Hq=129, Hkv=1, Nq=128, Nk=4096, D=64)
    assert (p.splits, p.workgroups, p.workspace_bytes) == (1, 129, 0)
    # between half a round and one round of workgroups (768 slots at head dim 64,
    # 512 at 128): slots - tiles tiles run as two halves, the jobs fill the slots,
    # a second launch merges; the workspace holds the halves' partials
    p = _plan(B=2, Hq=10, Hkv=10, Nq=4096, Nk=4096, D=64)      # SDXL: 640 tiles
    assert (p.splits, p.workgroups) == (2, 768)
    assert p.workspace_bytes == 128 * 2 * 128 * (64 * 2 + 8)
    assert _plan(B=1, Hq=767, Hkv=1, Nq=128, Nk=4096, D=64).workgroups == 768
    assert _plan(B=1, Hq=385, Hkv=1, Nq=128, Nk=4096, D=64).workgroups == 768
    p = _plan(B=1, Hq=384, Hkv=1, Nq=128, Nk=4096, D=64)      # half a round: unsplit
    assert (p.splits, p.workgroups, p.workspace_bytes) == (1, 384, 0)
    p = _plan(B=1, Hq=768, Hkv=1, Nq=128, Nk=4096, D=64)      # a full round: unsplit
    assert (p.splits, p.workgroups, p.workspace_bytes) == (1, 768, 0)
    p = _plan(B=1, Hq=300, Hkv=3, Nq=128, Nk=4096, D=128)
    assert (p.splits, p.workgroups) == (2, 512)
    assert _plan(B=1, Hq=300, Hkv=3, Nq=128, Nk=64, D=128).splits == 1     # one key tile
    # 85 tiles -> 3 parts; head dim 128 the same
    assert _plan(B=1, Hq=85, Hkv=1, Nq=128, Nk=4096, D=128).splits == 3
    # parts keep >= 2 key tiles each
    assert _plan(B=1, Hq=2, Hkv=2, Nq=256, Nk=4096, D=64).splits == 4
    assert _plan(B=1, Hq=2, Hkv=2, Nq=256, Nk=384, D=64).splits == 3
    assert _plan(B=1, Hq=2, Hkv=2, Nq=256, Nk=256, D=64).splits == 2
    assert _plan(B=1, Hq=2, Hkv=2, Nq=256, Nk=255, D=64).splits == 2    # 4 tiles, the last ragged
    assert _plan(B=1, Hq=2, Hkv=2, Nq=256, Nk=192, D=64).splits == 1
    # fp32 output: 4-byte partials, after the three bf16 staging copies
    p = _plan(B=1, Hq=2, Hkv=2, Nq=256, Nk=256, D=64, dtype=0)
    staging = 3 * 2 * 256 * 64 * 2
    assert p.workspace_bytes == staging + 256 + 8 * 128 * (64 * 4 + 8)
    # the quantised mode never splits this way
    assert _plan(B=1, Hq=8, Hkv=8, Nq=1024, Nk=4096, D=64, mode=sdpa.MODE_QUANT).splits == 1


def test_dispatch_boundaries(lib):
    import torch
    f16 = torch.float16
    # 32 packed rows decode, 34 do not
    assert _plan(B=1, Hq=8, Hkv=1, Nq=4, Nk=4096, D=128, dtype=1).kernel == sdpa.KERNEL_DECODE
    assert _plan(B=1, Hq=2, Hkv=1, Nq=17, Nk=4096, D=128, dtype=1).kernel == sdpa.KERNEL_PREFILL
    # fewer than 512 visible keys go to the prefill
    assert _plan(B=1, Hq=2, Hkv=1, Nq=1, Nk=511, D=128, dtype=1).kernel == sdpa.KERNEL_PREFILL
    assert _plan(B=1, Hq=2, Hkv=1, Nq=1, Nk=512, D=128, dtype=1).kernel == sdpa.KERNEL_DECODE
    # more than 65535 key/value heads cannot sit on the decode grid's y axis: prefill
    p = _plan(B=70000, Hq=2, Hkv=1, Nq=1, Nk=4096, D=128, dtype=1)
    assert p.kernel == sdpa.KERNEL_PREFILL and p.workspace_bytes == 0
    p = _plan(B=65535, Hq=2, Hkv=1, Nq=1, Nk=4096, D=128, dtype=1)
    assert p.kernel == sdpa.KERNEL_DECODE
    assert sdpa.fwd_workspace_bytes(70000, 2, 1, 1, 4096, 128, dtype=f16) == 0
    # the opt-in low-precision modes: one 128-row workgroup per query tile
    p = _plan(B=1, Hq=2, Hkv=2, Nq=256, Nk=256, D=128, mode=sdpa.MODE_MXD)
    assert (p.kernel, p.waves, p.rows, p.workgroups, p.pre_launches) == \
        (sdpa.KERNEL_PREFILL_MXD, 4, 128, 4, 4)
    assert _plan(B=1, Hq=2, Hkv=2, Nq=256, Nk=256, D=128, mode=sdpa.MODE_MX).kernel == \
        sdpa.KERNEL_PREFILL_MX
    # eight-wave prefill only for head dim 128 and grids of at least one round of
    # 256 workgroups whose last round is full, more than half full, or amortised
    # over eight rounds
    assert _plan(B=1, Hq=64, Hkv=64, Nq=8192, Nk=8192, D=128).waves == 8     # 2048
    assert _plan(B=1, Hq=63, Hkv=63, Nq=8192, Nk=8192, D=128).waves == 8     # 2016: 8 rounds - 32
    assert _plan(B=1, Hq=2, Hkv=2, Nq=32768, Nk=4096, D=128).waves == 8      # 256: one round
    assert _plan(B=1, Hq=1, Hkv=1, Nq=65280, Nk=4096, D=128).waves == 4      # 255
    assert _plan(B=1, Hq=20, Hkv=20, Nq=12800, Nk=4096, D=128).waves == 8    # 1000: tail 232
    assert _plan(B=1, Hq=11, Hkv=11, Nq=25600, Nk=4096, D=128).waves == 4    # 1100: tail 76
    assert _plan(B=1, Hq=4, Hkv=4, Nq=19200, Nk=4096, D=128).waves == 4      # 300: tail 44
    assert _plan(B=1, Hq=3, Hkv=3, Nq=32768, Nk=4096, D=128).waves == 4      # 384: tail 128
    assert _plan(B=1, Hq=13, Hkv=13, Nq=8192, Nk=4096, D=128).waves == 8     # 416: tail 160
    assert _plan(B=1, Hq=1, Hkv=1, Nq=98560, Nk=4096, D=128).waves == 8      # 385: tail 129
    assert _plan(B=2, Hq=1, Hkv=1, Nq=33024, Nk=4096, D=128).waves == 4      # 258: tail 2
    assert _plan(B=1, Hq=64, Hkv=64, Nq=8192, Nk=8192, D=64).waves == 4
    # under a per-row window narrower than 3072 keys the 128-row tiles compute
    # fewer masked scores: four waves even on a large grid
    win = dict(B=1, Hq=64, Hkv=64, Nq=8192, Nk=8192, D=128, causal=True)
    assert _plan(window=2048, **win).waves == 4
    assert _plan(window=3071, **win).waves == 4
    assert _plan(window=3072, **win).waves == 8
    assert _plan(window=2048, **win).workgroups == 64 * 8192 // 128
    # the MX mode, RoPE's extra pass and fp32 staging
    assert _plan(B=1, Hq=2, Hkv=2, Nq=256, Nk=256, D=64, mode=2).kernel == sdpa.KERNEL_PREFILL_MX
    assert _plan(B=1, Hq=2, Hkv=2, Nq=256, Nk=256, D=64, rope=True).pre_launches == 1
    assert _plan(B=1, Hq=2, Hkv=2, Nq=256, Nk=256, D=64, dtype=0, rope=True).pre_launches == 4
    # a per-row window: the decode over the window's tiles
    p = _plan(B=1, Hq=16, Hkv=8, Nq=4, Nk=4096, D=128, dtype=1, causal=True, pos0=4092,
              window=1024)
    assert p.kernel == sdpa.KERNEL_DECODE
    with pytest.raises(sdpa.AttnError):
        _plan(B=1, Hq=3, Hkv=2, Nq=4, Nk=4096, D=128)


def test_binding_quantize_qk_checks_pair_before_launch():
    # mismatched q, k pairs are refused before any device pointer is taken
    import torch
    q = torch.zeros(1, 4, 64, 128, dtype=torch.bfloat16)
    for k, what in ((torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16), "D"),
                    (torch.zeros(2, 2, 64, 128, dtype=torch.bfloat16), "B"),
                    (torch.zeros(1, 3, 64, 128, dtype=torch.bfloat16), "Hq % Hkv"),
                    (torch.zeros(1, 2, 64, 128, dtype=torch.float16), "dtype"),
                    (torch.zeros(2, 64, 128, dtype=torch.bfloat16), "rank")):
        with pytest.raises(sdpa.AttnError) as e:
            sdpa.quantize_qk(q, k)
        assert "device" not in str(e.value), what
    with pytest.raises(sdpa.AttnError, match="device"):
        sdpa.quantize_qk(q, torch.zeros(1, 2, 64, 128, dtype=torch.bfloat16))


# ---- allocation-free entry point: argument and size checks on the host -----------

def _noalloc(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, Hq=16, Hkv=8, Nq=4, Nk=4096, D=128,
             causal=1, window_lo=0, pos0=4092, scale=0.088, mode=0, dtype=1, stream=None)
    a.update(kw)
    return lib.attn_fwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["B"], a["Hq"], a["Hkv"],
                                a["Nq"], a["Nk"], a["D"], a["causal"], a["window_lo"], a["pos0"],
                                a["scale"], a["mode"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), E_INVALID),
    (dict(o=FAKE + 4), E_INVALID),
    (dict(Hq=12), E_INVALID),
    (dict(D=80), E_UNSUPPORTED),
    (dict(mode=1, dtype=0), E_UNSUPPORTED),
    (dict(scale=float("inf")), E_INVALID),
    # quantised mode at 8 x 8192 x 128: 25 MB of codes > the 16 MiB array
    (dict(Hq=8, Hkv=8, Nq=8192, Nk=8192, causal=0, pos0=0, mode=1, dtype=2), -5),
    # fp32 inputs staged as bf16 copies: 3 x 8 x 4096 x 128 x 2 bytes = 25 MB > 16 MiB
    (dict(B=1, Hq=8, Hkv=8, Nq=4096, Nk=4096, causal=0, pos0=0, dtype=0), -5),
])
def test_noalloc_rejects_before_touching_the_device(lib, kw, want):
    assert _noalloc(lib, **kw) == want


def test_noalloc_scratch_size_covers_the_decode(lib):
    # the decode workload's partials fit the fixed array many times over
    need = lib.attn_fwd_workspace_bytes(1, 16, 8, 4, 4096, 128, 1, 0, 4092, 0, 1)
    assert 0 < need < sdpa.NOALLOC_SCRATCH_BYTES // 8
    text = open(HEADER).read()
    assert "#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)" in text
    assert sdpa.NOALLOC_SCRATCH_BYTES == 16 << 20
