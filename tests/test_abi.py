"""The C-ABI library loads and exports every entry point include/attn.h
declares; argument checks reject bad calls before touching the GPU (CPU only:
no compute call is made)."""
import ctypes
import os
import re

import pytest

import scaled_dot_product_amd as sdpa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, E_INVALID, E_UNSUPPORTED, E_WORKSPACE = 0, -1, -2, -3


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(attn_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sdpa.LIB_PATH):
        from scaled_dot_product_amd import build
        build.build()
    return sdpa.load_library()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("attn_fwd", "attn_fwd_workspace_bytes", "attn_quantize_qk",
              "attn_quantize_v", "attn_decode_kvq", "attn_decode_kvq_workspace_bytes",
              "attn_fwd_sliding", "attn_fwd_sliding_workspace_bytes", "attn_quantize_mx",
              "attn_fwd_rope", "attn_fwd_rope_workspace_bytes",
              "attn_status_string", "attn_probe_mfma"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4, 7):
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



def test_probe_rejects_before_enqueue(lib):
    p = lib.attn_probe_mfma
    assert p(0, 4, 2, None, None) == E_INVALID          # no output buffer
    assert p(0, 4, 2, FAKE + 4, None) == E_INVALID      # misaligned
    assert p(3, 4, 2, FAKE, None) == E_INVALID          # unknown kind
    assert p(0, 0, 2, FAKE, None) == E_INVALID          # no iterations
    assert p(1, 4, 0, FAKE, None) == E_INVALID          # no workgroups
    assert p(2, 4, 65536, FAKE, None) == E_INVALID      # grid too large


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
