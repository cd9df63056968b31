// attn_api.cpp — the C ABI declared in include/attn.h: argument checks,
// workspace planning and kernel dispatch. Every check runs before anything is
// enqueued, and none of them touches the HIP runtime, so a rejected call has
// no effect on the device.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../include/attn.h"
#include "attn_internal.hpp"

namespace attn {

KeyRange key_range(const FwdArgs& a) {
  KeyRange r;
  r.lo = a.window_lo;
  // the lowest per-row bound is row 0's
  if (a.window_w > 0 && (int64_t)a.pos0 - a.window_w + 1 > r.lo) r.lo = a.pos0 - a.window_w + 1;
  r.hi = a.causal ? (int)(a.pos0 + (int64_t)a.Nq < a.Nk ? a.pos0 + a.Nq : a.Nk) : a.Nk;
  if (r.hi < r.lo) r.hi = r.lo;
  return r;
}

namespace {

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(int B, int Hq, int Hkv, int Nq, int Nk, int D, int dtype) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || D < 1) return ATTN_E_INVALID;
  if (Hq % Hkv != 0) return ATTN_E_INVALID;
  if (dtype != ATTN_DT_F32 && dtype != ATTN_DT_F16 && dtype != ATTN_DT_BF16) return ATTN_E_UNSUPPORTED;
  if (D != 64 && D != 128) return ATTN_E_UNSUPPORTED;
  return ATTN_OK;
}

int check_fwd(int B, int Hq, int Hkv, int Nq, int Nk, int D, int causal, int window_lo,
              int pos0, float scale, int mode, int dtype) {
  int st = check_shape(B, Hq, Hkv, Nq, Nk, D, dtype);
  if (st != ATTN_OK) return st;
  if (window_lo < 0 || pos0 < 0) return ATTN_E_INVALID;
  if (!isfinite(scale) || !(scale > 0.0f)) return ATTN_E_INVALID;
  if (mode != ATTN_MODE_EXACT && mode != ATTN_MODE_QUANT && mode != ATTN_MODE_MX &&
      mode != ATTN_MODE_MXD)
    return ATTN_E_UNSUPPORTED;
  if (mode != ATTN_MODE_EXACT && dtype == ATTN_DT_F32) return ATTN_E_UNSUPPORTED;
  return ATTN_OK;
}

// The quantised-cache decode packs the G * Nq query rows of a key/value head
// into one 32-column MFMA block and launches one grid row per key/value head.
int check_kvq(int B, int Hq, int Hkv, int Nq, int Nk, int D, int window_lo, int pos0,
              float scale, int dtype) {
  int st = check_shape(B, Hq, Hkv, Nq, Nk, D, dtype);
  if (st != ATTN_OK) return st;
  if (dtype == ATTN_DT_F32) return ATTN_E_UNSUPPORTED;
  if (window_lo < 0 || pos0 < 0) return ATTN_E_INVALID;
  if (!isfinite(scale) || !(scale > 0.0f)) return ATTN_E_INVALID;
  if ((int64_t)(Hq / Hkv) * Nq > 32) return ATTN_E_UNSUPPORTED;
  if ((int64_t)B * Hkv > 65535) return ATTN_E_UNSUPPORTED;
  return ATTN_OK;
}

int elem_size(int dtype) { return dtype == ATTN_DT_F32 ? 4 : 2; }

FwdArgs make_args(const void* q, const void* k, const void* v, void* o, int B, int Hq,
                  int Hkv, int Nq, int Nk, int D, int causal, int window_lo, int pos0,
                  float scale) {
  FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nk = Nk; a.D = D;
  a.causal = causal ? 1 : 0; a.window_lo = window_lo; a.pos0 = pos0; a.window_w = 0;
  memset(&a.rope, 0, sizeof a.rope);   // no rotation unless attn_fwd_rope sets it
  a.scale = scale;
  // Kept a normal float so that masked scores (-inf) times c stay -inf.
  a.c = fmaxf(scale * kLog2eHost, 1.17549435e-38f);
  return a;
}

// Workspace layout of one call. Offsets are 256-byte aligned.
struct Layout {
  size_t bf16_q = 0, bf16_k = 0, bf16_v = 0;       // fp32 inputs rounded to bf16
  size_t qc = 0, qs = 0, kc = 0, ks = 0, vc = 0, vs = 0;  // quantised mode
  size_t v4c = 0, v4s = 0, part = 0;                // MXFP4 V, row partials (diagonal-tiled)
  size_t dec = 0;                                  // decode partials
  size_t rk = 0;                                   // rotated K (exact mode with RoPE)
  size_t spl = 0;                                  // split-prefill counters and partials
  size_t total = 0;
  bool decode = false;
  DecodePlan plan{};
  PrefillSplit split{};
};

// force_decode >= 0: the decode kernel with that split request (0 = the
// library's own plan), whatever the key count; -1: attn_fwd's dispatch.
// allow_split: the exact prefill may split small grids (needs workspace).
Layout plan_layout(const FwdArgs& a, int mode, int dtype, int force_decode = -1,
                   bool allow_split = true) {
  Layout L;
  size_t off = 0;
  const size_t nq = (size_t)a.B * a.Hq * a.Nq * a.D;
  const size_t nk = (size_t)a.B * a.Hkv * a.Nk * a.D;
  if (mode == ATTN_MODE_MX || mode == ATTN_MODE_MXD) {
    const size_t tiles = (size_t)(a.Nk + 63) / 64;
    L.qc = off; off = round_up(off + nq);
    L.qs = off; off = round_up(off + (size_t)a.B * a.Hq * ((a.Nq + 63) / 64) * 4);
    L.kc = off; off = round_up(off + nk);
    L.ks = off; off = round_up(off + (size_t)a.B * a.Hkv * tiles * 4);
    L.vc = off; off = round_up(off + (size_t)a.B * a.Hkv * tiles * 64 * a.D);
    L.vs = off; off = round_up(off + (size_t)a.B * a.Hkv * tiles * 2 * a.D);
    if (mode == ATTN_MODE_MXD) {
      L.v4c = off; off = round_up(off + (size_t)a.B * a.Hkv * tiles * 32 * a.D);
      L.v4s = off; off = round_up(off + (size_t)a.B * a.Hkv * tiles * 2 * a.D);
      L.part = off; off = round_up(off + (size_t)a.B * a.Hq * a.Nq * (a.D * 2 + 16));
    }
    L.total = off;
    return L;
  }
  if (mode == ATTN_MODE_QUANT) {
    const size_t tiles = (size_t)(a.Nk + 63) / 64;
    L.qc = off; off = round_up(off + nq);
    L.qs = off; off = round_up(off + (size_t)a.B * a.Hq * ((a.Nq + 63) / 64) * 4);
    L.kc = off; off = round_up(off + nk);
    L.ks = off; off = round_up(off + (size_t)a.B * a.Hkv * tiles * 4);
    L.vc = off; off = round_up(off + (size_t)a.B * a.Hkv * tiles * 64 * a.D);
    L.vs = off; off = round_up(off + (size_t)a.B * a.Hkv * tiles * 4);
    L.total = off;
    return L;
  }
  if (dtype == ATTN_DT_F32) {
    L.bf16_q = off; off = round_up(off + nq * 2);
    L.bf16_k = off; off = round_up(off + nk * 2);
    L.bf16_v = off; off = round_up(off + nk * 2);
  } else if (a.rope.on) {
    L.rk = off; off = round_up(off + nk * 2);   // fp32 inputs rotate their bf16 copy in place
  }
  if (force_decode >= 0 || decode_eligible(a)) {
    L.decode = true;
    L.plan = decode_plan(a, force_decode > 0 ? force_decode : 0);
    L.dec = off; off = round_up(off + L.plan.ws_bytes);
  } else if (allow_split) {
    L.split = prefill_split_plan(a, dtype == ATTN_DT_F32 ? 4 : 2);
    if (L.split.ns > 1 || L.split.halves > 0) {
      L.spl = off; off = round_up(off + L.split.ws_bytes);
    }
  }
  L.total = off;
  return L;
}

// Rotary frequencies of attn_rope (the published rules; double precision):
// plain theta_i = base^(-2i/D); NTK: base * s^(D/(D-2)); YaRN: theta_i blended
// between theta_i / s and theta_i by the ramp over L theta_i / (2 pi), logits
// times (0.1 ln s + 1)^2. Stored as revolutions per position, hi + lo floats.
int make_rope(const attn_rope* p, int D, RopeArgs* r, double* logit_mult) {
  r->on = 0;
  r->style = 0;
  *logit_mult = 1.0;
  if (!p) return ATTN_OK;
  if (p->style != ATTN_ROPE_HALF && p->style != ATTN_ROPE_INTERLEAVED) return ATTN_E_INVALID;
  if (p->scaling != ATTN_ROPE_PLAIN && p->scaling != ATTN_ROPE_NTK && p->scaling != ATTN_ROPE_YARN)
    return ATTN_E_INVALID;
  if (!isfinite(p->base) || !(p->base > 0.0f)) return ATTN_E_INVALID;
  if (p->scaling != ATTN_ROPE_PLAIN && (!isfinite(p->factor) || !(p->factor >= 1.0f)))
    return ATTN_E_INVALID;
  if (p->scaling == ATTN_ROPE_YARN &&
      (p->orig_ctx < 1 || !isfinite(p->beta_fast) || !isfinite(p->beta_slow) ||
       !(p->beta_fast > p->beta_slow)))
    return ATTN_E_INVALID;
  const double two_pi = 6.283185307179586476925286766559;
  const double s = p->factor;
  double b = p->base;
  if (p->scaling == ATTN_ROPE_NTK) b = p->base * pow(s, (double)D / (double)(D - 2));
  for (int i = 0; i < kRopeMaxPairs; ++i) {
    double theta = 0.0;
    if (i < D / 2) {
      theta = pow(b, -2.0 * i / (double)D);
      if (p->scaling == ATTN_ROPE_YARN) {
        const double ratio = (double)p->orig_ctx * theta / two_pi;   // context over wavelength
        double g = (ratio - p->beta_slow) / ((double)p->beta_fast - p->beta_slow);
        g = g < 0.0 ? 0.0 : (g > 1.0 ? 1.0 : g);
        theta = (1.0 - g) * theta / s + g * theta;
      }
    }
    const double rev = theta / two_pi;
    r->rev_hi[i] = (float)rev;
    r->rev_lo[i] = (float)(rev - (double)r->rev_hi[i]);
  }
  if (p->scaling == ATTN_ROPE_YARN) {
    const double m = 0.1 * log(s) + 1.0;
    *logit_mult = m * m;
  }
  r->on = 1;
  r->style = p->style;
  return ATTN_OK;
}

// One validated forward call: workspace check and kernel dispatch.
int fwd_dispatch(FwdArgs a, int mode, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream, int force_decode = -1) {
  const int B = a.B, Hq = a.Hq, Hkv = a.Hkv, Nq = a.Nq, Nk = a.Nk, D = a.D;
  const void *q = a.q, *k = a.k, *v = a.v;
  Layout L = plan_layout(a, mode, dtype, force_decode);
  // A workspace too small for the split prefill runs it unsplit.
  if ((L.split.ns > 1 || L.split.halves > 0) && workspace_bytes < L.total)
    L = plan_layout(a, mode, dtype, force_decode, false);
  if (L.total > 0) {
    if (workspace_bytes < L.total) return ATTN_E_WORKSPACE;
    if (!workspace || ((uintptr_t)workspace & (kAlign - 1)) != 0) return ATTN_E_INVALID;
  }
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  hipError_t e = hipSuccess;

  const RopeArgs* rope = a.rope.on ? &a.rope : nullptr;   // fused into the INT8 quantiser
  if (mode == ATTN_MODE_MX || mode == ATTN_MODE_MXD) {
    const int elem = dtype == ATTN_DT_BF16 ? 2 : 1;
    const bool dg = mode == ATTN_MODE_MXD;
    e = launch_quant_int8(q, elem, (int64_t)B * Hq, Nq, D, (int8_t*)(ws + L.qc),
                          (float*)(ws + L.qs), s, rope, a.pos0);
    if (e == hipSuccess)
      e = launch_quant_int8(k, elem, (int64_t)B * Hkv, Nk, D, (int8_t*)(ws + L.kc),
                            (float*)(ws + L.ks), s, rope, 0);
    if (e == hipSuccess)
      e = launch_quant_mx(v, elem, (int64_t)B * Hkv, Nk, D, 1, 1, 0, (uint8_t*)(ws + L.vc),
                          (uint8_t*)(ws + L.vs), s);
    if (e == hipSuccess && dg)
      e = launch_quant_mx(v, elem, (int64_t)B * Hkv, Nk, D, 1, 1, 0, (uint8_t*)(ws + L.v4c),
                          (uint8_t*)(ws + L.v4s), s, true);
    if (e == hipSuccess)
      e = launch_prefill_mx(a, (const int8_t*)(ws + L.qc), (const float*)(ws + L.qs),
                            (const int8_t*)(ws + L.kc), (const float*)(ws + L.ks),
                            (const uint8_t*)(ws + L.vc), (const uint8_t*)(ws + L.vs),
                            dg ? (const uint8_t*)(ws + L.v4c) : nullptr,
                            dg ? (const uint8_t*)(ws + L.v4s) : nullptr,
                            dg ? (float*)(ws + L.part) : nullptr, elem, s);
    return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
  }
  if (mode == ATTN_MODE_QUANT) {
    const int elem = dtype == ATTN_DT_BF16 ? 2 : 1;
    e = launch_quant_int8(q, elem, (int64_t)B * Hq, Nq, D, (int8_t*)(ws + L.qc),
                          (float*)(ws + L.qs), s, rope, a.pos0);
    if (e == hipSuccess)
      e = launch_quant_int8(k, elem, (int64_t)B * Hkv, Nk, D, (int8_t*)(ws + L.kc),
                            (float*)(ws + L.ks), s, rope, 0);
    if (e == hipSuccess)
      e = launch_quant_e4m3(v, elem, (int64_t)B * Hkv, Nk, D, (uint8_t*)(ws + L.vc),
                            (float*)(ws + L.vs), 1, s);
    if (e == hipSuccess)
      e = launch_prefill_quant(a, (const int8_t*)(ws + L.qc), (const float*)(ws + L.qs),
                               (const int8_t*)(ws + L.kc), (const float*)(ws + L.ks),
                               (const uint8_t*)(ws + L.vc), (const float*)(ws + L.vs), elem, s);
    return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
  }

  int elem = dtype == ATTN_DT_F16 ? 1 : 2;
  const bool out_f32 = dtype == ATTN_DT_F32;
  if (out_f32) {
    const int64_t nq = (int64_t)B * Hq * Nq * D, nk = (int64_t)B * Hkv * Nk * D;
    e = launch_f32_to_bf16((const float*)q, ws + L.bf16_q, nq, s);
    if (e == hipSuccess) e = launch_f32_to_bf16((const float*)k, ws + L.bf16_k, nk, s);
    if (e == hipSuccess) e = launch_f32_to_bf16((const float*)v, ws + L.bf16_v, nk, s);
    if (e != hipSuccess) return ATTN_E_HIP;
    a.q = ws + L.bf16_q;
    a.k = ws + L.bf16_k;
    a.v = ws + L.bf16_v;
  }
  if (a.rope.on) {
    // K turned once per call, in one pass (the kernels turn Q themselves)
    void* dst = out_f32 ? (void*)(ws + L.bf16_k) : (void*)(ws + L.rk);
    e = launch_rope(a.k, dst, elem, (int64_t)B * Hkv, Nk, D, 0, a.rope, s);
    if (e != hipSuccess) return ATTN_E_HIP;
    a.k = dst;
  }
  if (L.decode)
    e = launch_decode(a, L.plan, elem, out_f32, ws + L.dec, s);
  else
    e = launch_prefill(a, elem, out_f32, L.split,
                       L.split.ns > 1 || L.split.halves > 0 ? ws + L.spl : nullptr, s);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

}  // namespace

size_t fwd_min_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int D, int causal,
                               int window_lo, int pos0, int mode, int dtype) {
  if (check_fwd(B, Hq, Hkv, Nq, Nk, D, causal, window_lo, pos0, 1.0f, mode, dtype) != ATTN_OK)
    return 0;
  FwdArgs a = make_args(nullptr, nullptr, nullptr, nullptr, B, Hq, Hkv, Nq, Nk, D, causal,
                        window_lo, pos0, 1.0f);
  return plan_layout(a, mode, dtype, -1, false).total;
}

int fwd_validate(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv,
                 int Nq, int Nk, int D, int causal, int window_lo, int pos0, float scale, int mode,
                 int dtype) {
  const int st = check_fwd(B, Hq, Hkv, Nq, Nk, D, causal, window_lo, pos0, scale, mode, dtype);
  if (st != ATTN_OK) return st;
  if (!q || !k || !v || !o) return ATTN_E_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_E_INVALID;
  return ATTN_OK;
}

}  // namespace attn

using namespace attn;

extern "C" {

size_t attn_fwd_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int D, int causal,
                                int window_lo, int pos0, int mode, int dtype) {
  if (check_fwd(B, Hq, Hkv, Nq, Nk, D, causal, window_lo, pos0, 1.0f, mode, dtype) != ATTN_OK)
    return 0;
  FwdArgs a = make_args(nullptr, nullptr, nullptr, nullptr, B, Hq, Hkv, Nq, Nk, D, causal,
                        window_lo, pos0, 1.0f);
  return plan_layout(a, mode, dtype).total;
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv,
             int Nq, int Nk, int D, int causal, int window_lo, int pos0, float scale, int mode,
             int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = attn::fwd_validate(q, k, v, o, B, Hq, Hkv, Nq, Nk, D, causal, window_lo, pos0,
                                    scale, mode, dtype);
  if (st != ATTN_OK) return st;
  FwdArgs a = make_args(q, k, v, o, B, Hq, Hkv, Nq, Nk, D, causal, window_lo, pos0, scale);
  return fwd_dispatch(a, mode, dtype, workspace, workspace_bytes, stream);
}

size_t attn_fwd_rope_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int D, int causal,
                                     int window_lo, int pos0, int mode, int dtype) {
  if (check_fwd(B, Hq, Hkv, Nq, Nk, D, causal, window_lo, pos0, 1.0f, mode, dtype) != ATTN_OK)
    return 0;
  FwdArgs a = make_args(nullptr, nullptr, nullptr, nullptr, B, Hq, Hkv, Nq, Nk, D, causal,
                        window_lo, pos0, 1.0f);
  a.rope.on = 1;
  return plan_layout(a, mode, dtype).total;
}

int attn_fwd_rope(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv,
                  int Nq, int Nk, int D, int causal, int window_lo, int pos0, float scale,
                  int mode, int dtype, const attn_rope* rope, void* workspace,
                  size_t workspace_bytes, void* stream) {
  int st = check_fwd(B, Hq, Hkv, Nq, Nk, D, causal, window_lo, pos0, scale, mode, dtype);
  if (st != ATTN_OK) return st;
  if (!q || !k || !v || !o) return ATTN_E_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_E_INVALID;
  FwdArgs a = make_args(q, k, v, o, B, Hq, Hkv, Nq, Nk, D, causal, window_lo, pos0, scale);
  double mult = 1.0;
  st = make_rope(rope, D, &a.rope, &mult);
  if (st != ATTN_OK) return st;
  if (mult != 1.0) {
    a.scale = (float)(scale * mult);
    a.c = fmaxf(a.scale * kLog2eHost, 1.17549435e-38f);
  }
  return fwd_dispatch(a, mode, dtype, workspace, workspace_bytes, stream);
}

int attn_fwd_sliding(const void* q, const void* k, const void* v, void* o, int B, int Hq,
                     int Hkv, int Nq, int Nk, int D, int causal, int window, int pos0,
                     float scale, int mode, int dtype, void* workspace, size_t workspace_bytes,
                     void* stream) {
  int st = check_fwd(B, Hq, Hkv, Nq, Nk, D, causal, 0, pos0, scale, mode, dtype);
  if (st != ATTN_OK) return st;
  if (window < 1) return ATTN_E_INVALID;
  if (!q || !k || !v || !o) return ATTN_E_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_E_INVALID;
  FwdArgs a = make_args(q, k, v, o, B, Hq, Hkv, Nq, Nk, D, causal, 0, pos0, scale);
  a.window_w = window;
  return fwd_dispatch(a, mode, dtype, workspace, workspace_bytes, stream);
}

size_t attn_fwd_sliding_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int D,
                                        int causal, int window, int pos0, int mode, int dtype) {
  if (window < 1 || check_fwd(B, Hq, Hkv, Nq, Nk, D, causal, 0, pos0, 1.0f, mode, dtype) != ATTN_OK)
    return 0;
  FwdArgs a = make_args(nullptr, nullptr, nullptr, nullptr, B, Hq, Hkv, Nq, Nk, D, causal, 0,
                        pos0, 1.0f);
  a.window_w = window;
  return plan_layout(a, mode, dtype).total;
}

int attn_quantize_qk(const void* q, const void* k, int8_t* q_codes, float* q_scales,
                     int8_t* k_codes, float* k_scales, int B, int Hq, int Hkv, int Nq, int Nk,
                     int D, int dtype, void* stream) {
  int st = check_shape(B, Hq, Hkv, Nq, Nk, D, dtype);
  if (st != ATTN_OK) return st;
  if (dtype == ATTN_DT_F32) return ATTN_E_UNSUPPORTED;
  if (!q || !k || !q_codes || !q_scales || !k_codes || !k_scales) return ATTN_E_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_codes) || !aligned16(k_codes) ||
      ((uintptr_t)q_scales & 3u) || ((uintptr_t)k_scales & 3u))
    return ATTN_E_INVALID;
  const int elem = dtype == ATTN_DT_BF16 ? 2 : 1;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_quant_int8(q, elem, (int64_t)B * Hq, Nq, D, q_codes, q_scales, s);
  if (e == hipSuccess) e = launch_quant_int8(k, elem, (int64_t)B * Hkv, Nk, D, k_codes, k_scales, s);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

int attn_quantize_v(const void* v, uint8_t* v_codes, float* v_scales, int B, int Hkv, int Nk,
                    int D, int dtype, void* stream) {
  int st = check_shape(B, Hkv, Hkv, 1, Nk, D, dtype);
  if (st != ATTN_OK) return st;
  if (dtype == ATTN_DT_F32) return ATTN_E_UNSUPPORTED;
  if (!v || !v_codes || !v_scales) return ATTN_E_INVALID;
  if (!aligned16(v) || !aligned16(v_codes) || ((uintptr_t)v_scales & 3u)) return ATTN_E_INVALID;
  const int elem = dtype == ATTN_DT_BF16 ? 2 : 1;
  hipError_t e = launch_quant_e4m3(v, elem, (int64_t)B * Hkv, Nk, D, v_codes, v_scales, 0,
                                   (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

int attn_quantize_mx(const void* x, uint8_t* codes, uint8_t* scales, int B, int H, int N, int D,
                     int axis, int dtype, void* stream) {
  int st = check_shape(B, H, H, N, 1, D, dtype);
  if (st != ATTN_OK) return st;
  if (dtype == ATTN_DT_F32) return ATTN_E_UNSUPPORTED;
  if (axis != 0 && axis != 1) return ATTN_E_INVALID;
  if (!x || !codes || !scales) return ATTN_E_INVALID;
  if (!aligned16(x) || !aligned16(codes)) return ATTN_E_INVALID;
  const int elem = dtype == ATTN_DT_BF16 ? 2 : 1;
  const hipError_t e = launch_quant_mx(x, elem, (int64_t)B * H, N, D, axis, 0, N, codes, scales,
                                       (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

int attn_quantize_mx4(const void* x, uint8_t* codes, uint8_t* scales, int B, int H, int N, int D,
                      int axis, int dtype, void* stream) {
  int st = check_shape(B, H, H, N, 1, D, dtype);
  if (st != ATTN_OK) return st;
  if (dtype == ATTN_DT_F32) return ATTN_E_UNSUPPORTED;
  if (axis != 0 && axis != 1) return ATTN_E_INVALID;
  if (!x || !codes || !scales) return ATTN_E_INVALID;
  if (!aligned16(x) || !aligned16(codes)) return ATTN_E_INVALID;
  const int elem = dtype == ATTN_DT_BF16 ? 2 : 1;
  const hipError_t e = launch_quant_mx(x, elem, (int64_t)B * H, N, D, axis, 0, N, codes, scales,
                                       (hipStream_t)stream, true);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

size_t attn_decode_kvq_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int D,
                                       int causal, int window_lo, int pos0, int dtype) {
  if (check_kvq(B, Hq, Hkv, Nq, Nk, D, window_lo, pos0, 1.0f, dtype) != ATTN_OK) return 0;
  FwdArgs a = make_args(nullptr, nullptr, nullptr, nullptr, B, Hq, Hkv, Nq, Nk, D, causal,
                        window_lo, pos0, 1.0f);
  return round_up(decode_plan(a).ws_bytes);
}

int attn_decode_kvq(const void* q, const int8_t* k_codes, const float* k_scales,
                    const uint8_t* v_codes, const float* v_scales, void* o, int B, int Hq,
                    int Hkv, int Nq, int Nk, int D, int causal, int window_lo, int pos0,
                    float scale, int dtype, void* workspace, size_t workspace_bytes,
                    void* stream) {
  int st = check_kvq(B, Hq, Hkv, Nq, Nk, D, window_lo, pos0, scale, dtype);
  if (st != ATTN_OK) return st;
  if (!q || !k_codes || !k_scales || !v_codes || !v_scales || !o) return ATTN_E_INVALID;
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(o) ||
      ((uintptr_t)k_scales & 3u) || ((uintptr_t)v_scales & 3u))
    return ATTN_E_INVALID;
  FwdArgs a = make_args(q, nullptr, nullptr, o, B, Hq, Hkv, Nq, Nk, D, causal, window_lo,
                        pos0, scale);
  const DecodePlan plan = decode_plan(a);
  if (workspace_bytes < round_up(plan.ws_bytes)) return ATTN_E_WORKSPACE;
  if (!workspace || ((uintptr_t)workspace & (kAlign - 1)) != 0) return ATTN_E_INVALID;
  const int elem = dtype == ATTN_DT_BF16 ? 2 : 1;
  const hipError_t e = launch_decode_kvq(a, plan, k_codes, k_scales, v_codes, v_scales, elem,
                                         workspace, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

size_t attn_fwd_decode_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int D, int causal,
                                       int window_lo, int pos0, int dtype, int splits) {
  if (check_fwd(B, Hq, Hkv, Nq, Nk, D, causal, window_lo, pos0, 1.0f, ATTN_MODE_EXACT, dtype) !=
          ATTN_OK ||
      splits < 0)
    return 0;
  FwdArgs a = make_args(nullptr, nullptr, nullptr, nullptr, B, Hq, Hkv, Nq, Nk, D, causal,
                        window_lo, pos0, 1.0f);
  if (!decode_supported(a)) return 0;
  return plan_layout(a, ATTN_MODE_EXACT, dtype, splits).total;
}

int attn_fwd_decode(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv,
                    int Nq, int Nk, int D, int causal, int window_lo, int pos0, float scale,
                    int dtype, int splits, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_fwd(B, Hq, Hkv, Nq, Nk, D, causal, window_lo, pos0, scale, ATTN_MODE_EXACT, dtype);
  if (st != ATTN_OK) return st;
  if (splits < 0) return ATTN_E_INVALID;
  if (!q || !k || !v || !o) return ATTN_E_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_E_INVALID;
  FwdArgs a = make_args(q, k, v, o, B, Hq, Hkv, Nq, Nk, D, causal, window_lo, pos0, scale);
  if (!decode_supported(a)) return ATTN_E_UNSUPPORTED;
  return fwd_dispatch(a, ATTN_MODE_EXACT, dtype, workspace, workspace_bytes, stream, splits);
}

int attn_fwd_plan(int B, int Hq, int Hkv, int Nq, int Nk, int D, int causal, int window_lo,
                  int window, int pos0, int mode, int dtype, int rope, attn_plan* plan) {
  int st = check_fwd(B, Hq, Hkv, Nq, Nk, D, causal, window_lo, pos0, 1.0f, mode, dtype);
  if (st != ATTN_OK) return st;
  if (window < 0 || (window > 0 && window_lo != 0) || !plan) return ATTN_E_INVALID;
  FwdArgs a = make_args(nullptr, nullptr, nullptr, nullptr, B, Hq, Hkv, Nq, Nk, D, causal,
                        window_lo, pos0, 1.0f);
  a.window_w = window;
  a.rope.on = rope ? 1 : 0;
  const Layout L = plan_layout(a, mode, dtype);
  attn_plan p;
  p.workspace_bytes = L.total;
  p.splits = 1;
  if (mode == ATTN_MODE_QUANT || mode == ATTN_MODE_MX || mode == ATTN_MODE_MXD) {
    p.kernel = mode == ATTN_MODE_QUANT ? ATTN_KERNEL_PREFILL_QUANT
               : mode == ATTN_MODE_MX  ? ATTN_KERNEL_PREFILL_MX
                                       : ATTN_KERNEL_PREFILL_MXD;
    p.waves = 4;
    p.rows = 128;
    p.workgroups = (long long)B * Hq * ((Nq + 127) / 128);
    // INT8 Q, INT8 K (rotated there with RoPE), V codes (and MXFP4 V codes)
    p.pre_launches = mode == ATTN_MODE_MXD ? 4 : 3;
  } else if (L.decode) {
    p.kernel = ATTN_KERNEL_DECODE;
    p.waves = L.plan.waves;
    p.rows = L.plan.rows;
    p.splits = L.plan.nsplit;
    p.workgroups = (long long)L.plan.nsplit * B * Hkv;
    p.pre_launches = (dtype == ATTN_DT_F32 ? 3 : 0) + (rope ? 1 : 0);
  } else {
    p.kernel = ATTN_KERNEL_PREFILL;
    p.waves = prefill_waves(a);
    p.rows = 32 * p.waves;
    p.splits = L.split.halves > 0 ? 2 : L.split.ns;
    p.workgroups = (long long)B * Hq * ((Nq + p.rows - 1) / p.rows) * L.split.ns + L.split.halves;
    p.pre_launches = (dtype == ATTN_DT_F32 ? 3 : 0) + (rope ? 1 : 0);
  }
  *plan = p;
  return ATTN_OK;
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_E_INVALID: return "invalid argument (null or misaligned pointer, bad size, position, window or scale)";
    case ATTN_E_UNSUPPORTED: return "unsupported head dimension, dtype, mode or shape";
    case ATTN_E_WORKSPACE: return "workspace smaller than the matching *_workspace_bytes() result";
    case ATTN_E_HIP: return "the HIP runtime refused a kernel launch";
    case ATTN_E_TOO_LARGE: return "the call needs more scratch than the allocation-free entry point holds (ATTN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
