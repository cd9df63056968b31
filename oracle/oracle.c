/*
 * oracle.c — plain, slow, obviously-correct CPU reference for the fused
 * attention forward and its low-precision preparation.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
 * calls this file; only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg do. It shares no code, header, table or constant with the
 * HIP path.
 *
 * What it computes (each function cites the passage it follows):
 *
 *   oracle_attn         exact attention, O = softmax(scale * Q K^T + mask) V,
 *                       in double precision, one query row at a time, with the
 *                       score row materialised (no tiling, no online softmax).
 *                       The pages name this operation ("attention" of shape
 *                       1 x 40 heads x 32 760 tokens x 128 in the table of
 *                       section 1 of "Attention kernels on a home RTX 5080")
 *                       but never write its formula; the textbook definition
 *                       of scaled-dot-product attention is used.
 *   oracle_quant_int8   symmetric per-block INT8 codes for Q and K ("INT8 QK",
 *                       same table), one fp32 scale per 64-token block of one
 *                       head.
 *   oracle_quant_e4m3   per-block FP8 E4M3 codes for V ("FP8 PV", same table).
 *   oracle_e4m3_encode  / oracle_e4m3_decode: the OCP FP8 E4M3 ("E4M3FN")
 *                       format, written from its definition (sign, 4 exponent
 *                       bits biased by 7, 3 mantissa bits, subnormals, no
 *                       infinities, 0x7F/0xFF NaN).
 *   oracle_attn_quant   the quantised-mode emulation: exact attention on the
 *                       dequantised Q, K, V with every softmax weight passed
 *                       through E4M3 at the static scale 448 (a diagnostic).
 *   oracle_attn_kvq     exact attention over a quantised KV cache: K and V
 *                       given as per-block INT8 / E4M3 codes and scales, Q as
 *                       is or through its own per-block INT8 codes.
 *   oracle_quant_mx     OCP Microscaling (MX) FP8 blocks: 32 E4M3 elements
 *                       sharing one power-of-two (E8M0) scale, along D or N.
 *   oracle_attn_mx      exact attention on the MX variant's inputs: INT8
 *                       Q, K blocks and V in MX blocks along the keys.
 *   oracle_e2m1_encode  / oracle_e2m1_decode: OCP FP4 E2M1.
 *   oracle_quant_mx4    OCP MX FP4 blocks: 32 E2M1 elements, one E8M0 scale.
 *   oracle_attn_mxd     the diagonal-tiled mixed MX variant: INT8 Q, K; per
 *                       row, P and V in MXFP8 on diagonal key tiles and in
 *                       MXFP4 elsewhere, every weight rounded as the variant
 *                       rounds it.
 *   oracle_rope_freqs   rotary frequencies: plain, NTK-aware, YaRN.
 *   oracle_rope_apply   the rotation of Q or K rows at their positions.
 *   oracle_attn_rope    exact attention on rotated Q and K.
 *
 * Readings taken where the pages are silent (listed again in the design
 * notes): query row i sits at absolute position pos0 + i and key j at j; a
 * key is visible iff j >= window_lo and (not causal or j <= pos0 + i) and,
 * with a per-row window of width W, j >= pos0 + i - W + 1; the KV
 * head of query head h is h / (Hq / Hkv); a row with no visible key is all
 * zeros (the measured-results section of "round 21 track b — qsa2" zeroes
 * rows outside the active region); quantisation blocks are 64 consecutive tokens of one
 * head, the last block holding the remainder.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 *        -pthread oracle.c -o liboracle.so -lm
 * (no contraction: the fp32 quantiser arithmetic must round after every op).
 */
#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Element types of the raw inputs. */
enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };

/* ---------------------------------------------------------------- inputs -- */

/* IEEE binary16 -> double, from the format definition (exact). */
static double half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int m = h & 1023;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24);
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + m), e - 25);
  }
  return sign ? -v : v;
}

/* bfloat16 -> double: the upper half of an IEEE binary32 (exact). */
static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double load_elem(const void* base, int dtype, int64_t idx) {
  switch (dtype) {
    case OR_F32: return (double)((const float*)base)[idx];
    case OR_F16: return half_to_double(((const uint16_t*)base)[idx]);
    default:     return bf16_to_double(((const uint16_t*)base)[idx]);
  }
}

/* Same, but to float (exact for all three types). */
static float load_elem_f(const void* base, int dtype, int64_t idx) {
  return (float)load_elem(base, dtype, idx);
}

/* ------------------------------------------------------ exact attention -- */

typedef struct {
  const void *q, *k, *v;
  int dtype;
  int B, Hq, Hkv, Nq, Nk, D;
  int causal, window_lo, pos0;
  int window_w;          /* > 0: per-row window, key j >= pos0 + i - window_w + 1 */
  double scale;
  const int64_t* rows;   /* NULL: all rows in order */
  int64_t nrows;
  double* out;           /* nrows x D */
  double* lse;           /* nrows, may be NULL */
  double* weights;       /* nrows x Nk, may be NULL */
  /* quantised-mode emulation (NULL for exact attention) */
  const double* qhat;    /* dequantised inputs, same layouts as q/k/v */
  const double* khat;
  const double* vhat;
  int quant_p;           /* 1: pass each weight through E4M3 at scale 448 */
  const double* vhat4;   /* non-NULL: the diagonal-tiled MX emulation, V through
                            MXFP4 off the diagonal (vhat: MXFP8 on it) */
  int64_t next;          /* work counter */
  pthread_mutex_t mu;
} attn_job;

uint8_t oracle_e4m3_encode(float y);
float oracle_e4m3_decode(uint8_t code);
uint8_t oracle_e2m1_encode(float y);
float oracle_e2m1_decode(uint8_t code);
static void mxd_row(const attn_job* J, int i, int64_t kvoff, const double* s, double m, double* o);

/* Key j is visible to query row i. */
static int visible(const attn_job* J, int i, int j) {
  if (j < J->window_lo) return 0;
  if (J->window_w > 0 && (int64_t)j < (int64_t)J->pos0 + i - J->window_w + 1) return 0;
  if (J->causal && j > J->pos0 + i) return 0;
  return j < J->Nk;
}

static double q_at(const attn_job* J, int64_t idx) {
  return J->qhat ? J->qhat[idx] : load_elem(J->q, J->dtype, idx);
}
static double k_at(const attn_job* J, int64_t idx) {
  return J->khat ? J->khat[idx] : load_elem(J->k, J->dtype, idx);
}
static double v_at(const attn_job* J, int64_t idx) {
  return J->vhat ? J->vhat[idx] : load_elem(J->v, J->dtype, idx);
}

/* One query row, by the definition: scores, max, exp, sum, weighted sum. */
static void attn_one_row(const attn_job* J, int64_t slot, double* s) {
  int64_t r = J->rows ? J->rows[slot] : slot;
  int i = (int)(r % J->Nq);
  int64_t bh = r / J->Nq;
  int h = (int)(bh % J->Hq);
  int b = (int)(bh / J->Hq);
  int g = h / (J->Hq / J->Hkv);
  int D = J->D, Nk = J->Nk;
  int64_t qoff = r * D;
  int64_t kvoff = ((int64_t)b * J->Hkv + g) * Nk * D;
  double* o = J->out + slot * D;

  double m = -INFINITY;
  int any = 0;
  for (int j = 0; j < Nk; ++j) {
    if (!visible(J, i, j)) continue;
    double acc = 0.0;
    for (int d = 0; d < D; ++d)
      acc += q_at(J, qoff + d) * k_at(J, kvoff + (int64_t)j * D + d);
    s[j] = J->scale * acc;
    if (s[j] > m) m = s[j];
    any = 1;
  }
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  if (J->weights)
    for (int j = 0; j < Nk; ++j) J->weights[slot * Nk + j] = 0.0;
  if (!any) {
    if (J->lse) J->lse[slot] = -INFINITY;
    return;
  }
  if (J->vhat4) {
    mxd_row(J, i, kvoff, s, m, o);
    return;
  }
  double l = 0.0;
  for (int j = 0; j < Nk; ++j) {
    if (!visible(J, i, j)) continue;
    double p = exp(s[j] - m);
    l += p;
    double pv = p;
    if (J->quant_p) {
      float scaled = (float)(448.0 * p);
      pv = (double)oracle_e4m3_decode(oracle_e4m3_encode(scaled)) / 448.0;
    }
    for (int d = 0; d < D; ++d) o[d] += pv * v_at(J, kvoff + (int64_t)j * D + d);
    s[j] = p;
  }
  for (int d = 0; d < D; ++d) o[d] /= l;
  if (J->lse) J->lse[slot] = m + log(l);
  if (J->weights)
    for (int j = 0; j < Nk; ++j)
      if (visible(J, i, j)) J->weights[slot * Nk + j] = s[j] / l;
}

static void* attn_worker(void* arg) {
  attn_job* J = (attn_job*)arg;
  double* s = (double*)malloc(sizeof(double) * (size_t)(J->Nk > 0 ? J->Nk : 1));
  if (!s) return (void*)1;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int64_t slot = J->next;
    J->next += 16;
    pthread_mutex_unlock(&J->mu);
    if (slot >= J->nrows) break;
    int64_t end = slot + 16 < J->nrows ? slot + 16 : J->nrows;
    for (; slot < end; ++slot) attn_one_row(J, slot, s);
  }
  free(s);
  return NULL;
}

static int run_attn(attn_job* J, int nthreads) {
  /* a row list must name rows that exist */
  if (J->nrows < 0) return -1;
  if (J->rows) {
    const int64_t total = (int64_t)J->B * J->Hq * J->Nq;
    for (int64_t s = 0; s < J->nrows; ++s)
      if (J->rows[s] < 0 || J->rows[s] >= total) return -1;
  }
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  J->next = 0;
  pthread_mutex_init(&J->mu, NULL);
  int started = 0, rc = 0;
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&th[t], NULL, attn_worker, J) != 0) break;
    ++started;
  }
  if (attn_worker(J) != NULL) rc = -1;
  for (int t = 1; t <= started; ++t) {
    void* res = NULL;
    pthread_join(th[t], &res);
    if (res != NULL) rc = -1;
  }
  pthread_mutex_destroy(&J->mu);
  return rc;
}

static int check_shape(int B, int Hq, int Hkv, int Nq, int Nk, int D) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || D < 1) return -1;
  if (Hq % Hkv != 0) return -1;
  return 0;
}

/*
 * Exact attention in double precision.
 *   q: [B][Hq][Nq][D], k and v: [B][Hkv][Nk][D], all of element type dtype,
 *   row-major with D innermost (the "1 x 40 heads x 32 760 tokens x 128"
 *   order of the table in section 1 of "Attention kernels on a home RTX
 *   5080").
 *   window_w: 0, or a per-row sliding window: row i (position pos0 + i) also
 *   needs key j >= pos0 + i - window_w + 1 (the per-row reading of the
 *   "sliding-window lower bound" in the summary of "perf(metal): widen
 *   four-row flash KV tiles").
 *   rows: flat row indices r = (b*Hq + h)*Nq + i to evaluate, or NULL for all
 *   B*Hq*Nq rows in order; out receives nrows x D doubles.
 *   lse (nullable): m + ln(l) per row, -inf for a row with no visible key.
 *   weights (nullable): nrows x Nk softmax weights, 0 where masked.
 * Returns 0, or -1 on a bad shape.
 */
int oracle_attn(const void* q, const void* k, const void* v, int dtype,
                int B, int Hq, int Hkv, int Nq, int Nk, int D,
                int causal, int window_lo, int pos0, int window_w, double scale,
                const int64_t* rows, int64_t nrows,
                double* out, double* lse, double* weights, int nthreads) {
  if (check_shape(B, Hq, Hkv, Nq, Nk, D)) return -1;
  if (dtype < OR_F32 || dtype > OR_BF16) return -1;
  attn_job J;
  memset(&J, 0, sizeof J);
  J.q = q; J.k = k; J.v = v; J.dtype = dtype;
  J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.Nq = Nq; J.Nk = Nk; J.D = D;
  J.causal = causal; J.window_lo = window_lo; J.pos0 = pos0; J.scale = scale;
  J.window_w = window_w > 0 ? window_w : 0;
  J.rows = rows;
  J.nrows = rows ? nrows : (int64_t)B * Hq * Nq;
  J.out = out; J.lse = lse; J.weights = weights;
  return run_attn(&J, nthreads);
}

/* ------------------------------------------------------------ FP8 E4M3 -- */

/*
 * Decode an OCP FP8 E4M3 code: sign bit, exponent field e (bias 7), mantissa
 * field m. e = 0 holds the subnormals m * 2^-9; e = 15 with m = 7 is NaN (the
 * format has no infinities, so e = 15, m < 7 are ordinary values up to 448).
 */
float oracle_e4m3_decode(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 15;
  int m = code & 7;
  float v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexpf((float)m, -9);
  else        v = ldexpf((float)(8 + m), e - 10);
  return sign ? -v : v;
}

/*
 * Encode to E4M3 by brute force: the nearest of the 127 non-negative finite
 * magnitudes (codes 0x00..0x7E), ties to the code with an even mantissa field
 * (round-to-nearest-even); sign carried separately. Inputs beyond 448 in
 * magnitude saturate to 448 (callers clamp first; the quantiser never sees
 * them). NaN input gives 0x7F.
 */
uint8_t oracle_e4m3_encode(float y) {
  if (isnan(y)) return 0x7F;
  uint8_t sign = signbit(y) ? 0x80 : 0x00;
  double a = fabs((double)y);
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    double err = fabs((double)oracle_e4m3_decode((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(sign | best);
}

/* ---------------------------------------------------------- quantisers -- */

/*
 * Per-block symmetric INT8 codes ("INT8 QK" in the table of section 1 of
 * "Attention kernels on a home RTX 5080"; one scale per block of 64 tokens of
 * one head).
 *   x: [BH][N][D] of element type dtype; codes: same layout, int8;
 *   scales: [BH][ceil(N/64)] fp32.
 * Per block, in fp32 with round-to-nearest-even after every operation:
 *   amax = max |x|;  amax == 0 -> scale 0, all codes 0;
 *   otherwise scale = amax / 127, inv = 127 / amax,
 *             code = clamp(rint(x * inv), -127, 127).
 * Dequantisation is code * scale.
 */
int oracle_quant_int8(const void* x, int dtype, int64_t BH, int N, int D,
                      int8_t* codes, float* scales) {
  if (BH < 1 || N < 1 || D < 1) return -1;
  int nblk = (N + 63) / 64;
  for (int64_t bh = 0; bh < BH; ++bh) {
    for (int t = 0; t < nblk; ++t) {
      int r0 = 64 * t, r1 = r0 + 64 < N ? r0 + 64 : N;
      int64_t base = (bh * N + r0) * (int64_t)D;
      int64_t cnt = (int64_t)(r1 - r0) * D;
      float amax = 0.0f;
      for (int64_t e = 0; e < cnt; ++e) {
        float a = fabsf(load_elem_f(x, dtype, base + e));
        if (a > amax) amax = a;
      }
      if (amax == 0.0f) {
        scales[bh * nblk + t] = 0.0f;
        for (int64_t e = 0; e < cnt; ++e) codes[base + e] = 0;
        continue;
      }
      volatile float s = amax / 127.0f;
      volatile float inv = 127.0f / amax;
      scales[bh * nblk + t] = s;
      for (int64_t e = 0; e < cnt; ++e) {
        volatile float prod = load_elem_f(x, dtype, base + e) * inv;
        float r = rintf(prod);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        codes[base + e] = (int8_t)r;
      }
    }
  }
  return 0;
}

/*
 * Per-block FP8 E4M3 codes ("FP8 PV", same table): as the INT8 quantiser but
 * scale = amax / 448, inv = 448 / amax, y = clamp(x * inv, -448, 448),
 * code = E4M3(y) rounded to nearest even. amax == 0 gives scale 0, codes 0.
 */
int oracle_quant_e4m3(const void* x, int dtype, int64_t BH, int N, int D,
                      uint8_t* codes, float* scales) {
  if (BH < 1 || N < 1 || D < 1) return -1;
  int nblk = (N + 63) / 64;
  for (int64_t bh = 0; bh < BH; ++bh) {
    for (int t = 0; t < nblk; ++t) {
      int r0 = 64 * t, r1 = r0 + 64 < N ? r0 + 64 : N;
      int64_t base = (bh * N + r0) * (int64_t)D;
      int64_t cnt = (int64_t)(r1 - r0) * D;
      float amax = 0.0f;
      for (int64_t e = 0; e < cnt; ++e) {
        float a = fabsf(load_elem_f(x, dtype, base + e));
        if (a > amax) amax = a;
      }
      if (amax == 0.0f) {
        scales[bh * nblk + t] = 0.0f;
        for (int64_t e = 0; e < cnt; ++e) codes[base + e] = 0;
        continue;
      }
      volatile float s = amax / 448.0f;
      volatile float inv = 448.0f / amax;
      scales[bh * nblk + t] = s;
      for (int64_t e = 0; e < cnt; ++e) {
        volatile float y = load_elem_f(x, dtype, base + e) * inv;
        float yc = y;
        if (yc > 448.0f) yc = 448.0f;
        if (yc < -448.0f) yc = -448.0f;
        codes[base + e] = oracle_e4m3_encode(yc);
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------ MX FP8 blocks -- */

/*
 * OCP Microscaling (MX) FP8 blocks, the block-scaled format of the MX
 * variant (per-block-scaled FP8/FP4 in the table of section 1 of "Attention
 * kernels on a home RTX 5080"; MXFP formats in "Transformers Get a Turbo Boost
 * with Mixed-Precision Magic"). The pages name the format only; the
 * definition followed is the OCP Microscaling Formats specification (v1.0):
 * 32 elements share one scale 2^e stored as an E8M0 byte e + 127, and each
 * element is an FP8 E4M3 code.
 *   x: [BH][N][D] of element type dtype; codes: the same layout, uint8 E4M3.
 *   axis 0: a block is 32 consecutive channels of one token (D % 32 == 0);
 *           scales [BH][N][D / 32].
 *   axis 1: a block is 32 consecutive tokens of one channel, the last block
 *           holding N mod 32 tokens; scales [BH][ceil(N / 32)][D].
 * Per block: amax = max |x| (fp32). amax == 0 gives scale byte 0 and zero
 * codes. Otherwise e = floor(log2 amax) - 8, 8 being the exponent of the
 * largest power of two in E4M3 (256); e is clamped to [-127, 127]; code =
 * E4M3(clamp(x * 2^-e, -448, 448)) rounded to nearest even (the product is
 * exact in fp32). Elements of the block above 448 * 2^e saturate.
 */
static int mx_block_exp(float amax) {
  int ex;
  frexpf(amax, &ex);           /* amax = m * 2^ex, m in [0.5, 1) */
  int e = (ex - 1) - 8;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

int oracle_quant_mx(const void* x, int dtype, int64_t BH, int N, int D, int axis,
                    uint8_t* codes, uint8_t* scales) {
  if (BH < 1 || N < 1 || D < 1) return -1;
  if (axis == 0 && D % 32 != 0) return -1;
  if (axis != 0 && axis != 1) return -1;
  int nb = axis == 0 ? D / 32 : (N + 31) / 32;   /* blocks per token (axis 0) or per head (axis 1) */
  for (int64_t bh = 0; bh < BH; ++bh) {
    int outer = axis == 0 ? N : nb;              /* token, or token block */
    int inner = axis == 0 ? nb : D;              /* channel block, or channel */
    for (int o = 0; o < outer; ++o) {
      for (int in = 0; in < inner; ++in) {
        int64_t idx[32];
        int cnt = 0;
        for (int j = 0; j < 32; ++j) {
          int tok = axis == 0 ? o : 32 * o + j;
          int ch = axis == 0 ? 32 * in + j : in;
          if (tok >= N) break;
          idx[cnt++] = (bh * N + tok) * (int64_t)D + ch;
        }
        float amax = 0.0f;
        for (int j = 0; j < cnt; ++j) {
          float a = fabsf(load_elem_f(x, dtype, idx[j]));
          if (a > amax) amax = a;
        }
        int64_t sidx = (bh * outer + o) * (int64_t)inner + in;
        if (amax == 0.0f) {
          scales[sidx] = 0;
          for (int j = 0; j < cnt; ++j) codes[idx[j]] = 0;
          continue;
        }
        int e = mx_block_exp(amax);
        scales[sidx] = (uint8_t)(e + 127);
        for (int j = 0; j < cnt; ++j) {
          float y = ldexpf(load_elem_f(x, dtype, idx[j]), -e);
          if (y > 448.0f) y = 448.0f;
          if (y < -448.0f) y = -448.0f;
          codes[idx[j]] = oracle_e4m3_encode(y);
        }
      }
    }
  }
  return 0;
}

static int dequant_int8(const void* x, int dtype, int64_t BH, int N, int D, double* out);

/* MX dequantisation into doubles: code value * 2^(scale byte - 127). */
static int dequant_mx(const void* x, int dtype, int64_t BH, int N, int D, int axis, double* out) {
  int64_t n = BH * (int64_t)N * D;
  int64_t ns = axis == 0 ? BH * (int64_t)N * (D / 32) : BH * (int64_t)((N + 31) / 32) * D;
  uint8_t* c = (uint8_t*)malloc((size_t)n);
  uint8_t* s = (uint8_t*)malloc((size_t)ns);
  if (!c || !s || oracle_quant_mx(x, dtype, BH, N, D, axis, c, s) != 0) { free(c); free(s); return -1; }
  for (int64_t e = 0; e < n; ++e) {
    int64_t bh = e / ((int64_t)N * D);
    int tok = (int)((e / D) % N), ch = (int)(e % D);
    int64_t si = axis == 0 ? (bh * N + tok) * (int64_t)(D / 32) + ch / 32
                           : (bh * ((N + 31) / 32) + tok / 32) * (int64_t)D + ch;
    out[e] = ldexp((double)oracle_e4m3_decode(c[e]), (int)s[si] - 127);
  }
  free(c); free(s);
  return 0;
}

/*
 * Exact attention (arguments and conventions of oracle_attn, no per-row
 * window) on the inputs of the MX variant: Q and K through their per-64-token
 * INT8 blocks (oracle_quant_int8) and V through MX blocks of 32 keys
 * (oracle_quant_mx, axis 1). This is the MX variant's reference up to the
 * rounding of the softmax weights, which it leaves exact.
 */
int oracle_attn_mx(const void* q, const void* k, const void* v, int dtype,
                   int B, int Hq, int Hkv, int Nq, int Nk, int D,
                   int causal, int window_lo, int pos0, double scale,
                   const int64_t* rows, int64_t nrows, double* out, int nthreads) {
  if (check_shape(B, Hq, Hkv, Nq, Nk, D) || D % 32 != 0) return -1;
  if (dtype < OR_F32 || dtype > OR_BF16) return -1;
  int64_t nq = (int64_t)B * Hq * Nq * D, nk = (int64_t)B * Hkv * Nk * D;
  double* qh = (double*)malloc(sizeof(double) * (size_t)nq);
  double* kh = (double*)malloc(sizeof(double) * (size_t)nk);
  double* vh = (double*)malloc(sizeof(double) * (size_t)nk);
  int rc = -1;
  if (qh && kh && vh &&
      dequant_int8(q, dtype, (int64_t)B * Hq, Nq, D, qh) == 0 &&
      dequant_int8(k, dtype, (int64_t)B * Hkv, Nk, D, kh) == 0 &&
      dequant_mx(v, dtype, (int64_t)B * Hkv, Nk, D, 1, vh) == 0) {
    attn_job J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.dtype = dtype;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.Nq = Nq; J.Nk = Nk; J.D = D;
    J.causal = causal; J.window_lo = window_lo; J.pos0 = pos0; J.scale = scale;
    J.rows = rows;
    J.nrows = rows ? nrows : (int64_t)B * Hq * Nq;
    J.out = out;
    J.qhat = qh; J.khat = kh; J.vhat = vh;
    rc = run_attn(&J, nthreads);
  }
  free(qh); free(kh); free(vh);
  return rc;
}

/* ---------------------------------------------------- MX FP4 blocks -- */

/*
 * The diagonal-tiled mixed-precision MX variant ("Diagonal-Tiled
 * Mixed-Precision Attention" in "Transformers Get a Turbo Boost with
 * Mixed-Precision Magic", section "The DMA breakthrough": two low-bit MXFP
 * computations combined at the tiling level, the diagonal treated apart; the
 * FP4 rows of the table in section 1 of "Attention kernels on a home RTX
 * 5080"). The pages give no arithmetic; the element format is OCP FP4 E2M1
 * (OCP Microscaling Formats v1.0): 1 sign bit, 2 exponent bits biased by 1,
 * 1 mantissa bit, exponent field 0 subnormal; magnitudes 0, 0.5, 1, 1.5, 2,
 * 3, 4, 6; no infinities or NaN.
 */
float oracle_e2m1_decode(uint8_t code) {
  int sign = (code >> 3) & 1;
  int e = (code >> 1) & 3;
  int m = code & 1;
  float v = e == 0 ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
  return sign ? -v : v;
}

/*
 * Encode to E2M1 by brute force: the nearest of the 8 magnitudes (codes
 * 0..7), ties to the even code (round-to-nearest-even); magnitudes above 6
 * saturate to 6 (callers clamp first). The sign is bit 3. NaN gives 0.
 */
uint8_t oracle_e2m1_encode(float y) {
  if (isnan(y)) return 0;
  uint8_t sign = signbit(y) ? 0x8 : 0x0;
  double a = fabs((double)y);
  if (a > 6.0) a = 6.0;   /* infinities included */
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c <= 7; ++c) {
    double err = fabs((double)oracle_e2m1_decode((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(sign | best);
}

/*
 * OCP MX FP4 blocks: as oracle_quant_mx, with E2M1 elements. Per block:
 * amax == 0 gives scale byte 0 and zero codes; otherwise e = floor(log2 amax)
 * - 2 (2: the exponent of the largest power of two in E2M1, 4), clamped to
 * [-127, 127], and code = E2M1(clamp(x * 2^-e, -6, 6)) rounded to nearest
 * even. codes: one byte per element (the 4-bit code in bits 0..3), same
 * layout as x; scales as oracle_quant_mx.
 */
int oracle_quant_mx4(const void* x, int dtype, int64_t BH, int N, int D, int axis,
                     uint8_t* codes, uint8_t* scales) {
  if (BH < 1 || N < 1 || D < 1) return -1;
  if (axis == 0 && D % 32 != 0) return -1;
  if (axis != 0 && axis != 1) return -1;
  int nb = axis == 0 ? D / 32 : (N + 31) / 32;
  for (int64_t bh = 0; bh < BH; ++bh) {
    int outer = axis == 0 ? N : nb;
    int inner = axis == 0 ? nb : D;
    for (int o = 0; o < outer; ++o) {
      for (int in = 0; in < inner; ++in) {
        int64_t idx[32];
        int cnt = 0;
        for (int j = 0; j < 32; ++j) {
          int tok = axis == 0 ? o : 32 * o + j;
          int ch = axis == 0 ? 32 * in + j : in;
          if (tok >= N) break;
          idx[cnt++] = (bh * N + tok) * (int64_t)D + ch;
        }
        float amax = 0.0f;
        for (int j = 0; j < cnt; ++j) {
          float a = fabsf(load_elem_f(x, dtype, idx[j]));
          if (a > amax) amax = a;
        }
        int64_t sidx = (bh * outer + o) * (int64_t)inner + in;
        if (amax == 0.0f) {
          scales[sidx] = 0;
          for (int j = 0; j < cnt; ++j) codes[idx[j]] = 0;
          continue;
        }
        int ex;
        frexpf(amax, &ex);                 /* amax = m * 2^ex, m in [0.5, 1) */
        int e = (ex - 1) - 2;
        if (e < -127) e = -127;
        if (e > 127) e = 127;
        scales[sidx] = (uint8_t)(e + 127);
        for (int j = 0; j < cnt; ++j) {
          float y = ldexpf(load_elem_f(x, dtype, idx[j]), -e);
          if (y > 6.0f) y = 6.0f;
          if (y < -6.0f) y = -6.0f;
          codes[idx[j]] = oracle_e2m1_encode(y);
        }
      }
    }
  }
  return 0;
}

/* MX FP4 dequantisation into doubles, axis 1 (blocks of 32 tokens). */
static int dequant_mx4(const void* x, int dtype, int64_t BH, int N, int D, double* out) {
  int64_t n = BH * (int64_t)N * D;
  int64_t ns = BH * (int64_t)((N + 31) / 32) * D;
  uint8_t* c = (uint8_t*)malloc((size_t)n);
  uint8_t* s = (uint8_t*)malloc((size_t)ns);
  if (!c || !s || oracle_quant_mx4(x, dtype, BH, N, D, 1, c, s) != 0) { free(c); free(s); return -1; }
  for (int64_t e = 0; e < n; ++e) {
    int64_t bh = e / ((int64_t)N * D);
    int tok = (int)((e / D) % N), ch = (int)(e % D);
    int64_t si = (bh * ((N + 31) / 32) + tok / 32) * (int64_t)D + ch;
    out[e] = ldexp((double)oracle_e2m1_decode(c[e]), (int)s[si] - 127);
  }
  free(c); free(s);
  return 0;
}

/*
 * Key tile t (keys 64 t .. 64 t + 63) is on the diagonal of query row i when
 * it holds the position of one of the rows of i's 32-row block r = i / 32,
 * i.e. [64 t, 64 t + 63] meets [pos0 + 32 r, pos0 + 32 r + 31] (row i sits
 * at position pos0 + i).
 */
static int mxd_diagonal(int pos0, int i, int j) {
  int64_t r0 = (int64_t)pos0 + 32 * (int64_t)(i / 32);
  int64_t k0 = 64 * (int64_t)(j / 64);
  return k0 <= r0 + 31 && k0 + 63 >= r0;
}

/*
 * One row of the diagonal-tiled MX emulation, given its scores s (natural
 * units, visible keys only) and their maximum m. The weights of each block of
 * 32 consecutive keys (keys 32 b .. 32 b + 31) are one MX block of the row:
 * with x_b the block's largest score in log2 units (scale * log2 e * q.k),
 * its scale is 2^E, E = floor(x_b) - 7 on diagonal tiles (E4M3 elements, all
 * below 256, none saturated) and E = floor(x_b) - 2 elsewhere (E2M1, the OCP
 * rule: elements clamped to 6); each weight 2^(x_j - E) is rounded to the
 * element format. V is MXFP8 on diagonal tiles and MXFP4 elsewhere (blocks of
 * 32 keys of one channel). O = sum_j P^_j V^_j / sum_j P^_j. Every quantity is
 * taken relative to the integer floor(m log2 e), which changes no rounding.
 */
static void mxd_row(const attn_job* J, int i, int64_t kvoff, const double* s, double m, double* o) {
  const double L2E = 1.4426950408889634;
  int D = J->D, Nk = J->Nk;
  double M = floor(m * L2E);
  double l = 0.0;
  for (int b0 = 0; b0 < Nk; b0 += 32) {
    int b1 = b0 + 32 < Nk ? b0 + 32 : Nk;
    double xb = -INFINITY;
    for (int j = b0; j < b1; ++j)
      if (visible(J, i, j) && s[j] * L2E - M > xb) xb = s[j] * L2E - M;
    if (xb == -INFINITY) continue;
    int diag = mxd_diagonal(J->pos0, i, b0);   /* a 32-key block lies in one tile */
    double E = floor(xb) - (diag ? 7.0 : 2.0);
    for (int j = b0; j < b1; ++j) {
      if (!visible(J, i, j)) continue;
      double w = exp2(s[j] * L2E - M - E);
      double pq;
      if (diag) {
        pq = (double)oracle_e4m3_decode(oracle_e4m3_encode((float)w));
      } else {
        float y = w > 6.0 ? 6.0f : (float)w;
        pq = (double)oracle_e2m1_decode(oracle_e2m1_encode(y));
      }
      pq = ldexp(pq, (int)E);
      l += pq;
      const double* vh = diag ? J->vhat : J->vhat4;
      for (int d = 0; d < D; ++d) o[d] += pq * vh[kvoff + (int64_t)j * D + d];
    }
  }
  for (int d = 0; d < D; ++d) o[d] = l > 0.0 ? o[d] / l : 0.0;
}

/*
 * The diagonal-tiled MX variant's reference (arguments of oracle_attn_mx,
 * plus the per-row window): Q and K through their per-64-token INT8 blocks,
 * then per row the weights and V as mxd_row describes.
 */
int oracle_attn_mxd(const void* q, const void* k, const void* v, int dtype,
                    int B, int Hq, int Hkv, int Nq, int Nk, int D,
                    int causal, int window_lo, int pos0, int window_w, double scale,
                    const int64_t* rows, int64_t nrows, double* out, int nthreads) {
  if (check_shape(B, Hq, Hkv, Nq, Nk, D) || D % 32 != 0 || window_w < 0) return -1;
  if (dtype < OR_F32 || dtype > OR_BF16) return -1;
  int64_t nq = (int64_t)B * Hq * Nq * D, nk = (int64_t)B * Hkv * Nk * D;
  double* qh = (double*)malloc(sizeof(double) * (size_t)nq);
  double* kh = (double*)malloc(sizeof(double) * (size_t)nk);
  double* vh = (double*)malloc(sizeof(double) * (size_t)nk);
  double* vh4 = (double*)malloc(sizeof(double) * (size_t)nk);
  int rc = -1;
  if (qh && kh && vh && vh4 &&
      dequant_int8(q, dtype, (int64_t)B * Hq, Nq, D, qh) == 0 &&
      dequant_int8(k, dtype, (int64_t)B * Hkv, Nk, D, kh) == 0 &&
      dequant_mx(v, dtype, (int64_t)B * Hkv, Nk, D, 1, vh) == 0 &&
      dequant_mx4(v, dtype, (int64_t)B * Hkv, Nk, D, vh4) == 0) {
    attn_job J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.dtype = dtype;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.Nq = Nq; J.Nk = Nk; J.D = D;
    J.causal = causal; J.window_lo = window_lo; J.pos0 = pos0; J.window_w = window_w;
    J.scale = scale;
    J.rows = rows;
    J.nrows = rows ? nrows : (int64_t)B * Hq * Nq;
    J.out = out;
    J.qhat = qh; J.khat = kh; J.vhat = vh; J.vhat4 = vh4;
    rc = run_attn(&J, nthreads);
  }
  free(qh); free(kh); free(vh); free(vh4);
  return rc;
}

/* ------------------------------------------------------------------ RoPE -- */

/*
 * Rotary position embedding with NTK or YaRN scaling, which section "Plans"
 * of "Attention kernels on a home RTX 5080" proposes to apply inside the
 * kernel. The page gives no formulas; the published definitions are followed.
 *   plain  theta_i = base^(-2 i / D), i = 0 .. D/2 - 1 (RoFormer);
 *   NTK    the same with base * s^(D / (D - 2)) (NTK-aware scaling, factor s);
 *   YaRN   theta_i' = (1 - g_i) theta_i / s + g_i theta_i, with
 *          g_i = clamp((r_i - beta_slow) / (beta_fast - beta_slow), 0, 1) and
 *          r_i = L theta_i / (2 pi) (the original context L over the
 *          wavelength), and the logits multiplied by (0.1 ln s + 1)^2.
 * scaling: 0 plain, 1 NTK, 2 YaRN. theta: D/2 doubles; *logit_mult: 1 unless
 * YaRN.
 */
int oracle_rope_freqs(int D, int scaling, double base, double factor, int orig_ctx,
                      double beta_fast, double beta_slow, double* theta, double* logit_mult) {
  if (D < 2 || D % 2 != 0 || !(base > 0.0) || scaling < 0 || scaling > 2) return -1;
  if (scaling != 0 && !(factor >= 1.0)) return -1;
  if (scaling == 2 && (orig_ctx < 1 || !(beta_fast > beta_slow))) return -1;
  double b = base;
  if (scaling == 1) b = base * pow(factor, (double)D / (double)(D - 2));
  for (int i = 0; i < D / 2; ++i) {
    double t = pow(b, -2.0 * i / (double)D);
    if (scaling == 2) {
      double r = (double)orig_ctx * t / (2.0 * M_PI);
      double g = (r - beta_slow) / (beta_fast - beta_slow);
      if (g < 0.0) g = 0.0;
      if (g > 1.0) g = 1.0;
      t = (1.0 - g) * t / factor + g * t;
    }
    theta[i] = t;
  }
  *logit_mult = 1.0;
  if (scaling == 2) {
    double m = 0.1 * log(factor) + 1.0;
    *logit_mult = m * m;
  }
  return 0;
}

/*
 * Rotate rows of x ([BH][N][D], element type dtype) into out (doubles): row n
 * of every head sits at position pos_base + n; pair i is (x_i, x_{i + D/2})
 * for style 0 (half-split) or (x_{2i}, x_{2i+1}) for style 1 (interleaved),
 * (a, b) -> (a cos(p theta_i) - b sin(p theta_i), a sin(p theta_i) + b cos(p theta_i)).
 */
int oracle_rope_apply(const void* x, int dtype, int64_t BH, int N, int D, int pos_base, int style,
                      const double* theta, double* out) {
  if (BH < 1 || N < 1 || D < 2 || D % 2 != 0 || (style != 0 && style != 1)) return -1;
  for (int64_t bh = 0; bh < BH; ++bh)
    for (int n = 0; n < N; ++n) {
      int64_t base = (bh * N + n) * (int64_t)D;
      double pos = (double)pos_base + n;
      for (int i = 0; i < D / 2; ++i) {
        int ia = style == 0 ? i : 2 * i;
        int ib = style == 0 ? i + D / 2 : 2 * i + 1;
        double a = load_elem(x, dtype, base + ia), b = load_elem(x, dtype, base + ib);
        double c = cos(pos * theta[i]), s = sin(pos * theta[i]);
        out[base + ia] = a * c - b * s;
        out[base + ib] = a * s + b * c;
      }
    }
  return 0;
}

/*
 * Exact attention (arguments and conventions of oracle_attn, no per-row
 * window) on Q rotated at positions pos0 + i and K at positions j, with the
 * scale multiplied by the YaRN logit factor.
 */
int oracle_attn_rope(const void* q, const void* k, const void* v, int dtype,
                     int B, int Hq, int Hkv, int Nq, int Nk, int D,
                     int causal, int window_lo, int pos0, double scale,
                     int style, int scaling, double base, double factor, int orig_ctx,
                     double beta_fast, double beta_slow,
                     const int64_t* rows, int64_t nrows, double* out, int nthreads) {
  if (check_shape(B, Hq, Hkv, Nq, Nk, D)) return -1;
  if (dtype < OR_F32 || dtype > OR_BF16) return -1;
  double* theta = (double*)malloc(sizeof(double) * (size_t)(D / 2 > 0 ? D / 2 : 1));
  double mult = 1.0;
  if (!theta || oracle_rope_freqs(D, scaling, base, factor, orig_ctx, beta_fast, beta_slow,
                                  theta, &mult) != 0) {
    free(theta);
    return -1;
  }
  int64_t nq = (int64_t)B * Hq * Nq * D, nk = (int64_t)B * Hkv * Nk * D;
  double* qh = (double*)malloc(sizeof(double) * (size_t)nq);
  double* kh = (double*)malloc(sizeof(double) * (size_t)nk);
  int rc = -1;
  if (qh && kh &&
      oracle_rope_apply(q, dtype, (int64_t)B * Hq, Nq, D, pos0, style, theta, qh) == 0 &&
      oracle_rope_apply(k, dtype, (int64_t)B * Hkv, Nk, D, 0, style, theta, kh) == 0) {
    attn_job J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.dtype = dtype;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.Nq = Nq; J.Nk = Nk; J.D = D;
    J.causal = causal; J.window_lo = window_lo; J.pos0 = pos0; J.scale = scale * mult;
    J.rows = rows;
    J.nrows = rows ? nrows : (int64_t)B * Hq * Nq;
    J.out = out;
    J.qhat = qh; J.khat = kh;
    rc = run_attn(&J, nthreads);
  }
  free(theta); free(qh); free(kh);
  return rc;
}

/* -------------------------------------------- quantised-mode emulation -- */

static int dequant_int8(const void* x, int dtype, int64_t BH, int N, int D, double* out) {
  int64_t n = BH * (int64_t)N * D;
  int nblk = (N + 63) / 64;
  int8_t* c = (int8_t*)malloc((size_t)n);
  float* s = (float*)malloc(sizeof(float) * (size_t)(BH * nblk));
  if (!c || !s) { free(c); free(s); return -1; }
  oracle_quant_int8(x, dtype, BH, N, D, c, s);
  for (int64_t e = 0; e < n; ++e) {
    int64_t bh = e / ((int64_t)N * D);
    int tok = (int)((e / D) % N);
    out[e] = (double)c[e] * (double)s[bh * nblk + tok / 64];
  }
  free(c); free(s);
  return 0;
}

static int dequant_e4m3(const void* x, int dtype, int64_t BH, int N, int D, double* out) {
  int64_t n = BH * (int64_t)N * D;
  int nblk = (N + 63) / 64;
  uint8_t* c = (uint8_t*)malloc((size_t)n);
  float* s = (float*)malloc(sizeof(float) * (size_t)(BH * nblk));
  if (!c || !s) { free(c); free(s); return -1; }
  oracle_quant_e4m3(x, dtype, BH, N, D, c, s);
  for (int64_t e = 0; e < n; ++e) {
    int64_t bh = e / ((int64_t)N * D);
    int tok = (int)((e / D) % N);
    out[e] = (double)oracle_e4m3_decode(c[e]) * (double)s[bh * nblk + tok / 64];
  }
  free(c); free(s);
  return 0;
}

/*
 * Quantised-mode emulation, a diagnostic for the INT8-QK / FP8-PV recipe of
 * the table in section 1 of "Attention kernels on a home RTX 5080": exact
 * attention (same arguments as oracle_attn) on Q^, K^ (INT8 blocks) and V^
 * (E4M3 blocks), where every softmax weight p_j = exp(s_j - m) of the final
 * row max m is replaced by E4M3(fp32(448 p_j)) / 448 in the weighted sum of V
 * while the denominator keeps the unquantised sum of p_j.
 */
int oracle_attn_quant(const void* q, const void* k, const void* v, int dtype,
                      int B, int Hq, int Hkv, int Nq, int Nk, int D,
                      int causal, int window_lo, int pos0, double scale,
                      const int64_t* rows, int64_t nrows,
                      double* out, int nthreads) {
  if (check_shape(B, Hq, Hkv, Nq, Nk, D)) return -1;
  if (dtype < OR_F32 || dtype > OR_BF16) return -1;
  int64_t nq = (int64_t)B * Hq * Nq * D, nk = (int64_t)B * Hkv * Nk * D;
  double* qh = (double*)malloc(sizeof(double) * (size_t)nq);
  double* kh = (double*)malloc(sizeof(double) * (size_t)nk);
  double* vh = (double*)malloc(sizeof(double) * (size_t)nk);
  int rc = -1;
  if (qh && kh && vh &&
      dequant_int8(q, dtype, (int64_t)B * Hq, Nq, D, qh) == 0 &&
      dequant_int8(k, dtype, (int64_t)B * Hkv, Nk, D, kh) == 0 &&
      dequant_e4m3(v, dtype, (int64_t)B * Hkv, Nk, D, vh) == 0) {
    attn_job J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.dtype = dtype;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.Nq = Nq; J.Nk = Nk; J.D = D;
    J.causal = causal; J.window_lo = window_lo; J.pos0 = pos0; J.scale = scale;
    J.rows = rows;
    J.nrows = rows ? nrows : (int64_t)B * Hq * Nq;
    J.out = out;
    J.qhat = qh; J.khat = kh; J.vhat = vh; J.quant_p = 1;
    rc = run_attn(&J, nthreads);
  }
  free(qh); free(kh); free(vh);
  return rc;
}

/*
 * Attention over a quantised KV cache: the INT8-QK / FP8-PV recipe of the
 * table in section 1 of "Attention kernels on a home RTX 5080" with K and V
 * stored as codes. Key j of key/value head (b, g) is
 *   K[j][d] = kc[j][d] * ks[b][g][j / 64],  V[j][d] = E4M3(vc[j][d]) * vs[b][g][j / 64]
 * (codes [B][Hkv][Nk][D], scales [B][Hkv][ceil(Nk/64)] fp32). The result is
 * exact attention (arguments and conventions of oracle_attn) on these K, V
 * and on Q as given (quant_q = 0) or on the dequantisation of Q's per-block
 * INT8 codes (quant_q = 1, oracle_quant_int8's recipe).
 */
int oracle_attn_kvq(const void* q, int dtype, const int8_t* kc, const float* ks,
                    const uint8_t* vc, const float* vs,
                    int B, int Hq, int Hkv, int Nq, int Nk, int D,
                    int causal, int window_lo, int pos0, double scale, int quant_q,
                    const int64_t* rows, int64_t nrows, double* out, int nthreads) {
  if (check_shape(B, Hq, Hkv, Nq, Nk, D)) return -1;
  if (dtype < OR_F32 || dtype > OR_BF16) return -1;
  int64_t nq = (int64_t)B * Hq * Nq * D, nk = (int64_t)B * Hkv * Nk * D;
  int nblk = (Nk + 63) / 64;
  double* qh = quant_q ? (double*)malloc(sizeof(double) * (size_t)nq) : NULL;
  double* kh = (double*)malloc(sizeof(double) * (size_t)nk);
  double* vh = (double*)malloc(sizeof(double) * (size_t)nk);
  int rc = -1;
  if (kh && vh && (!quant_q || qh) &&
      (!quant_q || dequant_int8(q, dtype, (int64_t)B * Hq, Nq, D, qh) == 0)) {
    for (int64_t e = 0; e < nk; ++e) {
      int64_t bg = e / ((int64_t)Nk * D);
      int tok = (int)((e / D) % Nk);
      kh[e] = (double)kc[e] * (double)ks[bg * nblk + tok / 64];
      vh[e] = (double)oracle_e4m3_decode(vc[e]) * (double)vs[bg * nblk + tok / 64];
    }
    attn_job J;
    memset(&J, 0, sizeof J);
    J.q = q; J.dtype = dtype;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.Nq = Nq; J.Nk = Nk; J.D = D;
    J.causal = causal; J.window_lo = window_lo; J.pos0 = pos0; J.scale = scale;
    J.rows = rows;
    J.nrows = rows ? nrows : (int64_t)B * Hq * Nq;
    J.out = out;
    J.qhat = qh; J.khat = kh; J.vhat = vh;
    rc = run_attn(&J, nthreads);
  }
  free(qh); free(kh); free(vh);
  return rc;
}
