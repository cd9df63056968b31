/*
 * attn.h — C ABI of the MI355X (gfx950) fused attention forward library.
 *
 * The operation is scaled-dot-product attention, O = softmax(scale * Q K^T +
 * mask) V, computed flash-style: K and V are streamed through on-chip memory
 * in tiles with a running maximum and running sum, and the Nq x Nk score
 * matrix is never stored. The pages that describe this path name it
 * ("attention" of shape 1 x 40 heads x 32 760 tokens x 128, bf16, in the
 * table of section 1 of "Attention kernels on a home RTX 5080") but do not
 * write its formula; the textbook definition is used.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller. The library
 *   never allocates, frees or synchronises; kernels are enqueued on `stream`
 *   (a hipStream_t; NULL = the default stream) and the call returns once they
 *   are enqueued.
 * - Layouts are row-major with D innermost (the "1 x 40 heads x 32 760 tokens
 *   x 128" order of that table): Q and O are [B][Hq][Nq][D], K and V are
 *   [B][Hkv][Nk][D], all contiguous. O has Q's element type.
 * - Tensor pointers must be 16-byte aligned; `workspace` 256-byte aligned.
 * - Every argument check runs before anything is enqueued: a call that
 *   returns an error has written nothing.
 * - Index arithmetic is 64-bit; each single dimension must fit in int.
 * - Calls are re-entrant; overlapping calls on different streams must use
 *   different workspaces.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
typedef enum {
  ATTN_OK = 0,
  ATTN_E_INVALID = -1,     /* null/misaligned pointer, bad size, bad scale  */
  ATTN_E_UNSUPPORTED = -2, /* head dim, dtype, mode or shape not supported  */
  ATTN_E_WORKSPACE = -3,   /* workspace below the matching *_workspace_bytes */
  ATTN_E_HIP = -4,         /* the HIP runtime refused a launch              */
  ATTN_E_TOO_LARGE = -5    /* the call needs more scratch than
                              attn_fwd_noalloc holds                         */
} attn_status;

/* Element types of Q, K, V and O. */
typedef enum { ATTN_DT_F32 = 0, ATTN_DT_F16 = 1, ATTN_DT_BF16 = 2 } attn_dtype;

/* Arithmetic mode. The default keeps full 16-bit operands; the quantised
 * mode is opt-in, as the explicit fast-precision policy of "Shmoosh update"
 * (section "An explicit fast-mode policy") keeps its high-fidelity default. */
typedef enum {
  ATTN_MODE_EXACT = 0, /* bf16/f16 matrix products, fp32 accumulation and
                          softmax; fp32 inputs are rounded to bf16 first */
  ATTN_MODE_QUANT = 1, /* INT8 Q K^T and FP8 (E4M3) P V with per-block
                          scales ("SageAttention 2 INT8 QK . FP8 PV" row of
                          the table in section 1 of "Attention kernels on a
                          home RTX 5080"); bf16/f16 inputs only */
  ATTN_MODE_MX = 2,    /* INT8 Q K^T as in ATTN_MODE_QUANT, and P V in OCP
                          MX FP8 blocks: V in blocks of 32 keys of each
                          channel (attn_quantize_mx, axis 1), the softmax
                          weights in blocks of 32 keys of each row, both E8M0
                          block scales applied by the scaled FP8 matrix cores
                          (the per-block-scaled low-precision kernels of that
                          table, MXFP as in "Transformers Get a Turbo Boost
                          with Mixed-Precision Magic"); bf16/f16 inputs only */
  ATTN_MODE_MXD = 3    /* the diagonal-tiled mixed MX variant ("Diagonal-
                          Tiled Mixed-Precision Attention", section "The DMA
                          breakthrough" of "Transformers Get a Turbo Boost
                          with Mixed-Precision Magic"; FP4 with per-block
                          scales in the table of section 1 of "Attention
                          kernels on a home RTX 5080"). INT8 Q K^T as above.
                          The map is tiled into 32-row blocks (rows 32 r ..
                          32 r + 31) and 64-key tiles; a tile holding the
                          position of one of its block's rows (key tile t
                          meets [pos0 + 32 r, pos0 + 32 r + 31]) is diagonal
                          and runs P V as ATTN_MODE_MX (MXFP8); every other
                          tile runs it in OCP MXFP4 (E2M1 elements): V in
                          blocks of 32 keys of each channel (attn_quantize_
                          mx4, axis 1), the weights of each 32-key block of a
                          row with scale 2^E, E = floor(log2 block max) - 2,
                          clamped to 6 and rounded to nearest even, on the
                          FP4 matrix cores at about twice the FP8 rate. Far
                          less precise (about 18 % relative error against
                          exact attention on normal inputs); bf16/f16 only */
} attn_mode;

/*
 * attn_fwd — one attention forward.
 *
 *   q, k, v, o   device tensors in the layouts above, element type `dtype`.
 *   B, Hq, Hkv   batch, query heads, key/value heads; Hq % Hkv == 0 and query
 *                head h reads key/value head h / (Hq / Hkv) (grouped-query
 *                attention, e.g. n_head=16 over n_kv=8 in the "Performance
 *                evidence" of "perf(metal): widen four-row flash KV tiles").
 *   Nq, Nk       query rows and keys per head (>= 1).
 *   D            head dimension: 64 or 128.
 *   causal       nonzero: query row i sits at absolute position pos0 + i and
 *                sees key j only if j <= pos0 + i (bottom-right aligned when
 *                pos0 = Nk - Nq, as in the rows=4, kv_len=4096, pos=4092
 *                decode of that page).
 *   window_lo    inclusive lower bound of visible keys for every row, with or
 *                without causal (the "sliding-window lower bound" of that
 *                page's summary); 0 = no window.
 *   pos0         position of query row 0 (>= 0); used only when causal.
 *   scale        multiplier of Q K^T, finite and > 0 (usually 1/sqrt(D)).
 *   mode         attn_mode.
 *   dtype        attn_dtype of q, k, v and o.
 *   workspace    device scratch of at least attn_fwd_workspace_bytes(...)
 *                bytes (may be NULL when that is 0); contents need no
 *                initialisation and are clobbered. 256-byte aligned.
 *                In the exact mode, a prefill whose grid fills the GPU
 *                less than once splits key ranges over several workgroups
 *                and merges their partials (at most 128 query tiles: each
 *                tile's keys over 2-4 workgroups; up to one round of
 *                workgroups, e.g. 2 x 10 heads x 4096 rows at head dim 64:
 *                enough tiles in two halves that every CU gets the same
 *                work, merged by a second launch); the workspace holds the
 *                partials. Given less than attn_fwd_workspace_bytes
 *                but at least what the unsplit schedule needs (0 for
 *                bf16/f16 inputs), the call runs unsplit: the same result
 *                up to rounding. The low-precision modes hold their codes
 *                and scales there; ATTN_MODE_MXD also V's MXFP4 codes and
 *                one partial row per query row (D 16-bit values and 4
 *                floats) that its second launch merges.
 *   stream       hipStream_t to enqueue on.
 *
 * A row with no visible key (window_lo > pos0 + i) is written as exact zeros.
 * Returns ATTN_OK or a negative attn_status; nothing is enqueued on error.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o,
             int B, int Hq, int Hkv, int Nq, int Nk, int D,
             int causal, int window_lo, int pos0, float scale, int mode,
             int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_fwd_workspace_bytes — workspace attn_fwd needs for these arguments
 * (same meaning as above), the split prefill's partials included.
 * Host-only; never touches the GPU. Returns 0 for arguments attn_fwd would
 * reject.
 */
size_t attn_fwd_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int D,
                                int causal, int window_lo, int pos0,
                                int mode, int dtype);

/*
 * Rotary position embedding (RoPE) of Q and K inside the kernel, with NTK or
 * YaRN scaling, as section "Plans" of "Attention kernels on a home RTX 5080"
 * proposes (the page gives no formulas; the published ones are used).
 * Query row i sits at position pos0 + i, key j at position j. Pair i of a row
 * (i = 0 .. D/2 - 1) turns by the angle position * theta_i:
 *   (a, b) -> (a cos - b sin, a sin + b cos).
 */
typedef enum {
  ATTN_ROPE_HALF = 0,        /* pairs (x_i, x_{i + D/2}) */
  ATTN_ROPE_INTERLEAVED = 1  /* pairs (x_{2i}, x_{2i+1}) */
} attn_rope_style;

typedef enum {
  ATTN_ROPE_PLAIN = 0,  /* theta_i = base^(-2i/D) */
  ATTN_ROPE_NTK = 1,    /* the same with base * factor^(D / (D - 2)) */
  ATTN_ROPE_YARN = 2    /* theta_i' = (1 - g_i) theta_i / factor + g_i theta_i with
                           g_i = clamp((r_i - beta_slow) / (beta_fast - beta_slow), 0, 1),
                           r_i = orig_ctx * theta_i / (2 pi); logits (scale) multiplied
                           by (0.1 ln factor + 1)^2 */
} attn_rope_scaling;

typedef struct {
  int style;        /* attn_rope_style */
  int scaling;      /* attn_rope_scaling */
  float base;       /* finite, > 0 (e.g. 10000) */
  float factor;     /* finite, >= 1 (NTK, YaRN) */
  int orig_ctx;     /* >= 1 (YaRN): the context the frequencies were trained on */
  float beta_fast;  /* YaRN ramp: beta_fast > beta_slow (e.g. 32 and 1) */
  float beta_slow;
} attn_rope;

/*
 * attn_fwd_rope — attn_fwd on rotary-embedded Q and K: the result is
 * attention on RoPE(Q) and RoPE(K) (same arguments, layouts, modes and error
 * behaviour as attn_fwd; `rope` NULL gives attn_fwd itself; invalid rope
 * fields give ATTN_E_INVALID). The kernels turn Q in registers as they load
 * it (once per workgroup); K is turned once per call: inside the INT8
 * quantiser in the quantised and MX modes, by one pass into the workspace in
 * the exact mode (a kernel that turned K on every load would redo it for
 * every query tile).
 *   workspace  at least attn_fwd_rope_workspace_bytes(...) bytes.
 */
int attn_fwd_rope(const void* q, const void* k, const void* v, void* o,
                  int B, int Hq, int Hkv, int Nq, int Nk, int D,
                  int causal, int window_lo, int pos0, float scale, int mode, int dtype,
                  const attn_rope* rope, void* workspace, size_t workspace_bytes,
                  void* stream);

/* Workspace attn_fwd_rope needs (host-only; 0 for rejected arguments). */
size_t attn_fwd_rope_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int D,
                                     int causal, int window_lo, int pos0, int mode,
                                     int dtype);

/*
 * attn_fwd_sliding — attn_fwd with a per-row sliding window instead of the
 * shared lower bound: query row i (absolute position pos0 + i) sees key j
 * only if j >= pos0 + i - window + 1, and, when causal, j <= pos0 + i; so a
 * causal row sees at most `window` keys, the newest ones. This is the other
 * reading of the "sliding-window lower bound" in the summary of "perf(metal):
 * widen four-row flash KV tiles" (there a single bound; here one per row, as
 * local attention uses it).
 *
 *   window     width W >= 1 (ATTN_E_INVALID otherwise).
 *   workspace  at least attn_fwd_sliding_workspace_bytes(...) bytes.
 *   Every other argument, the modes, layouts and the error behaviour are
 *   those of attn_fwd (window_lo is 0 here). Rows with no visible key are
 *   written as zeros.
 */
int attn_fwd_sliding(const void* q, const void* k, const void* v, void* o,
                     int B, int Hq, int Hkv, int Nq, int Nk, int D,
                     int causal, int window, int pos0, float scale, int mode,
                     int dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace attn_fwd_sliding needs (host-only; 0 for rejected arguments). */
size_t attn_fwd_sliding_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int D,
                                        int causal, int window, int pos0, int mode,
                                        int dtype);

/*
 * attn_quantize_qk — per-block symmetric INT8 codes of Q and K (the "INT8 QK"
 * half of the quantised mode).
 *
 * A block is 64 consecutive tokens of one (batch, head) across all D
 * channels; the last block of a head holds the remaining N % 64 tokens. Per
 * block, in fp32 with round-to-nearest-even after every operation:
 *   amax = max |x|; amax == 0 gives scale 0 and all-zero codes; otherwise
 *   scale = amax / 127, inv = 127 / amax, code = clamp(rint(x * inv), -127, 127).
 * Dequantisation is code * scale.
 *
 *   q, k          device inputs [B][Hq][Nq][D] and [B][Hkv][Nk][D], bf16/f16.
 *   q_codes       device int8 [B][Hq][Nq][D]; k_codes [B][Hkv][Nk][D].
 *   q_scales      device fp32 [B][Hq][ceil(Nq/64)]; k_scales [B][Hkv][ceil(Nk/64)].
 * Codes and scales are bit-exact with the CPU oracle's definition.
 */
int attn_quantize_qk(const void* q, const void* k, int8_t* q_codes, float* q_scales,
                     int8_t* k_codes, float* k_scales,
                     int B, int Hq, int Hkv, int Nq, int Nk, int D, int dtype,
                     void* stream);

/*
 * attn_quantize_v — per-block FP8 codes of V (the "FP8 PV" half). Blocks as
 * above; scale = amax / 448, inv = 448 / amax, y = clamp(x * inv, -448, 448),
 * code = OCP FP8 E4M3 of y rounded to nearest even (sign kept, subnormals
 * kept, 448 = 0x7E the largest magnitude). amax == 0 gives scale 0, codes 0.
 *
 *   v          device input [B][Hkv][Nk][D], bf16/f16.
 *   v_codes    device uint8 [B][Hkv][Nk][D].
 *   v_scales   device fp32 [B][Hkv][ceil(Nk/64)].
 */
int attn_quantize_v(const void* v, uint8_t* v_codes, float* v_scales,
                    int B, int Hkv, int Nk, int D, int dtype, void* stream);

/*
 * attn_quantize_mx — OCP Microscaling (MX) FP8 blocks of the MX mode: 32
 * elements share one power-of-two scale 2^e, stored as an E8M0 byte e + 127,
 * and each element is an OCP FP8 E4M3 code. Per block, in fp32: amax = max
 * |x|; amax == 0 gives scale byte 0 and zero codes; otherwise e = floor(log2
 * amax) - 8 clamped to [-127, 127] and code = E4M3(clamp(x * 2^-e, -448,
 * 448)) rounded to nearest even (elements above 448 * 2^e saturate).
 *
 *   x        device [B][H][N][D], bf16/f16 (`dtype`); D = 64 or 128.
 *   codes    device uint8 [B][H][N][D].
 *   scales   device uint8: axis 0 (blocks of 32 consecutive channels of one
 *            token) [B][H][N][D/32]; axis 1 (blocks of 32 consecutive tokens
 *            of one channel, the last holding N mod 32) [B][H][ceil(N/32)][D].
 * Codes and scales are bit-exact with the CPU oracle's definition.
 */
int attn_quantize_mx(const void* x, uint8_t* codes, uint8_t* scales, int B, int H, int N,
                     int D, int axis, int dtype, void* stream);

/*
 * attn_quantize_mx4 — OCP Microscaling (MX) FP4 blocks of ATTN_MODE_MXD's
 * off-diagonal tiles (OCP Microscaling Formats v1.0; the pages name FP4 and
 * MXFP without a format): 32 elements share one scale 2^e stored as an E8M0
 * byte e + 127, and each element is an E2M1 code (sign, 2 exponent bits
 * biased by 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6). Per
 * block, in fp32: amax == 0 gives scale byte 0 and zero codes; otherwise e =
 * floor(log2 amax) - 2 clamped to [-127, 127] and code = E2M1(clamp(x * 2^-e,
 * -6, 6)) rounded to nearest even.
 *
 *   x        device [B][H][N][D], bf16/f16 (`dtype`); D = 64 or 128.
 *   codes    device uint8 [B][H][N][D / 2]: byte c of a row holds channel 2c
 *            in bits 0..3 and channel 2c + 1 in bits 4..7.
 *   scales   device uint8, as attn_quantize_mx: axis 0 [B][H][N][D/32],
 *            axis 1 [B][H][ceil(N/32)][D].
 * Codes and scales are bit-exact with the CPU oracle's definition. Errors as
 * attn_quantize_mx; nothing is allocated.
 */
int attn_quantize_mx4(const void* x, uint8_t* codes, uint8_t* scales, int B, int H, int N,
                      int D, int axis, int dtype, void* stream);

/*
 * attn_decode_kvq — decode over a quantised KV cache: the split-KV decode of
 * attn_fwd reading K and V as the per-block codes that attn_quantize_qk (its
 * K half) and attn_quantize_v write, at half the bytes of a 16-bit cache.
 * This is the "INT8 QK . FP8 PV" recipe of the table in section 1 of
 * "Attention kernels on a home RTX 5080" applied to the cache; the pages'
 * own kernels quantise a 16-bit cache on every call instead.
 *
 *   q          device [B][Hq][Nq][D], f16 or bf16 (`dtype`).
 *   k_codes    device int8 [B][Hkv][Nk][D]; key j of a head dequantises to
 *              k_codes * k_scales[b][h][j / 64].
 *   k_scales   device fp32 [B][Hkv][ceil(Nk/64)].
 *   v_codes    device uint8 [B][Hkv][Nk][D], OCP FP8 E4M3 codes; value
 *              E4M3(code) * v_scales[b][h][j / 64].
 *   v_scales   device fp32 [B][Hkv][ceil(Nk/64)].
 *   o          device [B][Hq][Nq][D], `dtype`.
 *   B .. scale, stream: as for attn_fwd. (Hq / Hkv) * Nq must be <= 32 (all
 *              query rows of a key/value head fit one 32-column matrix-core
 *              block) and B * Hkv <= 65535; otherwise ATTN_E_UNSUPPORTED.
 *   workspace  device scratch of at least attn_decode_kvq_workspace_bytes(...)
 *              bytes, 256-byte aligned, no initialisation needed.
 *
 * In the kernel, Q is quantised with the INT8 recipe of attn_quantize_qk (the
 * Nq <= 32 rows of one head are one block), Q K^T is computed exactly in
 * int32 and scaled by the block scales, and each softmax weight enters P V as
 * an E4M3 code (fp32 accumulation; the denominator sums the unrounded
 * weights). Scales may be 0 (a block of zero codes); codes 0x7F/0xFF (NaN)
 * give NaN outputs. A row with no visible key is written as zeros. Returns
 * ATTN_OK or a negative attn_status; nothing is enqueued on error.
 */
int attn_decode_kvq(const void* q, const int8_t* k_codes, const float* k_scales,
                    const uint8_t* v_codes, const float* v_scales, void* o,
                    int B, int Hq, int Hkv, int Nq, int Nk, int D,
                    int causal, int window_lo, int pos0, float scale, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Workspace attn_decode_kvq needs (host-only; 0 for arguments it rejects). */
size_t attn_decode_kvq_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int D,
                                       int causal, int window_lo, int pos0, int dtype);

/*
 * attn_fwd_decode — the split-KV decode of attn_fwd with a caller-chosen
 * split count (serving loops tune it to the batch and the cache length; the
 * tests use it to check that the result does not depend on it).
 *
 * The G * Nq query rows of a key/value head (G = Hq / Hkv) are packed into one
 * matrix-core block; the visible keys are cut into 64-key tiles, `splits`
 * workgroups share a key/value head's tiles (contiguous ranges), each keeps
 * an online-softmax partial (running max, running sum, unnormalised O), and
 * the last workgroup of the head to finish merges the partials with
 * log-sum-exp weights in split order: the chunked attention + merge structure
 * of "round 21 track b — qsa2" (sections "implementation and review",
 * "measured results").
 *
 *   splits     workgroups per key/value head: 0 = the library's own plan
 *              (what attn_fwd uses); otherwise at most this many, fewer when
 *              the visible range has fewer 64-key tiles (at most 64).
 *   Every other argument, layout and error is as for attn_fwd in the exact
 *   mode (mode is implied). (Hq / Hkv) * Nq must be <= 32 and B * Hkv <=
 *   65535, else ATTN_E_UNSUPPORTED; splits < 0 gives ATTN_E_INVALID.
 *   workspace  at least attn_fwd_decode_workspace_bytes(...) bytes.
 * Unlike attn_fwd, the decode kernel runs for any number of visible keys
 * (attn_fwd takes it only for >= 512). Rows with no visible key are zeros.
 */
int attn_fwd_decode(const void* q, const void* k, const void* v, void* o,
                    int B, int Hq, int Hkv, int Nq, int Nk, int D,
                    int causal, int window_lo, int pos0, float scale, int dtype, int splits,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Workspace attn_fwd_decode needs (host-only; 0 for arguments it rejects). */
size_t attn_fwd_decode_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int D,
                                       int causal, int window_lo, int pos0, int dtype,
                                       int splits);

/*
 * attn_fwd_plan — which kernels a call would launch, without launching
 * anything (host-only; the dispatch stays inside the library, as the
 * resolver of "perf(metal): widen four-row flash KV tiles" keeps it, and this
 * makes it observable).
 *
 * Arguments as for attn_fwd (window > 0 describes attn_fwd_sliding with that
 * width, window_lo must then be 0; rope nonzero describes attn_fwd_rope).
 * Fills *plan and returns ATTN_OK, or the status attn_fwd would return for
 * these sizes (plan untouched).
 */
typedef enum {
  ATTN_KERNEL_PREFILL = 1,        /* exact-mode prefill (bf16/f16 matrix cores) */
  ATTN_KERNEL_DECODE = 2,         /* exact-mode split-KV decode, fused merge */
  ATTN_KERNEL_PREFILL_QUANT = 3,  /* INT8 Q K^T, FP8 P V */
  ATTN_KERNEL_PREFILL_MX = 4,     /* INT8 Q K^T, MX FP8 P V */
  ATTN_KERNEL_PREFILL_MXD = 5     /* INT8 Q K^T, MX FP8 / FP4 P V by tile */
} attn_kernel;

typedef struct {
  int kernel;              /* attn_kernel of the attention launch */
  int waves;               /* waves of 64 lanes per workgroup */
  int rows;                /* prefill: query rows per workgroup; decode: packed
                              query rows per key/value head (G * Nq) */
  int splits;              /* decode: workgroups per key/value head; exact
                              prefill: workgroups per query tile (1; 2-4 for
                              grids of at most 128 query tiles; 2 for some
                              tiles of a grid between half a round and one
                              round of workgroups, which then takes a second,
                              merging launch), given the full workspace;
                              else 1 */
  long long workgroups;    /* workgroups of the attention launch */
  int pre_launches;        /* launches enqueued before it (fp32 -> bf16
                              conversions, quantisers, the K rotation pass) */
  size_t workspace_bytes;  /* what the matching *_workspace_bytes returns */
} attn_plan;

int attn_fwd_plan(int B, int Hq, int Hkv, int Nq, int Nk, int D, int causal, int window_lo,
                  int window, int pos0, int mode, int dtype, int rope, attn_plan* plan);

/*
 * attn_fwd_noalloc — attn_fwd for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. It allocates nothing (no hipMalloc, hipFree or allocating
 * library call): the workspace attn_fwd would need comes from one fixed array
 * of ATTN_NOALLOC_SCRATCH_BYTES in device memory that the library holds on
 * every GPU it runs on until the process ends. Its device address is looked
 * up once per device, on the first call on that device.
 *
 * Arguments, layouts, modes and results are those of attn_fwd (the same
 * kernels run); the caller passes only inputs and outputs. Errors:
 *   every attn_fwd argument error, checked first (nothing enqueued);
 *   ATTN_E_TOO_LARGE  the call needs more workspace than ATTN_NOALLOC_SCRATCH_BYTES
 *                     even unsplit (e.g. the quantised modes at long sequences,
 *                     fp32 inputs beyond about 2 M elements); a split prefill
 *                     whose partials do not fit runs unsplit instead;
 *   ATTN_E_INVALID    `stream` belongs to another device than the current one;
 *   ATTN_E_HIP        the device address could not be looked up, or a launch
 *                     failed.
 * Calls on one GPU share its array, which keeps the last call's contents (no
 * kernel here needs it cleared: the arrival counters of the decode and of the
 * split prefill carry a per-call tag), so calls that overlap on one GPU (different streams, or concurrent host
 * threads) race and must be serialised by the caller.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                     int B, int Hq, int Hkv, int Nq, int Nk, int D,
                     int causal, int window_lo, int pos0, float scale, int mode,
                     int dtype, void* stream);

/* Static English text for a status code. */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
