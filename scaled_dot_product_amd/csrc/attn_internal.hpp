// attn_internal.hpp — host-side launch plans shared by the C ABI and the
// kernel translation units. Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

constexpr float kLog2eHost = 1.4426950408889634f;

// Rotary position embedding of one call: pair i turns by 2 pi pos * rev_i
// revolutions, rev_i = theta_i / (2 pi) held as the sum of two floats.
constexpr int kRopeMaxPairs = 64;
struct RopeArgs {
  int on;      // 0: no rotation
  int style;   // 0: pairs (c, c + D/2); 1: pairs (2i, 2i + 1)
  float rev_hi[kRopeMaxPairs];
  float rev_lo[kRopeMaxPairs];
};

// Arguments of one forward call after validation.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int B, Hq, Hkv, Nq, Nk, D;
  int causal, window_lo, pos0;
  int window_w;  // > 0: row i also needs key >= pos0 + i - window_w + 1
  float scale;
  float c;  // scale * log2(e): scores are exponentiated with exp2
  RopeArgs rope;   // rotation of Q in the kernels (K is rotated before them)
};

// The argument checks of attn_fwd (everything but the workspace): ATTN_OK or
// the status attn_fwd returns. Host-only, touches no runtime state.
int fwd_validate(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv,
                 int Nq, int Nk, int D, int causal, int window_lo, int pos0, float scale, int mode,
                 int dtype);
// The least workspace attn_fwd accepts for these sizes (the split prefill
// off); attn_fwd_workspace_bytes gives the size that enables it.
size_t fwd_min_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int D, int causal,
                               int window_lo, int pos0, int mode, int dtype);

// Visible key range [lo, hi) over all rows of a call (hi <= lo: none).
struct KeyRange {
  int lo, hi;
};
KeyRange key_range(const FwdArgs& a);

// ---- exact-mode prefill (bf16/f16 MFMA) ----------------------------------
// Split of each query tile's key range over ns workgroups (ns = 1: none). A
// grid of few query tiles leaves most CUs idle; ns parts of about equal
// length per tile put them to work. Each part publishes its normalised
// partial (O / l in the output type, m and l in fp32) and the last part of a
// query tile to arrive merges them.
struct PrefillSplit {
  int ns = 1;              // parts per query tile (merged by the last to arrive)
  int halves = 0;          // or: the last `halves` tiles run as two halves each,
                           // merged by a second launch (the balanced schedule)
  int64_t tiles = 0;       // query tiles (the unsplit grid)
  int rows = 0;            // query rows per tile
  size_t ctr_bytes = 0;    // arrival counters, one per query tile
  size_t ws_bytes = 0;     // counters + partials
};
// out_bytes: bytes per output element (2, or 4 for fp32 output).
PrefillSplit prefill_split_plan(const FwdArgs& a, int out_bytes);
// elem: 1 = f16, 2 = bf16 operands; out_f32: write fp32 output. ws: the
// split's workspace (ws_bytes of sp), unused when sp.ns == 1.
hipError_t launch_prefill(const FwdArgs& a, int elem, bool out_f32, const PrefillSplit& sp,
                          void* ws, hipStream_t s);
// Waves (of 32 query rows each) per prefill workgroup for this call: 4 or 8.
int prefill_waves(const FwdArgs& a);
// A different value for every launch (tags of the arrival counters).
unsigned long long next_generation();

// ---- split-KV decode + log-sum-exp merge ---------------------------------
struct DecodePlan {
  int rows;       // G * Nq query rows per key/value head (<= 32)
  int t_lo;       // first 64-key tile
  int ntiles;     // tiles in the visible range
  int nsplit;     // workgroups per key/value head
  int tiles_per_wg;
  int waves;      // waves per workgroup (1, 2 or 4), one 64-key tile each per step
  size_t ctr_bytes;  // arrival counters at the start of the workspace
  size_t ws_bytes;
};
// The decode kernel packs G * Nq <= 32 rows and puts B * Hkv on grid.y.
bool decode_supported(const FwdArgs& a);
// attn_fwd takes the decode kernel for supported shapes with >= 512 visible keys.
bool decode_eligible(const FwdArgs& a);
// splits: 0 = the library's plan, else at most this many workgroups per head.
DecodePlan decode_plan(const FwdArgs& a, int splits = 0);
hipError_t launch_decode(const FwdArgs& a, const DecodePlan& p, int elem, bool out_f32,
                         void* ws, hipStream_t s);

// Decode over a quantised KV cache (INT8 K codes, E4M3 V codes, fp32 scales
// per 64-key block) with the plan above; elem: 1 = f16, 2 = bf16 Q and O.
hipError_t launch_decode_kvq(const FwdArgs& a, const DecodePlan& p, const int8_t* kc,
                             const float* ks, const uint8_t* vc, const float* vs, int elem,
                             void* ws, hipStream_t s);

// ---- fp32 inputs: rounded to bf16 before the MFMA path --------------------
hipError_t launch_f32_to_bf16(const float* x, void* y, int64_t n, hipStream_t s);

// ---- quantised mode ------------------------------------------------------
// rope (optional): rotate each row at position pos_base + n before quantising.
hipError_t launch_quant_int8(const void* x, int elem, int64_t BH, int N, int D,
                             int8_t* codes, float* scales, hipStream_t s,
                             const RopeArgs* rope = nullptr, int pos_base = 0);
// Rows of x ([BH][N][D]) rotated at positions pos_base + n into y (may be x).
hipError_t launch_rope(const void* x, void* y, int elem, int64_t BH, int N, int D, int pos_base,
                       const RopeArgs& rope, hipStream_t s);
// layout 0: codes [BH][N][D]; layout 1: per 64-key tile, transposed
// [BH][ceil(N/64)][D][64] with zero codes for keys past N.
hipError_t launch_quant_e4m3(const void* x, int elem, int64_t BH, int N, int D,
                             uint8_t* codes, float* scales, int layout, hipStream_t s);
hipError_t launch_prefill_quant(const FwdArgs& a, const int8_t* qc, const float* qs,
                                const int8_t* kc, const float* ks, const uint8_t* vct,
                                const float* vs, int elem_out, hipStream_t s);

// ---- MX variants (OCP MX FP8 / FP4 blocks, scaled MFMA) -------------------
// axis 0: blocks of 32 channels, scales [BH][srows][D/32] (srows >= N);
// axis 1: blocks of 32 tokens; layout 0: codes [BH][N][D], scales
// [BH][ceil(N/32)][D]; layout 1: codes [BH][ceil(N/64)][D][64] (zero past N),
// scales [BH][2 ceil(N/64)][D]. fp4: E2M1 codes two per byte (the lower
// index in the low nibble), so code rows and tile rows hold half the bytes.
hipError_t launch_quant_mx(const void* x, int elem, int64_t BH, int N, int D, int axis, int layout,
                           int srows, uint8_t* codes, uint8_t* scales, hipStream_t s,
                           bool fp4 = false);
// Q and K as per-64-token INT8 blocks (launch_quant_int8), V as MXFP8
// transposed tiles + scale bytes (axis 1, layout 1); with v4t (MXFP4 tiles)
// and v4s non-null, the diagonal-tiled mixed variant in two launches, which
// pass per-row partials through `part` ([B][Hq][Nq] rows of D output-type
// elements and 4 floats).
hipError_t launch_prefill_mx(const FwdArgs& a, const int8_t* qc, const float* qs,
                             const int8_t* kc, const float* ks, const uint8_t* vct,
                             const uint8_t* vs, const uint8_t* v4t, const uint8_t* v4s,
                             float* part, int elem_out, hipStream_t s);


}  // namespace attn
