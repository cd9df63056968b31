// attn_decode.hip — split-KV decode for few query rows per key/value head.
//
// Decode reads every visible K/V byte once and does little arithmetic per
// byte, so it is bound by HBM bandwidth, not by the matrix cores. All
// G * Nq query rows that share a key/value head (G = Hq / Hkv) are packed
// into the 32 columns of one MFMA block, so each K/V byte feeds every one of
// them. The visible keys are cut into 64-key tiles; each wave takes one tile
// (K straight from global memory into A-operand registers, V transposed
// through a private LDS slab) and produces an unnormalised partial
// (O_s, m_s, l_s); the four waves of a workgroup merge theirs in LDS and write
// one partial per workgroup; a second kernel merges the partials of all
// workgroups with log-sum-exp weights. This is the chunked attention + merge
// structure of "round 21 track b — qsa2" (its attention kernel writes
// partial buffers that a merge kernel combines with cached maxima and
// weights and a denominator computed once), written for wave64 MFMA.
#include "attn_common.hpp"
#include "attn_internal.hpp"

namespace attn {

namespace {

constexpr int kWaves = 4;          // waves per workgroup, one 64-key tile each
constexpr int kKeysPerWg = 64 * kWaves;

struct DecodeArgs {
  int rows, t_lo, t_hi, nsplit;
  float* opart;  // [B*Hkv][nsplit][rows][D], unnormalised
  float* mpart;  // [B*Hkv][nsplit][rows], running max in exp2 units
  float* lpart;  // [B*Hkv][nsplit][rows]
};

template <typename T, int D>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256)))
decode_partial_kernel(FwdArgs a, DecodeArgs p) {
  using E = Elem<T>;
  using V8 = typename E::vec8;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int VLD = 64 + 8;
  constexpr int CPR = D / 8;               // 16-byte chunks per key row
  constexpr int LOADS = 64 * CPR / 64;     // per lane, one tile of V
  // Per-wave V^T slabs; reused after a barrier for the cross-wave merge.
  constexpr int SLAB = D * VLD * 2;        // bytes per wave
  constexpr int MERGE = kWaves * 32 * D * 4 + 2 * kWaves * 32 * 4;
  constexpr int LDS_BYTES = (kWaves * SLAB > MERGE) ? kWaves * SLAB : MERGE;
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int split = blockIdx.x, bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int64_t kvbase = (int64_t)bg * a.Nk * D;
  const T* __restrict__ Kp = (const T*)a.k + kvbase;
  const T* __restrict__ Vp = (const T*)a.v + kvbase;
  T* slab = (T*)(lds + wave * SLAB);

  // Column -> (query head within the group, row): n = hh * Nq + i.
  const bool cvalid = col < p.rows;
  const int hh = col / a.Nq, qi = col - hh * a.Nq;
  const T* Qrow = (const T*)a.q + (((int64_t)b * a.Hq + g * G + hh) * a.Nq + qi) * D;

  const int t = p.t_lo + split * kWaves + wave;
  const bool has_tile = t < p.t_hi;
  const int k0 = t * 64;

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[db][j] = 0.0f;
  float m = -INFINITY, l = 0.0f;

  // Phase 1: issue every load of the tile, then stage V^T in this wave's slab.
  u32x4 kreg[2][KS];
  V8 qv[KS];
  if (has_tile) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int key = k0 + 32 * mb + swap23(col);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kreg[mb][ks] = key < a.Nk ? ld16(Kp + (int64_t)key * D + 16 * ks + 8 * half)
                                  : u32x4{0, 0, 0, 0};
    }
    // V: lane -> keys 4*(lane%16) + r, chunk columns lane/16 + 4*u.
    const int kg = lane & 15, c0 = lane >> 4;
    u32x4 vreg[LOADS / 4][4];
#pragma unroll
    for (int u = 0; u < LOADS / 4; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 4 * kg + r;
        const int cc = c0 + 4 * u;
        vreg[u][r] = key < a.Nk ? ld16(Vp + (int64_t)key * D + 8 * cc) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 raw = {0, 0, 0, 0};
      if (cvalid) raw = ld16(Qrow + 16 * ks + 8 * half);
      qv[ks] = __builtin_bit_cast(V8, raw);
    }
#pragma unroll
    for (int u = 0; u < LOADS / 4; ++u) {
      const int cc = c0 + 4 * u;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        u32x2 pk;
        pk[0] = __builtin_amdgcn_perm(vreg[u][1][e >> 1], vreg[u][0][e >> 1], sel);
        pk[1] = __builtin_amdgcn_perm(vreg[u][3][e >> 1], vreg[u][2][e >> 1], sel);
        *(u32x2*)&slab[(8 * cc + e) * VLD + 4 * kg] = pk;
      }
    }
  }
  __syncthreads();

  // Phase 2: S^T = K Q^T, mask, softmax of the tile, O^T = V^T P^T.
  if (has_tile) {
    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) s[mb][j] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        s[mb] = E::mma(__builtin_bit_cast(V8, kreg[mb][ks]), qv[ks], s[mb]);
    }
    // Mask every element: one tile per wave, so this is cheap.
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = k0 + 32 * mb + 16 * (j >> 3) + 8 * half + (j & 7);
        const bool vis = cvalid && key >= a.window_lo && key < a.Nk &&
                         (!a.causal || key <= a.pos0 + qi);
        if (!vis) s[mb][j] = -INFINITY;
      }
    float mx = s[0][0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = fmaxf(mx, s[0][j]);
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[1][j]);
    m = halves_max(mx) * a.c;
    const float mu = m == -INFINITY ? 0.0f : m;
    V8 pv[2][2];
    float lsum = 0.0f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(s[mb][8 * tt + i], a.c, -mu));
          lsum += e;
          pv[mb][tt][i] = E::from_float(e);
        }
    l = halves_sum(lsum);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const V8 va = *(const V8*)&slab[(32 * db + col) * VLD + 32 * mb + 16 * tt + 8 * half];
          oacc[db] = E::mma(va, pv[mb][tt], oacc[db]);
        }
  }

  // Merge the four waves: publish (m, l, O) per column, then every thread
  // combines one (row, 4 channels) slot over the waves in a fixed order.
  __syncthreads();
  float* so = (float*)lds;                              // [wave][32][D]
  float* sm = so + kWaves * 32 * D;                     // [wave][32]
  float* sl = sm + kWaves * 32;                         // [wave][32]
  if (cvalid) {
    if (half == 0) {
      sm[wave * 32 + col] = m;
      sl[wave * 32 + col] = l;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d = 32 * db + 8 * a4 + 4 * half;
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = oacc[db][4 * a4 + r];
        *(f32x4*)&so[(wave * 32 + col) * D + d] = v;
      }
  }
  __syncthreads();
  constexpr int SLOTS = D / 4;   // threads per row
  const int64_t pbase = ((int64_t)bg * p.nsplit + split) * p.rows;
  for (int idx = tid; idx < p.rows * SLOTS; idx += 256) {
    const int n = idx / SLOTS, d = (idx - n * SLOTS) * 4;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm[w * 32 + n]);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float L = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(sm[w * 32 + n] - M);
        L += f * sl[w * 32 + n];
        const f32x4 v = *(const f32x4*)&so[(w * 32 + n) * D + d];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += f * v[r];
      }
    }
    *(f32x4*)&p.opart[(pbase + n) * D + d] = acc;
    if (d == 0) {
      p.mpart[pbase + n] = M;
      p.lpart[pbase + n] = L;
    }
  }
}

// Log-sum-exp merge over the splits of one key/value head: the maxima are
// read once, the weights 2^(m_s - M) computed once per (row, split), and the
// denominator once per row.
template <typename TO, int D>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256)))
decode_merge_kernel(FwdArgs a, DecodeArgs p) {
  constexpr int SLOTS = D / 4;
  const int bg = blockIdx.x, b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  for (int idx = threadIdx.x; idx < p.rows * SLOTS; idx += 256) {
    const int n = idx / SLOTS, d = (idx - n * SLOTS) * 4;
    const int64_t base = (int64_t)bg * p.nsplit * p.rows + n;
    float M = -INFINITY;
    for (int sp = 0; sp < p.nsplit; ++sp) M = fmaxf(M, p.mpart[base + (int64_t)sp * p.rows]);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float L = 0.0f;
    if (M != -INFINITY) {
      for (int sp = 0; sp < p.nsplit; ++sp) {
        const int64_t r = base + (int64_t)sp * p.rows;
        const float f = __builtin_amdgcn_exp2f(p.mpart[r] - M);
        L += f * p.lpart[r];
        const f32x4 v = *(const f32x4*)&p.opart[r * D + d];
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] += f * v[k];
      }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const int hh = n / a.Nq, qi = n - hh * a.Nq;
    TO* orow = (TO*)a.o + (((int64_t)b * a.Hq + g * G + hh) * a.Nq + qi) * D + d;
    if constexpr (sizeof(TO) == 4) {
      f32x4 o;
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = acc[k] * inv;
      *(f32x4*)orow = o;
    } else {
      TO o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = Elem<TO>::from_float(acc[k] * inv);
      *(u32x2*)orow = *(const u32x2*)o;
    }
  }
}

template <typename T, typename TO, int D>
hipError_t launch_t(const FwdArgs& a, const DecodePlan& pl, void* ws, hipStream_t s) {
  DecodeArgs p;
  p.rows = pl.rows;
  p.t_lo = pl.t_lo;
  p.t_hi = pl.t_lo + pl.ntiles;
  p.nsplit = pl.nsplit;
  const int64_t nrow = (int64_t)a.B * a.Hkv * pl.nsplit * pl.rows;
  p.opart = (float*)ws;
  p.mpart = p.opart + nrow * D;
  p.lpart = p.mpart + nrow;
  hipLaunchKernelGGL((decode_partial_kernel<T, D>), dim3(pl.nsplit, a.B * a.Hkv), dim3(256), 0, s, a, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<TO, D>), dim3(a.B * a.Hkv), dim3(256), 0, s, a, p);
  return hipGetLastError();
}

}  // namespace

bool decode_eligible(const FwdArgs& a) {
  const int rows = (a.Hq / a.Hkv) * a.Nq;
  const KeyRange r = key_range(a);
  return rows <= 32 && r.hi - r.lo >= 512;
}

DecodePlan decode_plan(const FwdArgs& a) {
  DecodePlan p;
  const KeyRange r = key_range(a);
  p.rows = (a.Hq / a.Hkv) * a.Nq;
  p.t_lo = r.lo / 64;
  const int t_hi = r.hi > r.lo ? (r.hi + 63) / 64 : p.t_lo;
  p.ntiles = t_hi - p.t_lo;
  p.nsplit = (p.ntiles + kWaves - 1) / kWaves;
  if (p.nsplit < 1) p.nsplit = 1;
  const size_t nrow = (size_t)a.B * a.Hkv * p.nsplit * p.rows;
  p.ws_bytes = nrow * (size_t)(a.D + 2) * sizeof(float);
  return p;
}

hipError_t launch_decode(const FwdArgs& a, const DecodePlan& p, int elem, bool out_f32,
                         void* ws, hipStream_t s) {
  if (elem == 2) {
    if (out_f32) return a.D == 64 ? launch_t<__bf16, float, 64>(a, p, ws, s) : launch_t<__bf16, float, 128>(a, p, ws, s);
    return a.D == 64 ? launch_t<__bf16, __bf16, 64>(a, p, ws, s) : launch_t<__bf16, __bf16, 128>(a, p, ws, s);
  }
  return a.D == 64 ? launch_t<_Float16, _Float16, 64>(a, p, ws, s) : launch_t<_Float16, _Float16, 128>(a, p, ws, s);
}

}  // namespace attn
