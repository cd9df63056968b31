// attn_decode.hip — split-KV decode for few query rows per key/value head.
//
// Decode reads every visible K/V byte once and does little arithmetic per
// byte, so it is bound by HBM bandwidth and latency, not by the matrix cores.
// All G * Nq query rows that share a key/value head (G = Hq / Hkv) are packed
// into the 32 columns of one MFMA block, so each K/V byte feeds every one of
// them. The visible keys are cut into 64-key tiles; each wave takes one tile
// at a time (K straight from global memory into A-operand registers, V
// transposed through a private LDS slab) and keeps an online-softmax partial
// (O_s, m_s, l_s); the waves of a workgroup merge theirs in LDS and publish one
// partial per workgroup. The last workgroup of a key/value head to publish
// merges all partials of that head with log-sum-exp weights and writes O, so
// one kernel launch does the whole decode. This is the chunked attention +
// merge structure of "round 21 track b — qsa2" (partial buffers combined by a
// merge with cached maxima and weights and a denominator computed once),
// written for wave64 MFMA and fused into one launch.
#include <atomic>
#include <chrono>

#include "attn_common.hpp"
#include "attn_internal.hpp"

namespace attn {

namespace {

constexpr int kMaxSplits = 32;     // workgroups per key/value head, at most

struct DecodeArgs {
  int rows, t_lo, t_hi, nsplit, tiles_per_wg;
  float* opart;  // [B*Hkv][nsplit][rows][D], unnormalised
  float* mpart;  // [B*Hkv][nsplit][rows], running max in exp2 units
  float* lpart;  // [B*Hkv][nsplit][rows]
  unsigned long long* ctr;  // [B*Hkv] arrivals: (generation << 24) | count
  unsigned long long gen;   // in [1, 2^40), different for every call
};

// Partials cross workgroups that may sit on different XCDs, whose L2 caches
// are not coherent with each other. They are written and read with
// agent-scope atomic accesses (write-through / L2-bypassing), so no L2
// write-back or invalidate is needed; a workgroup counts its arrival only
// after all its partial stores are acknowledged.
__device__ __forceinline__ void put4(float* dst, f32x4 v) {
  unsigned long long* d = (unsigned long long*)dst;
  const u32x4 u = __builtin_bit_cast(u32x4, v);
  __hip_atomic_store(d, (unsigned long long)u[0] | ((unsigned long long)u[1] << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(d + 1, (unsigned long long)u[2] | ((unsigned long long)u[3] << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4 get4(const float* src) {
  unsigned long long* s = (unsigned long long*)src;
  const unsigned long long a = __hip_atomic_load(s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned long long b = __hip_atomic_load(s + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const u32x4 u = {(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
  return __builtin_bit_cast(f32x4, u);
}
__device__ __forceinline__ void put1(float* dst, float v) {
  __hip_atomic_store((unsigned*)dst, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get1(const float* src) {
  return __uint_as_float(__hip_atomic_load((unsigned*)src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Arrival counting for the fused merge. The counter of a key/value head is
// (generation << 24) | arrivals. At kernel start (off the critical path, while
// the tile loads are in flight) one thread of each workgroup claims the
// counter for this call: a counter whose tag is not this call's generation
// (left by an earlier call, or uninitialised workspace) is swapped for
// (generation << 24). A failed swap means another workgroup already claimed
// it, so at most one swap per workgroup is tried. Arrival is then a single
// atomic add; the workgroup that sees nsplit - 1 earlier arrivals is last.
// It resets the counter to 0, a tag no call uses, so replays of a captured
// graph (same generation) claim it again. Claims all precede the reset, as
// every workgroup claims before it arrives.
__device__ void claim_counter(unsigned long long* c, unsigned long long gen) {
  const unsigned long long cur = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((cur >> 24) != gen) atomicCAS(c, cur, gen << 24);
}
__device__ bool arrive_last(unsigned long long* c, int nsplit) {
  const unsigned long long old = atomicAdd(c, 1ull);
  return (int)(old & 0xffffffull) == nsplit - 1;
}

template <typename T, typename TO, int D, int kWaves>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * kWaves, 64 * kWaves)))
decode_kernel(FwdArgs a, DecodeArgs p) {
  using E = Elem<T>;
  using V8 = typename E::vec8;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int VLD = 64 + 8;
  constexpr int UV = D / 32;               // V loads per lane per tile, in groups of 4 keys
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

  // Column -> (query head within the group, row): n = hh * Nq + i. Columns past
  // the packed rows read row 0 and are masked out.
  const bool cvalid = col < p.rows;
  const int ccol = cvalid ? col : 0;
  const int hh = ccol / a.Nq, qi = ccol - hh * a.Nq;
  const T* Qrow = (const T*)a.q + (((int64_t)b * a.Hq + g * G + hh) * a.Nq + qi) * D;
  V8 qv[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qv[ks] = __builtin_bit_cast(V8, ld16(Qrow + 16 * ks + 8 * half));

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[db][j] = 0.0f;
  float m = -INFINITY, l = 0.0f;
  bool claimed = false;   // uniform: the counter is claimed after the first loads

  // This workgroup's tiles: [t0, t1); wave w takes t0 + w, t0 + w + kWaves, ...
  const int t0 = p.t_lo + split * p.tiles_per_wg;
  const int t1 = min(t0 + p.tiles_per_wg, p.t_hi);
  const int kg = lane & 15, c0 = lane >> 4;
  for (int tb = t0; tb < t1; tb += kWaves) {
    const int t = tb + wave;
    const bool has_tile = t < t1;
    const int k0 = t * 64;
    // Phase 1: every load of the tile issued back to back. Rows past Nk are
    // clamped to a real row (finite values) and masked below.
    u32x4 kreg[2][KS];
    if (has_tile) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int key = min(k0 + 32 * mb + swap23(col), a.Nk - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kreg[mb][ks] = ld16(Kp + (int64_t)key * D + 16 * ks + 8 * half);
      }
      u32x4 vreg[UV][4];
#pragma unroll
      for (int u = 0; u < UV; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = min(k0 + 4 * kg + r, a.Nk - 1);
          vreg[u][r] = ld16(Vp + (int64_t)key * D + 8 * (c0 + 4 * u));
        }
      // claim while this wave's tile loads are in flight (its wait on the
      // counter read then overlaps the wait on the tile)
      if (!claimed && tid == 0) claim_counter(p.ctr + bg, p.gen);
      // V^T into this wave's slab.
#pragma unroll
      for (int u = 0; u < UV; ++u) {
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

    // Phase 2: S^T = K Q^T, mask, online softmax, O^T += V^T P^T.
    if (has_tile) {
      // four independent accumulators (even/odd k-steps) shorten the MFMA chains
      f32x16 s[2][2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int j = 0; j < 16; ++j) s[mb][h2][j] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          s[mb][ks & 1] = E::mma(__builtin_bit_cast(V8, kreg[mb][ks]), qv[ks], s[mb][ks & 1]);
      float sc[2][16];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = k0 + 32 * mb + 16 * (j >> 3) + 8 * half + (j & 7);
          const bool vis = cvalid && key >= a.window_lo && key < a.Nk &&
                           (!a.causal || key <= a.pos0 + qi);
          sc[mb][j] = vis ? s[mb][0][j] + s[mb][1][j] : -INFINITY;
        }
      float mx = sc[0][0];
#pragma unroll
      for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sc[0][j]);
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sc[1][j]);
      mx = halves_max(mx) * a.c;
      const float m_new = fmaxf(m, mx);
      const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m - m_new);
      m = m_new;
      const float mu = m == -INFINITY ? 0.0f : m;
      V8 pv[2][2];
      float lsum = 0.0f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float e = __builtin_amdgcn_exp2f(fmaf(sc[mb][8 * tt + i], a.c, -mu));
            lsum += e;
            pv[mb][tt][i] = E::from_float(e);
          }
      l = l * alpha + halves_sum(lsum);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const V8 va = *(const V8*)&slab[(32 * db + col) * VLD + 32 * mb + 16 * tt + 8 * half];
            oacc[db] = E::mma(va, pv[mb][tt], oacc[db]);
          }
      }
    }
    __syncthreads();
    claimed = true;
  }
  // A workgroup without tiles still claims before it arrives.
  if (!claimed && tid == 0) claim_counter(p.ctr + bg, p.gen);

  // 1. Publish this workgroup's partial.
  const int64_t pbase = ((int64_t)bg * p.nsplit + split) * p.rows;
  if constexpr (kWaves == 1) {
    // One wave: its partial goes straight from registers to the workspace.
    if (cvalid) {
      if (half == 0) {
        put1(&p.mpart[pbase + col], m);
        put1(&p.lpart[pbase + col], l);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int d = 32 * db + 8 * a4 + 4 * half;
          f32x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = oacc[db][4 * a4 + r];
          put4(&p.opart[(pbase + col) * D + d], v);
        }
    }
  } else {
    // Merge the waves in LDS, in a fixed order, then publish.
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
    for (int idx = tid; idx < p.rows * SLOTS; idx += 64 * kWaves) {
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
      put4(&p.opart[(pbase + n) * D + d], acc);
      if (d == 0) {
        put1(&p.mpart[pbase + n], M);
        put1(&p.lpart[pbase + n], L);
      }
    }
  }

  // 2. Arrive; the last workgroup of this key/value head merges all splits.
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);   // every partial store of this thread acknowledged
  __syncthreads();
  if (tid == 0) s_last = arrive_last(p.ctr + bg, p.nsplit);
  __syncthreads();
  if (!s_last) return;

  // Final merge, one thread per (row, 4 channels): all loads of a chunk of
  // splits first (one memory round trip per 16 splits), then an online
  // log-sum-exp merge in registers, in split order.
  constexpr int NT = 64 * kWaves;
  constexpr int SLOTS = D / 4;
  constexpr int CH = 16;
  const int ns = p.nsplit, rows = p.rows;
  const int64_t hbase = (int64_t)bg * ns * rows;
  for (int idx = tid; idx < rows * SLOTS; idx += NT) {
    const int n = idx / SLOTS, d = (idx - n * SLOTS) * 4;
    float M = -INFINITY, L = 0.0f;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < ns; s0 += CH) {
      float mv[CH], lv[CH];
      f32x4 ov[CH];
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int sp = min(s0 + u, ns - 1);
        const int64_t r = hbase + (int64_t)sp * rows + n;
        mv[u] = get1(&p.mpart[r]);
        lv[u] = get1(&p.lpart[r]);
        ov[u] = get4(&p.opart[r * D + d]);
      }
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        if (s0 + u >= ns || mv[u] == -INFINITY) continue;
        if (mv[u] > M) {
          const float f = __builtin_amdgcn_exp2f(M - mv[u]);   // 0 while M = -inf
          L = L * f + lv[u];
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[c] = acc[c] * f + ov[u][c];
          M = mv[u];
        } else {
          const float f = __builtin_amdgcn_exp2f(mv[u] - M);
          L += f * lv[u];
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[c] += f * ov[u][c];
        }
      }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const int hh2 = n / a.Nq, qi2 = n - hh2 * a.Nq;
    TO* orow = (TO*)a.o + (((int64_t)b * a.Hq + g * G + hh2) * a.Nq + qi2) * D + d;
    if constexpr (sizeof(TO) == 4) {
      f32x4 o;
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = acc[c] * inv;
      *(f32x4*)orow = o;
    } else {
      TO o[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = Elem<TO>::from_float(acc[c] * inv);
      *(u32x2*)orow = *(const u32x2*)o;
    }
  }
  if (tid == 0) __hip_atomic_store(p.ctr + bg, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A different generation for every launch, from a per-process random start
// (so that counters left in a reused workspace by another process never match).
unsigned long long next_generation() {
  static std::atomic<unsigned long long> counter{
      ((unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count() ^
       (unsigned long long)(uintptr_t)&counter) * 0x9E3779B97F4A7C15ull};
  const unsigned long long g = counter.fetch_add(1, std::memory_order_relaxed);
  return (g % ((1ull << 40) - 1)) + 1;
}

template <typename T, typename TO, int D>
hipError_t launch_t(const FwdArgs& a, const DecodePlan& pl, void* ws, hipStream_t s) {
  DecodeArgs p;
  p.rows = pl.rows;
  p.t_lo = pl.t_lo;
  p.t_hi = pl.t_lo + pl.ntiles;
  p.nsplit = pl.nsplit;
  p.tiles_per_wg = pl.tiles_per_wg;
  const int64_t nrow = (int64_t)a.B * a.Hkv * pl.nsplit * pl.rows;
  p.ctr = (unsigned long long*)ws;
  p.opart = (float*)((char*)ws + pl.ctr_bytes);
  p.mpart = p.opart + nrow * D;
  p.lpart = p.mpart + nrow;
  p.gen = next_generation();
  const dim3 grid(pl.nsplit, a.B * a.Hkv);
  if (pl.waves == 1)
    hipLaunchKernelGGL((decode_kernel<T, TO, D, 1>), grid, dim3(64), 0, s, a, p);
  else if (pl.waves == 2)
    hipLaunchKernelGGL((decode_kernel<T, TO, D, 2>), grid, dim3(128), 0, s, a, p);
  else
    hipLaunchKernelGGL((decode_kernel<T, TO, D, 4>), grid, dim3(256), 0, s, a, p);
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
  // Four waves (one 64-key tile each) per workgroup and at most kMaxSplits
  // workgroups per key/value head; longer ranges give each wave several
  // tiles. Fewer, fuller workgroups keep the final merge (on the critical
  // path, in the last workgroup) short.
  p.waves = 4;
  const int per_wave = (p.ntiles + p.waves * kMaxSplits - 1) / (p.waves * kMaxSplits);
  p.tiles_per_wg = p.waves * (per_wave < 1 ? 1 : per_wave);
  p.nsplit = (p.ntiles + p.tiles_per_wg - 1) / p.tiles_per_wg;
  if (p.nsplit < 1) p.nsplit = 1;
  const size_t nrow = (size_t)a.B * a.Hkv * p.nsplit * p.rows;
  p.ctr_bytes = ((size_t)a.B * a.Hkv * sizeof(unsigned long long) + 255) / 256 * 256;
  p.ws_bytes = p.ctr_bytes + nrow * (size_t)(a.D + 2) * sizeof(float);
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
