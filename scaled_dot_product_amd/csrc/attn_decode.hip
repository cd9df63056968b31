// attn_decode.hip — split-KV decode for few query rows per key/value head.
//
// Decode reads every visible K/V byte once and does little arithmetic per
// byte, so it is bound by HBM bandwidth and latency, not by the matrix cores.
// All G * Nq query rows that share a key/value head (G = Hq / Hkv) are packed
// into the 32 columns of one MFMA block, so each K/V byte feeds every one of
// them. The visible keys are cut into 64-key tiles; each wave streams its own
// tiles through a private pair of LDS tiles (direct global-to-LDS loads, the
// prefill's swizzles; V^T operands by transpose reads; a wave's first scores
// are computed as soon as its K tile lands, while V is still arriving) and
// keeps an online-softmax partial (O_s, m_s, l_s); the waves of a workgroup
// merge theirs in LDS and publish one partial per workgroup, O_s normalised by
// l_s and rounded to the output element type (half the bytes the merging
// workgroup must read, at the output's own precision). The last workgroup of a
// key/value head to publish merges all partials of that head with log-sum-exp
// weights and writes O, so one kernel launch does the whole decode. This is the chunked attention +
// merge structure of "round 21 track b — qsa2" (partial buffers combined by a
// merge with cached maxima and weights and a denominator computed once),
// written for wave64 MFMA and fused into one launch.
#include <atomic>
#include <chrono>

#include "attn_common.hpp"
#include "attn_internal.hpp"

namespace attn {

namespace {

constexpr int kMaxSplits = 32;     // workgroups per key/value head in the library's plan
constexpr int kMaxRequestedSplits = 64;   // ... and when the caller chooses

struct DecodeArgs {
  int rows, t_lo, t_hi, nsplit, tiles_per_wg;
  float* opart;  // [B*Hkv][nsplit][rows][D] of O_s / l_s in the output type (fp32-sized area)
  float* mpart;  // [B*Hkv][nsplit][rows], running max in exp2 units
  float* lpart;  // [B*Hkv][nsplit][rows]
  unsigned long long* ctr;  // [B*Hkv] arrivals: (generation << 24) | count
  unsigned long long gen;   // in [1, 2^40), different for every call
};

// Partials cross workgroups that may sit on different XCDs, whose L2 caches
// are not coherent with each other. They are written and read with
// agent-scope atomic accesses, and a workgroup counts its arrival only after
// all its partial stores are acknowledged and its waves have met at a
// barrier; the arrival is an agent-scope acquire-release add, so the merging
// workgroup (whose add reads the others') sees every partial by the memory
// model's happens-before (workgroup barrier, then agent-scope release and
// acquire), not by a property of this hardware.
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
// Four partial values in the output element type: one 64-bit word (16-bit
// types) or two (fp32).
template <typename TO>
__device__ __forceinline__ void put_part(float* base, int64_t idx, f32x4 v) {
  if constexpr (sizeof(TO) == 2) {
    TO o4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) o4[c] = Elem<TO>::from_float(v[c]);
    unsigned long long w;
    __builtin_memcpy(&w, o4, 8);
    __hip_atomic_store((unsigned long long*)((TO*)base + idx), w, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  } else {
    put4(base + idx, v);
  }
}
template <typename TO>
__device__ __forceinline__ f32x4 get_part(const float* base, int64_t idx) {
  if constexpr (sizeof(TO) == 2) {
    const unsigned long long w = __hip_atomic_load((unsigned long long*)((const TO*)base + idx),
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    TO o4[4];
    __builtin_memcpy(o4, &w, 8);
    return f32x4{(float)o4[0], (float)o4[1], (float)o4[2], (float)o4[3]};
  } else {
    return get4(base + idx);
  }
}
__device__ __forceinline__ void put1(float* dst, float v) {
  __hip_atomic_store((unsigned*)dst, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get1(const float* src) {
  return __uint_as_float(__hip_atomic_load((unsigned*)src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// After the tiles: the counter claim, the merge of the waves' partials in LDS
// (so: kWaves x 32 x D floats, sml: 2 x kWaves x 32 floats), the workgroup's
// partial published, the arrival, and in the last workgroup of the KV head
// the merge of all splits into O.
template <typename TO, int D, int kWaves>
__device__ __forceinline__ void decode_finish(const FwdArgs& a, const DecodeArgs& p, float m,
                                              float l, f32x16 (&oacc)[D / 32], float* so_base,
                                              float* sml, unsigned long long ctr_seen) {
  constexpr int DB = D / 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int split = blockIdx.x, bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const bool cvalid = col < p.rows;
  if (tid == 0 && (ctr_seen >> 24) != p.gen) atomicCAS(p.ctr + bg, ctr_seen, p.gen << 24);
  __syncthreads();   // every wave is done with its tiles before the merge reuses LDS


  // 1. Publish this workgroup's partial.
  const int64_t pbase = ((int64_t)bg * p.nsplit + split) * p.rows;
  if constexpr (kWaves == 1) {
    // One wave: its partial goes straight from registers to the workspace.
    if (cvalid) {
      if (half == 0) {
        put1(&p.mpart[pbase + col], m);
        put1(&p.lpart[pbase + col], l);
      }
      const float r = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int d = 32 * db + 8 * a4 + 4 * half;
          f32x4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = oacc[db][4 * a4 + q] * r;
          put_part<TO>(p.opart, (pbase + col) * D + d, v);
        }
    }
  } else {
    // Merge the waves in LDS, in a fixed order, then publish.
    float* so = so_base;                                  // [wave][32][D]
    float* sm = sml;                                      // [wave][32]
    float* sl = sml + kWaves * 32;                        // [wave][32]
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
      const float r = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] *= r;
      put_part<TO>(p.opart, (pbase + n) * D + d, acc);
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
  // splits first (one memory round trip per 16 splits), then the chunk's
  // largest maximum, then its weights 2^(m_s - M) l_s and the weighted sum of
  // the normalised partials, without branches; chunks combine online.
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
        mv[u] = s0 + u < ns ? get1(&p.mpart[r]) : -INFINITY;
        lv[u] = get1(&p.lpart[r]);
        ov[u] = get_part<TO>(p.opart, r * D + d);
      }
      float Mc = M;
#pragma unroll
      for (int u = 0; u < CH; ++u) Mc = fmaxf(Mc, mv[u]);
      // (no split with a visible key yet: nothing to scale)
      const float sc = Mc == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(M - Mc);
      L *= sc;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] *= sc;
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        // a split with no visible key has m = -inf and weight 0
        const float wgt = __builtin_amdgcn_exp2f(mv[u] - Mc) * lv[u];
        const float w = mv[u] == -INFINITY ? 0.0f : wgt;
        L += w;
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = fmaf(w, ov[u][c], acc[c]);
      }
      M = Mc;
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

template <typename T, typename TO, int D, int kWaves>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * kWaves, 64 * kWaves)))
decode_kernel(FwdArgs a, DecodeArgs p) {
  using E = Elem<T>;
  using V8 = typename E::vec8;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int CPR = D / 8;               // 16-byte chunks per K/V row
  constexpr int RPI = 64 / CPR;            // rows one 64-lane direct load covers
  constexpr int NL = 64 / RPI;             // direct loads per 64-row tile
  constexpr int TILE = 64 * D;             // elements of one K or V tile
  constexpr float kLag = 2.0f;             // see the rescale below (log2 units)
  // Each wave streams its own tiles through a K and a V tile of its own in
  // LDS. The cross-wave merge reuses the K tiles' bytes (32 x D floats per
  // wave).
  __shared__ __attribute__((aligned(16))) T sk_all[kWaves * TILE];
  __shared__ __attribute__((aligned(16))) T sv_all[kWaves * TILE];
  __shared__ float sml[2 * kWaves * 32];
  static_assert(sizeof(T) * TILE == 32 * D * sizeof(float), "merge area must fit a K tile");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int split = blockIdx.x, bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int64_t kvbase = (int64_t)bg * a.Nk * D;
  const T* __restrict__ Kp = (const T*)a.k + kvbase;
  const T* __restrict__ Vp = (const T*)a.v + kvbase;
  T* sk = sk_all + wave * TILE;
  T* sv = sv_all + wave * TILE;

  // Column -> (query head within the group, row): n = hh * Nq + i. Columns past
  // the packed rows read row 0 and are masked out.
  const bool cvalid = col < p.rows;
  const int ccol = cvalid ? col : 0;
  const int hh = ccol / a.Nq, qi = ccol - hh * a.Nq;
  // Column (hh, qi) sees keys [row_lo, row_hi] (none for columns past the
  // packed rows); tiles inside the bounds common to all rows,
  // [wave_lo, wave_hi], are not masked.
  const int wrow = a.window_w > 0 ? a.pos0 - a.window_w + 1 : -(1 << 30);   // row i: key >= i + wrow
  const int row_lo = cvalid ? max(a.window_lo, qi + wrow) : a.Nk;
  const int row_hi = a.causal ? min(a.pos0 + qi, a.Nk - 1) : a.Nk - 1;
  const int wave_lo = max(a.window_lo, a.Nq - 1 + wrow);
  const int wave_hi = a.causal ? min(a.pos0, a.Nk - 1) : a.Nk - 1;
  const T* Qrow = (const T*)a.q + (((int64_t)b * a.Hq + g * G + hh) * a.Nq + qi) * D;
  V8 qv[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qv[ks] = __builtin_bit_cast(V8, ld16(Qrow + 16 * ks + 8 * half));
  // rotary position embedding of the row at position pos0 + qi (K arrives rotated)
  if (a.rope.on)
    rope_lane_row<T, KS>(qv, (float)(a.pos0 + qi), half, a.rope.style, a.rope.rev_hi, a.rope.rev_lo);

  // Tiles go straight into LDS (16 bytes per lane, 1 KB per instruction) with
  // the XOR chunk swizzles and K row order of the prefill: K row r holds key
  // (r & ~31) | swap23(r & 31), V row r key r; rows past Nk clamp to the last.
  auto kswz = [](int r) { return CPR == 16 ? (r & 15) : ((r >> 1) & 7); };
  auto vswz = [](int r) { return CPR == 16 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); };
  auto load_k = [&](int t) {
    const char* base = (const char*)(Kp + (int64_t)64 * t * D);
    const int last = a.Nk - 1 - 64 * t;
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int r = RPI * u + lane / CPR, pos = lane % CPR;
      const int kk = (r & ~31) | swap23(r & 31);
      load_to_lds16(base, (uint32_t)(min(kk, last) * (D * 2) + 16 * (pos ^ kswz(r))), sk + RPI * u * D);
    }
  };
  auto load_v = [&](int t) {
    const char* base = (const char*)(Vp + (int64_t)64 * t * D);
    const int last = a.Nk - 1 - 64 * t;
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int r = RPI * u + lane / CPR, pos = lane % CPR;
      load_to_lds16(base, (uint32_t)(min(r, last) * (D * 2) + 16 * (pos ^ vswz(r))), sv + RPI * u * D);
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[db][j] = 0.0f;
  float m = -INFINITY, l = 0.0f;

  // This workgroup's tiles: [t0, t1); wave w takes t0 + w, t0 + w + kWaves, ...
  // K of the next tile is loaded once S of this one has read its K tile, V
  // of the next once P V has read its V tile.
  const int t0 = p.t_lo + split * p.tiles_per_wg;
  const int t1 = min(t0 + p.tiles_per_wg, p.t_hi);
  int t = t0 + wave;
  if (t < t1) {
    load_k(t);
    load_v(t);
  }
  // Claim the arrival counter in two parts: its read is issued here, behind
  // the tile loads, and the swap (if any) after the tiles, when the read has
  // long returned; neither waits on the critical path.
  unsigned long long ctr_seen = 0;
  if (tid == 0) ctr_seen = __hip_atomic_load(p.ctr + bg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  auto tile = [&](int t) {
    const int k0 = t * 64;
    const bool more = t + kWaves < t1;
    const bool first = t == t0 + wave;
    // The direct loads are not tracked by the compiler, so these waits are
    // ours. A wave's first tile: only its K tile has to have landed here (the
    // NL loads of V were issued after it, and in wave 0 the counter read
    // after those); later tiles wait for everything issued before.
    if (first) {
      if (wave == 0)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(NL + 1));
      else
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(NL));
    } else {
      vmem_wait_all();
    }
    // S^T = K Q^T: four independent accumulators (even/odd k-steps).
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
      for (int mb = 0; mb < 2; ++mb) {
        const int r = 32 * mb + col;
        const V8 ka = *(const V8*)&sk[r * D + 8 * ((2 * ks + half) ^ kswz(r))];
        s[mb][ks & 1] = E::mma(ka, qv[ks], s[mb][ks & 1]);
      }
    // every K read of this wave has returned before the next K tile lands
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    if (more) load_k(t + kWaves);
    float sc[2][16];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) sc[mb][j] = s[mb][0][j] + s[mb][1][j];
    // Only tiles that straddle a bound are masked (columns past the packed
    // rows compute finite values that are never published).
    if (k0 < wave_lo || k0 + 63 > wave_hi) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = k0 + 32 * mb + 16 * (j >> 3) + 8 * half + (j & 7);
          const bool vis = key >= row_lo && key <= row_hi;
          if (!vis) sc[mb][j] = -INFINITY;
        }
    }
    float mx = sc[0][0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sc[0][j]);
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sc[1][j]);
    mx = halves_max(mx) * a.c;
    // O and l are rescaled only when a column's maximum runs more than kLag
    // ahead of m; the weights meanwhile stay below 2^kLag.
    if (__builtin_amdgcn_ballot_w64(mx > m + kLag)) {
      asm volatile("" ::: "memory");
      const float m_new = fmaxf(m, mx);
      const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
      m = m_new;
    }
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
    l += halves_sum(lsum);
    // The first tile's V has landed (a next K tile, if any, was issued after it).
    if (first) {
      if (more)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(NL));
      else
        vmem_wait_all();
    }
    // O^T += V^T P^T; the V^T operands come through transpose reads (as in the
    // prefill): lane r of a 16-lane group names key kb + r/4 at channel d0 + 4 (r % 4).
    const int gq = lane >> 4, rr = lane & 15;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          s16x4 part[2];
#pragma unroll
          for (int rd = 0; rd < 2; ++rd) {
            const int key = 32 * mb + 16 * tt + 8 * (gq >> 1) + 4 * rd + (rr >> 2);
            const int d0 = 32 * db + 16 * (gq & 1) + 4 * (rr & 3);
            part[rd] = lds_read_tr16(&sv[key * D + 8 * ((d0 >> 3) ^ vswz(key)) + (d0 & 7)]);
          }
          const s16x8 both = {part[0][0], part[0][1], part[0][2], part[0][3],
                              part[1][0], part[1][1], part[1][2], part[1][3]};
          oacc[db] = E::mma(__builtin_bit_cast(V8, both), pv[mb][tt], oacc[db]);
        }
    }
    if (more) {
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): V reads returned
      load_v(t + kWaves);
    }
  };
  for (; t < t1; t += kWaves) tile(t);
  decode_finish<TO, D, kWaves>(a, p, m, l, oacc, (float*)sk_all, sml, ctr_seen);
}

// Decode over a quantised KV cache: K as INT8 codes and V as FP8 E4M3 codes,
// each with one fp32 scale per 64-key block of a key/value head (what
// attn_quantize_qk and attn_quantize_v write). This is the "INT8 QK . FP8 PV"
// recipe of the table in section 1 of "Attention kernels on a home RTX 5080"
// applied to the cache, which halves the bytes decode streams. Same split,
// tiles and merge as decode_kernel; per tile:
//   S_int^T = Kc Qc^T             i8 MFMA 32x32x32, exact int32 (Q is
//                                 quantised here with the same per-block
//                                 recipe: a head's Nq <= 32 rows are one block)
//   z = S_int * s_q * s_k * scale * log2(e)     (log2 units)
//   P^ = E4M3(448 * 2^-(margin + 3) * 2^(z - m) * s_v / s_ref)
//   O_acc += Vc^T P^T              fp8 MFMA 32x32x64, fp32 accumulation
//   l += sum of 2^(z - m) (unquantised)
// m is a running maximum allowed to trail the scores by up to 2 (log2 units)
// and s_ref a reference V block scale allowed to trail the wave's largest by
// up to a factor 2; only when either is exceeded are they raised and O_acc
// and l rescaled. So every weight stays <= 448, and
// O = O_acc * s_ref * 2^(margin + 3) / 448 / l.
template <typename TO, int D, int kWaves>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * kWaves, 64 * kWaves)))
decode_kvq_kernel(FwdArgs a, DecodeArgs p, const int8_t* __restrict__ kc,
                  const float* __restrict__ ks, const uint8_t* __restrict__ vc,
                  const float* __restrict__ vs) {
  constexpr int KS = D / 32;            // i8 k-steps of 32 channels
  constexpr int DB = D / 32;
  constexpr int CPR = D / 16;           // 16-byte chunks per code row
  constexpr int RPI = 64 / CPR;         // code rows one 64-lane direct load covers
  constexpr int NL = 64 / RPI;          // direct loads per 64-row code tile
  constexpr int TILEB = 64 * D;         // bytes of one K or V code tile
  constexpr int CQ = D / 8;             // 16-byte chunks per 16-bit Q row
  constexpr int NQI = 32 * CQ / 64;     // direct loads for 32 Q rows
  static_assert(NQI % kWaves == 0, "Q rows split evenly over the waves");
  constexpr float kLog2_448 = 8.807354922057604f;
  // exp2 rounds within an ulp or so; lowering the weights by 2^-12 keeps every
  // one <= 448 (the largest E4M3 magnitude) without a clamp
  constexpr float kMargin = 2.44140625e-4f;
  constexpr float kOff = 12582912.0f;   // 1.5 * 2^23
  // lags (log2 units) of the running maximum and of the V-scale reference
  // before O is rescaled; the weights' FP8 scale is lowered by 2^(kLag + kLagV)
  constexpr float kLag = 2.0f, kLagV = 1.0f;
  // Per wave two K and two V code tiles (the tile in hand and the next one
  // stay in flight together); the cross-wave merge reuses the first half of
  // them (32 x D floats per wave). Q comes in through a staging area of its own.
  __shared__ __attribute__((aligned(16))) uint8_t lds[kWaves * 4 * TILEB];
  __shared__ __attribute__((aligned(16))) uint8_t sqst[32 * D * 2];
  __shared__ float sml[2 * kWaves * 32];
  static_assert(2 * TILEB == 32 * D * (int)sizeof(float), "merge area must fit the tiles");
  static_assert(4 * NL < 64, "outstanding loads must fit the vmcnt counter");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int split = blockIdx.x, bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int nkt = (a.Nk + 63) / 64;
  const int8_t* Kc = kc + (int64_t)bg * a.Nk * D;
  const uint8_t* Vc = vc + (int64_t)bg * a.Nk * D;
  const float* Ks = ks + (int64_t)bg * nkt;
  const float* Vs = vs + (int64_t)bg * nkt;
  // slot s of this wave: K tile at sk + 2 s TILEB, V tile TILEB above it
  uint8_t* sk = lds + wave * 4 * TILEB;

  // The G * Nq query rows of this key/value head are contiguous in Q (heads
  // g G .. g G + G - 1): column n = hh * Nq + i is row n of that block. They
  // come into LDS by direct loads (rows past the packed ones repeat the last),
  // chunk c of row n at position c ^ qswz(n).
  auto qswz = [](int n) { return CQ == 16 ? (n & 15) : ((n >> 1) & 7); };
  {
    const char* qbase = (const char*)((const TO*)a.q + ((int64_t)b * a.Hq + g * G) * a.Nq * D);
#pragma unroll
    for (int u0 = 0; u0 < NQI / kWaves; ++u0) {
      const int u = u0 * kWaves + wave;
      const int n = (64 * u + lane) / CQ, pos = lane % CQ;
      load_to_lds16(qbase, (uint32_t)((min(n, p.rows - 1) * D + 8 * (pos ^ qswz(n))) * 2),
                    sqst + 1024 * u);
    }
  }

  // K code row r holds key 32 h + 16 blk + 4 a + c for r = 32 blk + 8 a + 4 h + c
  // (lane half h's 32 scores are keys 32 h .. 32 h + 31 in B-operand order); V
  // code rows are keys in order. Chunk c of a row sits at c ^ kswz(r) or
  // c ^ vswz(r): the operand reads of a 16- or 32-lane group hit distinct
  // banks. Rows past Nk clamp to the last key (masked).
  auto kswz = [](int r) { return CPR == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3); };
  auto vswz = [](int r) { return CPR == 8 ? (r & 7) : 2 * ((r >> 2) & 1); };
  auto load_k = [&](int t, int slot) {
    const int8_t* base = Kc + (int64_t)64 * t * D;
    uint8_t* dst = sk + 2 * TILEB * slot;
    const int last = a.Nk - 1 - 64 * t;
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int r = RPI * u + lane / CPR, pos = lane % CPR;
      const int key = 32 * ((r >> 2) & 1) + 16 * (r >> 5) + 4 * ((r >> 3) & 3) + (r & 3);
      load_to_lds16(base, (uint32_t)(min(key, last) * D + 16 * (pos ^ kswz(r))), dst + RPI * u * D);
    }
  };
  auto load_v = [&](int t, int slot) {
    const uint8_t* base = Vc + (int64_t)64 * t * D;
    uint8_t* dst = sk + 2 * TILEB * slot + TILEB;
    const int last = a.Nk - 1 - 64 * t;
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int r = RPI * u + lane / CPR, pos = lane % CPR;
      load_to_lds16(base, (uint32_t)(min(r, last) * D + 16 * (pos ^ vswz(r))), dst + RPI * u * D);
    }
  };

  const int t0 = p.t_lo + split * p.tiles_per_wg;
  const int t1 = min(t0 + p.tiles_per_wg, p.t_hi);
  int t = t0 + wave;
  float kst = 0.0f, vst = 0.0f;   // block scales of the tile in hand
  // this wave's first two tiles go in flight behind its Q loads, which must
  // land first (loads complete in issue order)
  if (t + kWaves < t1) {
    load_k(t, 0);
    load_v(t, 0);
    load_k(t + kWaves, 1);
    load_v(t + kWaves, 1);
    kst = Ks[t];
    vst = Vs[t];
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(4 * NL));
  } else if (t < t1) {
    load_k(t, 0);
    load_v(t, 0);
    kst = Ks[t];
    vst = Vs[t];
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * NL));
  } else {
    vmem_wait_all();
  }
  __syncthreads();   // every wave's share of Q is in LDS

  // Q codes while the first tiles are in flight. Lane (col, half) holds, for
  // k-step k, channels 32 k + 16 half + (0..15) of row col (B-operand order).
  const bool cvalid = col < p.rows;
  const int ccol = cvalid ? col : 0;
  const int hh = ccol / a.Nq, qi = ccol - hh * a.Nq;
  // Column (hh, qi) sees keys [row_lo, row_hi] (none for columns past the
  // packed rows); tiles inside the bounds common to all rows,
  // [wave_lo, wave_hi], are not masked.
  const int wrow = a.window_w > 0 ? a.pos0 - a.window_w + 1 : -(1 << 30);   // row i: key >= i + wrow
  const int row_lo = cvalid ? max(a.window_lo, qi + wrow) : a.Nk;
  const int row_hi = a.causal ? min(a.pos0 + qi, a.Nk - 1) : a.Nk - 1;
  const int wave_lo = max(a.window_lo, a.Nq - 1 + wrow);
  const int wave_hi = a.causal ? min(a.pos0, a.Nk - 1) : a.Nk - 1;
  float x[KS][16];
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < KS; ++k)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int ch = 4 * k + 2 * half + c;
      unpack8<TO>(*(const u32x4*)&sqst[(ccol * CQ + (ch ^ qswz(ccol))) * 16], &x[k][8 * c]);
    }
#pragma unroll
  for (int k = 0; k < KS; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[k][i]));
  amax = halves_max(amax);
  float hmax = 0.0f;   // over the Nq rows of query head hh
  for (int j = 0; j < a.Nq; ++j) hmax = fmaxf(hmax, __shfl(amax, hh * a.Nq + j, 64));
  // fp32, correctly rounded: the block recipe of the INT8 quantiser
  const float sq = hmax > 0.0f ? hmax / 127.0f : 0.0f;
  const float qinv = hmax > 0.0f ? 127.0f / hmax : 0.0f;
  i32x4 qv[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k)
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float r = __builtin_rintf(x[k][4 * w4 + i] * qinv);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        w |= ((uint32_t)(int)r & 0xffu) << (8 * i);
      }
      qv[k][w4] = (int)w;
    }
  const float cfq = sq * a.c;

  unsigned long long ctr_seen = 0;
  if (tid == 0) ctr_seen = __hip_atomic_load(p.ctr + bg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[db][j] = 0.0f;
  float m = -INFINITY, l = 0.0f;
  float lref = -INFINITY;   // log2 of the largest V block scale seen so far

  // The int32 scores start from 0x4B400000, the bit pattern of 1.5 * 2^23:
  // |S| < 2^22, so each accumulator read as a float is exactly 1.5 * 2^23 + S.
  i32x16 magic;
#pragma unroll
  for (int j = 0; j < 16; ++j) magic[j] = 0x4B400000;
  asm volatile("" : "+v"(magic));

  auto tile = [&](int t, int slot) {
    const int k0 = t * 64;
    const bool next = t + kWaves < t1;       // loads in flight behind this tile's
    const bool more = t + 2 * kWaves < t1;   // a tile to load into this slot
    const float kst_c = kst, vst_c = vst;
    if (next) {
      // uniform index: scalar loads, which do not wait behind the tile loads
      const int tn = __builtin_amdgcn_readfirstlane(t + kWaves);
      kst = Ks[tn];
      vst = Vs[tn];
    }
    // this tile's code tiles have landed (untracked loads; only the next
    // tile's may still be in flight)
    if (next)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * NL));
    else
      vmem_wait_all();
    const uint8_t* tk = sk + 2 * TILEB * slot;
    const uint8_t* tv = tk + TILEB;
    i32x16 s[2];
#pragma unroll
    for (int k = 0; k < KS; ++k)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int r = 32 * mb + col;
        const i32x4 ka = *(const i32x4*)&tk[r * D + 16 * ((2 * k + half) ^ kswz(r))];
        s[mb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka, qv[k], k == 0 ? magic : s[mb], 0, 0, 0);
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): K reads returned
    if (more) load_k(t + 2 * kWaves, slot);

    // A block of zero codes has scale 0; the floor keeps masked scores at
    // -inf (-inf * 0 would be NaN) and changes nothing else.
    const float cf = fmaxf(cfq * kst_c, 1.17549435e-38f);
    float sf[2][16];   // kOff + S, exact
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) sf[mb][j] = __builtin_bit_cast(f32x16, s[mb])[j];
    // Only tiles that straddle a bound are masked (columns past the packed
    // rows compute finite values that are never published).
    if (k0 < wave_lo || k0 + 63 > wave_hi) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = k0 + 32 * half + 16 * mb + 4 * (j >> 2) + (j & 3);
          const bool vis = key >= row_lo && key <= row_hi;
          if (!vis) sf[mb][j] = -INFINITY;
        }
    }
    float mx = sf[0][0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sf[0][j]);
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sf[1][j]);
    mx = (halves_max(mx) - kOff) * cf;   // exact subtraction
    const float lv = __builtin_amdgcn_logf(fmaxf(vst_c, 1.17549435e-38f));
    // O and l are rescaled only when a column's maximum runs more than kLag
    // ahead of m, or the V scale more than kLagV ahead of the reference; the
    // weights' FP8 scale leaves room for both, so none exceeds 448 meanwhile.
    if (__builtin_amdgcn_ballot_w64(mx > m + kLag) || lv > lref + kLagV) {
      asm volatile("" ::: "memory");
      const float m_new = fmaxf(m, mx);
      const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m - m_new);
      const float lref_new = fmaxf(lref, lv);
      const float ab = alpha * __builtin_amdgcn_exp2f(lref - lref_new);   // 0 before any tile
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] *= ab;
      m = m_new;
      lref = lref_new;
    }
    const float bias = (lv - lref) + (kLog2_448 - kMargin - kLag - kLagV);
    const float mu = (m == -INFINITY ? 0.0f : m) - bias;
    // exponent = S cf - mu = (kOff + S) cf - (kOff cf + mu): one FMA per score.
    // Rounding kOff cf + mu moves every exponent of the tile by at most
    // 2^-24 |kOff cf + mu| < 0.9 cf + 2^-21, far below the INT8 rounding of
    // the scores and within the headroom to the E4M3 rounding boundary 464 for
    // cf < 0.03; larger factors take the exact form.
    float C = fmaf(kOff, cf, mu);
    if (cf >= 0.03f) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) sf[mb][j] -= kOff;
      C = mu;
    }
    i32x8 pb;
    float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float e[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          e[k] = __builtin_amdgcn_exp2f(fmaf(sf[mb][4 * q4 + k], cf, -C));
          ls[k] += e[k];
        }
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], pk, true);
        pb[4 * mb + q4] = pk;
      }
    // the denominator takes the weights back to their unscaled values
    l += halves_sum((ls[0] + ls[1]) + (ls[2] + ls[3])) * __builtin_amdgcn_exp2f(-bias);

    // O^T += V^T P^T: lane 16 g + tt of a transpose read names key
    // 32 (g / 2) + 8 q + tt / 2 at channels 32 db + 16 (g % 2) + 8 (tt % 2) + (0..7);
    // four reads give lane (col, half) channel 32 db + col of keys 32 half + (0..31).
    const int gq = lane >> 4, tt = lane & 15;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int c16 = 2 * db + (gq & 1);
      i32x8 va;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int key = 32 * (gq >> 1) + 8 * q + (tt >> 1);
        const u32x2 w = lds_read_tr8(&tv[key * D + 16 * (c16 ^ vswz(key)) + 8 * (tt & 1)]);
        va[2 * q] = (int)w[0];
        va[2 * q + 1] = (int)w[1];
      }
      oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, oacc[db], 0, 0, 0, 127, 0, 127);
    }
    if (more) {
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): V reads returned
      load_v(t + 2 * kWaves, slot);
    }
  };
  for (int i = 0; t < t1; t += kWaves, ++i) tile(t, __builtin_amdgcn_readfirstlane(i & 1));

  // back to V units: O_acc * s_ref * 2^(margin + lags) / 448
  const float fac = lref == -INFINITY
                        ? 0.0f
                        : __builtin_amdgcn_exp2f(lref + (kMargin + kLag + kLagV)) * (1.0f / 448.0f);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[db][j] *= fac;
  decode_finish<TO, D, kWaves>(a, p, m, l, oacc, (float*)lds, sml, ctr_seen);
}

DecodeArgs decode_args(const FwdArgs& a, const DecodePlan& pl, void* ws) {
  DecodeArgs p;
  p.rows = pl.rows;
  p.t_lo = pl.t_lo;
  p.t_hi = pl.t_lo + pl.ntiles;
  p.nsplit = pl.nsplit;
  p.tiles_per_wg = pl.tiles_per_wg;
  const int64_t nrow = (int64_t)a.B * a.Hkv * pl.nsplit * pl.rows;
  p.ctr = (unsigned long long*)ws;
  p.opart = (float*)((char*)ws + pl.ctr_bytes);
  p.mpart = p.opart + nrow * a.D;
  p.lpart = p.mpart + nrow;
  p.gen = next_generation();
  return p;
}

template <typename T, typename TO, int D>
hipError_t launch_t(const FwdArgs& a, const DecodePlan& pl, void* ws, hipStream_t s) {
  const DecodeArgs p = decode_args(a, pl, ws);
  const dim3 grid(pl.nsplit, a.B * a.Hkv);
  if (pl.waves == 1)
    hipLaunchKernelGGL((decode_kernel<T, TO, D, 1>), grid, dim3(64), 0, s, a, p);
  else if (pl.waves == 2)
    hipLaunchKernelGGL((decode_kernel<T, TO, D, 2>), grid, dim3(128), 0, s, a, p);
  else
    hipLaunchKernelGGL((decode_kernel<T, TO, D, 4>), grid, dim3(256), 0, s, a, p);
  return hipGetLastError();
}

template <typename TO, int D>
hipError_t launch_kvq_t(const FwdArgs& a, const DecodePlan& pl, const int8_t* kc,
                        const float* ks, const uint8_t* vc, const float* vs, void* ws,
                        hipStream_t s) {
  if (pl.waves != 4) return hipErrorInvalidConfiguration;
  const DecodeArgs p = decode_args(a, pl, ws);
  const dim3 grid(pl.nsplit, a.B * a.Hkv);
  hipLaunchKernelGGL((decode_kvq_kernel<TO, D, 4>), grid, dim3(256), 0, s, a, p, kc, ks, vc, vs);
  return hipGetLastError();
}

}  // namespace

// A different generation for every launch, from a per-process random start
// (so that counters left in a reused workspace by another process never match).
unsigned long long next_generation() {
  static std::atomic<unsigned long long> counter{
      ((unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count() ^
       (unsigned long long)(uintptr_t)&counter) * 0x9E3779B97F4A7C15ull};
  const unsigned long long g = counter.fetch_add(1, std::memory_order_relaxed);
  return (g % ((1ull << 40) - 1)) + 1;
}

bool decode_supported(const FwdArgs& a) {
  return (int64_t)(a.Hq / a.Hkv) * a.Nq <= 32 && (int64_t)a.B * a.Hkv <= 65535;
}

bool decode_eligible(const FwdArgs& a) {
  const KeyRange r = key_range(a);
  return decode_supported(a) && r.hi - r.lo >= 512;
}

DecodePlan decode_plan(const FwdArgs& a, int splits) {
  DecodePlan p;
  const KeyRange r = key_range(a);
  p.rows = (a.Hq / a.Hkv) * a.Nq;
  p.t_lo = r.lo / 64;
  const int t_hi = r.hi > r.lo ? (r.hi + 63) / 64 : p.t_lo;
  p.ntiles = t_hi - p.t_lo;
  if (splits > 0) {
    // At most `splits` workgroups, each a contiguous range of tiles, with up
    // to four waves (one tile each per step).
    const int ns = splits < kMaxRequestedSplits ? splits : kMaxRequestedSplits;
    const int per = p.ntiles > 0 ? (p.ntiles + ns - 1) / ns : 1;
    p.waves = per >= 4 ? 4 : (per >= 2 ? 2 : 1);
    p.tiles_per_wg = per;
  } else {
    // Four waves (one 64-key tile each) per workgroup and at most kMaxSplits
    // workgroups per key/value head; longer ranges give each wave several
    // tiles. Fewer, fuller workgroups keep the final merge (on the critical
    // path, in the last workgroup) short.
    p.waves = 4;
    // Up to two tiles per wave, 16 splits merge faster than 32 splits run a
    // second tile: 32 only for longer ranges.
    const int cap = p.ntiles <= 2 * p.waves * 16 ? 16 : kMaxSplits;
    const int per_wave = (p.ntiles + p.waves * cap - 1) / (p.waves * cap);
    p.tiles_per_wg = p.waves * (per_wave < 1 ? 1 : per_wave);
  }
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

hipError_t launch_decode_kvq(const FwdArgs& a, const DecodePlan& p, const int8_t* kc,
                             const float* ks, const uint8_t* vc, const float* vs, int elem,
                             void* ws, hipStream_t s) {
  if (elem == 2)
    return a.D == 64 ? launch_kvq_t<__bf16, 64>(a, p, kc, ks, vc, vs, ws, s)
                     : launch_kvq_t<__bf16, 128>(a, p, kc, ks, vc, vs, ws, s);
  return a.D == 64 ? launch_kvq_t<_Float16, 64>(a, p, kc, ks, vc, vs, ws, s)
                   : launch_kvq_t<_Float16, 128>(a, p, kc, ks, vc, vs, ws, s);
}

}  // namespace attn
