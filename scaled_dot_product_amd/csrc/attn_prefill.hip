// attn_prefill.hip — exact-mode flash attention forward for gfx950.
//
// One workgroup of 4 waves owns 128 query rows of one (batch, query head);
// each wave owns 32 rows, two workgroups share a CU (2 waves per SIMD; three
// at head dim 64). The
// workgroup streams the visible keys of its key/value head in tiles of 64:
// K and V go from HBM/L2 straight into LDS (global_load_lds, 16 bytes per
// lane, no register staging) in row-major tiles with an XOR swizzle of the
// 16-byte chunks, and every wave runs
//     S^T = K Q^T                   (bf16/f16 MFMA, fp32 accumulation)
//     mask (boundary tiles only)
//     online softmax in exp2 units  (running max, running sum, lazy rescale)
//     O^T += V^T P^T                (P rounded to the operand type; the V^T
//                                   operands come from the row-major V tile
//                                   through ds_read_b64_tr_b16 transposes)
// before the epilogue divides by the running sum. The N x N score matrix is
// never stored.
//
// The loop is software-pipelined so that both halves of the work always have
// matrix-core instructions beside them: iteration i first accumulates P V of
// tile i-1 on the MFMA pipe while the vector ALU exponentiates half of tile
// i, then computes S of tile i+1 beside the other half. The weights are
// taken against the running maximum as it stands; the tile's row maxima are
// computed only in the rare branch that raises it.
// K tiles are loaded two iterations ahead, V tiles one (both issued at the
// start of the S half); K and V use separate LDS double buffers and one
// barrier per iteration suffices. The instruction
// interleave inside each half is fixed with scheduling-group barriers.
//
// 64-key tiles follow the 64-position KV chunk of "perf(metal): widen
// four-row flash KV tiles" (its 128-position chunk is a different trade-off,
// for a four-row shape on another GPU).
#include <type_traits>

#include "attn_common.hpp"
#include "attn_internal.hpp"

namespace attn {

namespace {

// The running maximum is raised only when some weight against it could
// exceed this bound (a lane's partial row sum of a tile does); until then the
// weights stay <= 2^12, which bf16, f16 and fp32 hold in range. Exactness is
// unaffected: numerator and denominator share the stale maximum.
constexpr float kLazyMax = 4096.0f;

// Scheduling-group masks (see the AMDGPU backend's sched_group_barrier).
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// LDS operand reads issued ahead of the MFMA that consumes them (K reads in
// the S half, V transpose-read pairs in the P V half).
#ifndef PREFILL_KPRE
#define PREFILL_KPRE 4
#endif
#ifndef PREFILL_VPRE
#define PREFILL_VPRE 4
#endif
constexpr int kKPre = PREFILL_KPRE;
constexpr int kVPre = PREFILL_VPRE;

// The split of the query tiles' key ranges (one launch; ns = 1: no split).
struct SplitArgs {
  int ns;                    // parts per query tile (fused merge; 1: none)
  int halves;                // > 0: the last `halves` tiles run as two halves, merged
                             // by prefill_merge_kernel afterwards (ns is then 1)
  unsigned long long* ctr;   // [tiles] arrivals: (generation << 24) | count
  unsigned long long gen;    // in [1, 2^40), different for every launch
  void* opart;               // ns > 1: [tiles][ns][rows][D], halves: [halves][2][rows][D]
                             // of O_s / l_s in the output type
  float* mlpart;             // the same slots x [2]: m_s (exp2 units), l_s
};

// The balanced schedule: `tiles` query tiles of which the last `halves` run
// as two halves, tiles + halves workgroups in all. Workgroup ids go round the
// 8 XCDs (id % 8) and, inside an XCD, fill one slot of every CU before the
// next; so each XCD's share lists its whole tiles first and its halves last,
// which puts the halves into the last slot the CUs fill: with as many jobs as
// slots, every CU then runs the same work. Returns the tile; part is -1 for
// a whole tile, else 0 or 1.
__device__ __forceinline__ int balanced_job(int id, int tiles, int halves, int& part) {
  const int jobs = tiles + halves, whole = tiles - halves;
  const int x = id % 8, local = id / 8;
  const int wx = whole / 8 + (x < whole % 8 ? 1 : 0);
  const int w0 = x * (whole / 8) + min(x, whole % 8);
  if (local < wx) {
    part = -1;
    return w0 + local;
  }
  const int j0 = x * (jobs / 8) + min(x, jobs % 8);   // this XCD's first job
  const int h = (j0 - w0) + (local - wx);              // half index, XCD by XCD
  part = h & 1;
  return whole + (h >> 1);
}

// Store 4 consecutive channels of one row in the output element type.
template <typename TO>
__device__ __forceinline__ void put4(TO* p, const float (&v)[4]) {
  if constexpr (sizeof(TO) == 4) {
    *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
  } else {
    TO o4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) o4[r] = Elem<TO>::from_float(v[r]);
    *(u32x2*)p = *(const u32x2*)o4;
  }
}
template <typename TO>
__device__ __forceinline__ void get4(const TO* p, float (&v)[4]) {
  if constexpr (sizeof(TO) == 4) {
    const f32x4 x = *(const f32x4*)p;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = x[r];
  } else {
    const u32x2 x = *(const u32x2*)p;
    const TO* e = (const TO*)&x;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = (float)e[r];
  }
}

// The end of one part of a split query tile: publish the normalised partial
// (O / l in the output type, m and l in fp32), arrive, and in the tile's
// last part to arrive merge the ns partials with log-sum-exp weights
// 2^(m_s - M) l_s and write O. Lane (col, half) holds channels
// 32 db + 8 a4 + 4 half + (0..3) of row qrow, as in the plain epilogue.
template <typename TO, int D, int BM>
__device__ __forceinline__ void split_finish(const FwdArgs& a, const SplitArgs& sp,
                                             unsigned long long ctr_seen, int tile, int part,
                                             int q0, int qrow, float l, float inv, float m_run,
                                             const f32x16 (&oacc)[D / 32]) {
  constexpr int DB = D / 32;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  if (tid == 0 && (ctr_seen >> 24) != sp.gen) atomicCAS(sp.ctr + tile, ctr_seen, sp.gen << 24);
  TO* op = (TO*)sp.opart;
  const int64_t slot0 = (int64_t)tile * sp.ns * BM + (qrow - q0);   // this row, part 0
  if (qrow < a.Nq) {
    const int64_t r = slot0 + (int64_t)part * BM;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = oacc[db][4 * a4 + q] * inv;
        put4<TO>(op + r * D + 32 * db + 8 * a4 + 4 * half, v);
      }
    if (half == 0) {
      sp.mlpart[2 * r] = m_run;
      sp.mlpart[2 * r + 1] = l;
    }
  }
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);   // every partial store of this thread acknowledged
  __syncthreads();
  if (tid == 0) s_last = arrive_last(sp.ctr + tile, sp.ns);
  __syncthreads();
  if (!s_last) return;
  if (qrow < a.Nq) {
    float M = -INFINITY;
    for (int s = 0; s < sp.ns; ++s) M = fmaxf(M, sp.mlpart[2 * (slot0 + (int64_t)s * BM)]);
    float L = 0.0f;
    float acc[DB][4][4] = {};
    for (int s = 0; s < sp.ns; ++s) {
      const int64_t r = slot0 + (int64_t)s * BM;
      const float ms = sp.mlpart[2 * r], ls = sp.mlpart[2 * r + 1];
      // a part with no visible key has m = -inf and weight 0
      const float w = ms == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms - M) * ls;
      L += w;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          float v[4];
          get4<TO>(op + r * D + 32 * db + 8 * a4 + 4 * half, v);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[db][a4][q] = fmaf(w, v[q], acc[db][a4][q]);
        }
    }
    const float invL = L > 0.0f ? 1.0f / L : 0.0f;
    TO* orow = (TO*)a.o + ((int64_t)(tile / ((a.Nq + BM - 1) / BM)) * a.Nq + qrow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = acc[db][a4][q] * invL;
        put4<TO>(orow + 32 * db + 8 * a4 + 4 * half, v);
      }
  }
  if (tid == 0) __hip_atomic_store(sp.ctr + tile, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Head dim 128 runs 2 waves per SIMD; head dim 64 fits 3 (168 VGPRs, a few
// spills outside the loop), which measured 1-3 % faster on the SDXL shape
// and on long sequences.
template <typename T, typename TO, int D, int W>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * W, 64 * W),
                               amdgpu_waves_per_eu(D == 64 ? 3 : 2, D == 64 ? 3 : 2)))
prefill_kernel(FwdArgs a, int ntq, SplitArgs sp) {
  using E = Elem<T>;
  using V8 = typename E::vec8;
  constexpr int BM = 32 * W;       // W waves of 32 query rows
  constexpr int KS = D / 16;       // 16-wide k-steps of Q K^T
  constexpr int DB = D / 32;       // 32-row blocks of O^T
  constexpr int CPR = D / 8;       // 16-byte chunks per K/V row
  constexpr int RPI = 64 / CPR;    // rows one 64-lane direct load covers
  __shared__ __attribute__((aligned(16))) T sk[2][64 * D];
  __shared__ __attribute__((aligned(16))) T sv[2][64 * D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int half = lane >> 5, col = lane & 31;
  // Workgroup -> (query tile, part of its key range); the parts of a tile
  // run on one XCD.
  int tile, part, nparts;
  if (sp.halves > 0) {
    tile = balanced_job(blockIdx.x, gridDim.x - sp.halves, sp.halves, part);
    nparts = part < 0 ? 1 : 2;
    part = part < 0 ? 0 : part;
  } else {
    const int job = xcd_remap(blockIdx.x, gridDim.x);
    tile = job / sp.ns;
    part = job - tile * sp.ns;
    nparts = sp.ns;
  }
  const int bh = tile / ntq, qt_in = tile - bh * ntq;
  // Causal rows see more keys the later they sit: a head's heaviest q-tiles
  // are dispatched first, so the light ones fill the end of the grid.
  const int qt = a.causal ? ntq - 1 - qt_in : qt_in;
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const int q0 = qt * BM;
  const int64_t kvbase = ((int64_t)b * a.Hkv + g) * a.Nk * D;
  const T* __restrict__ Qp = (const T*)a.q + (int64_t)bh * a.Nq * D;
  const T* __restrict__ Kp = (const T*)a.k + kvbase;
  const T* __restrict__ Vp = (const T*)a.v + kvbase;
  TO* __restrict__ Op = (TO*)a.o + (int64_t)bh * a.Nq * D;

  // Visible keys of this workgroup's rows, as tiles [t_lo, t_lo + nt).
  const int qlast = min(q0 + BM, a.Nq) - 1;
  // (a per-row window: row q0 has the lowest bound)
  const int kv_lo = a.window_w > 0 ? max(a.window_lo, a.pos0 + q0 - a.window_w + 1) : a.window_lo;
  const int kv_hi = a.causal ? min(a.Nk, a.pos0 + qlast + 1) : a.Nk;
  const int t_lo0 = kv_lo / 64;
  const int nt0 = kv_hi > kv_lo ? (kv_hi + 63) / 64 - t_lo0 : 0;
  // this part's tiles: [t_lo, t_lo + nt), ns nearly equal parts (some may be empty)
  const int chunk = (nt0 + nparts - 1) / nparts;
  const int t_lo = t_lo0 + part * chunk;
  const int nt = max(0, min(chunk, nt0 - part * chunk));

  // Q^T as B operands, held for the whole loop: column = query row,
  // lane half h of k-step ks holds d = 16 ks + 8 h + (0..7).
  const int qw0 = q0 + wave * 32;   // first row of this wave
  const int qrow = qw0 + col;
  V8 qv[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 raw = {0, 0, 0, 0};
    if (qrow < a.Nq) raw = ld16(Qp + (int64_t)qrow * D + 16 * ks + 8 * half);
    qv[ks] = __builtin_bit_cast(V8, raw);
  }
  // rotary position embedding of the row at position pos0 + qrow, once per
  // workgroup in registers (K arrives rotated)
  if (a.rope.on)
    rope_lane_row<T, KS>(qv, (float)(a.pos0 + qrow), half, a.rope.style, a.rope.rev_hi, a.rope.rev_lo);
  // a split call: the tile's arrival counter, read now, claimed after the tiles
  unsigned long long ctr_seen = 0;
  if (sp.ns > 1 && tid == 0)
    ctr_seen = __hip_atomic_load(sp.ctr + tile, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // LDS tiles are 64 unpadded rows of D elements; chunk c of row r sits at
  // chunk position c ^ swz(r). K row r holds key (r & ~31) | swap23(r & 31)
  // (so P^T lands in B-operand order), V row r holds key r. The swizzles make
  // the 16 lanes of a K operand read (16 rows, one logical chunk) and the 32
  // lanes of a V transpose read (4 rows x 8 chunks) hit distinct banks.
  auto kswz = [](int r) { return CPR == 16 ? (r & 15) : ((r >> 1) & 7); };
  auto vswz = [](int r) { return CPR == 16 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); };
  // Direct loads: a tile takes NLK instructions of RPI rows each for K and as
  // many for V (lane i -> row i / CPR, chunk position i % CPR). With at least
  // W of them, wave w loads NL consecutive instructions of each tile; with
  // fewer (head dim 64, 8 waves), waves 0 .. NLK-1 load K and the last NLK
  // waves load V, one instruction each. The per-lane byte offsets inside a
  // tile are loop invariant; the tile enters as a uniform base pointer. In
  // the ragged last tile, rows past Nk are clamped to the last row (finite
  // values; masked).
  constexpr int NLK = 64 / RPI;
  constexpr bool kSplitKV = NLK < W;
  constexpr int NL = kSplitKV ? 1 : NLK / W;   // K (and V) instructions per wave
  static_assert(kSplitKV ? 2 * NLK == W : NL * W == NLK, "direct loads must split evenly");
  const bool loads_k = !kSplitKV || wave < NLK;
  const bool loads_v = !kSplitKV || wave >= W - NLK;
  const int kr0 = kSplitKV ? RPI * wave : RPI * NL * wave;             // first K row
  const int vr0 = kSplitKV ? RPI * (wave - (W - NLK)) : RPI * NL * wave;  // first V row
  auto krow = [](int r) { return (r & ~31) | swap23(r & 31); };   // key held by K row r
  uint32_t kofs[NL], vofs[NL];
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const int pos = lane % CPR;
    const int rk = kr0 + RPI * u + lane / CPR, rv = vr0 + RPI * u + lane / CPR;
    kofs[u] = (uint32_t)(krow(rk) * (D * 2) + 16 * (pos ^ kswz(rk)));
    vofs[u] = (uint32_t)(rv * (D * 2) + 16 * (pos ^ vswz(rv)));
  }
  auto load_k = [&](int t, int buf) {
    if (!loads_k) return;
    const char* base = (const char*)(Kp + (int64_t)64 * t * D);
    const int last = a.Nk - 1 - 64 * t;   // rows past it clamp to the last key
    if (last >= 63) {
#pragma unroll
      for (int u = 0; u < NL; ++u) load_to_lds16(base, kofs[u], &sk[buf][(kr0 + RPI * u) * D]);
    } else {
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const int r0 = kr0 + RPI * u;
        const int r = r0 + lane / CPR, pos = lane % CPR;
        load_to_lds16(base, (uint32_t)(min(krow(r), last) * (D * 2) + 16 * (pos ^ kswz(r))),
                      &sk[buf][r0 * D]);
      }
    }
  };
  auto load_v = [&](int t, int buf) {
    if (!loads_v) return;
    const char* base = (const char*)(Vp + (int64_t)64 * t * D);
    const int last = a.Nk - 1 - 64 * t;
    if (last >= 63) {
#pragma unroll
      for (int u = 0; u < NL; ++u) load_to_lds16(base, vofs[u], &sv[buf][(vr0 + RPI * u) * D]);
    } else {
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const int r0 = vr0 + RPI * u;
        const int r = r0 + lane / CPR, pos = lane % CPR;
        load_to_lds16(base, (uint32_t)(min(r, last) * (D * 2) + 16 * (pos ^ vswz(r))),
                      &sv[buf][r0 * D]);
      }
    }
  };

  // Row qrow sees keys [row_lo, row_hi]: the shared lower bound, a per-row
  // window's lower edge, the causal diagonal and the last key. Only tiles
  // reaching outside the bounds common to the wave's 32 rows are masked.
  const int wrow = a.window_w > 0 ? a.pos0 - a.window_w + 1 : -(1 << 30);   // row r: key >= r + wrow
  const int row_lo = max(kv_lo, qrow + wrow);
  const int row_hi = a.causal ? min(a.pos0 + qrow, a.Nk - 1) : a.Nk - 1;
  const int wave_lo = max(kv_lo, qw0 + 31 + wrow);                            // largest row_lo
  const int wave_hi = a.causal ? min(a.pos0 + qw0, a.Nk - 1) : a.Nk - 1;     // smallest row_hi
  auto apply_mask = [&](f32x16 (&s)[2], int t) {
    const int k0 = 64 * t;
    if (k0 < wave_lo || k0 + 63 > wave_hi) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = k0 + 32 * mb + 16 * (j >> 3) + 8 * half + (j & 7);
          if (key < row_lo || key > row_hi) s[mb][j] = -INFINITY;
        }
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[db][j] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  // P^T of the previous tile, waiting for its P V product.
  V8 pprev[2][2];

  // S^T of one tile from an LDS K buffer (two independent MFMA chains).
  auto s_mma = [&](int buf, f32x16 (&s)[2]) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) s[mb][j] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int r = 32 * mb + col;
        const V8 ka = *(const V8*)&sk[buf][r * D + 8 * ((2 * ks + half) ^ kswz(r))];
        s[mb] = E::mma(ka, qv[ks], s[mb]);
      }
  };

  // O^T += V^T P^T for one tile (4 k-steps of 16 keys, DB chains). In each
  // 16-lane group the transpose read hands lane 4a + e element e of the rows
  // named by lanes a, a+4, a+8, a+12: lane r names key kb + r/4 at channel
  // d0 + 4 (r % 4), so lane (col, half) gets channel col of keys kb..kb+3,
  // i.e. four B-operand slots of P^T's order.
  auto pv_mma = [&](int vb) {
    const int gq = lane >> 4, rr = lane & 15;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          s16x4 part[2];
#pragma unroll
          for (int rd = 0; rd < 2; ++rd) {
            const int key = 32 * mb + 16 * tt + 8 * (gq >> 1) + 4 * rd + (rr >> 2);
            const int d0 = 32 * db + 16 * (gq & 1) + 4 * (rr & 3);
            const int off = key * D + 8 * ((d0 >> 3) ^ vswz(key)) + (d0 & 7);
            part[rd] = lds_read_tr16(&sv[vb][off]);
          }
          const s16x8 both = {part[0][0], part[0][1], part[0][2], part[0][3],
                              part[1][0], part[1][1], part[1][2], part[1][3]};
          const V8 va = __builtin_bit_cast(V8, both);
          oacc[db] = E::mma(va, pprev[mb][tt], oacc[db]);
        }
  };

  // One pipeline step for tile i (scores in cur): P V of tile i - 1, then S
  // of tile i + 1 into nxt, each beside half of the exponentials of tile i.
  auto step = [&](auto first, int i, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
    constexpr bool kFirst = decltype(first)::value;
    const int t = t_lo + i;
    apply_mask(cur, t);

    // Weights of one 32-key block of tile i: the B operands of P V (rounded
    // to the operand type) against the reference mu.
    auto weights = [&](int mb, float mu_, V8 (&p)[2]) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int q = 0; q < 8; ++q)
          p[tt][q] = E::from_float(__builtin_amdgcn_exp2f(fmaf(cur[mb][8 * tt + q], a.c, -mu_)));
    };

    // The weights of tile i are taken against the running maximum as it
    // stands; the row maxima of the tile are needed only when a weight may
    // exceed kLazyMax or the row has no maximum yet. A lane's partial row sum
    // bounds each of its weights, so the sums the denominator needs anyway
    // decide that, and the maxima are found in the rare rescale branch.
    // First half: P V of tile i - 1 on the MFMA pipe beside the weights of
    // the first 32 keys; second half: S of tile i + 1 beside the other 32.
    // Eight-wave tiles: waves w and w + 4 share a SIMD; the second of them
    // takes issue priority through the P V half (every wave of the CU enters
    // it together at the barrier) and gives it back for the S half. Paired
    // A/B: 0.4 % faster on the video shape, 0.5 % causal; priority in the S
    // half instead changed nothing, alternating it was 0.8 % slower, and the
    // same by workgroup slot on four-wave tiles (SDXL) 5 % slower.
    if (W == 8 && (wave & 4)) __builtin_amdgcn_s_setprio(1);
    if constexpr (!kFirst) pv_mma((i - 1) & 1);
    const float mu = m_run == -INFINITY ? 0.0f : m_run;
    V8 pa[2], pb[2];
    weights(0, mu, pa);
    float ls[4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) ls[tt] = E::sum8(pa[tt], 0.0f);
    if constexpr (!kFirst) {
      // 4 DB MFMAs with the vector work spread between them; transpose reads
      // run ahead of the MFMAs that use them.
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kVPre, 0);
#pragma unroll
      for (int k = 0; k < 4 * DB; ++k) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 48 / (4 * DB), 0);
        if (k < 4 * DB - kVPre) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      }
    }
    {
      // keep the first weights in this half (the compiler would sink them
      // into the second)
      u32x4 w0 = __builtin_bit_cast(u32x4, pa[0]);
      u32x4 w1 = __builtin_bit_cast(u32x4, pa[1]);
      asm volatile("" : "+v"(w0), "+v"(w1), "+v"(ls[0]), "+v"(ls[1]));
      pa[0] = __builtin_bit_cast(V8, w0);
      pa[1] = __builtin_bit_cast(V8, w1);
    }

    // K tile i + 2 goes where K tile i was (read before the previous
    // barrier), V tile i where V tile i - 2 was (its P V ran in the previous
    // step); both land during the S half and are published by the closing
    // barrier. Issued here rather than at the top of the step, they stay out
    // of the burst of transpose reads with which every wave of the CU starts
    // its P V half right after the barrier (3 % faster on SDXL, 1.5-2.6 %
    // on the video shape).
    if (W == 8 && (wave & 4)) __builtin_amdgcn_s_setprio(0);
    if (i + 2 < nt) load_k(t + 2, i & 1);
    load_v(t, i & 1);
    s_mma((i + 1) & 1, nxt);
    weights(1, mu, pb);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) ls[2 + tt] = E::sum8(pb[tt], 0.0f);
    // 2*KS MFMAs with the vector work spread between them; the K reads run
    // ahead of the MFMAs that use them.
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kKPre, 0);
#pragma unroll
    for (int k = 0; k < 2 * KS - kKPre; ++k) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, 48 / (2 * KS), 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, kKPre, 0);
    float lsum = (ls[0] + ls[1]) + (ls[2] + ls[3]);
    // (!(x <= y) also catches a NaN partial sum)
    if (__builtin_amdgcn_ballot_w64(!(lsum <= kLazyMax) || m_run == -INFINITY)) {
      // rare after a row's first tile; the empty asm keeps this a real branch.
      // O already holds tile i - 1 here.
      asm volatile("" ::: "memory");
      float mx = cur[0][0];
#pragma unroll
      for (int j = 1; j < 16; ++j) mx = fmaxf(mx, cur[0][j]);
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, cur[1][j]);
      mx = halves_max(mx) * a.c;
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
      m_run = m_new;
      const float mu2 = m_run == -INFINITY ? 0.0f : m_run;
      weights(0, mu2, pa);
      weights(1, mu2, pb);
      lsum = 0.0f;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) lsum = E::sum8(pb[tt], E::sum8(pa[tt], lsum));
    }
    l_run += lsum;
    // Pin the weights here: left alone, the compiler sinks the exponentials
    // past the barrier to their first use in the next step, where the P V
    // MFMAs would wait on them and no MFMA would run beside them.
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      u32x4 w0 = __builtin_bit_cast(u32x4, pa[tt]);
      u32x4 w1 = __builtin_bit_cast(u32x4, pb[tt]);
      asm volatile("" : "+v"(w0), "+v"(w1));
      pprev[0][tt] = __builtin_bit_cast(V8, w0);
      pprev[1][tt] = __builtin_bit_cast(V8, w1);
    }

    vmem_wait_all();   // this wave's direct-to-LDS loads have landed
    __syncthreads();
  };

  if (nt > 0) {
    // Prologue: K tiles 0 and 1 in LDS, S of tile 0.
    load_k(t_lo, 0);
    if (nt > 1) load_k(t_lo + 1, 1);
    vmem_wait_all();
    __syncthreads();
    f32x16 s0[2], s1[2];
    s_mma(0, s0);
    __syncthreads();   // step 0 overwrites the K buffer just read
    using First = std::true_type;
    using Later = std::false_type;
    step(First{}, 0, s0, s1);
    int i = 1;
    for (; i + 1 < nt; i += 2) {
      step(Later{}, i, s1, s0);
      step(Later{}, i + 1, s0, s1);
    }
    if (i < nt) step(Later{}, i, s1, s0);
    // P V of the last tile (its V tile was published by the last barrier).
    pv_mma((nt - 1) & 1);
  }

  // Epilogue: O = O_acc / l; rows with no visible key are written as zeros.
  const float l = halves_sum(l_run);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  if (sp.ns > 1) {
    split_finish<TO, D, BM>(a, sp, ctr_seen, tile, part, q0, qrow, l, inv, m_run, oacc);
    return;
  }
  if (nparts > 1) {
    // a half of the balanced schedule: publish; the merge kernel combines
    const int first = gridDim.x - 2 * sp.halves;   // the first tile run in halves
    if (qrow < a.Nq) {
      const int64_t r = ((int64_t)(tile - first) * 2 + part) * BM + (qrow - q0);
      TO* op = (TO*)sp.opart;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = oacc[db][4 * a4 + q] * inv;
          put4<TO>(op + r * D + 32 * db + 8 * a4 + 4 * half, v);
        }
      if (half == 0) {
        sp.mlpart[2 * r] = m_run;
        sp.mlpart[2 * r + 1] = l;
      }
    }
    return;
  }
  if (qrow < a.Nq) {
    TO* orow = Op + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d = 32 * db + 8 * a4 + 4 * half;
        if constexpr (sizeof(TO) == 4) {
          f32x4 o4;
#pragma unroll
          for (int r = 0; r < 4; ++r) o4[r] = oacc[db][4 * a4 + r] * inv;
          *(f32x4*)(orow + d) = o4;
        } else {
          TO o4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) o4[r] = Elem<TO>::from_float(oacc[db][4 * a4 + r] * inv);
          *(u32x2*)(orow + d) = *(const u32x2*)o4;
        }
      }
  }
}

// The balanced schedule's merge: one thread per (row, 4 channels) of the
// tiles run in halves (all their loads in flight at once): weights
// 2^(m_s - M) l_s, O = the weighted sum of the two normalised halves over the
// sum of the weights.
template <typename TO, int D>
__global__ void __launch_bounds__(256) prefill_merge_kernel(FwdArgs a, int ntq, int rows, int first,
                                                            int halves, SplitArgs sp) {
  constexpr int CH = D / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)halves * rows * CH) return;
  const int sidx = (int)(idx / (rows * CH));
  const int rem = (int)(idx - (int64_t)sidx * rows * CH);
  const int n = rem / CH, d = (rem - n * CH) * 4;
  const int tile = first + sidx;
  const int bh = tile / ntq, qt_in = tile - bh * ntq;
  const int qt = a.causal ? ntq - 1 - qt_in : qt_in;
  const int qrow = qt * rows + n;
  if (qrow >= a.Nq) return;
  const TO* op = (const TO*)sp.opart;
  const int64_t r0 = (int64_t)sidx * 2 * rows + n, r1 = r0 + rows;
  const float m0 = sp.mlpart[2 * r0], l0 = sp.mlpart[2 * r0 + 1];
  const float m1 = sp.mlpart[2 * r1], l1 = sp.mlpart[2 * r1 + 1];
  float v0[4], v1[4], o[4];
  get4<TO>(op + r0 * D + d, v0);
  get4<TO>(op + r1 * D + d, v1);
  const float M = fmaxf(m0, m1);
  // a half with no visible key has m = -inf and weight 0
  const float w0 = m0 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m0 - M) * l0;
  const float w1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - M) * l1;
  const float L = w0 + w1;
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c) o[c] = fmaf(w1, v1[c], w0 * v0[c]) * inv;
  put4<TO>((TO*)a.o + ((int64_t)bh * a.Nq + qrow) * D + d, o);
}

template <typename T, typename TO, int D, int W>
hipError_t launch_w(const FwdArgs& a, const PrefillSplit& pl, void* ws, hipStream_t s) {
  constexpr int BM = 32 * W;
  const int ntq = (a.Nq + BM - 1) / BM;
  const int64_t tiles = (int64_t)a.B * a.Hq * ntq;
  SplitArgs sp{1, 0, nullptr, 0, nullptr, nullptr};
  if (pl.ns > 1 || pl.halves > 0) {
    if (pl.tiles != tiles || pl.rows != BM || ws == nullptr) return hipErrorInvalidValue;
    const int64_t nrow = pl.ns > 1 ? tiles * pl.ns * BM : (int64_t)pl.halves * 2 * BM;
    sp.ns = pl.ns;
    sp.halves = pl.halves;
    sp.ctr = (unsigned long long*)ws;
    sp.opart = (char*)ws + pl.ctr_bytes;
    sp.mlpart = (float*)((char*)ws + pl.ctr_bytes + ((size_t)nrow * D * sizeof(TO) + 255) / 256 * 256);
    sp.gen = next_generation();
  }
  const int64_t grid = tiles * sp.ns + sp.halves;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((prefill_kernel<T, TO, D, W>), dim3((unsigned)grid), dim3(64 * W), 0, s, a, ntq,
                     sp);
  if (sp.halves > 0) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t items = (int64_t)sp.halves * BM * (D / 4);
    hipLaunchKernelGGL((prefill_merge_kernel<TO, D>), dim3((unsigned)((items + 255) / 256)), dim3(256),
                       0, s, a, ntq, BM, (int)(tiles - sp.halves), sp.halves, sp);
  }
  return hipGetLastError();
}

template <typename T, typename TO, int D>
hipError_t launch_t(const FwdArgs& a, const PrefillSplit& pl, void* ws, hipStream_t s) {
  if (prefill_waves(a) == 8) return launch_w<T, TO, D, 8>(a, pl, ws, s);
  return launch_w<T, TO, D, 4>(a, pl, ws, s);
}

}  // namespace

// Eight waves (256 query rows) per workgroup halve the direct-load traffic
// into LDS per flop (about 5 % faster per full round at head dim 128), but
// one such workgroup fills a CU, so a partial last round costs a whole round.
// Four-wave workgroups run two to a CU; when their last round holds at most
// 256 of them each runs alone on a CU, at 0.7-0.9 of a shared round's time.
// So eight waves need at least one full round of 256 workgroups and either
// no partial round, a last round more than half full, or eight rounds to
// amortise it (measured: 256, 416, 512, 1000, 1024, 1184, 1536 and 2016
// workgroups 4-9 % faster on eight waves; 300, 384, 640 and 1100, whose last
// rounds are 17, 50, 50 and 30 % full, 9.4, 4.1, 7.0 and 0.6 % slower). Under a
// per-row window of W keys a query tile of R rows covers W + R - 1 keys of
// which each row uses W, so taller tiles compute more masked scores; below
// 3072 keys the 128-row tiles win (measured: W = 1024 and 2048 run 8.6 % and
// 2.3-3.7 % faster on four waves, 3072-6144 are even, 8192 and 16384 run
// 0.6 % and 6.5 % slower).
int prefill_waves(const FwdArgs& a) {
  const int64_t grid8 = (int64_t)a.B * a.Hq * ((a.Nq + 255) / 256);
  if (a.window_w > 0 && a.window_w < 3072) return 4;
  if (a.D != 128 || grid8 < 256) return 4;
  const int64_t tail = grid8 % 256;
  return grid8 >= 8 * 256 || tail == 0 || tail > 128 ? 8 : 4;
}

// Parts per query tile: grids of at most 128 query tiles are split into 2
// to 4 parts of at least two key tiles each, as many as keep the split grid
// within one workgroup per CU (256). Each part's publication and the merge
// cost an agent-scope release and acquire, which write back and invalidate
// the XCD's L2; with one workgroup per CU that is cheap (1.7-2.6 times
// faster on 16-64 tiles), with several per CU the invalidations cost the
// other workgroups their cached K/V tiles (a 640-tile grid split in two took
// 30 % longer), so larger grids run unsplit.
PrefillSplit prefill_split_plan(const FwdArgs& a, int out_bytes) {
  PrefillSplit p;
  const int W = prefill_waves(a);
  p.rows = 32 * W;
  p.tiles = (int64_t)a.B * a.Hq * ((a.Nq + p.rows - 1) / p.rows);
  const KeyRange r = key_range(a);
  const int nt = r.hi > r.lo ? (r.hi + 63) / 64 - r.lo / 64 : 0;
  int ns = 1;
  if (p.tiles * 2 <= 256) {
    ns = (int)(256 / p.tiles);
    ns = ns > 4 ? 4 : ns;
    while (ns > 1 && nt < 2 * ns) --ns;
  }
  p.ns = ns;
  // Between half a round and one round of workgroups (slots: 256 CUs times
  // the four-wave workgroups one holds, 3 at head dim 64, 2 at 128) some CUs
  // run one workgroup more than others. Running slots - tiles of the tiles as
  // two halves makes the jobs exactly fill the slots, one half in every CU's
  // last slot (see balanced_job), and a second launch merges the halves: no
  // fences in the main kernel. SDXL (640 tiles, 768 slots): 104 -> 93 us.
  const int64_t slots = 256LL * (a.D == 64 ? 3 : 2);
  if (ns == 1 && W == 4 && p.tiles < slots && 2 * p.tiles > slots && nt >= 2)
    p.halves = (int)(slots - p.tiles);
  if (ns > 1) {
    const size_t nrow = (size_t)p.tiles * ns * p.rows;
    p.ctr_bytes = ((size_t)p.tiles * sizeof(unsigned long long) + 255) / 256 * 256;
    p.ws_bytes = p.ctr_bytes + (nrow * a.D * out_bytes + 255) / 256 * 256 + nrow * 2 * sizeof(float);
  } else if (p.halves > 0) {
    const size_t nrow = (size_t)p.halves * 2 * p.rows;
    p.ws_bytes = (nrow * a.D * out_bytes + 255) / 256 * 256 + nrow * 2 * sizeof(float);
  }
  return p;
}

hipError_t launch_prefill(const FwdArgs& a, int elem, bool out_f32, const PrefillSplit& sp,
                          void* ws, hipStream_t s) {
  if (elem == 2) {
    if (out_f32)
      return a.D == 64 ? launch_t<__bf16, float, 64>(a, sp, ws, s) : launch_t<__bf16, float, 128>(a, sp, ws, s);
    return a.D == 64 ? launch_t<__bf16, __bf16, 64>(a, sp, ws, s) : launch_t<__bf16, __bf16, 128>(a, sp, ws, s);
  }
  return a.D == 64 ? launch_t<_Float16, _Float16, 64>(a, sp, ws, s)
                   : launch_t<_Float16, _Float16, 128>(a, sp, ws, s);
}

// fp32 -> bf16, round to nearest even (the hardware conversion).
__global__ void f32_to_bf16_kernel(const float* __restrict__ x, __bf16* __restrict__ y, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i + 3 < n) {
    const f32x4 v = *(const f32x4*)(x + i);
    __bf16 o[4] = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    *(u32x2*)(y + i) = *(const u32x2*)o;
  } else {
    for (int64_t j = i; j < n; ++j) y[j] = (__bf16)x[j];
  }
}

hipError_t launch_f32_to_bf16(const float* x, void* y, int64_t n, hipStream_t s) {
  const int64_t threads = (n + 3) / 4;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, (__bf16*)y, n);
  return hipGetLastError();
}

}  // namespace attn
