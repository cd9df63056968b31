// attn_prefill.hip — exact-mode flash attention forward for gfx950.
//
// One workgroup of 4 waves owns 128 query rows of one (batch, query head);
// each wave owns 32 rows, two workgroups share a CU (2 waves per SIMD). The
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
// The loop is software-pipelined so the matrix cores do not wait for the
// softmax: iteration i computes S for tile i+1 on the MFMA pipe while the
// vector ALU exponentiates tile i, then accumulates P V for tile i. K tile
// i+1 and V tile i are resident together, so K and V use separate LDS double
// buffers offset by one tile, and one barrier per iteration suffices. The
// instruction interleave inside an iteration is fixed with scheduling-group
// barriers.
//
// 64-key tiles follow the 64-position KV chunk of "perf(metal): widen
// four-row flash KV tiles" (its 128-position chunk is a different trade-off,
// for a four-row shape on another GPU).
#include "attn_common.hpp"
#include "attn_internal.hpp"

#ifndef PREFILL_QB128
#define PREFILL_QB128 1
#endif

namespace attn {

namespace {

// The running maximum is raised only when a new score exceeds it by more
// than this many powers of two; until then exponents stay <= 2^8, which bf16,
// f16 and fp32 hold exactly in range. Exactness is unaffected: numerator and
// denominator share the stale maximum.
constexpr float kLazyLog2 = 8.0f;

// Scheduling-group masks (see the AMDGPU backend's sched_group_barrier).
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

template <typename T, typename TO, int D, int QB>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256),
                               amdgpu_waves_per_eu(QB == 1 ? 2 : 1, QB == 1 ? 2 : 1)))
prefill_kernel(FwdArgs a, int ntq) {
  using E = Elem<T>;
  using V8 = typename E::vec8;
  constexpr int BM = 128 * QB;
  constexpr int KS = D / 16;       // 16-wide k-steps of Q K^T
  constexpr int DB = D / 32;       // 32-row blocks of O^T
  constexpr int CPR = D / 8;       // 16-byte chunks per K/V row
  constexpr int RPI = 64 / CPR;    // rows one 64-lane direct load covers
  __shared__ __attribute__((aligned(16))) T sk[2][64 * D];
  __shared__ __attribute__((aligned(16))) T sv[2][64 * D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int half = lane >> 5, col = lane & 31;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / ntq, qt = tile - bh * ntq;
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
  const int kv_lo = a.window_lo;
  const int kv_hi = a.causal ? min(a.Nk, a.pos0 + qlast + 1) : a.Nk;
  const int t_lo = kv_lo / 64;
  const int nt = kv_hi > kv_lo ? (kv_hi + 63) / 64 - t_lo : 0;

  // Q^T as B operands, held for the whole loop: column = query row,
  // lane half h of k-step ks holds d = 16 ks + 8 h + (0..7). A wave owns
  // QB blocks of 32 rows.
  const int qw0 = q0 + wave * 32 * QB;  // first row of this wave
  int qrow[QB];
  V8 qv[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qrow[qb] = qw0 + 32 * qb + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 raw = {0, 0, 0, 0};
      if (qrow[qb] < a.Nq) raw = ld16(Qp + (int64_t)qrow[qb] * D + 16 * ks + 8 * half);
      qv[qb][ks] = __builtin_bit_cast(V8, raw);
    }
  }

  // LDS tiles are 64 unpadded rows of D elements; chunk c of row r sits at
  // chunk position c ^ swz(r). K row r holds key (r & ~31) | swap23(r & 31)
  // (so P^T lands in B-operand order), V row r holds key r. The swizzles make
  // the 16 lanes of a K operand read (16 rows, one logical chunk) and the 32
  // lanes of a V transpose read (4 rows x 8 chunks) hit distinct banks.
  auto kswz = [](int r) { return CPR == 16 ? (r & 15) : ((r >> 1) & 7); };
  auto vswz = [](int r) { return CPR == 16 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); };
  // Direct loads: each wave fills 16 rows of the K and of the V tile, RPI
  // rows per instruction (lane i -> row i / CPR, chunk position i % CPR).
  // Rows past Nk are clamped to the last row (finite values; masked).
  // Per-lane parts of the direct loads are loop invariant; the tile enters
  // as a uniform base pointer and a clamp on the row.
  auto load_k = [&](int t, int buf) {
    const char* base = (const char*)(Kp + (int64_t)64 * t * D);
    const int last = a.Nk - 1 - 64 * t;   // rows past it clamp to the last key
#pragma unroll
    for (int u = 0; u < 16 / RPI; ++u) {
      const int r0 = 16 * wave + RPI * u;
      const int r = r0 + lane / CPR, pos = lane % CPR;
      const int kk = (r & ~31) | swap23(r & 31);
      const uint32_t off = (uint32_t)(min(kk, last) * (D * 2) + 16 * (pos ^ kswz(r)));
      load_to_lds16(base + off, &sk[buf][r0 * D]);
    }
  };
  auto load_v = [&](int t, int buf) {
    const char* base = (const char*)(Vp + (int64_t)64 * t * D);
    const int last = a.Nk - 1 - 64 * t;
#pragma unroll
    for (int u = 0; u < 16 / RPI; ++u) {
      const int r0 = 16 * wave + RPI * u;
      const int r = r0 + lane / CPR, pos = lane % CPR;
      const uint32_t off = (uint32_t)(min(r, last) * (D * 2) + 16 * (pos ^ vswz(r)));
      load_to_lds16(base + off, &sv[buf][r0 * D]);
    }
  };

  // Boundary tiles only: window edge, ragged end, causal diagonal.
  auto apply_mask = [&](f32x16 (&s)[2][QB], int t) {
    const int k0 = 64 * t;
    const bool need = (k0 < kv_lo) || (k0 + 64 > a.Nk) || (a.causal && k0 + 63 > a.pos0 + qw0);
    if (need) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = k0 + 32 * mb + 16 * (j >> 3) + 8 * half + (j & 7);
            const bool vis = key >= kv_lo && key < a.Nk && (!a.causal || key <= a.pos0 + qrow[qb]);
            if (!vis) s[mb][qb][j] = -INFINITY;
          }
    }
  };

  f32x16 oacc[DB][QB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[db][qb][j] = 0.0f;
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.0f;
  }

  // S^T of one tile from an LDS K buffer (2 * QB independent MFMA chains;
  // every K operand read feeds QB MFMAs).
  auto s_mma = [&](int buf, f32x16 (&s)[2][QB]) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int j = 0; j < 16; ++j) s[mb][qb][j] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int r = 32 * mb + col;
        const V8 ka = *(const V8*)&sk[buf][r * D + 8 * ((2 * ks + half) ^ kswz(r))];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[mb][qb] = E::mma(ka, qv[qb][ks], s[mb][qb]);
      }
  };

  // One pipeline step: softmax and P V of tile i (scores in cur), S of tile
  // i + 1 into nxt, then the stores and loads that keep K two tiles and V one
  // tile ahead.
  auto step = [&](int i, f32x16 (&cur)[2][QB], f32x16 (&nxt)[2][QB]) {
    const int t = t_lo + i;
    // K tile i + 2 goes where K tile i was, V tile i + 1 where V tile i - 1
    // was (both last read before the previous barrier); they land during
    // this step and are published by its closing barrier.
    if (i + 2 < nt) load_k(t + 2, i & 1);
    if (i + 1 < nt) load_v(t + 1, (i + 1) & 1);
    apply_mask(cur, t);
    float mu[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = cur[0][qb][0];
#pragma unroll
      for (int j = 1; j < 16; ++j) mx = fmaxf(mx, cur[0][qb][j]);
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, cur[1][qb][j]);
      mx = halves_max(mx) * a.c;
      if (__builtin_amdgcn_ballot_w64(mx > m_run[qb] + kLazyLog2)) {
        // rare after the first tiles; the empty asm keeps this a real branch
        // (the compiler would otherwise run the rescale on every tile)
        asm volatile("" ::: "memory");
        const float m_new = fmaxf(m_run[qb], mx);
        const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j) oacc[db][qb][j] *= alpha;
        m_run[qb] = m_new;
      }
      mu[qb] = m_run[qb] == -INFINITY ? 0.0f : m_run[qb];
    }

    // S of tile i + 1 (MFMA) interleaved with the exponentials of tile i.
    __builtin_amdgcn_s_setprio(1);
    s_mma((i + 1) & 1, nxt);
    V8 pv[QB][2][2];
    float ls[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int k = 0; k < 4; ++k) ls[qb][k] = 0.0f;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          V8 p;
#pragma unroll
          for (int q = 0; q < 8; ++q)
            p[q] = E::from_float(__builtin_amdgcn_exp2f(fmaf(cur[mb][qb][8 * tt + q], a.c, -mu[qb])));
          pv[qb][mb][tt] = p;
          // the denominator sums the rounded weights the P V product uses
          ls[qb][2 * mb + tt] = E::sum8(p, ls[qb][2 * mb + tt]);
        }
    // 2*KS*QB MFMAs with the exponentials spread between them; the K reads
    // run ahead of the MFMAs that use them.
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
#pragma unroll
    for (int k = 0; k < 2 * KS - 2; ++k) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 64 / KS, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * QB, 0);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_run[qb] += (ls[qb][0] + ls[qb][1]) + (ls[qb][2] + ls[qb][3]);

    // O^T += V^T P^T for tile i (4 k-steps of 16 keys, DB * QB chains). In
    // each 16-lane group the transpose read hands lane 4a + e element e of
    // the rows named by lanes a, a+4, a+8, a+12: lane r names key kb + r/4
    // at channel d0 + 4 (r % 4), so lane (col, half) gets channel col of keys
    // kb..kb+3, i.e. four B-operand slots of P^T's order.
    const int vb = i & 1;
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
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = E::mma(va, pv[qb][mb][tt], oacc[db][qb]);
        }

    __builtin_amdgcn_s_setprio(0);
    vmem_wait_all();   // this wave's direct-to-LDS loads have landed
    __syncthreads();
  };

  if (nt > 0) {
    // Prologue: K tiles 0 and 1 and V tile 0 in LDS, S of tile 0.
    load_k(t_lo, 0);
    load_v(t_lo, 0);
    if (nt > 1) load_k(t_lo + 1, 1);
    vmem_wait_all();
    __syncthreads();
    f32x16 s0[2][QB], s1[2][QB];
    s_mma(0, s0);
    __syncthreads();   // step 0 overwrites the K buffer just read
    int i = 0;
    for (; i + 1 < nt; i += 2) {
      step(i, s0, s1);
      step(i + 1, s1, s0);
    }
    if (i < nt) step(i, s0, s1);
  }

  // Epilogue: O = O_acc / l; rows with no visible key are written as zeros.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = halves_sum(l_run[qb]);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (qrow[qb] >= a.Nq) continue;
    TO* orow = Op + (int64_t)qrow[qb] * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d = 32 * db + 8 * a4 + 4 * half;
        if constexpr (sizeof(TO) == 4) {
          f32x4 o4;
#pragma unroll
          for (int r = 0; r < 4; ++r) o4[r] = oacc[db][qb][4 * a4 + r] * inv;
          *(f32x4*)(orow + d) = o4;
        } else {
          TO o4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) o4[r] = Elem<TO>::from_float(oacc[db][qb][4 * a4 + r] * inv);
          *(u32x2*)(orow + d) = *(const u32x2*)o4;
        }
      }
  }
}

template <typename T, typename TO, int D, int QB>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
  constexpr int BM = 128 * QB;
  const int ntq = (a.Nq + BM - 1) / BM;
  const int64_t grid = (int64_t)a.B * a.Hq * ntq;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((prefill_kernel<T, TO, D, QB>), dim3((unsigned)grid), dim3(256), 0, s, a, ntq);
  return hipGetLastError();
}

}  // namespace

// Rows per wave: 64 for head dim 128 (one wave per SIMD, 512 registers),
// 32 for head dim 64 (two waves per SIMD).
hipError_t launch_prefill(const FwdArgs& a, int elem, bool out_f32, hipStream_t s) {
  constexpr int QB128 = PREFILL_QB128;
  if (elem == 2) {
    if (out_f32) return a.D == 64 ? launch_t<__bf16, float, 64, 1>(a, s) : launch_t<__bf16, float, 128, QB128>(a, s);
    return a.D == 64 ? launch_t<__bf16, __bf16, 64, 1>(a, s) : launch_t<__bf16, __bf16, 128, QB128>(a, s);
  }
  return a.D == 64 ? launch_t<_Float16, _Float16, 64, 1>(a, s) : launch_t<_Float16, _Float16, 128, QB128>(a, s);
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
