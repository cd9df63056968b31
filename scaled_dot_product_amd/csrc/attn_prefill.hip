// attn_prefill.hip — exact-mode flash attention forward for gfx950.
//
// One workgroup of 4 waves owns BM = 4 * 32 * QB query rows of one
// (batch, query head); each wave owns 32 * QB rows. The workgroup streams the
// visible keys of its key/value head in tiles of 64: K and V are read from
// HBM/L2 with 16-byte loads, staged in double-buffered LDS (K row-major, V
// transposed), and every wave runs
//     S^T = K Q^T                   (bf16/f16 MFMA, fp32 accumulation)
//     mask (boundary tiles only)
//     online softmax in exp2 units  (running max, running sum, lazy rescale)
//     O^T += V^T P^T                (P rounded to the operand type)
// before the epilogue divides by the running sum. The N x N score matrix is
// never stored. 64-key tiles follow the 64-position KV chunk of
// "perf(metal): widen four-row flash KV tiles" (its 128-position chunk is a
// different trade-off for a four-row shape on another GPU).
#include "attn_common.hpp"
#include "attn_internal.hpp"

namespace attn {

namespace {

// The running maximum is raised only when a new score exceeds it by more
// than this many powers of two; until then exponents stay <= 2^8, which bf16,
// f16 and fp32 hold exactly in range. Exactness is unaffected: numerator and
// denominator share the stale maximum.
constexpr float kLazyLog2 = 8.0f;

template <typename T, typename TO, int D, int QB>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256),
                               amdgpu_waves_per_eu(QB == 1 ? 2 : 1, QB == 1 ? 2 : 1)))
prefill_kernel(FwdArgs a, int ntq) {
  using E = Elem<T>;
  using V8 = typename E::vec8;
  constexpr int BM = 4 * 32 * QB;
  constexpr int KS = D / 16;       // 16-wide k-steps of Q K^T
  constexpr int DB = D / 32;       // 32-row blocks of O^T
  constexpr int KLD = D + 8;       // K tile row stride (elements): +16 B pad
  constexpr int VLD = 64 + 8;      // V^T tile row stride (elements): +16 B pad
  constexpr int KPT = D / 32;      // keys per thread in a tile load
  constexpr int KG = 64 / KPT;     // key groups per tile
  __shared__ __attribute__((aligned(16))) T sk[2][64 * KLD];
  __shared__ __attribute__((aligned(16))) T sv[2][D * VLD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

  // Visible keys of this workgroup's rows.
  const int qlast = min(q0 + BM, a.Nq) - 1;
  const int kv_lo = a.window_lo;
  const int kv_hi = a.causal ? min(a.Nk, a.pos0 + qlast + 1) : a.Nk;
  const int t_lo = kv_lo / 64;
  const int t_hi = kv_hi > kv_lo ? (kv_hi + 63) / 64 : t_lo;

  // Q^T as B operands, held for the whole loop: column = query row,
  // lane half h of k-step ks holds d = 16 ks + 8 h + (0..7).
  V8 qv[QB][KS];
  int qrow[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qrow[qb] = q0 + (wave * QB + qb) * 32 + col;
    const bool ok = qrow[qb] < a.Nq;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 raw = {0, 0, 0, 0};
      if (ok) raw = ld16(Qp + (int64_t)qrow[qb] * D + 16 * ks + 8 * half);
      qv[qb][ks] = __builtin_bit_cast(V8, raw);
    }
  }
  const int qw0 = q0 + wave * QB * 32;  // first row of this wave

  // Tile loads: thread -> key group kg (KPT consecutive keys) and 16-byte
  // column cc. Rows past Nk are clamped to the last row, so every load is
  // unconditional (no branches between them); those keys are masked.
  const int kg = tid % KG, cc = tid / KG;
  u32x4 kreg[KPT], vreg[KPT];
  auto gload = [&](int k0) {
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int key = min(k0 + kg * KPT + r, a.Nk - 1);
      kreg[r] = ld16(Kp + (int64_t)key * D + 8 * cc);
      vreg[r] = ld16(Vp + (int64_t)key * D + 8 * cc);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int kk = kg * KPT + r;
      const int row = (kk & ~31) | swap23(kk & 31);
      st16(&sk[buf][row * KLD + 8 * cc], kreg[r]);
    }
    // V^T: element e of every key's chunk goes to row d = 8 cc + e.
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      T* dst = &sv[buf][(8 * cc + e) * VLD + kg * KPT];
      if constexpr (KPT == 4) {
        u32x2 pk;
        pk[0] = __builtin_amdgcn_perm(vreg[1][e >> 1], vreg[0][e >> 1], sel);
        pk[1] = __builtin_amdgcn_perm(vreg[3][e >> 1], vreg[2][e >> 1], sel);
        *(u32x2*)dst = pk;
      } else {
        *(uint32_t*)dst = __builtin_amdgcn_perm(vreg[1][e >> 1], vreg[0][e >> 1], sel);
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

  if (t_lo < t_hi) {
    gload(t_lo * 64);
    lstore(0);
    __syncthreads();
  }
  for (int t = t_lo; t < t_hi; ++t) {
    const int buf = (t - t_lo) & 1;
    const int k0 = t * 64;
    if (t + 1 < t_hi) gload(k0 + 64);

    // S^T = K Q^T for 64 keys x 32*QB queries; even and odd k-steps go to
    // separate accumulators so that four MFMA chains are in flight.
    f32x16 s[2][QB], s2[2][QB];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int j = 0; j < 16; ++j) s[mb][qb][j] = s2[mb][qb][j] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ks += 2) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const V8 ka = *(const V8*)&sk[buf][(32 * mb + col) * KLD + 16 * ks + 8 * half];
        const V8 kb = *(const V8*)&sk[buf][(32 * mb + col) * KLD + 16 * ks + 16 + 8 * half];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          s[mb][qb] = E::mma(ka, qv[qb][ks], s[mb][qb]);
          s2[mb][qb] = E::mma(kb, qv[qb][ks + 1], s2[mb][qb]);
        }
      }
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int j = 0; j < 16; ++j) s[mb][qb][j] += s2[mb][qb][j];

    // Boundary tiles only: window edge, ragged end, causal diagonal.
    const bool need_mask = (k0 < kv_lo) || (k0 + 64 > a.Nk) ||
                           (a.causal && k0 + 63 > a.pos0 + qw0);
    if (need_mask) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = k0 + 32 * mb + 16 * (j >> 3) + 8 * half + (j & 7);
            const bool vis = key >= kv_lo && key < a.Nk &&
                             (!a.causal || key <= a.pos0 + qrow[qb]);
            if (!vis) s[mb][qb][j] = -INFINITY;
          }
    }

    // Online softmax (exp2 units) and P^T as B operands.
    V8 pv[QB][2][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = s[0][qb][0];
#pragma unroll
      for (int j = 1; j < 16; ++j) mx = fmaxf(mx, s[0][qb][j]);
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[1][qb][j]);
      mx = halves_max(mx) * a.c;
      const bool grow = mx > m_run[qb] + kLazyLog2;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = fmaxf(m_run[qb], mx);
        const float alpha =
            m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j) oacc[db][qb][j] *= alpha;
        m_run[qb] = m_new;
      }
      const float mu = m_run[qb] == -INFINITY ? 0.0f : m_run[qb];
      float lsum = 0.0f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          V8 p;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float e = __builtin_amdgcn_exp2f(fmaf(s[mb][qb][8 * tt + i], a.c, -mu));
            lsum += e;
            p[i] = E::from_float(e);
          }
          pv[qb][mb][tt] = p;
        }
      l_run[qb] += lsum;
    }

    // O^T += V^T P^T over the 64 keys (4 k-steps of 16).
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const V8 va =
              *(const V8*)&sv[buf][(32 * db + col) * VLD + 32 * mb + 16 * tt + 8 * half];
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = E::mma(va, pv[qb][mb][tt], oacc[db][qb]);
        }

    if (t + 1 < t_hi) lstore(buf ^ 1);
    __syncthreads();
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
  constexpr int BM = 4 * 32 * QB;
  const int ntq = (a.Nq + BM - 1) / BM;
  const int64_t grid = (int64_t)a.B * a.Hq * ntq;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((prefill_kernel<T, TO, D, QB>), dim3((unsigned)grid), dim3(256), 0, s, a, ntq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const FwdArgs& a, int elem, bool out_f32, hipStream_t s) {
  constexpr int QB = 1;
  if (elem == 2) {
    if (out_f32) return a.D == 64 ? launch_t<__bf16, float, 64, QB>(a, s) : launch_t<__bf16, float, 128, QB>(a, s);
    return a.D == 64 ? launch_t<__bf16, __bf16, 64, QB>(a, s) : launch_t<__bf16, __bf16, 128, QB>(a, s);
  }
  return a.D == 64 ? launch_t<_Float16, _Float16, 64, QB>(a, s) : launch_t<_Float16, _Float16, 128, QB>(a, s);
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
