// attn_quant.hip — the opt-in low-precision mode: INT8 Q K^T and FP8 P V.
//
// The recipe is the "SageAttention 2 INT8 QK . FP8 PV" row of the table in
// section 1 of "Attention kernels on a home RTX 5080": Q and K become
// symmetric INT8 codes with one fp32 scale per 64-token block of one head,
// V becomes OCP FP8 E4M3 codes with one scale per 64-token block, and the
// softmax weights are rounded to E4M3 at the static scale 448 (each weight is
// at most 1 because the running maximum is always current in this kernel).
//
//   quant_int8_kernel   per block: amax, scale = amax/127, inv = 127/amax,
//                       code = clamp(rint(x*inv), -127, 127)  (bit-exact)
//   quant_e4m3_kernel   per block: scale = amax/448, inv = 448/amax,
//                       code = E4M3(clamp(x*inv, -448, 448)) via the gfx950
//                       conversion (OCP E4M3, round to nearest even)
//   prefill_quant_kernel
//     S_int^T = Kc Qc^T              i8 MFMA 32x32x32, exact int32
//     exponent = S_int * (s_q s_k scale log2 e) - m   (one FMA per score)
//     P^ = E4M3(448 * 2^exponent), l += 448 * 2^exponent
//     T^T = Vc^T P^T                 fp8 MFMA 32x32x64, fp32 accumulation
//     O_acc = alpha O_acc + s_v T    (s_v: the tile's V block scale)
//   O = O_acc / l.
#include "attn_common.hpp"
#include "attn_internal.hpp"

namespace attn {

namespace {

template <typename T>
__device__ __forceinline__ float elem_to_float(uint32_t bits16);
template <>
__device__ __forceinline__ float elem_to_float<__bf16>(uint32_t b) {
  return __uint_as_float(b << 16);
}
template <>
__device__ __forceinline__ float elem_to_float<_Float16>(uint32_t b) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)b);
  return (float)h;
}

// Unpack one 16-byte chunk (8 elements) to floats (exact widening).
template <typename T>
__device__ __forceinline__ void unpack8(u32x4 raw, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = elem_to_float<T>(raw[i] & 0xffffu);
    x[2 * i + 1] = elem_to_float<T>(raw[i] >> 16);
  }
}

// Block amax over the workgroup (256 threads), identical in every thread.
__device__ __forceinline__ float block_amax(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// One workgroup per 64-token block of one head. Thread -> (token, chunk).
template <typename T, int D>
__global__ void __launch_bounds__(256) quant_int8_kernel(const T* __restrict__ x, int N,
                                                          int8_t* __restrict__ codes,
                                                          float* __restrict__ scales) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per token row
  constexpr int PER = 64 * CPR / 256;        // chunks per thread
  __shared__ float red[4];
  const int nblk = (N + 63) / 64;
  const int64_t bh = blockIdx.x / nblk;
  const int t = blockIdx.x - (int)(bh * nblk);
  const int r0 = 64 * t;
  const int rows = min(64, N - r0);
  const T* src = x + (bh * N + r0) * D;
  int8_t* dst = codes + (bh * N + r0) * D;
  float vals[PER][8];
  bool live[PER];
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int chunk = threadIdx.x + 256 * u;
    const int row = chunk / CPR, c = chunk - row * CPR;
    live[u] = row < rows;
    u32x4 raw = {0, 0, 0, 0};
    if (live[u]) raw = ld16(src + (int64_t)row * D + 8 * c);
    unpack8<T>(raw, vals[u]);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(vals[u][i]));
  }
  amax = block_amax(amax, red);
  float inv = 0.0f;
  if (amax > 0.0f) inv = 127.0f / amax;   // correctly rounded fp32 division
  if (threadIdx.x == 0) scales[bh * nblk + t] = amax > 0.0f ? amax / 127.0f : 0.0f;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    if (!live[u]) continue;
    const int chunk = threadIdx.x + 256 * u;
    const int row = chunk / CPR, c = chunk - row * CPR;
    uint32_t w[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float r = __builtin_rintf(vals[u][i] * inv);
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      w[i >> 2] |= ((uint32_t)(int)r & 0xffu) << (8 * (i & 3));
    }
    *(u32x2*)(dst + (int64_t)row * D + 8 * c) = u32x2{w[0], w[1]};
  }
}

// E4M3 codes. layout 0: [BH][N][D]; layout 1: per 64-token block, transposed
// [BH][nblk][D][64] with zero codes past N (the tile the quantised kernel
// copies straight into LDS).
template <typename T, int D>
__global__ void __launch_bounds__(256) quant_e4m3_kernel(const T* __restrict__ x, int N,
                                                          uint8_t* __restrict__ codes,
                                                          float* __restrict__ scales, int layout) {
  constexpr int CPR = D / 8;
  constexpr int PER = 64 * CPR / 256;
  constexpr int TLD = D + 8;                 // LDS row stride (bytes), keeps 8-byte stores aligned
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint8_t tileb[64 * TLD];
  const int nblk = (N + 63) / 64;
  const int64_t bh = blockIdx.x / nblk;
  const int t = blockIdx.x - (int)(bh * nblk);
  const int r0 = 64 * t;
  const int rows = min(64, N - r0);
  const T* src = x + (bh * N + r0) * D;
  float vals[PER][8];
  bool live[PER];
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int chunk = threadIdx.x + 256 * u;
    const int row = chunk / CPR, c = chunk - row * CPR;
    live[u] = row < rows;
    u32x4 raw = {0, 0, 0, 0};
    if (live[u]) raw = ld16(src + (int64_t)row * D + 8 * c);
    unpack8<T>(raw, vals[u]);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(vals[u][i]));
  }
  amax = block_amax(amax, red);
  float inv = 0.0f;
  if (amax > 0.0f) inv = 448.0f / amax;
  if (threadIdx.x == 0) scales[bh * nblk + t] = amax > 0.0f ? amax / 448.0f : 0.0f;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int chunk = threadIdx.x + 256 * u;
    const int row = chunk / CPR, c = chunk - row * CPR;
    uint32_t w[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float y[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        y[k] = fminf(fmaxf(vals[u][4 * i + k] * inv, -448.0f), 448.0f);
      int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], pk, true);
      w[i] = (uint32_t)pk;
    }
    if (!live[u]) w[0] = w[1] = 0;
    if (layout == 0) {
      if (live[u]) *(u32x2*)(codes + (bh * N + r0 + row) * D + 8 * c) = u32x2{w[0], w[1]};
    } else {
      *(u32x2*)&tileb[row * TLD + 8 * c] = u32x2{w[0], w[1]};
    }
  }
  if (layout == 1) {
    __syncthreads();
    // Transposed tile: 16-byte chunk (d, keys 16j..16j+15).
    uint8_t* dst = codes + (bh * nblk + t) * (int64_t)D * 64;
    for (int ch = threadIdx.x; ch < D * 4; ch += 256) {
      const int d = ch >> 2, j = ch & 3;
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t v = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) v |= (uint32_t)tileb[(16 * j + 4 * q + k) * TLD + d] << (8 * k);
        w[q] = v;
      }
      st16(dst + (int64_t)d * 64 + 16 * j, u32x4{w[0], w[1], w[2], w[3]});
    }
  }
}

// ---------------------------------------------------------------------------
// Quantised prefill: 4 waves x 32 query rows, 64-key tiles.
template <typename TO, int D>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
prefill_quant_kernel(FwdArgs a, int ntq, const int8_t* __restrict__ qc,
                     const float* __restrict__ qs, const int8_t* __restrict__ kc,
                     const float* __restrict__ ks, const uint8_t* __restrict__ vct,
                     const float* __restrict__ vs) {
  constexpr int BM = 128;
  constexpr int KS = D / 32;      // i8 k-steps (32 channels each)
  constexpr int DB = D / 32;
  constexpr int KLD = D + 16;     // K code tile row stride (bytes)
  constexpr int VLD = 64 + 16;    // V^T code tile row stride (bytes)
  constexpr int KCH = 64 * D / 16 / 256;   // 16-byte K chunks per thread
  constexpr int VCH = D * 64 / 16 / 256;   // 16-byte V^T chunks per thread
  constexpr float kP = 8.807354922057604f; // log2(448)
  __shared__ __attribute__((aligned(16))) uint8_t sk[2][64 * KLD];
  __shared__ __attribute__((aligned(16))) uint8_t sv[2][D * VLD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / ntq, qt = tile - bh * ntq;
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const int bg = b * a.Hkv + g;
  const int q0 = qt * BM;
  const int nkt = (a.Nk + 63) / 64;
  const int8_t* Qc = qc + (int64_t)bh * a.Nq * D;
  const int8_t* Kc = kc + (int64_t)bg * a.Nk * D;
  const uint8_t* Vt = vct + (int64_t)bg * nkt * D * 64;
  const float* Ks = ks + (int64_t)bg * nkt;
  const float* Vs = vs + (int64_t)bg * nkt;
  TO* Op = (TO*)a.o + (int64_t)bh * a.Nq * D;

  const int qlast = min(q0 + BM, a.Nq) - 1;
  const int kv_lo = a.window_lo;
  const int kv_hi = a.causal ? min(a.Nk, a.pos0 + qlast + 1) : a.Nk;
  const int t_lo = kv_lo / 64;
  const int t_hi = kv_hi > kv_lo ? (kv_hi + 63) / 64 : t_lo;

  const int qrow = q0 + wave * 32 + col;
  const int qw0 = q0 + wave * 32;
  // Q codes as B operands: lane half h of k-step ks holds channels 32 ks + 16 h + (0..15).
  i32x4 qv[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    u32x4 raw = {0, 0, 0, 0};
    if (qrow < a.Nq) raw = ld16(Qc + (int64_t)qrow * D + 32 * k + 16 * half);
    qv[k] = __builtin_bit_cast(i32x4, raw);
  }
  // The wave's 32 rows lie in one 64-row block (q0 is a multiple of 128).
  const float sq = qs[(int64_t)bh * ((a.Nq + 63) / 64) + min(qw0, a.Nq - 1) / 64];
  const float cq = sq * a.c;

  u32x4 kreg[KCH], vreg[VCH];
  auto gload = [&](int t) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int ch = tid + 256 * u;
      const int kk = ch / (D / 16), c = ch - kk * (D / 16);
      const int key = min(64 * t + kk, a.Nk - 1);   // clamped rows are masked
      kreg[u] = ld16(Kc + (int64_t)key * D + 16 * c);
    }
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int ch = tid + 256 * u;
      vreg[u] = ld16(Vt + (int64_t)t * D * 64 + 16 * ch);
    }
  };
  // K code row for key kk in the tile: C-row m = 8a + 4h + b of block blk holds
  // key 32h + 16blk + 4a + b, so lane half h's 32 scores are keys 32h..32h+31.
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int ch = tid + 256 * u;
      const int kk = ch / (D / 16), c = ch - kk * (D / 16);
      const int hh = kk >> 5, blk = (kk >> 4) & 1, aa = (kk >> 2) & 3, bb = kk & 3;
      const int row = 32 * blk + 8 * aa + 4 * hh + bb;
      st16(&sk[buf][row * KLD + 16 * c], kreg[u]);
    }
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int ch = tid + 256 * u;
      const int d = ch >> 2, j = ch & 3;
      st16(&sv[buf][d * VLD + 16 * j], vreg[u]);
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[db][j] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  if (t_lo < t_hi) {
    gload(t_lo);
    lstore(0);
    __syncthreads();
  }
  for (int t = t_lo; t < t_hi; ++t) {
    const int buf = (t - t_lo) & 1;
    const int k0 = 64 * t;
    if (t + 1 < t_hi) gload(t + 1);

    i32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) s[mb][j] = 0;
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const i32x4 ka = *(const i32x4*)&sk[buf][(32 * mb + col) * KLD + 32 * k + 16 * half];
        s[mb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka, qv[k], s[mb], 0, 0, 0);
      }
    }
    // A block of zero codes has scale 0; a positive floor keeps masked scores
    // at -inf (-inf * 0 would be NaN) and changes nothing else, as every score
    // of such a block is exactly 0.
    const float cf = fmaxf(cq * Ks[t], 1.17549435e-38f);
    float sf[2][16];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) sf[mb][j] = (float)s[mb][j];
    const bool need_mask = (k0 < kv_lo) || (k0 + 64 > a.Nk) || (a.causal && k0 + 63 > a.pos0 + qw0);
    if (need_mask) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = k0 + 32 * half + 16 * mb + 4 * (j >> 2) + (j & 3);
          const bool vis = key >= kv_lo && key < a.Nk && (!a.causal || key <= a.pos0 + qrow);
          if (!vis) sf[mb][j] = -INFINITY;
        }
    }
    float mx = sf[0][0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sf[0][j]);
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sf[1][j]);
    mx = halves_max(mx) * cf;
    float alpha = 1.0f;
    if (__builtin_amdgcn_ballot_w64(mx > m_run)) {
      const float m_new = fmaxf(m_run, mx);
      alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
    }
    // 448 * P, one E4M3 code per score; the running max is current, so <= 448.
    const float mu = (m_run == -INFINITY ? 0.0f : m_run) - kP;
    i32x8 pb;
    float lsum = 0.0f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float e[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          e[k] = __builtin_amdgcn_exp2f(fmaf(sf[mb][4 * q4 + k], cf, -mu));
          lsum += e[k];
          e[k] = fminf(e[k], 448.0f);  // exp2 rounding may land a hair above 448
        }
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], pk, true);
        pb[4 * mb + q4] = pk;
      }
    l_run += lsum;

    // T^T = Vc^T P^T (fp8 x fp8 -> fp32), then O_acc = alpha O_acc + s_v T.
    const float sv_t = Vs[t];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const uint8_t* vp = &sv[buf][(32 * db + col) * VLD + 32 * half];
      const u32x4 lo = ld16(vp), hi = ld16(vp + 16);
      const i32x8 va = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                        (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      f32x16 tacc;
#pragma unroll
      for (int j = 0; j < 16; ++j) tacc[j] = 0.0f;
      tacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, tacc, 0, 0, 0, 127, 0, 127);
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[db][j] = fmaf(oacc[db][j], alpha, sv_t * tacc[j]);
    }

    if (t + 1 < t_hi) lstore(buf ^ 1);
    __syncthreads();
  }

  const float l = halves_sum(l_run);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  if (qrow < a.Nq) {
    TO* orow = Op + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d = 32 * db + 8 * a4 + 4 * half;
        TO o4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o4[r] = Elem<TO>::from_float(oacc[db][4 * a4 + r] * inv);
        *(u32x2*)(orow + d) = *(const u32x2*)o4;
      }
  }
}

template <typename T>
hipError_t quant_int8_t(const void* x, int64_t BH, int N, int D, int8_t* c, float* s,
                        hipStream_t st) {
  const int64_t grid = BH * ((N + 63) / 64);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (D == 64)
    hipLaunchKernelGGL((quant_int8_kernel<T, 64>), dim3((unsigned)grid), dim3(256), 0, st, (const T*)x, N, c, s);
  else
    hipLaunchKernelGGL((quant_int8_kernel<T, 128>), dim3((unsigned)grid), dim3(256), 0, st, (const T*)x, N, c, s);
  return hipGetLastError();
}

template <typename T>
hipError_t quant_e4m3_t(const void* x, int64_t BH, int N, int D, uint8_t* c, float* s, int layout,
                        hipStream_t st) {
  const int64_t grid = BH * ((N + 63) / 64);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (D == 64)
    hipLaunchKernelGGL((quant_e4m3_kernel<T, 64>), dim3((unsigned)grid), dim3(256), 0, st, (const T*)x, N, c, s, layout);
  else
    hipLaunchKernelGGL((quant_e4m3_kernel<T, 128>), dim3((unsigned)grid), dim3(256), 0, st, (const T*)x, N, c, s, layout);
  return hipGetLastError();
}

template <typename TO, int D>
hipError_t prefill_quant_t(const FwdArgs& a, const int8_t* qc, const float* qs, const int8_t* kc,
                           const float* ks, const uint8_t* vct, const float* vs, hipStream_t st) {
  const int ntq = (a.Nq + 127) / 128;
  const int64_t grid = (int64_t)a.B * a.Hq * ntq;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((prefill_quant_kernel<TO, D>), dim3((unsigned)grid), dim3(256), 0, st, a, ntq,
                     qc, qs, kc, ks, vct, vs);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_int8(const void* x, int elem, int64_t BH, int N, int D, int8_t* codes,
                             float* scales, hipStream_t s) {
  return elem == 2 ? quant_int8_t<__bf16>(x, BH, N, D, codes, scales, s)
                   : quant_int8_t<_Float16>(x, BH, N, D, codes, scales, s);
}

hipError_t launch_quant_e4m3(const void* x, int elem, int64_t BH, int N, int D, uint8_t* codes,
                             float* scales, int layout, hipStream_t s) {
  return elem == 2 ? quant_e4m3_t<__bf16>(x, BH, N, D, codes, scales, layout, s)
                   : quant_e4m3_t<_Float16>(x, BH, N, D, codes, scales, layout, s);
}

hipError_t launch_prefill_quant(const FwdArgs& a, const int8_t* qc, const float* qs,
                                const int8_t* kc, const float* ks, const uint8_t* vct,
                                const float* vs, int elem_out, hipStream_t s) {
  if (elem_out == 2)
    return a.D == 64 ? prefill_quant_t<__bf16, 64>(a, qc, qs, kc, ks, vct, vs, s)
                     : prefill_quant_t<__bf16, 128>(a, qc, qs, kc, ks, vct, vs, s);
  return a.D == 64 ? prefill_quant_t<_Float16, 64>(a, qc, qs, kc, ks, vct, vs, s)
                   : prefill_quant_t<_Float16, 128>(a, qc, qs, kc, ks, vct, vs, s);
}

}  // namespace attn
