// attn_mx.hip — the MX variants: OCP Microscaling FP8 (and FP4) blocks on
// the scaled matrix cores of gfx950.
//
// The table in section 1 of "Attention kernels on a home RTX 5080" puts
// per-block-scaled low-precision kernels at the top of its speed list, and
// "Transformers Get a Turbo Boost with Mixed-Precision Magic" runs attention
// on MXFP formats. Neither gives the arithmetic, so the format is the OCP
// Microscaling (MX) one: 32 FP8 E4M3 elements share one power-of-two scale
// stored as an E8M0 byte. gfx950's v_mfma_scale_f32_32x32x64_f8f6f4 takes one
// such scale per lane and 32-element block of each operand, so the matrix
// core applies every block scale of the P V product itself.
//
// Q K^T stays in the per-64-token-block INT8 of the quantised mode: the INT8
// matrix cores run at the FP8 rate, and E4M3 on Q and K alone costs about
// 3.5 % relative error, which with V's and P's E4M3 rounding would use up
// the 6 % budget.
//
// MX quantisation follows the OCP rule: e = floor(log2 amax) - 8, code =
// E4M3(clamp(x * 2^-e, +-448)) rounded to nearest even; with FP4 (E2M1)
// elements, for the diagonal-tiled variant below, e = floor(log2 amax) - 2
// and code = E2M1(clamp(x * 2^-e, +-6)), two codes per byte.
#include "attn_common.hpp"
#include "attn_internal.hpp"

namespace attn {

namespace {

// Block exponent of the OCP rule from a block maximum (> 0): floor(log2 amax)
// - 8, clamped to the E8M0 range [-127, 127].
__device__ __forceinline__ int mx_exp(float amax) {
  const int ex = __builtin_amdgcn_frexp_expf(amax);   // amax = m 2^ex, m in [0.5, 1)
  return min(max(ex - 1 - 8, -127), 127);
}

// Four E4M3 codes of x * 2^-e (clamped to +-448), packed little-endian.
__device__ __forceinline__ uint32_t mx_pack4(float a, float b, float c, float d, int e) {
  auto y = [&](float x) { return fminf(fmaxf(__builtin_amdgcn_ldexpf(x, -e), -448.0f), 448.0f); };
  int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y(a), y(b), 0, false);
  pk = __builtin_amdgcn_cvt_pk_fp8_f32(y(c), y(d), pk, true);
  return (uint32_t)pk;
}

// The FP4 (E2M1) block exponent of the OCP rule: floor(log2 amax) - 2, 2
// being the exponent of the largest power of two in E2M1 (4).
__device__ __forceinline__ int mx4_exp(float amax) {
  const int ex = __builtin_amdgcn_frexp_expf(amax);
  return min(max(ex - 1 - 2, -127), 127);
}

// Eight E2M1 codes of x * 2^-e (clamped to +-6), nibble i = element i.
__device__ __forceinline__ uint32_t mx4_pack8(const float* x, int e) {
  auto y = [&](float v) { return fminf(fmaxf(__builtin_amdgcn_ldexpf(v, -e), -6.0f), 6.0f); };
  uint32_t pk = 0;
  pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, y(x[0]), y(x[1]), 1.0f, 0);
  pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, y(x[2]), y(x[3]), 1.0f, 1);
  pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, y(x[4]), y(x[5]), 1.0f, 2);
  pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, y(x[6]), y(x[7]), 1.0f, 3);
  return pk;
}

// Blocks of 32 channels: one thread per (token, block). Scales go to
// [BH][srows][D / 32] with srows >= N rows per head (padding rows untouched).
// FP8: one code byte per element; FP4: two per byte, the even channel in
// the low nibble (rows of D / 2 bytes).
template <typename T, int D, bool FP4>
__global__ void __launch_bounds__(256) quant_mx_rows_kernel(const T* __restrict__ x, int64_t BH,
                                                            int N, int srows,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  constexpr int NB = D / 32;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= BH * N * NB) return;
  const int64_t row = id / NB;
  const int blk = (int)(id - row * NB);
  const int64_t bh = row / N;
  const int tok = (int)(row - bh * N);
  const T* src = x + row * D + 32 * blk;
  float v[32];
#pragma unroll
  for (int c = 0; c < 4; ++c) unpack8<T>(ld16(src + 8 * c), &v[8 * c]);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  uint8_t sb = 0;
  if (amax > 0.0f) {
    const int e = FP4 ? mx4_exp(amax) : mx_exp(amax);
    sb = (uint8_t)(e + 127);
    if constexpr (FP4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = mx4_pack8(&v[8 * i], e);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = mx_pack4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3], e);
    }
  }
  if constexpr (FP4) {
    st16(codes + row * (D / 2) + 16 * blk, u32x4{w[0], w[1], w[2], w[3]});
  } else {
    uint8_t* dst = codes + row * D + 32 * blk;
    st16(dst, u32x4{w[0], w[1], w[2], w[3]});
    st16(dst + 16, u32x4{w[4], w[5], w[6], w[7]});
  }
  scales[(bh * srows + tok) * NB + blk] = sb;
}

// Blocks of 32 tokens of one channel: one workgroup per (head, 64-token tile).
// FP8 (one code byte per element):
//   layout 0: codes [BH][N][D], scales [BH][ceil(N/32)][D] (blocks past N not
//             written);
//   layout 1: codes as transposed tiles [BH][ceil(N/64)][D][64] with zero
//             codes past N, scales [BH][2 ceil(N/64)][D] (a block past N:
//             scale byte 0).
// FP4 (two codes per byte, the lower index in the low nibble): layout 0
// codes [BH][N][D / 2] (channel pairs), layout 1 transposed tiles
// [BH][ceil(N/64)][D][32] (token pairs); scales as for FP8.
template <typename T, int D, bool FP4>
__global__ void __launch_bounds__(256) quant_mx_cols_kernel(const T* __restrict__ x, int N,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales,
                                                            int layout) {
  constexpr int CPR = D / 8;
  constexpr int TLD = D + 1;
  __shared__ float tile[64 * TLD];
  __shared__ __attribute__((aligned(16))) uint8_t ctile[64 * D];   // FP4: one nibble per byte
  const int nt = (N + 63) / 64;
  const int64_t bh = blockIdx.x / nt;
  const int t = (int)(blockIdx.x - bh * nt);
  const int r0 = 64 * t;
  const T* src = x + (bh * N + r0) * (int64_t)D;
  for (int ch = threadIdx.x; ch < 64 * CPR; ch += 256) {
    const int r = ch / CPR, c = ch - r * CPR;
    float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (r0 + r < N) unpack8<T>(ld16(src + (int64_t)r * D + 8 * c), v);
#pragma unroll
    for (int i = 0; i < 8; ++i) tile[r * TLD + 8 * c + i] = v[i];
  }
  __syncthreads();
  const int nblk32 = (N + 31) / 32;
  for (int task = threadIdx.x; task < 2 * D; task += 256) {
    const int d = task % D, j = task / D;
    const int tok0 = r0 + 32 * j;
    const int cnt = min(max(N - tok0, 0), 32);
    float amax = 0.0f;
    for (int i = 0; i < cnt; ++i) amax = fmaxf(amax, fabsf(tile[(32 * j + i) * TLD + d]));
    uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint8_t sb = 0;
    if (amax > 0.0f) {
      const int e = FP4 ? mx4_exp(amax) : mx_exp(amax);
      sb = (uint8_t)(e + 127);
      if constexpr (FP4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float col[8];
#pragma unroll
          for (int b = 0; b < 8; ++b) col[b] = tile[(32 * j + 8 * q + b) * TLD + d];   // rows past N are 0
          w[q] = mx4_pack8(col, e);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float* col = &tile[(32 * j + 4 * q) * TLD + d];
          w[q] = mx_pack4(col[0], col[TLD], col[2 * TLD], col[3 * TLD], e);   // rows past N are 0
        }
      }
    }
    if (layout == 1) {
      if constexpr (FP4) {
        st16(codes + ((bh * nt + t) * (int64_t)D + d) * 32 + 16 * j, u32x4{w[0], w[1], w[2], w[3]});
      } else {
        uint8_t* dst = codes + ((bh * nt + t) * (int64_t)D + d) * 64 + 32 * j;
        st16(dst, u32x4{w[0], w[1], w[2], w[3]});
        st16(dst + 16, u32x4{w[4], w[5], w[6], w[7]});
      }
      scales[((bh * nt + t) * 2 + j) * (int64_t)D + d] = sb;
    } else {
      if constexpr (FP4) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int b = 0; b < 8; ++b) ctile[(32 * j + 8 * q + b) * D + d] = (uint8_t)((w[q] >> (4 * b)) & 15);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int b = 0; b < 4; ++b) ctile[(32 * j + 4 * q + b) * D + d] = (uint8_t)(w[q] >> (8 * b));
      }
      if (cnt > 0) scales[(bh * nblk32 + 2 * t + j) * (int64_t)D + d] = sb;
    }
  }
  if (layout == 0) {
    __syncthreads();
    if constexpr (FP4) {
      // row r: D / 2 bytes, byte c = channels 2c (low nibble) and 2c + 1
      for (int ch = threadIdx.x; ch < 64 * (D / 32); ch += 256) {
        const int r = ch / (D / 32), c = ch - r * (D / 32);
        if (r0 + r < N) {
          uint32_t w4[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t wq = 0;
#pragma unroll
            for (int b = 0; b < 8; ++b) wq |= (uint32_t)ctile[r * D + 32 * c + 8 * q + b] << (4 * b);
            w4[q] = wq;
          }
          st16(codes + (bh * N + r0 + r) * (int64_t)(D / 2) + 16 * c, u32x4{w4[0], w4[1], w4[2], w4[3]});
        }
      }
    } else {
      for (int ch = threadIdx.x; ch < 64 * (D / 16); ch += 256) {
        const int r = ch / (D / 16), c = ch - r * (D / 16);
        if (r0 + r < N)
          st16(codes + (bh * N + r0 + r) * (int64_t)D + 16 * c, *(const u32x4*)&ctile[r * D + 16 * c]);
      }
    }
  }
}

// Four consecutive elements of a row in the output type, as floats.
template <typename TO>
__device__ __forceinline__ void get4(const TO* p, float (&v)[4]) {
  const u32x2 x = *(const u32x2*)p;
  const TO* e = (const TO*)&x;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = (float)e[r];
}

// ---------------------------------------------------------------------------
// MX attention: the quantised kernel's skeleton (4 waves x 32 query rows,
// 64-key tiles, two workgroups per CU, code tiles by direct loads into
// double buffers, one barrier per tile, S of tile i+1 beside the weights of
// tile i) with the P V product in MX blocks:
//   S_int^T = Kc Qc^T          i8 MFMA 32x32x32, exact int32; Q, K per-64-token
//                               INT8 blocks (attn_quantize_qk)
//   P^ = MX blocks of 32 keys of each query row, made in the kernel (scale
//        2^E, E = floor(log2 block max) - 7: every element below 256)
//   O^T += V^ P^T              v_mfma_scale_f32_32x32x64_f8f6f4 with V's and
//                               P's E8M0 block scales as operands
// so O accumulates in true units; the only rescale is the running-maximum one.
//
// Operand layout of the scaled FP8 MFMA (checked on the GPU): lane half h
// holds k-slots 16 h + (0..15) in its bytes 0..15 and 32 + 16 h + (0..15) in
// bytes 16..31; bytes 0..15 of both halves are scale block 0 (the scale comes
// from lane half 0), bytes 16..31 block 1 (from lane half 1). With FP4
// operands (E2M1, format 4) lane half h holds k-slots 32 h + (0..31) as the
// nibbles of its first 16 bytes (nibble i: bits 4 (i % 8) of dword i / 8),
// and its scale is that of block h. The FP4 x FP4 product runs at about
// twice the FP8 rate; an FP4 x FP8 product runs at the FP8 rate.
//
// The diagonal-tiled mixed variant ("Diagonal-Tiled Mixed-Precision
// Attention" of "Transformers Get a Turbo Boost with Mixed-Precision Magic",
// section "The DMA breakthrough": two low-bit MXFP products chosen per tile,
// the diagonal apart) runs in two passes of this kernel. A wave's 32 rows
// form one row block; the key tiles holding the positions of its rows (1 or
// 2) are its diagonal tiles.
//   PASS 1: every tile but the wave's diagonal ones (masked out), in MXFP4:
//           V from its MXFP4 copy (blocks of 32 keys of one channel), the
//           weights of each 32-key block with scale 2^E, E = floor(log2
//           block max) - 2, clamped to 6 and rounded to E2M1. The K rows are
//           permuted so that lane half h holds the scores of keys 32 h +
//           (0..31), the k-slots of the FP4 operand. Writes O / l (in the
//           output type), m and l (fp32) of every row to the partial buffer.
//   PASS 2: only the workgroup's diagonal tiles, each wave keeping its own,
//           in MXFP8 as in the MX mode; merges its result with the row's
//           pass 1 partial by log-sum-exp weights and writes O.
// Both passes keep the running maximum an integer, so a block's scale and
// its rounded weights do not depend on when the maximum was last raised, and
// splitting the keys over two passes changes no rounding.
template <typename TO, int D, int PASS>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
prefill_mx_kernel(FwdArgs a, int ntq, const int8_t* __restrict__ qc, const float* __restrict__ qs,
                  const int8_t* __restrict__ kc, const float* __restrict__ ks,
                  const uint8_t* __restrict__ vct, const uint8_t* __restrict__ vs,
                  float* __restrict__ part) {
  constexpr bool FP4 = PASS == 1;   // V^T tiles of D rows x 32 bytes (E2M1 pairs)
  constexpr int BM = 128;
  constexpr int KS = D / 32;       // i8 k-steps (32 channels each)
  constexpr int DB = D / 32;       // 32-channel blocks of O^T
  constexpr int KCPR = D / 16;     // 16-byte chunks per K code row
  constexpr int KRPI = 64 / KCPR;  // K rows per direct-load instruction
  constexpr float kLag = 2.0f;     // the running maximum may trail by this (log2)
  constexpr float kOff = 12582912.0f;   // 1.5 * 2^23
  __shared__ __attribute__((aligned(16))) uint8_t sk[2][64 * D];
  __shared__ __attribute__((aligned(16))) uint8_t sv[2][FP4 ? D * 32 : D * 64];
  __shared__ __attribute__((aligned(16))) uint8_t svs[2][2 * D];   // V scales [block][channel]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / ntq, qt_in = tile - bh * ntq;
  const int qt = a.causal ? ntq - 1 - qt_in : qt_in;   // heaviest causal q-tiles first
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const int bg = b * a.Hkv + g;
  const int q0 = qt * BM;
  const int nkt = (a.Nk + 63) / 64;
  const int8_t* Qc = qc + (int64_t)bh * a.Nq * D;
  const int8_t* Kc = kc + (int64_t)bg * a.Nk * D;
  const float* Ks = ks + (int64_t)bg * nkt;
  const uint8_t* Vt = vct + (int64_t)bg * nkt * D * (FP4 ? 32 : 64);
  const uint8_t* Vs = vs + (int64_t)bg * nkt * 2 * D;
  TO* Op = (TO*)a.o + (int64_t)bh * a.Nq * D;

  const int qlast = min(q0 + BM, a.Nq) - 1;
  const int kv_lo = a.window_w > 0 ? max(a.window_lo, a.pos0 + q0 - a.window_w + 1) : a.window_lo;
  const int kv_hi = a.causal ? min(a.Nk, a.pos0 + qlast + 1) : a.Nk;
  int t_lo = kv_lo / 64;
  int nt = kv_hi > kv_lo ? (kv_hi + 63) / 64 - t_lo : 0;
  // the diagonal key tiles of the workgroup's 128 rows and of this wave's 32
  const int64_t gpos = (int64_t)a.pos0 + q0, wpos = (int64_t)a.pos0 + q0 + 32 * wave;
  const int64_t wd_lo = wpos / 64, wd_hi = (wpos + 31) / 64;
  if constexpr (PASS == 2) {
    // only the workgroup's diagonal tiles that hold visible keys
    const int g_lo = (int)min(max(gpos / 64, (int64_t)t_lo), (int64_t)(t_lo + nt));
    const int g_hi = (int)min(max((gpos + 127) / 64 + 1, (int64_t)g_lo), (int64_t)(t_lo + nt));
    t_lo = g_lo;
    nt = g_hi - g_lo;
  }

  const int qrow = q0 + wave * 32 + col;
  const int qw0 = q0 + wave * 32;
  // Row qrow sees keys [row_lo, row_hi]; tiles inside the bounds common to
  // the wave's rows, [wave_lo, wave_hi], are not masked.
  const int wrow = a.window_w > 0 ? a.pos0 - a.window_w + 1 : -(1 << 30);
  const int row_lo = max(kv_lo, qrow + wrow);
  const int row_hi = a.causal ? min(a.pos0 + qrow, a.Nk - 1) : a.Nk - 1;
  const int wave_lo = max(kv_lo, qw0 + 31 + wrow);
  const int wave_hi = a.causal ? min(a.pos0 + qw0, a.Nk - 1) : a.Nk - 1;

  // Q codes as B operands of the i8 MFMA: lane half h of k-step k holds
  // channels 32 k + 16 h + (0..15); the wave's rows share one 64-row block.
  i32x4 qv[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    u32x4 raw = {0, 0, 0, 0};
    if (qrow < a.Nq) raw = ld16(Qc + (int64_t)qrow * D + 32 * k + 16 * half);
    qv[k] = __builtin_bit_cast(i32x4, raw);
  }
  const float cq = qs[(int64_t)bh * ((a.Nq + 63) / 64) + min(qw0, a.Nq - 1) / 64] * a.c;

  // K code row r holds key 32 blk + 16 h + 4 a + c for r = 32 blk + 8 a + 4 h + c:
  // lane half h's scores of 32-key block blk are keys 32 blk + 16 h + (0..15),
  // the bytes of P^T that the scaled MFMA wants, and each 32-key block of a
  // row is one scale block. Chunk c of a row sits at c ^ kswz(r), chunk c of
  // V^T row d at c ^ vswz(d).
  auto kswz = [](int r) { return KCPR == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3); };
  auto vswz = [](int d) { return (d >> 2) & 3; };
  auto kperm = [](int r) {
    return FP4 ? 32 * ((r >> 2) & 1) + 16 * (r >> 5) + 4 * ((r >> 3) & 3) + (r & 3)
               : 32 * (r >> 5) + 16 * ((r >> 2) & 1) + 4 * ((r >> 3) & 3) + (r & 3);
  };
  constexpr int NK = 16 / KRPI, NV = FP4 ? 1 : D / 64;
  uint32_t kofs[NK], vofs[NV];
#pragma unroll
  for (int u = 0; u < NK; ++u) {
    const int r = 16 * wave + KRPI * u + lane / KCPR, pos = lane % KCPR;
    kofs[u] = (uint32_t)(kperm(r) * D + 16 * (pos ^ kswz(r)));
  }
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int d = (D / 4) * wave + 16 * u + lane / 4, pos = lane % 4;
    // FP4: the tile's 16-byte chunk (row d, half h) sits at global chunk 2 d + h
    // and at LDS chunk 32 (d / 16) + 16 h + d % 16, so that the 16 lanes of
    // one LDS access read 256 contiguous bytes (conflict-free); lane i of the
    // wave lands LDS chunk 64 wave + i and reads the matching global chunk
    vofs[u] = FP4 ? (uint32_t)(16 * (32 * (lane >> 5) + 2 * (lane & 15) + ((lane >> 4) & 1)))
                  : (uint32_t)(d * 64 + 16 * (pos ^ vswz(d)));
  }
  constexpr int NVS = 2 * D / 16;   // 16-byte pieces of a V scale tile
  auto load_k = [&](int t, int buf) {
    const int8_t* base = Kc + (int64_t)64 * t * D;
    const int last = a.Nk - 1 - 64 * t;
    if (last >= 63) {
#pragma unroll
      for (int u = 0; u < NK; ++u) load_to_lds16(base, kofs[u], &sk[buf][(16 * wave + KRPI * u) * D]);
    } else {
#pragma unroll
      for (int u = 0; u < NK; ++u) {
        const int r0 = 16 * wave + KRPI * u;
        const int r = r0 + lane / KCPR, pos = lane % KCPR;
        load_to_lds16(base, (uint32_t)(min(kperm(r), last) * D + 16 * (pos ^ kswz(r))), &sk[buf][r0 * D]);
      }
    }
  };
  auto load_v = [&](int t, int buf) {
    if constexpr (FP4) {
      // D x 32 contiguous bytes: 1 KB per wave (waves 0-1 at head dim 64)
      if (D == 128 || wave < 2)
        load_to_lds16(Vt + (int64_t)t * D * 32 + 1024 * wave, vofs[0], &sv[buf][1024 * wave]);
    } else {
      const uint8_t* base = Vt + (int64_t)t * D * 64;
#pragma unroll
      for (int u = 0; u < NV; ++u) load_to_lds16(base, vofs[u], &sv[buf][((D / 4) * wave + 16 * u) * 64]);
    }
    // the tile's 2 D scale bytes ride along (wave 1)
    // (the byte offset is rebuilt from the lane id on the spot: kept across
    // the loop, it is spilled at head dim 128)
    if (wave == 1 && lane < NVS) {
      uint32_t ofs;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0\n\tv_lshlrev_b32 %0, 4, %0"
                   : "=v"(ofs));
      load_to_lds16(Vs + (int64_t)t * 2 * D, ofs, &svs[buf][0]);
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[db][j] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  // The int32 scores start from 0x4B400000, the bit pattern of 1.5 * 2^23:
  // |S| < 2^22, so each accumulator read as a float is exactly 1.5 * 2^23 + S.
  i32x16 magic;
#pragma unroll
  for (int j = 0; j < 16; ++j) magic[j] = 0x4B400000;
  asm volatile("" : "+v"(magic));
  auto s_mma = [&](int buf, i32x16 (&s)[2]) {
#pragma unroll
    for (int k = 0; k < KS; ++k)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int r = 32 * mb + col;
        const i32x4 ka = *(const i32x4*)&sk[buf][r * D + 16 * ((2 * k + half) ^ kswz(r))];
        s[mb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka, qv[k], k == 0 ? magic : s[mb], 0, 0, 0);
      }
  };

  // E4M3 (pass 1: E2M1) 1.0 in every byte (nibble), and a zero accumulator
  i32x8 ones8;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones8[j] = FP4 ? 0x22222222 : 0x38383838;
  f32x16 fzero;
#pragma unroll
  for (int j = 0; j < 16; ++j) fzero[j] = 0.0f;
  auto step = [&](int i, i32x16 (&cur)[2], i32x16 (&nxt)[2]) {
    const int t = t_lo + i;
    if (i + 2 < nt) load_k(t + 2, i & 1);
    if (i + 1 < nt) load_v(t + 1, (i + 1) & 1);
    // A block of zero codes has scale 0; the floor keeps masked scores at
    // -inf (-inf * 0 would be NaN) and changes nothing else.
    const float cf = fmaxf(cq * Ks[t], 1.17549435e-38f);
    float sf[2][16];   // kOff + S, exact
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) sf[mb][j] = __builtin_bit_cast(f32x16, cur[mb])[j];
    const int k0 = 64 * t;
    if constexpr (PASS != 0) {
      // pass 1 leaves out the wave's diagonal tiles, pass 2 keeps only them
      const bool dg = t >= wd_lo && t <= wd_hi;
      if (PASS == 1 ? dg : !dg) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int j = 0; j < 16; ++j) sf[mb][j] = -INFINITY;
      }
    }
    if (k0 < wave_lo || k0 + 63 > wave_hi) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = FP4 ? k0 + 32 * half + 16 * mb + 4 * (j >> 2) + (j & 3)
                              : k0 + 32 * mb + 16 * half + 4 * (j >> 2) + (j & 3);
          if (key < row_lo || key > row_hi) sf[mb][j] = -INFINITY;
        }
    }
    // per 32-key block: the largest kOff + S (pass 1: the lane holds all 32
    // keys of its block h, bm[0] = bm[1])
    float bm[2], rowm;
    if constexpr (FP4) {
      float b = sf[0][0];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) b = fmaxf(b, sf[mb][j]);
      bm[0] = bm[1] = b;
      rowm = halves_max(b);
    } else {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        bm[mb] = sf[mb][0];
#pragma unroll
        for (int j = 1; j < 16; ++j) bm[mb] = fmaxf(bm[mb], sf[mb][j]);
        bm[mb] = halves_max(bm[mb]);
      }
      rowm = fmaxf(bm[0], bm[1]);
    }
    const float mx = (rowm - kOff) * cf;   // exact subtraction
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kLag)) {
      asm volatile("" ::: "memory");
      const float m_new = PASS != 0 ? ceilf(fmaxf(m_run, mx)) : fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
      m_run = m_new;
    }
    const float mu = m_run == -INFINITY ? 0.0f : m_run;
    // exponent = S cf - mu = (kOff + S) cf - (kOff cf + mu): one FMA per
    // score; the rounding of kOff cf + mu (< 0.9 cf + 2^-21) is far below the
    // INT8 rounding of the scores for cf < 0.03, larger factors take the
    // exact form. The diagonal-tiled passes always take it: a common error of
    // that size would move weights across E2M1 rounding midpoints (steps of
    // up to a third of a weight) that the exact exponent keeps.
    float C = fmaf(kOff, cf, mu);
    if (PASS != 0 || cf >= 0.03f) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) sf[mb][j] -= kOff;
        bm[mb] -= kOff;
      }
      C = mu;
    }
    // Each 32-key block mb of a row's weights (16 in each lane half) is one
    // MX block with scale 2^E, E = floor(log2 of its largest weight) - 7, so
    // its elements lie below 256. The largest weight's exponent is the block
    // maximum through the same FMA, and 2^-E folds into the FMA's constant:
    // the weights come out already scaled.
    int E[2];
    float Cm[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const float x = fmaf(bm[mb], cf, -C);
      E[mb] = bm[mb] == -INFINITY ? -127 : max((int)__builtin_floorf(x) - (FP4 ? 2 : 7), -127);
      Cm[mb] = C + (float)E[mb];   // exact: C's ulp is below 1 and E an integer
    }

    // S of tile i + 1 after the weights of tile i (K operand reads, vector
    // work, then the MFMAs; the other wave of the SIMD fills the gaps).
    s_mma((i + 1) & 1, nxt);
    i32x8 pb;
    if constexpr (FP4) {
      // E2M1 weights, nibble 16 mb + j = key 32 h + 16 mb + j (FP4 operands
      // read dwords 0..3 only). The weights lie below 8; the conversion
      // itself saturates everything from 6 up to infinity to 6 (checked on
      // the GPU), which is the clamp the rounding rule asks for.
      asm volatile("" : "=v"(pb));
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          float e[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) e[k] = __builtin_amdgcn_exp2f(fmaf(sf[mb][8 * w + k], cf, -Cm[0]));
          uint32_t pk = 0;
          pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, e[0], e[1], 1.0f, 0);
          pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, e[2], e[3], 1.0f, 1);
          pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, e[4], e[5], 1.0f, 2);
          pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, e[6], e[7], 1.0f, 3);
          pb[2 * mb + w] = (int)pk;
        }
    } else {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          float e[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) e[k] = __builtin_amdgcn_exp2f(fmaf(sf[mb][4 * q4 + k], cf, -Cm[mb]));
          // (the second conversion writes the upper half, so the first one may
          // start from whatever the register holds: no zeroing move)
          int pk;
          asm volatile("" : "=v"(pk));
          pk = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], pk, false);
          pk = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], pk, true);
          pb[4 * mb + q4] = pk;
        }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * KS, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 80, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * KS, 0);
    const int psc = (half ? E[1] : E[0]) + 127;   // lane half h: scale of block h
    // The denominator: the tile's row sums of the weights the numerator uses,
    // in unscaled units, from one more scaled MFMA against an all-ones block
    // (every row of the product is the same column sum).
    constexpr int fmt = FP4 ? 4 : 0;   // E2M1 or E4M3 operands
    const f32x16 rs = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones8, pb, fzero, fmt, fmt, 0, 127, 0, psc);

    // O^T += V^T P^T for tile i: one scaled FP8 MFMA per 32 channels (a
    // scheduling fence keeps the V operand reads from being hoisted above
    // the weights, which would run the wave out of registers).
    __builtin_amdgcn_sched_barrier(0);
    const int vb = i & 1;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = 32 * db + col;
      i32x8 va;
      if constexpr (FP4) {
        // keys 32 h + (0..31) of channel d: LDS chunk 32 (d / 16) + 16 h + d % 16
        const u32x4 x = ld16(&sv[vb][16 * (32 * (d >> 4) + 16 * half + (d & 15))]);
        asm volatile("" : "=v"(va));
        va[0] = (int)x[0];
        va[1] = (int)x[1];
        va[2] = (int)x[2];
        va[3] = (int)x[3];
      } else {
        const uint8_t* row = &sv[vb][d * 64];
        const u32x4 lo = ld16(row + 16 * (half ^ vswz(d)));         // keys 16 h + (0..15)
        const u32x4 hi = ld16(row + 16 * ((2 + half) ^ vswz(d)));   // keys 32 + 16 h + (0..15)
        va = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
      const int vsc = svs[vb][half * D + d];
      oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, oacc[db], fmt, fmt, 0, vsc, 0, psc);
    }
    l_run += rs[0];
    vmem_wait_all();
    __syncthreads();
  };

  if (nt > 0) {
    load_k(t_lo, 0);
    load_v(t_lo, 0);
    if (nt > 1) load_k(t_lo + 1, 1);
    vmem_wait_all();
    __syncthreads();
    i32x16 s0[2], s1[2];
    s_mma(0, s0);
    __syncthreads();   // step 0 overwrites the K buffer just read
    int i = 0;
    for (; i + 1 < nt; i += 2) {
      step(i, s0, s1);
      step(i + 1, s1, s0);
    }
    if (i < nt) step(i, s0, s1);
  }

  const float l = l_run;   // both lane halves hold the row's full sum
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  if (qrow >= a.Nq) return;
  // the partial of row qrow (diagonal-tiled passes), D * sizeof(TO) + 16
  // bytes: O / l in the output type, then m (exp2 units, an integer or -inf)
  // and l in fp32
  TO* prow = (TO*)((char*)part + ((int64_t)bh * a.Nq + qrow) * (D * (int)sizeof(TO) + 16));
  float* pml = (float*)(prow + D);
  if constexpr (PASS == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d = 32 * db + 8 * a4 + 4 * half;
        TO o4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o4[r] = Elem<TO>::from_float(oacc[db][4 * a4 + r] * inv);
        *(u32x2*)(prow + d) = *(const u32x2*)o4;
      }
    if (half == 0) *(f32x4*)pml = f32x4{m_run, l, 0.0f, 0.0f};
    return;
  }
  float w1 = 0.0f, w2 = 1.0f;   // the weights of the pass 1 partial and of this result
  if constexpr (PASS == 2) {
    const f32x4 ml = *(const f32x4*)pml;
    const float M = fmaxf(ml[0], m_run);
    w1 = ml[0] == -INFINITY ? 0.0f : ml[1] * __builtin_amdgcn_exp2f(ml[0] - M);
    w2 = m_run == -INFINITY ? 0.0f : l * __builtin_amdgcn_exp2f(m_run - M);
    const float L = w1 + w2;
    const float r = L > 0.0f ? 1.0f / L : 0.0f;
    w1 *= r;
    w2 *= r;
  }
  TO* orow = Op + (int64_t)qrow * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d = 32 * db + 8 * a4 + 4 * half;
      float o1[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (PASS == 2) get4<TO>(prow + d, o1);
      TO o4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) o4[r] = Elem<TO>::from_float(fmaf(w2, oacc[db][4 * a4 + r] * inv, w1 * o1[r]));
      *(u32x2*)(orow + d) = *(const u32x2*)o4;
    }
}

template <typename TO, int D>
hipError_t prefill_mx_t(const FwdArgs& a, const int8_t* qc, const float* qs, const int8_t* kc,
                        const float* ks, const uint8_t* vct, const uint8_t* vs, const uint8_t* v4t,
                        const uint8_t* v4s, float* part, hipStream_t st) {
  const int ntq = (a.Nq + 127) / 128;
  const int64_t grid = (int64_t)a.B * a.Hq * ntq;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (v4t == nullptr) {
    hipLaunchKernelGGL((prefill_mx_kernel<TO, D, 0>), dim3((unsigned)grid), dim3(256), 0, st, a, ntq,
                       qc, qs, kc, ks, vct, vs, nullptr);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((prefill_mx_kernel<TO, D, 1>), dim3((unsigned)grid), dim3(256), 0, st, a, ntq,
                     qc, qs, kc, ks, v4t, v4s, part);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prefill_mx_kernel<TO, D, 2>), dim3((unsigned)grid), dim3(256), 0, st, a, ntq,
                     qc, qs, kc, ks, vct, vs, part);
  return hipGetLastError();
}

template <typename T, bool FP4>
hipError_t quant_mx_t(const void* x, int64_t BH, int N, int D, int axis, int layout, int srows,
                      uint8_t* codes, uint8_t* scales, hipStream_t st) {
  if (axis == 0) {
    const int64_t blocks = (BH * N * (D / 32) + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (D == 64)
      hipLaunchKernelGGL((quant_mx_rows_kernel<T, 64, FP4>), dim3((unsigned)blocks), dim3(256), 0,
                         st, (const T*)x, BH, N, srows, codes, scales);
    else
      hipLaunchKernelGGL((quant_mx_rows_kernel<T, 128, FP4>), dim3((unsigned)blocks), dim3(256), 0,
                         st, (const T*)x, BH, N, srows, codes, scales);
  } else {
    const int64_t grid = BH * ((N + 63) / 64);
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (D == 64)
      hipLaunchKernelGGL((quant_mx_cols_kernel<T, 64, FP4>), dim3((unsigned)grid), dim3(256), 0, st,
                         (const T*)x, N, codes, scales, layout);
    else
      hipLaunchKernelGGL((quant_mx_cols_kernel<T, 128, FP4>), dim3((unsigned)grid), dim3(256), 0,
                         st, (const T*)x, N, codes, scales, layout);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_mx(const void* x, int elem, int64_t BH, int N, int D, int axis, int layout,
                           int srows, uint8_t* codes, uint8_t* scales, hipStream_t s, bool fp4) {
  if (fp4)
    return elem == 2 ? quant_mx_t<__bf16, true>(x, BH, N, D, axis, layout, srows, codes, scales, s)
                     : quant_mx_t<_Float16, true>(x, BH, N, D, axis, layout, srows, codes, scales, s);
  return elem == 2 ? quant_mx_t<__bf16, false>(x, BH, N, D, axis, layout, srows, codes, scales, s)
                   : quant_mx_t<_Float16, false>(x, BH, N, D, axis, layout, srows, codes, scales, s);
}

hipError_t launch_prefill_mx(const FwdArgs& a, const int8_t* qc, const float* qs,
                             const int8_t* kc, const float* ks, const uint8_t* vct,
                             const uint8_t* vs, const uint8_t* v4t, const uint8_t* v4s,
                             float* part, int elem_out, hipStream_t s) {
  if (elem_out == 2)
    return a.D == 64 ? prefill_mx_t<__bf16, 64>(a, qc, qs, kc, ks, vct, vs, v4t, v4s, part, s)
                     : prefill_mx_t<__bf16, 128>(a, qc, qs, kc, ks, vct, vs, v4t, v4s, part, s);
  return a.D == 64 ? prefill_mx_t<_Float16, 64>(a, qc, qs, kc, ks, vct, vs, v4t, v4s, part, s)
                   : prefill_mx_t<_Float16, 128>(a, qc, qs, kc, ks, vct, vs, v4t, v4s, part, s);
}

}  // namespace attn
