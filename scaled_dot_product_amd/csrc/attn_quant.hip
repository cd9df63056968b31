// attn_quant.hip — the opt-in low-precision mode: INT8 Q K^T and FP8 P V.
//
// The recipe is the "SageAttention 2 INT8 QK . FP8 PV" row of the table in
// section 1 of "Attention kernels on a home RTX 5080": Q and K become
// symmetric INT8 codes with one fp32 scale per 64-token block of one head,
// V becomes OCP FP8 E4M3 codes with one scale per 64-token block, and the
// softmax weights are rounded to E4M3 with a per-key-block scale (each weight
// is at most 4: the running maximum trails the scores by at most 2 in log2).
//
//   quant_int8_kernel   per block: amax, scale = amax/127, inv = 127/amax,
//                       code = clamp(rint(x*inv), -127, 127)  (bit-exact)
//   quant_e4m3_kernel   per block: scale = amax/448, inv = 448/amax,
//                       code = E4M3(clamp(x*inv, -448, 448)) via the gfx950
//                       conversion (OCP E4M3, round to nearest even)
//   prefill_quant_kernel
//     S_int^T = Kc Qc^T              i8 MFMA 32x32x32, exact int32
//     exponent = S_int * (s_q s_k scale log2 e) - m   (one FMA per score)
//     P^ = E4M3(112 P s_v / s_ref)   (s_v: the tile's V block scale, s_ref
//                                     the largest one the query tile sees;
//                                     folded into the exponent's bias)
//     O_acc += Vc^T P^T              fp8 MFMA 32x32x64, fp32 accumulation
//     l += (row sums of P^) * s_ref / (112 s_v)   (the sums from one more fp8
//                                     MFMA against an all-ones block)
//   O = O_acc * s_ref / 112 / l.
#include "attn_common.hpp"
#include "attn_internal.hpp"

namespace attn {

namespace {

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
// With rope.on, each row is first turned by its rotary position embedding at
// position pos_base + n (the rotation fused into the pass that reads the
// row anyway).
template <typename T, int D>
__global__ void __launch_bounds__(256) quant_int8_kernel(const T* __restrict__ x, int N,
                                                          int8_t* __restrict__ codes,
                                                          float* __restrict__ scales,
                                                          RopeArgs rope, int pos_base) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per token row
  constexpr int PER = 64 * CPR / 256;        // chunks per thread
  static_assert(256 % CPR == 0, "a thread keeps one chunk position");
  __shared__ float red[4];
  __shared__ float rh[kRopeMaxPairs], rl[kRopeMaxPairs];
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
  }
  if (rope.on) {
    if (threadIdx.x < kRopeMaxPairs) {
      rh[threadIdx.x] = rope.rev_hi[threadIdx.x];
      rl[threadIdx.x] = rope.rev_lo[threadIdx.x];
    }
    __syncthreads();
    const int c = threadIdx.x % CPR;         // the same chunk position for every u
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const float pos = (float)(pos_base + r0 + (int)((threadIdx.x + 256 * u) / CPR));
      if (rope.style == 0) {
        // channel 8 c + e pairs with the one D/2 away: chunk c ^ (CPR/2), the
        // same row in lane ^ (CPR/2) of this wave
        constexpr int HP = CPR / 2;
        const bool first = c < HP;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float other = __shfl_xor(vals[u][e], HP, 64);
          const int i = (c % HP) * 8 + e;
          float xa = first ? vals[u][e] : other, xb = first ? other : vals[u][e];
          rope_rotate(xa, xb, pos, rh[i], rl[i]);
          vals[u][e] = first ? xa : xb;
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = 4 * c + q;
          rope_rotate(vals[u][2 * q], vals[u][2 * q + 1], pos, rh[i], rl[i]);
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < PER; ++u)
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(vals[u][i]));
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
// Quantised prefill: 4 waves x 32 query rows, 64-key tiles, two workgroups
// per CU, software-pipelined like the exact kernel (S of tile i+1 issued
// right after the exponentials of tile i, while the SIMD's other wave runs
// its own vector work; code tiles go straight from HBM into XOR-swizzled LDS
// tiles).
//
// The V block scale s_v changes from tile to tile. Rather than rescale the
// fp32 output by s_v after every tile, each tile's weights are quantised as
// E4M3(112 P s_v / s_ref) with s_ref the largest V block scale the query tile
// sees: the factor 112 s_v / s_ref <= 112 goes into the exponent's bias
// (free), the fp8 products accumulate straight into O, and the epilogue
// multiplies by s_ref / 112 once. The denominator sums the quantised
// weights the numerator uses, taken back by the same per-tile factor.
template <typename TO, int D>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
prefill_quant_kernel(FwdArgs a, int ntq, const int8_t* __restrict__ qc,
                     const float* __restrict__ qs, const int8_t* __restrict__ kc,
                     const float* __restrict__ ks, const uint8_t* __restrict__ vct,
                     const float* __restrict__ vs) {
  constexpr int BM = 128;
  constexpr int KS = D / 32;       // i8 k-steps (32 channels each)
  constexpr int DB = D / 32;
  constexpr int KCPR = D / 16;     // 16-byte chunks per K code row
  constexpr int KRPI = 64 / KCPR;  // K rows per direct-load instruction
  constexpr float kLog2_448 = 8.807354922057604f;
  // exp2 rounds within an ulp or so; lowering the bias by 2^-12 keeps every
  // scaled weight <= 448 (the largest E4M3 magnitude) without a clamp
  constexpr float kMargin = 2.44140625e-4f;
  // The running maximum may trail the true one by up to kLag powers of two
  // before O is rescaled; the weights' FP8 scale is lowered by 2^kLag so that
  // none of them exceeds 448 meanwhile (relative FP8 precision is unchanged,
  // the smallest weights reach the subnormal range 2 powers of two earlier).
  constexpr float kLag = 2.0f;
  __shared__ __attribute__((aligned(16))) uint8_t sk[2][64 * D];
  __shared__ __attribute__((aligned(16))) uint8_t sv[2][D * 64];
  __shared__ float sred[4];
  // Per visible V block: the exponent bias log2(s_v / s_ref) + const and
  // 2^-bias (the denominator's factor), taken once per workgroup for the
  // first kTileCache blocks instead of once per wave and block.
  constexpr int kTileCache = 1024;
  __shared__ float2 stile[kTileCache];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  // (a per-row window: row q0 has the lowest bound)
  const int kv_lo = a.window_w > 0 ? max(a.window_lo, a.pos0 + q0 - a.window_w + 1) : a.window_lo;
  const int kv_hi = a.causal ? min(a.Nk, a.pos0 + qlast + 1) : a.Nk;
  const int t_lo = kv_lo / 64;
  const int nt = kv_hi > kv_lo ? (kv_hi + 63) / 64 - t_lo : 0;

  // s_ref over the visible tiles (0 only when every one of those V blocks is 0).
  float sref = 0.0f;
  for (int t = t_lo + tid; t < t_lo + nt; t += 256) sref = fmaxf(sref, Vs[t]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sref = fmaxf(sref, __shfl_xor(sref, off, 64));
  if (lane == 0) sred[wave] = sref;
  __syncthreads();
  sref = fmaxf(fmaxf(sred[0], sred[1]), fmaxf(sred[2], sred[3]));
  // (the tile factor s_v / s_ref scales a tile's numerator and denominator
  // alike, so a reciprocal's rounding cancels)
  const float inv_sref = sref > 0.0f ? 1.0f / sref : 0.0f;
  auto tile_bias = [&](int t) {
    const float ratio = sref > 0.0f ? fmaxf(Vs[t] * inv_sref, 9.5367431640625e-7f) : 1.0f;
    const float bias = __builtin_amdgcn_logf(ratio) + (kLog2_448 - kMargin - kLag);   // log2
    return float2{bias, __builtin_amdgcn_exp2f(-bias)};
  };
  for (int u = tid; u < min(nt, kTileCache); u += 256) stile[u] = tile_bias(t_lo + u);
  __syncthreads();

  const int qrow = q0 + wave * 32 + col;
  const int qw0 = q0 + wave * 32;
  // Row qrow sees keys [row_lo, row_hi] (shared lower bound, per-row window,
  // causal diagonal, last key); tiles inside the bounds common to the wave's
  // rows, [wave_lo, wave_hi], are not masked.
  const int wrow = a.window_w > 0 ? a.pos0 - a.window_w + 1 : -(1 << 30);   // row r: key >= r + wrow
  const int row_lo = max(kv_lo, qrow + wrow);
  const int row_hi = a.causal ? min(a.pos0 + qrow, a.Nk - 1) : a.Nk - 1;
  const int wave_lo = max(kv_lo, qw0 + 31 + wrow);
  const int wave_hi = a.causal ? min(a.pos0 + qw0, a.Nk - 1) : a.Nk - 1;
  // Q codes as B operands: lane half h of k-step k holds channels 32 k + 16 h + (0..15).
  i32x4 qv[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    u32x4 raw = {0, 0, 0, 0};
    if (qrow < a.Nq) raw = ld16(Qc + (int64_t)qrow * D + 32 * k + 16 * half);
    qv[k] = __builtin_bit_cast(i32x4, raw);
  }
  // The wave's 32 rows lie in one 64-row block (q0 is a multiple of 128).
  const float cq = qs[(int64_t)bh * ((a.Nq + 63) / 64) + min(qw0, a.Nq - 1) / 64] * a.c;

  // K code row r holds key 32 h + 16 blk + 4 a + b for r = 32 blk + 8 a + 4 h + b,
  // so lane half h's 32 scores of a tile are keys 32 h .. 32 h + 31 in B-operand
  // slot order. Chunk c of a row sits at position c ^ kswz(r), chunk c of V^T row
  // d (64 keys) at c ^ vswz(d): the 16 lanes of an operand read hit distinct banks.
  auto kswz = [](int r) { return KCPR == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3); };
  auto vswz = [](int d) { return (d >> 2) & 3; };
  // Per-lane byte offsets inside a tile are loop invariant; in the ragged last
  // K tile, rows past Nk clamp to the last key (masked).
  constexpr int NK = 16 / KRPI, NV = D / 64;
  uint32_t kofs[NK], vofs[NV];
#pragma unroll
  for (int u = 0; u < NK; ++u) {
    const int r = 16 * wave + KRPI * u + lane / KCPR, pos = lane % KCPR;
    const int key = 32 * ((r >> 2) & 1) + 16 * (r >> 5) + 4 * ((r >> 3) & 3) + (r & 3);
    kofs[u] = (uint32_t)(key * D + 16 * (pos ^ kswz(r)));
  }
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int d = (D / 4) * wave + 16 * u + lane / 4, pos = lane % 4;
    vofs[u] = (uint32_t)(d * 64 + 16 * (pos ^ vswz(d)));
  }
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
        const int key = 32 * ((r >> 2) & 1) + 16 * (r >> 5) + 4 * ((r >> 3) & 3) + (r & 3);
        const uint32_t off = (uint32_t)(min(key, last) * D + 16 * (pos ^ kswz(r)));
        load_to_lds16(base, off, &sk[buf][r0 * D]);
      }
    }
  };
  auto load_v = [&](int t, int buf) {
    const uint8_t* base = Vt + (int64_t)t * D * 64;
#pragma unroll
    for (int u = 0; u < NV; ++u) load_to_lds16(base, vofs[u], &sv[buf][((D / 4) * wave + 16 * u) * 64]);
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[db][j] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  // The int32 scores start from 0x4B400000, the bit pattern of 1.5 * 2^23:
  // |S| < 2^22, so each accumulator, read as a float, is exactly 1.5 * 2^23 + S
  // and no int-to-float conversion is needed.
  i32x16 magic;
#pragma unroll
  for (int j = 0; j < 16; ++j) magic[j] = 0x4B400000;
  // opaque to the compiler: the constant stays in its 16 registers instead of
  // being copied in again from scalar registers before every tile
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

  // E4M3 1.0 in every byte, and a zero accumulator
  i32x8 ones8;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones8[j] = 0x38383838;
  asm volatile("" : "+v"(ones8));   // kept in registers, not rebuilt per tile
  f32x16 fzero;
#pragma unroll
  for (int j = 0; j < 16; ++j) fzero[j] = 0.0f;
  auto step = [&](int i, i32x16 (&cur)[2], i32x16 (&nxt)[2]) {
    const int t = t_lo + i;
    if (i + 2 < nt) load_k(t + 2, i & 1);
    if (i + 1 < nt) load_v(t + 1, (i + 1) & 1);
    // A block of zero codes has scale 0; a positive floor keeps masked scores
    // at -inf (-inf * 0 would be NaN) and changes nothing else, as every score
    // of such a block is exactly 0.
    const float cf = fmaxf(cq * Ks[t], 1.17549435e-38f);
    const float2 tb = i < kTileCache ? stile[i] : tile_bias(t);
    const float bias = tb.x;
    constexpr float kOff = 12582912.0f;   // 1.5 * 2^23
    float sf[2][16];                      // kOff + S
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) sf[mb][j] = __builtin_bit_cast(f32x16, cur[mb])[j];
    // (the whole vector is reinterpreted: a bit cast of one element of the
    // accumulator vector was miscompiled into copies of element 0)
    const int k0 = 64 * t;
    if (k0 < wave_lo || k0 + 63 > wave_hi) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = k0 + 32 * half + 16 * mb + 4 * (j >> 2) + (j & 3);
          if (key < row_lo || key > row_hi) sf[mb][j] = -INFINITY;
        }
    }
    float mx = sf[0][0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sf[0][j]);
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sf[1][j]);
    mx = (halves_max(mx) - kOff) * cf;   // exact subtraction
    // the running maximum must be within kLag of the scores: every scaled
    // weight stays <= 448
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kLag)) {
      asm volatile("" ::: "memory");
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
      m_run = m_new;
    }
    const float mu = (m_run == -INFINITY ? 0.0f : m_run) - bias;
    // exponent = S cf - mu = (kOff + S) cf - (kOff cf + mu): one FMA per score.
    // The rounding of kOff cf + mu shifts every exponent of the tile by at
    // most 2^-24 |kOff cf + mu| < 0.9 cf + 2^-21, far below the effect of the
    // INT8 rounding of the scores; it must also stay below the headroom from
    // 448 up to the E4M3 rounding boundary 464 (0.05 in log2), which holds for
    // cf < 0.03. Larger factors (from large block maxima or a large scale;
    // with scale 1/sqrt(128), a product of Q and K block maxima above about
    // 3800) take the exact form.
    float C = fmaf(kOff, cf, mu);
    if (cf >= 0.03f) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) sf[mb][j] -= kOff;
      C = mu;
    }

    // S of tile i + 1 (i8 MFMA) and the weights of tile i. The groups below
    // ask for the K operand reads, then the vector work, then the MFMAs; the
    // compiler still sinks the weights past the closing barrier, where they
    // run beside the P V MFMAs. Measured: about 1 % faster than one MFMA per
    // tenth of the vector work; pinning the weights before the barrier was
    // 1-2 % slower.
    s_mma((i + 1) & 1, nxt);
    i32x8 pb;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float e[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) e[k] = __builtin_amdgcn_exp2f(fmaf(sf[mb][4 * q4 + k], cf, -C));
        // (the second conversion writes the upper half, so the first one may
        // start from whatever the register holds: no zeroing move)
        int pk;
        asm volatile("" : "=v"(pk));
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], pk, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], pk, true);
        pb[4 * mb + q4] = pk;
      }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * KS, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 80, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * KS, 0);
    // The tile's row sums of the FP8 weights, from one more MFMA against an
    // all-ones block (every row of the product is the same column sum), taken
    // back to unscaled weights for the denominator.
    const f32x16 rs = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones8, pb, fzero, 0, 0, 0, 127, 0, 127);

    // O^T += V^T P^T (fp8 x fp8 -> fp32) for tile i: one MFMA per 32 channels.
    const int vb = i & 1;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = 32 * db + col;
      const uint8_t* row = &sv[vb][d * 64];
      const u32x4 lo = ld16(row + 16 * ((2 * half) ^ vswz(d)));
      const u32x4 hi = ld16(row + 16 * ((2 * half + 1) ^ vswz(d)));
      const i32x8 va = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                        (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, oacc[db], 0, 0, 0, 127, 0, 127);
    }
    l_run += rs[0] * tb.y;
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
  // undo the fp8 weight scaling: 448 * 2^-(margin + lag) / s_ref
  const float inv = l > 0.0f ? (sref * __builtin_amdgcn_exp2f(kMargin + kLag) / 448.0f) / l : 0.0f;
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
                        hipStream_t st, const RopeArgs& rope, int pos_base) {
  const int64_t grid = BH * ((N + 63) / 64);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (D == 64)
    hipLaunchKernelGGL((quant_int8_kernel<T, 64>), dim3((unsigned)grid), dim3(256), 0, st, (const T*)x,
                       N, c, s, rope, pos_base);
  else
    hipLaunchKernelGGL((quant_int8_kernel<T, 128>), dim3((unsigned)grid), dim3(256), 0, st, (const T*)x,
                       N, c, s, rope, pos_base);
  return hipGetLastError();
}

// Rotary position embedding of whole rows (for K in the exact mode, one pass
// in and out): row n of each head at position pos_base + n. Style 0: one
// thread per (row, chunk c < CPR/2) turns chunks c and c + CPR/2 together;
// style 1: one thread per (row, chunk). x and y may be the same buffer.
template <typename T, int D>
__global__ void __launch_bounds__(256) rope_kernel(const T* x, T* y, int64_t nrows, int N,
                                                   int pos_base, RopeArgs rope) {
  constexpr int CPR = D / 8;
  __shared__ float rh[kRopeMaxPairs], rl[kRopeMaxPairs];
  if (threadIdx.x < kRopeMaxPairs) {
    rh[threadIdx.x] = rope.rev_hi[threadIdx.x];
    rl[threadIdx.x] = rope.rev_lo[threadIdx.x];
  }
  __syncthreads();
  const int per_row = rope.style == 0 ? CPR / 2 : CPR;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= nrows * per_row) return;
  const int64_t row = id / per_row;
  const int c = (int)(id - row * per_row);
  const float pos = (float)(pos_base + (int)(row % N));
  const T* src = x + row * D;
  T* dst = y + row * D;
  if (rope.style == 0) {
    float a[8], b[8];
    unpack8<T>(ld16(src + 8 * c), a);
    unpack8<T>(ld16(src + 8 * (c + CPR / 2)), b);
#pragma unroll
    for (int e = 0; e < 8; ++e) rope_rotate(a[e], b[e], pos, rh[8 * c + e], rl[8 * c + e]);
    T oa[8], ob[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      oa[e] = Elem<T>::from_float(a[e]);
      ob[e] = Elem<T>::from_float(b[e]);
    }
    st16(dst + 8 * c, *(const u32x4*)oa);
    st16(dst + 8 * (c + CPR / 2), *(const u32x4*)ob);
  } else {
    float v[8];
    unpack8<T>(ld16(src + 8 * c), v);
#pragma unroll
    for (int q = 0; q < 4; ++q) rope_rotate(v[2 * q], v[2 * q + 1], pos, rh[4 * c + q], rl[4 * c + q]);
    T o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = Elem<T>::from_float(v[e]);
    st16(dst + 8 * c, *(const u32x4*)o);
  }
}

template <typename T>
hipError_t rope_t(const void* x, void* y, int64_t BH, int N, int D, int pos_base,
                  const RopeArgs& rope, hipStream_t st) {
  const int64_t nrows = BH * N;
  const int per_row = rope.style == 0 ? D / 16 : D / 8;
  const int64_t grid = (nrows * per_row + 255) / 256;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (D == 64)
    hipLaunchKernelGGL((rope_kernel<T, 64>), dim3((unsigned)grid), dim3(256), 0, st, (const T*)x,
                       (T*)y, nrows, N, pos_base, rope);
  else
    hipLaunchKernelGGL((rope_kernel<T, 128>), dim3((unsigned)grid), dim3(256), 0, st, (const T*)x,
                       (T*)y, nrows, N, pos_base, rope);
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
                             float* scales, hipStream_t s, const RopeArgs* rope, int pos_base) {
  RopeArgs none;
  none.on = 0;
  none.style = 0;
  const RopeArgs& r = rope ? *rope : none;
  return elem == 2 ? quant_int8_t<__bf16>(x, BH, N, D, codes, scales, s, r, pos_base)
                   : quant_int8_t<_Float16>(x, BH, N, D, codes, scales, s, r, pos_base);
}

hipError_t launch_rope(const void* x, void* y, int elem, int64_t BH, int N, int D, int pos_base,
                       const RopeArgs& rope, hipStream_t s) {
  return elem == 2 ? rope_t<__bf16>(x, y, BH, N, D, pos_base, rope, s)
                   : rope_t<_Float16>(x, y, BH, N, D, pos_base, rope, s);
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
