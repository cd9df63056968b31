// attn_common.hpp — device helpers shared by the gfx950 attention kernels.
//
// Matrix-core conventions used throughout (v_mfma_*_32x32x{16,32,64}):
//   A operand: lane l holds row (l % 32) of A, K-slots of lane half (l / 32).
//   B operand: lane l holds column (l % 32) of B, same K-slots.
//   C/D:       lane l, register j holds row 8*(j/4) + 4*(l/32) + (j%4),
//              column l % 32.
// A and B pair K-slots symmetrically, so any consistent slot -> K-index map
// gives the same product; the kernels pick the map that keeps every operand
// a contiguous 16-byte read.
//
// Scores are computed transposed, S^T = K Q^T, so that a lane owns one query
// column: the row maximum and sum of the softmax are in-lane reductions plus
// one exchange between the two lane halves, and the probabilities are already
// in B-operand position for O^T += V^T P^T.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// 16-bit element traits: the 8-wide operand vector and the MFMA on it.
template <typename T> struct Elem;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <> struct Elem<__bf16> {
  typedef bf16x8 vec8;
  // acc + (sum of the 8 elements of v), as 4 packed dot products with 1
  static __device__ __forceinline__ float sum8(vec8 v, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[2 * i], v[2 * i + 1]}, one, acc, false);
    return acc;
  }
  static __device__ __forceinline__ f32x16 mma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ __bf16 from_float(float x) { return (__bf16)x; }
};
template <> struct Elem<_Float16> {
  typedef f16x8 vec8;
  static __device__ __forceinline__ float sum8(vec8 v, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2(f16x2{v[2 * i], v[2 * i + 1]}, one, acc, false);
    return acc;
  }
  static __device__ __forceinline__ f32x16 mma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ _Float16 from_float(float x) { return (_Float16)x; }
};

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *(u32x4*)p = v; }

// Reductions across the two lane halves (lane l with lane l ^ 32) with one
// v_permlane32_swap: with both operands x, the first result holds x of the
// low half in every lane and the second holds x of the high half.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Arrival counting for a fused merge of partials (split-KV decode, split
// prefill). A counter is (generation << 24) | arrivals. One thread of each
// workgroup claims it for this call in two parts kept off the critical path:
// it reads the counter behind its tile loads, and after its tiles, if the tag
// read is not this call's generation (left by an earlier call, or
// uninitialised workspace), it swaps the value read for (generation << 24). A
// failed swap means another workgroup already claimed it. Arrival is then a
// single agent-scope acquire-release add (after the workgroup's partial
// stores have been acknowledged and its waves have met at a barrier); the
// workgroup that sees nsplit - 1 earlier arrivals is last. It resets the
// counter to 0, a tag no call uses, so replays of a captured graph (same
// generation) claim it again. Every swap precedes its own workgroup's
// arrival, so all of them precede the reset.
__device__ __forceinline__ bool arrive_last(unsigned long long* c, int nsplit) {
  const unsigned long long old =
      __hip_atomic_fetch_add(c, 1ull, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  return (int)(old & 0xffffffull) == nsplit - 1;
}

// gfx950 LDS transpose read (ds_read_b64_tr_b16). Within each 16-lane group,
// lane 4a + e receives element e of the four 8-byte rows whose addresses
// lanes a, a+4, a+8 and a+12 supply. The body exists only in the device pass
// (the host pass cannot type the LDS address-space cast).
__device__ __forceinline__ s16x4 lds_read_tr16(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
#else
  (void)p;
  return s16x4{0, 0, 0, 0};
#endif
}

// gfx950 LDS transpose read of bytes (ds_read_b64_tr_b8). Within each
// 16-lane group, lane 8h + c receives as its byte k (k = 0..7) byte c of the
// 8 bytes whose address lane h + 2k supplies.
__device__ __forceinline__ u32x2 lds_read_tr8(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p));
#else
  (void)p;
  return u32x2{0, 0};
#endif
}

// 16-bit element bits -> float (exact widening).
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

// Unpack one 16-byte chunk (8 elements) to floats.
template <typename T>
__device__ __forceinline__ void unpack8(u32x4 raw, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = elem_to_float<T>(raw[i] & 0xffffu);
    x[2 * i + 1] = elem_to_float<T>(raw[i] >> 16);
  }
}

// Direct global -> LDS load of 16 bytes per lane: lane i's 16 bytes, read
// from base + off_i, land at lds_base + 16 i (base and lds_base must be the
// same for the whole wave; M0 carries the LDS address). Written as inline asm
// so that the compiler does not order later LDS reads of other tiles behind
// it: it would otherwise make every LDS read wait for all direct loads still
// in flight. The caller makes the tile visible with vmem_wait_all() and a
// workgroup barrier before any wave reads it.
__device__ __forceinline__ void load_to_lds16(const void* base, uint32_t off, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_base;
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "{m0}"(m0) : "memory");
#else
  (void)base;
  (void)off;
  (void)lds_base;
#endif
}

// Wait until every vector-memory operation of this wave has completed,
// including global -> LDS loads (s_waitcnt vmcnt(0); the other counters are
// left alone).
__device__ __forceinline__ void vmem_wait_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt immediate that waits until at most n (< 64) vector-memory
// operations of this wave are outstanding (they complete in issue order).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// Workgroup id -> logical tile so that tiles [x*T/8, (x+1)*T/8) run on XCD x
// (the dispatcher places workgroup w on XCD w % 8); neighbouring tiles, which
// share K/V, then share one L2.
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int per = total / 8, rem = total % 8;
  const int xcd = w % 8, local = w / 8;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// Rotary position embedding of one pair: (x, y) turns by the angle
// 2 pi pos (rhi + rlo). The product pos * rhi is split exactly (FMA residual)
// and reduced to its fraction before the hardware sine and cosine, which take
// revolutions, so large positions keep their precision.
__device__ __forceinline__ void rope_rotate(float& x, float& y, float pos, float rhi, float rlo) {
  const float a = pos * rhi;
  const float lo = fmaf(pos, rhi, -a) + pos * rlo;
  const float f = (a - __builtin_rintf(a)) + lo;   // |f| <= 0.5 + 2^-20
  const float c = __builtin_amdgcn_cosf(f), s = __builtin_amdgcn_sinf(f);
  const float x2 = x * c - y * s;
  y = x * s + y * c;
  x = x2;
}

// Rotate the query row a lane holds as MFMA operands: KS vectors of 8
// elements, vector ks holding channels 16 ks + 8 half + (0..7) (D = 16 KS).
// style 0 pairs channel c with c + D/2 (vector ks with ks + KS/2, same lane);
// style 1 pairs 2i with 2i + 1 (inside one vector). rh/rl: revolutions per
// position of each pair, indexed by compile-time constants only.
template <typename T, int KS>
__device__ __forceinline__ void rope_lane_row(typename Elem<T>::vec8 (&v)[KS], float pos, int half,
                                              int style, const float* rh, const float* rl) {
  float x[KS][8];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) x[ks][e] = (float)v[ks][e];
  if (style == 0) {
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i0 = 16 * ks + e;
        rope_rotate(x[ks][e], x[ks + KS / 2][e], pos, half ? rh[i0 + 8] : rh[i0],
                    half ? rl[i0 + 8] : rl[i0]);
      }
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i0 = 8 * ks + u;
        rope_rotate(x[ks][2 * u], x[ks][2 * u + 1], pos, half ? rh[i0 + 4] : rh[i0],
                    half ? rl[i0 + 4] : rl[i0]);
      }
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) v[ks][e] = Elem<T>::from_float(x[ks][e]);
}

// Key index inside a 32-key block held by C-row m of S^T: swapping bits 2 and
// 3 makes lane half h's registers j = 8t + i hold keys 16t + 8h + i, i.e. a
// contiguous 8-key B-operand slice for each 16-key step of P V. It is its own
// inverse, so it also maps a key to the LDS row the kernels store it in.
__device__ __forceinline__ int swap23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

}  // namespace attn
