// attn_probe.hip — measurement probes (libattn_probe.so, include/attn_probe.h).
//
// Not part of the attention path: these kernels measure what this part
// sustains, the "measured achievable" figures printed beside the data-sheet
// peaks, and the floors a short kernel cannot go below.
//   attn_probe_mfma   matrix cores with register operands only (no memory
//                     traffic, no vector work), four independent accumulators
//   attn_probe_read   a bare streaming read of n bytes (16 bytes per lane,
//                     four loads in flight per lane), the floor of a
//                     bandwidth-bound kernel of that size
//   attn_probe_empty  a launch that does nothing, the floor of any kernel
//   attn_probe_valu   the issue cost of one kind of vector instruction (16
//                     independent chains per wave), for the softmax's
//                     instruction mix: exponential, FMA, bf16 and fp8 packing,
//                     three-way maximum, bf16 pair dot product
//   attn_probe_mix    the bf16 MFMA rate with nv vector instructions (one
//                     exponential to two FMAs) issued beside every 4 MFMAs
//   attn_probe_phase  two waves per SIMD alternating a block of vector work
//                     and a block of MFMAs between workgroup barriers, all
//                     in the same order or the second wave of each SIMD in
//                     the opposite order (matrix block first)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/attn_probe.h"
#include "attn_common.hpp"

namespace attn {

namespace {

// kind 0: bf16 32x32x16 (32768 flop), 1: i8 32x32x32 (65536 op),
// 2: fp8 32x32x64 with unit block scales (131072 op).
template <int KIND>
__global__ void __launch_bounds__(256) probe_mfma_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  float sum = 0.0f;
  if constexpr (KIND == 0) {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(0.001f * (lane + i));
      b[i] = (__bf16)(0.002f * (i - lane));
    }
    f32x16 c[4] = {};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < 16; ++k) c[k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k & 3], 0, 0, 0);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int j = 0; j < 16; ++j) sum += c[k][j];
  } else if constexpr (KIND == 1) {
    i32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = 0x01010101 * ((lane + i) & 7);
      b[i] = 0x01020304 + i;
    }
    i32x16 c[4] = {};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < 16; ++k) c[k & 3] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[k & 3], 0, 0, 0);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int j = 0; j < 16; ++j) sum += (float)c[k][j];
  } else {
    i32x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = 0x30303030 + ((lane + i) & 7);   // small E4M3 values
      b[i] = 0x28282828 + i;
    }
    f32x16 c[4] = {};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < 16; ++k)
        c[k & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c[k & 3], 0, 0, 0, 127, 0, 127);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int j = 0; j < 16; ++j) sum += c[k][j];
  }
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

// Each lane reads 16-byte chunks with a grid stride, four in flight, and folds
// them into one word so the loads cannot be dropped; one word per workgroup
// is written. n16: number of 16-byte chunks.
__global__ void __launch_bounds__(256) probe_read_kernel(const u32x4* __restrict__ x, int64_t n16,
                                                         uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = x[i], b = x[i + stride], c = x[i + 2 * stride], d = x[i + 3 * stride];
    acc ^= (a[0] ^ a[1] ^ a[2] ^ a[3]) + (b[0] ^ b[1] ^ b[2] ^ b[3]) +
           (c[0] ^ c[1] ^ c[2] ^ c[3]) + (d[0] ^ d[1] ^ d[2] ^ d[3]);
  }
  for (; i < n16; i += stride) {
    const u32x4 a = x[i];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < 256; ++t) r ^= red[t];
    out[blockIdx.x] = r;
  }
}

__global__ void probe_empty_kernel() {}

// Vector-instruction issue cost: iters rounds of 16 independent instructions
// of one kind per wave (each register its own dependency chain).
template <int KIND>
__global__ void __launch_bounds__(256) probe_valu_kernel(float* out, int iters) {
  float r[16], s[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    r[i] = 0.37f * (i + 1) + 1e-3f * threadIdx.x;
    s[i] = 0.5f * r[i];
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (KIND == 0) asm volatile("v_exp_f32 %0, %0" : "+v"(r[i]));
      if constexpr (KIND == 1) asm volatile("v_fma_f32 %0, %0, %1, %1" : "+v"(r[i]) : "v"(s[i]));
      if constexpr (KIND == 2) asm volatile("v_cvt_pk_bf16_f32 %0, %0, %1" : "+v"(r[i]) : "v"(s[i]));
      if constexpr (KIND == 3) asm volatile("v_cvt_pk_fp8_f32 %0, %1, %1" : "+v"(r[i]) : "v"(s[i]));
      if constexpr (KIND == 4) asm volatile("v_max3_f32 %0, %0, %1, %1" : "+v"(r[i]) : "v"(s[i]));
      if constexpr (KIND == 5) asm volatile("v_dot2c_f32_bf16 %0, %1, %1" : "+v"(r[i]) : "v"(s[i]));
    }
  }
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) sum += r[i];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

// bf16 32x32x16 MFMAs on four independent accumulators, each group of four
// followed by NV vector instructions (an exponential, then two FMAs, repeating,
// on 16 chains that the MFMAs do not touch).
template <int NV>
__global__ void __launch_bounds__(256) probe_mix_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (lane + i));
    b[i] = (__bf16)(0.002f * (i - lane));
  }
  float r[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = 0.37f * (i + 1) + 1e-3f * threadIdx.x;
  f32x16 c[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
#pragma unroll
      for (int v = 0; v < NV / 4; ++v) {
        const int i = (NV / 4 * k + v) & 15;
        if ((NV / 4 * k + v) % 3 == 0)
          asm volatile("v_exp_f32 %0, %0" : "+v"(r[i]));
        else
          asm volatile("v_fma_f32 %0, %0, %0, %0" : "+v"(r[i]));
      }
    }
  }
  float sum = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int j = 0; j < 16; ++j) sum += c[k][j];
#pragma unroll
  for (int i = 0; i < 16; ++i) sum += r[i];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

// 8 waves (two per SIMD); per round a vector block of NV instructions (one
// v_exp_f32 to two v_fma_f32 on 16 chains) and a matrix block of NM
// v_mfma_f32_32x32x16_bf16 on four accumulators, then a barrier. Waves 4..7
// (the second wave of each SIMD) run the matrix block first when late != 0.
template <int NV, int NM>
__global__ void __launch_bounds__(512) probe_phase_kernel(float* out, int iters, int late) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (lane + i));
    b[i] = (__bf16)(0.002f * (i - lane));
  }
  float r[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = 0.37f * (i + 1) + 1e-3f * threadIdx.x;
  f32x16 c[4] = {};
  const bool mfirst = late != 0 && __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >= 4;
  auto vblock = [&]() {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (i % 3 == 0)
        asm volatile("v_exp_f32 %0, %0" : "+v"(r[i & 15]));
      else
        asm volatile("v_fma_f32 %0, %0, %0, %0" : "+v"(r[i & 15]));
    }
  };
  auto mblock = [&]() {
#pragma unroll
    for (int k = 0; k < NM; ++k) c[k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k & 3], 0, 0, 0);
  };
  for (int it = 0; it < iters; ++it) {
    if (mfirst) {
      mblock();
      vblock();
    } else {
      vblock();
      mblock();
    }
    __syncthreads();
  }
  float sum = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int j = 0; j < 16; ++j) sum += c[k][j];
#pragma unroll
  for (int i = 0; i < 16; ++i) sum += r[i];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

}  // namespace

}  // namespace attn

extern "C" {

int attn_probe_mfma(int kind, int iters, int blocks, float* out, void* stream) {
  if (out == nullptr || ((uintptr_t)out & 15u) || kind < 0 || kind > 2 || iters < 1 || blocks < 1 ||
      blocks > 65535)
    return -1;
  const hipStream_t s = (hipStream_t)stream;
  if (kind == 0)
    hipLaunchKernelGGL((attn::probe_mfma_kernel<0>), dim3(blocks), dim3(256), 0, s, out, iters);
  else if (kind == 1)
    hipLaunchKernelGGL((attn::probe_mfma_kernel<1>), dim3(blocks), dim3(256), 0, s, out, iters);
  else
    hipLaunchKernelGGL((attn::probe_mfma_kernel<2>), dim3(blocks), dim3(256), 0, s, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int attn_probe_read(const void* x, size_t nbytes, int blocks, uint32_t* out, void* stream) {
  if (x == nullptr || out == nullptr || ((uintptr_t)x & 15u) || ((uintptr_t)out & 3u) ||
      (nbytes & 15u) || nbytes == 0 || blocks < 1 || blocks > 65535)
    return -1;
  hipLaunchKernelGGL(attn::probe_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (const attn::u32x4*)x, (int64_t)(nbytes / 16), out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int attn_probe_valu(int kind, int iters, int blocks, float* out, void* stream) {
  if (out == nullptr || ((uintptr_t)out & 3u) || kind < 0 || kind > 5 || iters < 1 || blocks < 1 ||
      blocks > 65535)
    return -1;
  const hipStream_t s = (hipStream_t)stream;
  switch (kind) {
    case 0: hipLaunchKernelGGL((attn::probe_valu_kernel<0>), dim3(blocks), dim3(256), 0, s, out, iters); break;
    case 1: hipLaunchKernelGGL((attn::probe_valu_kernel<1>), dim3(blocks), dim3(256), 0, s, out, iters); break;
    case 2: hipLaunchKernelGGL((attn::probe_valu_kernel<2>), dim3(blocks), dim3(256), 0, s, out, iters); break;
    case 3: hipLaunchKernelGGL((attn::probe_valu_kernel<3>), dim3(blocks), dim3(256), 0, s, out, iters); break;
    case 4: hipLaunchKernelGGL((attn::probe_valu_kernel<4>), dim3(blocks), dim3(256), 0, s, out, iters); break;
    default: hipLaunchKernelGGL((attn::probe_valu_kernel<5>), dim3(blocks), dim3(256), 0, s, out, iters); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int attn_probe_mix(int nv, int iters, int blocks, float* out, void* stream) {
  if (out == nullptr || ((uintptr_t)out & 3u) || iters < 1 || blocks < 1 || blocks > 65535)
    return -1;
  const hipStream_t s = (hipStream_t)stream;
  switch (nv) {
    case 0: hipLaunchKernelGGL((attn::probe_mix_kernel<0>), dim3(blocks), dim3(256), 0, s, out, iters); break;
    case 4: hipLaunchKernelGGL((attn::probe_mix_kernel<4>), dim3(blocks), dim3(256), 0, s, out, iters); break;
    case 8: hipLaunchKernelGGL((attn::probe_mix_kernel<8>), dim3(blocks), dim3(256), 0, s, out, iters); break;
    case 12: hipLaunchKernelGGL((attn::probe_mix_kernel<12>), dim3(blocks), dim3(256), 0, s, out, iters); break;
    case 16: hipLaunchKernelGGL((attn::probe_mix_kernel<16>), dim3(blocks), dim3(256), 0, s, out, iters); break;
    case 24: hipLaunchKernelGGL((attn::probe_mix_kernel<24>), dim3(blocks), dim3(256), 0, s, out, iters); break;
    case 32: hipLaunchKernelGGL((attn::probe_mix_kernel<32>), dim3(blocks), dim3(256), 0, s, out, iters); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int attn_probe_phase(int kind, int late, int iters, int blocks, float* out, void* stream) {
  if (out == nullptr || ((uintptr_t)out & 3u) || iters < 1 || blocks < 1 || blocks > 65535 ||
      (late != 0 && late != 1))
    return -1;
  const hipStream_t s = (hipStream_t)stream;
  switch (kind) {
    case 0: hipLaunchKernelGGL((attn::probe_phase_kernel<96, 16>), dim3(blocks), dim3(512), 0, s, out, iters, late); break;
    case 1: hipLaunchKernelGGL((attn::probe_phase_kernel<96, 0>), dim3(blocks), dim3(512), 0, s, out, iters, late); break;
    case 2: hipLaunchKernelGGL((attn::probe_phase_kernel<0, 16>), dim3(blocks), dim3(512), 0, s, out, iters, late); break;
    case 3: hipLaunchKernelGGL((attn::probe_phase_kernel<48, 16>), dim3(blocks), dim3(512), 0, s, out, iters, late); break;
    case 4: hipLaunchKernelGGL((attn::probe_phase_kernel<144, 16>), dim3(blocks), dim3(512), 0, s, out, iters, late); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int attn_probe_empty(int blocks, void* stream) {
  if (blocks < 1 || blocks > 65535) return -1;
  hipLaunchKernelGGL(attn::probe_empty_kernel, dim3(blocks), dim3(64), 0, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
