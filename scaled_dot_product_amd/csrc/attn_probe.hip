// attn_probe.hip — matrix-core rate probe for the measurement report.
//
// Every wave runs a fixed number of MFMAs with register operands (no memory
// traffic, no vector work) on four independent accumulators, so the launch
// measures what the matrix cores of this part sustain at its clock under that
// load: the "measured achievable" figure printed beside the data-sheet peak.
// Not part of the attention path.
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

}  // namespace

hipError_t launch_probe_mfma(int kind, int iters, int blocks, float* out, hipStream_t s) {
  if (kind == 0)
    hipLaunchKernelGGL((probe_mfma_kernel<0>), dim3(blocks), dim3(256), 0, s, out, iters);
  else if (kind == 1)
    hipLaunchKernelGGL((probe_mfma_kernel<1>), dim3(blocks), dim3(256), 0, s, out, iters);
  else
    hipLaunchKernelGGL((probe_mfma_kernel<2>), dim3(blocks), dim3(256), 0, s, out, iters);
  return hipGetLastError();
}

}  // namespace attn
