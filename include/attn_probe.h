/*
 * attn_probe.h — C ABI of libattn_probe.so: measurement probes for the
 * report of the attention library, not attention themselves. They give the
 * "measured achievable" figures printed beside the data-sheet peaks and the
 * floors below which no short kernel of a given size can go.
 *
 * Conventions: pointers are caller-owned DEVICE memory; nothing is allocated,
 * freed or synchronised; kernels go on `stream` (a hipStream_t, NULL = the
 * default stream). Return 0 on success, -1 for an invalid argument (checked
 * before anything is enqueued, nothing written), -4 if the HIP runtime refused
 * the launch.
 */
#ifndef ATTN_PROBE_H
#define ATTN_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core rate with register operands only: `blocks` workgroups of 4 waves,
 * each wave `iters` x 16 MFMAs on four independent accumulators.
 *   kind 0: v_mfma_f32_32x32x16_bf16   (32 768 flop each)
 *   kind 1: v_mfma_i32_32x32x32_i8     (65 536 op each)
 *   kind 2: v_mfma_scale_f32_32x32x64_f8f6f4, FP8 E4M3, unit scales (131 072 op)
 *   out: blocks * 256 floats (16-byte aligned), written with the accumulator
 *        sums so the work cannot be dropped.
 * Invalid: out NULL or misaligned, kind outside 0..2, iters < 1, blocks
 * outside 1..65535. */
int attn_probe_mfma(int kind, int iters, int blocks, float* out, void* stream);

/* A bare streaming read of `nbytes` bytes at x (16-byte chunks, a grid stride
 * over `blocks` workgroups of 256 lanes, four loads in flight per lane); one
 * 32-bit word per workgroup is written to out. The time of this launch on
 * a cold x is the floor of any kernel that must read nbytes once.
 * Invalid: a NULL or misaligned pointer (x 16 bytes, out 4), nbytes zero or
 * not a multiple of 16, blocks outside 1..65535. */
int attn_probe_read(const void* x, size_t nbytes, int blocks, uint32_t* out, void* stream);

/* A launch of `blocks` workgroups of 64 lanes that do nothing: the fixed cost
 * of one kernel. Invalid: blocks outside 1..65535. */
int attn_probe_empty(int blocks, void* stream);

/* Issue cost of one kind of vector instruction: `blocks` workgroups of 4
 * waves, each wave `iters` x 16 instructions on 16 independent chains.
 *   kind 0: v_exp_f32   1: v_fma_f32   2: v_cvt_pk_bf16_f32
 *   kind 3: v_cvt_pk_fp8_f32   4: v_max3_f32   5: v_dot2c_f32_bf16
 *   out: blocks * 256 floats (4-byte aligned), written with the chain values
 *        so the work cannot be dropped.
 * Invalid: out NULL or misaligned, kind outside 0..5, iters < 1, blocks
 * outside 1..65535. */
int attn_probe_valu(int kind, int iters, int blocks, float* out, void* stream);

/* The bf16 MFMA rate beside vector work: per wave `iters` rounds of 4
 * v_mfma_f32_32x32x16_bf16 on four independent accumulators, each followed by
 * nv / 4 vector instructions (v_exp_f32 and v_fma_f32 in the ratio 1 : 2) on
 * registers the MFMAs do not use. nv in {0, 4, 8, 12, 16, 24, 32}.
 *   out: blocks * 256 floats (4-byte aligned).
 * Invalid: out NULL or misaligned, another nv, iters < 1, blocks outside
 * 1..65535. */
int attn_probe_mix(int nv, int iters, int blocks, float* out, void* stream);

/* Whether two waves of one SIMD gain from running opposite phases: `blocks`
 * workgroups of 8 waves (two per SIMD), each wave `iters` rounds of a vector
 * block (v_exp_f32 and v_fma_f32 in the ratio 1 : 2, 16 chains) and a matrix
 * block (v_mfma_f32_32x32x16_bf16 on four accumulators), then a workgroup
 * barrier. late = 0: every wave runs vector then matrix; late = 1: waves 4..7
 * (the second wave of each SIMD) run matrix then vector.
 *   kind 0: 96 vector + 16 MFMA   1: 96 vector only   2: 16 MFMA only
 *   kind 3: 48 vector + 16 MFMA   4: 144 vector + 16 MFMA
 *   out: blocks * 512 floats (4-byte aligned).
 * Invalid: out NULL or misaligned, kind outside 0..4, late not 0 or 1,
 * iters < 1, blocks outside 1..65535. */
int attn_probe_phase(int kind, int late, int iters, int blocks, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBE_H */
