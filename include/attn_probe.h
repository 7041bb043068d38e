/*
 * attn_probe.h - measurement kernels reported beside the attention
 * benchmark: measured ceilings of the GPU (the matrix cores' bf16 rate, a
 * plain HBM streaming read) and its shader clock, next to the published
 * peaks the roofline fractions use (the roofline framing of the
 * AIInfraGuide "Self-Attention" page, section 11.2).  Not part of the
 * attention path; built into its own library (libattn_probe.so).
 *
 * Every pointer is a device pointer owned by the caller; each call only
 * enqueues one kernel on `stream` (a hipStream_t, NULL = null stream) and
 * returns the hipError_t of the launch (0 on success, hipErrorInvalidValue
 * for bad arguments, checked before launching).
 */
#ifndef ATTN_PROBE_H
#define ATTN_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* n_wg workgroups of 8 waves; every wave runs iters x 4 independent
 * v_mfma_f32_32x32x16_bf16 (32768 FLOP each) on register operands.
 *   out     float [n_wg * 512]: one checksum per lane
 *   cycles  uint64 [n_wg * 8][2]: per wave, shader-clock cycles and 100 MHz
 *           reference ticks over its loop */
int attn_probe_mfma(int n_wg, int iters, float* out, unsigned long long* cycles, void* stream);

/* The same with pseudo-random bf16 operands spread like N(0,1) (eight
 * register sets, both operands change on every MFMA): every wave runs
 * iters x 32 MFMAs.  The chip's power limit, and so its clock, depends on
 * the operand bits, so this is the matrix-core ceiling for random data.
 * Same arguments and outputs as attn_probe_mfma. */
int attn_probe_mfma_random(int n_wg, int iters, float* out, unsigned long long* cycles, void* stream);

/* Reads bytes of src once (16-byte non-temporal loads written straight to
 * LDS, the decode kernel's access pattern), split over n_wg workgroups of
 * 4 waves; bytes / n_wg must be a multiple of 64 KiB and below 2 GiB.
 *   sink  uint32 [n_wg]: one checksum word per workgroup */
int attn_probe_stream_read(const void* src, size_t bytes, unsigned* sink, int n_wg, void* stream);

/* One wave samples the shader clock and the 100 MHz reference clock ticks
 * reference ticks apart (at most 2^26 sleep rounds).
 *   out  uint64 [2]: shader cycles, reference ticks */
int attn_probe_clock(unsigned long long* out, int ticks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBE_H */
