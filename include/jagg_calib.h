/*
 * jagg_calib.h -- machine-peak probes used by the benchmark (library
 * libjagg_calib.so, separate from the executor).
 *
 * "Stax (5): Caching and Measurement", Section 13.1 ("Machine parameters"):
 * a roofline is read against the rates the machine actually reaches, so the
 * benchmark measures them beside the nominal datasheet peaks.  The HBM rate
 * is a plain device copy (timed by the caller); the matrix-core rates are
 * these probes: loops of bf16 or fp32 MFMAs on operands held in registers.
 */
#ifndef JAGG_CALIB_H
#define JAGG_CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Launches, on `hip_stream`, `n_blocks` workgroups of 4 wavefronts; each
 * wavefront loads eight 32x16 bf16 operand fragments from `operands`
 * (device, at least 4096 bf16 values, any distribution; the values set the
 * chip's power draw and with it the clock) and runs `iters` rounds of the
 * 4 x 4 products of four A and four B fragments into 16 fp32 32x32
 * accumulators (v_mfma_f32_32x32x16_bf16, 32768 FLOP each), then writes one
 * float per wavefront to `sink` (device, n_blocks * 4 floats) so the work is
 * kept.  FLOPs of one launch: n_blocks * 4 * iters * 16 * 32768.
 * Returns 0, or -6 when the launch fails. */
int jagg_calib_mfma_bf16(void *hip_stream, const void *operands, float *sink, int n_blocks, int iters);

/* The fp32 form of the same probe: each wavefront loads eight fp32 operand
 * registers from `operands` (device, at least 512 floats) and runs `iters`
 * rounds of the 4 x 4 products into 16 fp32 32x32 accumulators with
 * v_mfma_f32_32x32x2f32 (4096 FLOP each).  FLOPs of one launch:
 * n_blocks * 4 * iters * 16 * 4096.  Returns 0, or -6 when the launch
 * fails. */
int jagg_calib_mfma_f32(void *hip_stream, const float *operands, float *sink, int n_blocks, int iters);

#ifdef __cplusplus
}
#endif
#endif /* JAGG_CALIB_H */
