/*
 * colibri_ceilings.h -- two measurement kernels (libcolibri_ceilings.so) that
 * give the achieved ceilings of an MI355X, beside which the MoE layer's
 * kernels are reported.  They are not part of the layer's C ABI
 * (colibri_moe.h) and are used only by the benchmark.
 *
 * Return codes: 0 = launched, -1 = invalid argument, -4 = HIP launch error.
 * Nothing is allocated or synchronised; work goes on `stream`.
 */
#ifndef COLIBRI_CEILINGS_H
#define COLIBRI_CEILINGS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a multiple of 16) of device memory at src (16-byte aligned)
 * with `blocks` workgroups of 256 lanes, 16 bytes per lane per load,
 * grid-stride; lane i of the grid writes one word to sink[i]
 * (sink: blocks * 256 uint32). */
int colibri_ceiling_stream_read(const void *src, size_t bytes, uint32_t *sink, int blocks, hipStream_t stream);

/* `blocks` workgroups of 4 waves; each wave runs `iters` rounds of 8
 * independent v_mfma_f32_32x32x16_bf16 on register operands; lane i of the
 * grid writes one float to sink[i] (sink: blocks * 256 floats). */
int colibri_ceiling_mfma_loop(int iters, float *sink, int blocks, hipStream_t stream);

/* Flops of one colibri_ceiling_mfma_loop call. */
double colibri_ceiling_mfma_flops(int iters, int blocks);

#ifdef __cplusplus
}
#endif

#endif /* COLIBRI_CEILINGS_H */
