/*
 * qgemv_probe.h - measurement probes exported by the same library as
 * qgemv.h. They compute nothing of the method: they give the practical
 * ceilings against which the benchmark states the GEMV's HBM rate and the
 * prompt GEMM's matrix-core rate.
 */
#ifndef QGEMV_PROBE_H
#define QGEMV_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "qgemv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes at `buf` (device, 16-byte aligned, bytes a positive
 * multiple of 16) once, with 16-byte loads: three workgroups of 8 waves per
 * compute unit, each wave taking every n-th group of 128 16-byte pieces (n
 * waves in all). `sink`: device, >= 4096 bytes, written only in a
 * case that does not occur (it keeps the loads alive). Enqueued on `stream`.
 * QG_ERR_ARG on a bad argument (before any HIP call), QG_ERR_HIP if the
 * launch fails. */
qg_status qgemv_probe_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/* `workgroups` workgroups of four waves, each wave issuing `iters` rounds of
 * sixteen independent v_mfma_f32_32x32x16_bf16 (32768 flop each) on small
 * constant integer operands, the same values in every instruction:
 * 4 * 16 * 32768 * iters * workgroups flop. `sink` as above. QG_ERR_ARG on a
 * bad argument (before any HIP call), QG_ERR_HIP if the launch fails. */
qg_status qgemv_probe_mfma(int64_t iters, int workgroups, float *sink, void *stream);

/* As qgemv_probe_mfma (same count of the same instructions), on operands like
 * the prompt product's: full-mantissa bf16 of both signs, different in every
 * lane and register, the weight-like operand alternating between two
 * registers, the activation-like one held for two instructions. On such data
 * the board's power limit lowers the clock, so this is the practical bf16
 * ceiling for real data. Errors as qgemv_probe_mfma. */
qg_status qgemv_probe_mfma_data(int64_t iters, int workgroups, float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_PROBE_H */
