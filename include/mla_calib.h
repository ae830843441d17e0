/*
 * Device calibration calls of libmla_kv.so: the achievable rates that the decode's roofline
 * fractions are also quoted against, beside the published MI355X peaks (8 TB/s HBM3E,
 * 2.5 PFLOP/s dense bf16 MFMA).  They time nothing themselves: the caller brackets them
 * with events on `stream`.  Not part of the decode path.
 *
 * Errors: MLA_ERR_NULL (NULL pointer), MLA_ERR_SHAPE (count out of range), MLA_ERR_ALIGN,
 * MLA_ERR_LAUNCH; checked before any launch.  Every buffer is the caller's.
 */
#ifndef MLA_CALIB_H
#define MLA_CALIB_H

#include "mla_kv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroups of mla_calib_mfma (4 waves each, one per SIMD); `out` needs grid * 256 floats. */
int32_t mla_calib_mfma_grid(void);

/* Back-to-back v_mfma_f32_32x32x16_bf16 on every SIMD: 4 independent accumulator chains per
 * wave, `iters` rounds.  out: device, mla_calib_mfma_grid() * 256 floats (written, unused). */
mla_status_t mla_calib_mfma(int32_t iters, float* out, hipStream_t stream);

/* FLOPs one mla_calib_mfma(iters) launch performs (0 for iters < 1). */
double mla_calib_mfma_flop(int32_t iters);

/* Streaming read of the first mla_calib_read_bytes(bytes, workgroups) bytes of src (device,
 * 16-byte aligned) by `workgroups` workgroups, each a contiguous slice in 36 KiB tiles of
 * 16-byte direct-to-LDS loads (the decode's load form).  out: device, `workgroups` floats. */
mla_status_t mla_calib_read(const void* src, int64_t bytes, int32_t workgroups, float* out,
                            hipStream_t stream);

/* Bytes one mla_calib_read(src, bytes, workgroups) launch reads (0 on bad arguments). */
int64_t mla_calib_read_bytes(int64_t bytes, int32_t workgroups);

#ifdef __cplusplus
}
#endif

#endif /* MLA_CALIB_H */
