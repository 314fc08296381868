/*
 * pisa_roofline.h -- on-device roofline probes of libpisa (MI355X, gfx950).
 *
 * The denominators the benchmark reports kernel efficiency against, measured
 * on the machine instead of taken from the datasheet alone (the chip clocks
 * below its rated frequency under sustained matrix load).  Not part of the
 * attention method; plain throughput loops.  Asynchronous on `stream`; the
 * caller times them (HIP events) and owns every buffer.
 *
 * pisa_probe_mfma_bf16  every wave runs four independent accumulator chains
 *                       of v_mfma_f32_32x32x16_bf16 for `iters` rounds on
 *                       register operands, over `workgroups` workgroups of
 *                       four waves.  Dense bf16 FLOPs executed:
 *                       workgroups * 4 * iters * 4 * 32768.  `sink` (fp32,
 *                       at least workgroups * 256 values, 16-byte aligned)
 *                       receives a result so the loop is not removed.
 * pisa_probe_hbm_copy   dst[i] = src[i] over `bytes` bytes (a multiple of 16,
 *                       both 16-byte aligned): `bytes` read plus `bytes`
 *                       written.
 * pisa_probe_hbm_read   reads `bytes` bytes of src (a multiple of 16,
 *                       16-byte aligned) and writes one fp32 per workgroup
 *                       to `sink` (at least 65536 floats).
 * Return PISA_OK, PISA_E_ARG for a bad argument (checked before any launch),
 * or PISA_E_HIP for a failed launch.
 */
#ifndef PISA_ROOFLINE_H
#define PISA_ROOFLINE_H

#include <stddef.h>
#include <stdint.h>

#include "pisa.h"

#ifdef __cplusplus
extern "C" {
#endif

pisa_status pisa_probe_mfma_bf16(int32_t workgroups, int32_t iters, float *sink, hipStream_t stream);
pisa_status pisa_probe_hbm_copy(void *dst, const void *src, size_t bytes, hipStream_t stream);
pisa_status pisa_probe_hbm_read(const void *src, size_t bytes, float *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* PISA_ROOFLINE_H */
