/*
 * ppmeasure.h -- measurement aid shipped with libppattn (not part of the
 * attention path).
 *
 * The decode step's kernels are judged against the HBM roofline.  The
 * published MI355X figure (8 TB/s) is a nominal peak; what a kernel that only
 * reads can actually pull from HBM on a given device is measured here, with a
 * plain streaming read of a caller buffer of known size, so that achieved
 * bandwidths can be stated against both the nominal and the measured
 * ceiling, and so that HBM byte counters (rocprofv3 FETCH_SIZE) can be
 * calibrated on a launch whose bytes are known exactly.
 */
#ifndef PPMEASURE_H
#define PPMEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "ppattn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads every byte of buf[0, bytes) once (16-byte vector loads, grid-stride,
 * 8 loads in flight per lane), folds them into an XOR that is written to
 * sink[0] only when it equals a fixed improbable value (so the loads cannot
 * be dropped and nearly nothing is written).  One launch of
 * blocks_per_cu x (compute units) workgroups of 256 lanes on hip_stream.
 *   buf            caller-owned device memory, 16-byte aligned, read only
 *   bytes          a multiple of 16, >= 16
 *   sink           caller-owned device uint32[1] (written at most once)
 *   blocks_per_cu  workgroups per compute unit, in [1, 64]
 * Errors: PP_ERR_INVALID_ARG for a null or misaligned pointer, a size that
 * is not a positive multiple of 16, or blocks_per_cu out of range;
 * PP_ERR_HIP for a failed launch or device query. */
pp_status_t pp_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t blocks_per_cu,
                           void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* PPMEASURE_H */
