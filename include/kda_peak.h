/*
 * kda_peak.h -- measurement probes for the rooflines the KDA prefill is measured
 * against on MI355X (not part of the KDA path): the HBM bandwidth a plain stream
 * of the chunk kernel's read/write mix reaches, and the bf16 matrix-core rate a
 * loop of independent MFMAs reaches.  Both enqueue one kernel on `stream`,
 * allocate nothing and never synchronise; they return KDA_ERR_* codes like the
 * rest of the library (KDA_ERR_NULL for NULL pointers, KDA_ERR_SHAPE for a
 * zero or too large size, KDA_ERR_HIP for a launch failure).
 */
#ifndef KDA_PEAK_H
#define KDA_PEAK_H

#include <stddef.h>
#include <stdint.h>

#include "kda.h"

#ifdef __cplusplus
extern "C" {
#endif

/* out[i] = in[0][i] ^ in[1][i] ^ ... ^ in[4][i] over n16 16-byte elements: five bytes read
 * for every byte written, the ratio of the chunk kernel's traffic (1,284 bytes of q, k, v,
 * g and beta read per 256 bytes of out written, per token-head).  in[0..4] and out are
 * device pointers to n16 * 16 bytes each, 16-byte aligned; out may not overlap the inputs. */
kda_status_t kda_peak_stream(const void *const in[5], void *out, int64_t n16, void *stream);

/* A loop of bf16 32x32x16 MFMAs (8 independent accumulators per wave, operands held in
 * registers): `workgroups` workgroups of 4 waves, `iters` iterations of 8 MFMAs each, so
 * workgroups * 4 * iters * 8 * 32768 flops.  Each wave writes one float (the sum of its
 * accumulators) to out[wave], so out holds workgroups * 4 floats. */
kda_status_t kda_peak_mfma(float *out, int32_t workgroups, int32_t iters, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* KDA_PEAK_H */
