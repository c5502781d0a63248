/*
 * ssm_calib.h - calibration probes of libssm.so for the measurement harness.
 *
 * These are not part of the selective scan.  They measure, on the device at hand,
 * the two resources the scan's rooflines are stated against: the achievable HBM
 * bandwidth (a plain streaming copy, which is also the reference kernel that HBM
 * byte counters are scaled by) and the issue rates of fp32 FMAs and of the
 * hardware exp2 (the scan spends one exp per element).  Same conventions as
 * ssm.h: device pointers, asynchronous on `stream` (a hipStream_t, NULL = the null
 * stream), argument errors returned before anything is enqueued.
 */
#ifndef SSM_CALIB_H
#define SSM_CALIB_H

#include <stddef.h>
#include <stdint.h>

#include "ssm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * dst[0 .. bytes) = src[0 .. bytes) with 16-byte vector loads and stores over a
 * grid-stride loop: `bytes` read and `bytes` written.  src and dst must be 16-byte
 * aligned, bytes a multiple of 16, and the two ranges disjoint
 * (SSM_ERR_INVALID_ARG otherwise); SSM_ERR_HIP if the launch fails.
 */
ssm_status ssm_calib_copy(const void *src, void *dst, size_t bytes, void *stream);

/*
 * Issue-rate probe: `blocks` workgroups of 256 lanes, each lane running 8
 * independent chains for `iters` iterations of
 *   kind 0: x = fma(x, a, b)              (one v_fma_f32 per chain and iteration)
 *   kind 1: x = exp2(x * -0.5)            (one v_mul_f32 and one v_exp_f32)
 * and storing the sum of its chains to out[lane] (out holds blocks * 256 floats).
 * ssm_calib_alu_ops gives the chain steps one call performs (blocks * 256 * iters * 8).
 * SSM_ERR_INVALID_ARG for a NULL out, blocks outside [1, 2^31), iters <= 0 or an
 * unknown kind; SSM_ERR_HIP if the launch fails.
 */
ssm_status ssm_calib_alu(int kind, float *out, int64_t blocks, int iters, void *stream);
int64_t ssm_calib_alu_ops(int64_t blocks, int iters);

#ifdef __cplusplus
}
#endif

#endif /* SSM_CALIB_H */
