/*
 * astr_ceiling.h -- attainable-rate probes exported by libastr beside the
 * attention path.  They compute nothing the path needs: a roofline is only as
 * informative as its denominator, so the benchmark runs these two plain
 * kernels on the same device and reports each attention kernel's rate both
 * against the nominal MI355X peaks (8 TB/s HBM3E, 2.5 PFLOP/s dense bf16)
 * and against what these probes attain.
 *
 * Same conventions as astr.h: device pointers are owned by the caller,
 * nothing is allocated or synchronised, the work is enqueued on `stream`
 * (a hipStream_t; NULL = default stream), arguments are checked on the host
 * first and a non-OK status leaves a message in astr_last_error().
 */
#ifndef ASTR_CEILING_H
#define ASTR_CEILING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` bytes of `buf` once (16-byte loads, eight in flight per lane,
 * grid-stride over `workgroups` workgroups of 256 lanes; non-temporal loads
 * when nontemporal is nonzero).  Each workgroup stores one 32-bit fold of what it read into
 * sink[workgroup], so that no load can be elided.
 *   buf    device, 16-byte aligned, `bytes` a positive multiple of 16
 *   sink   device uint32 [workgroups], written
 * Errors: INVAL (null pointer, misaligned or empty buffer, workgroups < 1),
 * LAUNCH.
 */
int astr_ceiling_stream_read(const void *buf, size_t bytes, int workgroups, int nontemporal,
                             uint32_t *sink, void *stream);

/*
 * `workgroups` workgroups of 4 waves; every wave issues `iters` rounds of 8
 * independent v_mfma_f32_16x16x32_bf16 products (16 x 16 x 32 multiply-adds
 * each) on register operands: 2 * 16 * 16 * 32 * 8 * iters flop per wave.
 * Each lane stores one float (the sum of its accumulators) to
 * sink[256 * workgroup + lane_in_workgroup].
 *   sink   device float32 [256 * workgroups], written
 * Errors: INVAL (workgroups < 1, iters < 1, null sink), LAUNCH.
 */
int astr_ceiling_mfma_loop(int workgroups, int iters, float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ASTR_CEILING_H */
