/*
 * qgemv_tuning.h -- measurement and tuning hooks of libqgemv.so.
 *
 * Not part of the product surface (qgemv.h): these calls exist for launch-
 * shape sweeps, kernel timing and the bandwidth probe.  Three of them set
 * state of the CALLING THREAD that changes later calls of qgemv.h's entry
 * points made from that thread:
 *   - qg_set_gemv_shape / qg_set_prefill_shape fix launch-shape fields until
 *     they are called again with zeros (-1 for xl and engine);
 *   - qg_time_next_launch arms a one-shot timing hook for the next launch.
 * A caller that never includes this header never sees that state.  Other
 * threads are not affected.
 */
#ifndef QGEMV_TUNING_H
#define QGEMV_TUNING_H

#include <stddef.h>
#include <stdint.h>

#include "qgemv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Arm kernel timing for the next launch this library makes from the calling
 * thread: that kernel records its own start and end into `start` and `stop`
 * (hipEvent_t, created by the caller) through hipExtLaunchKernel, so
 * hipEventElapsedTime(start, stop) is the kernel's execution time without
 * queueing gaps.  One-shot: the next launch consumes it.  Pass NULLs to
 * disarm.  Entry points that launch more than one kernel time the first. */
void qg_time_next_launch(void *start, void *stop);

/* Number of compute units the launch heuristics assume on `device`
 * (QG_ERR_DEVICE if the query fails). */
qg_status qg_device_cus(int device, int *cus);

/* Tuning knob for launch-shape sweeps of qgemv_* / qmoe_gemv_q4_0: fixes J
 * (blocks per lane per row, J * M <= 8), R (row sets per group: 1, 2 or 4),
 * ksplit (waves sharing a row along K), teams per workgroup, the total
 * number of teams, xl (activations of 1-4 tokens staged once per workgroup
 * in LDS, whole rows per wave: 1; kept in each lane's registers: 0), engine
 * (vector-ALU kernel: 0; matrix-core kernel for 2..8 tokens and rows of at
 * most 256 blocks, for q2w an even number: 1, where ksplit is its number of
 * waves along K, teams_per_wg its teams of such waves per workgroup sharing
 * one staged copy of the activations (1 or 2; 2 for slices of at most 16
 * blocks per wave) and teams its number of persistent workgroups) and
 * lanes_per_row (lanes of a wave that share one row in the vector-ALU
 * kernel: 16, 32 or 64; below 64 one token only) for later calls from the
 * calling thread.  A zero (-1 for xl and engine) keeps the built-in
 * per-shape choice for that field.  An impossible combination makes the
 * later calls return QG_ERR_SHAPE. */
void qg_set_gemv_shape(int J, int R, int ksplit, int teams_per_wg, int64_t teams, int xl, int engine,
                       int lanes_per_row);

/* Tuning knob for sweeps of qgemm_q4_0_prefill, for later calls from the
 * calling thread: `wgs` fixes the number of persistent workgroups among
 * which the (tile, K step) iterations are split (a workgroup whose range
 * covers part of a tile adds it atomically into a zero-filled Y); `tile`
 * picks the tile configuration (tokens x rows): 64 (64 x 128, two
 * workgroups per CU), 66 (64 x 256, two per CU), 128 (128 x 256, one per CU),
 * 130 (128 x 128, two per CU), 136 (128 x 256 with eight waves, one per
 * CU), 257 (256 x 64, waves 2 x 2, one per CU), or
 * 16: the kernel for up to 64 tokens (activations in registers, 16-row
 * weight tiles; `wgs` is then its number of workgroups along N, and more
 * than 64 tokens return QG_ERR_SHAPE).  0 keeps the built-in choice; an
 * unknown tile makes the later calls return QG_ERR_SHAPE. */
void qg_set_prefill_shape(int wgs, int tile);

/* Memory-bandwidth probe on the GEMV kernels' load path: a streaming read of
 * `bytes` (rounded down to a multiple of 16, at most 2^40) of device memory
 * at `buf` (16-byte aligned) with non-temporal 16-byte buffer loads.  The
 * buffer is cut into tiles of loads x 4 KiB, handed round-robin to `wgs`
 * workgroups of 256 threads, each lane keeping `loads` (2, 4, 8 or 16)
 * loads of a tile in flight and issuing its next tile's before folding the
 * current one; a lane of workgroup g writes sink[g] (device, >= wgs words)
 * only if its fold of the data equals a fixed value, so the reads cannot be
 * dropped (sink's contents are meaningless).  The measured roofline
 * beside the spec sheet [sm8x-bench, methodology: a bandwidth probe gives
 * the measured roofline]. */
qg_status qg_read_probe(const void *buf, size_t bytes, uint32_t *sink, int wgs, int loads, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_TUNING_H */
