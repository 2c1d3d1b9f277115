/*
 * gclip_stamps.h -- the phase timeline of the fused clip kernel, a
 * diagnostic build of libgclip.
 *
 * The grad clip lesson (unhomeschool.com, ru), section "ANDREA's three-kernel
 * pipeline", splits the clip into a summing pass, a final reduction with the
 * decision, and a scaling pass.  The fused kernels (gclip_clip_ and
 * gclip_accumulate_clip_ on the fused path) run all three in one launch; this
 * build records, per workgroup, the wall-clock time at which each of its
 * phases ended, so that the time of one launch can be split between them.
 * With the += the summing pass also writes the sums of the streamed region,
 * and the scaling pass rescales the scale chunks the workgroup claims.  The
 * one-launch per-tensor clip (gclip_clip_per_tensor_ on the fused path)
 * records the same points over pieces: its streamed run summed, its resident
 * pieces read, its tensors counted and completed, the decision seen, its
 * resident pieces written, its claimed pieces scaled.
 *
 * Only the library built with -DGCLIP_PHASE_STAMPS exports gclip_phase_stamps
 * (`python -m global_l2_norm_amd.build --phase-stamps` writes it to
 * global_l2_norm_amd/_stamps/libgclip.so); the library itself records
 * nothing and does not export it.  The stamps are kept in one device array
 * per process that every fused launch on the device overwrites; a workgroup
 * that hands its block back records no phase after GCLIP_STAMP_BLOCK_READ,
 * so its later slots keep older values (earlier than its own start).
 */
#ifndef GCLIP_STAMPS_H
#define GCLIP_STAMPS_H

#include <stdint.h>

#include "gclip.h"

/* Workgroups recorded (workgroups beyond it record nothing) and slots per
 * workgroup. */
#define GCLIP_STAMP_WORKERS 1024
#define GCLIP_STAMP_POINTS 8

/* Slot k of a workgroup's stamps: the wall clock when it ... */
#define GCLIP_STAMP_START 0           /* started */
#define GCLIP_STAMP_CHUNKS_SUMMED 1   /* had summed its chunks of the streamed region */
#define GCLIP_STAMP_BLOCK_READ 2      /* had read its block into VGPRs and LDS */
#define GCLIP_STAMP_DECISION_SEEN 3   /* knew the decision (every wave) */
#define GCLIP_STAMP_BLOCK_WRITTEN 4   /* had issued the writes of its block (when it writes) */
#define GCLIP_STAMP_CHUNKS_SCALED 5   /* had scaled its chunks of the streamed region (when it writes) */
#define GCLIP_STAMP_END 6             /* was done, finish ticket included (the per-tensor clip: taken) */
#define GCLIP_STAMP_TENSORS_DONE 7    /* the per-tensor clip: had counted its pieces and summed the
                                         tensors it completed */

#ifdef __cplusplus
extern "C" {
#endif

/* Copy the stamps of workgroups 0 .. n_workers - 1 of the last fused launch
 * on the current device (synchronously: the caller has waited for it) into
 * host[n_workers * GCLIP_STAMP_POINTS], slot k of workgroup w at
 * host[w * GCLIP_STAMP_POINTS + k], in ticks of the device's wall clock,
 * whose rate (ticks per second) goes to *ticks_per_s.
 *   host          host memory owned by the caller
 *   n_workers     0 .. GCLIP_STAMP_WORKERS (gclip_list_info's n_workers)
 * Returns GCLIP_EINVAL for a NULL pointer or n_workers out of range,
 * GCLIP_EHIP for a failed HIP call. */
gclip_status gclip_phase_stamps(uint64_t* host, int32_t n_workers, int64_t* ticks_per_s);

#ifdef __cplusplus
}
#endif

#endif /* GCLIP_STAMPS_H */
