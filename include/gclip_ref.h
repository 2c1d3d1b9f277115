/*
 * gclip_ref.h -- attainable-bandwidth reference kernels of libgclip.
 *
 * The grad clip lesson (unhomeschool.com, ru), section "ANDREA's three-kernel
 * pipeline", makes the clip two full passes over the gradients: a read (the
 * partial sums of squares) and, when the norm exceeds the threshold, a read
 * and a write (the scale).  These two calls move the same kinds of bytes and
 * do nothing else, so the rates they reach on a device bound the rates the
 * clip's passes can reach there; the benchmark reports the clip against
 * them.  They are not part of the clip itself.
 *
 * Both take device addresses on the current device, enqueue one kernel on
 * `stream` (a hipStream_t; NULL = the default stream), allocate nothing and
 * never block.  Argument errors return GCLIP_EINVAL with nothing enqueued.
 */
#ifndef GCLIP_REF_H
#define GCLIP_REF_H

#include <stdint.h>

#include "gclip.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read every 16-byte vector of [d_src, d_src + bytes) once, with
 * nontemporal dwordx4 loads, one workgroup per 128 KB.
 *   d_src   16-byte aligned (may be NULL when bytes == 0)
 *   bytes   >= 0, a multiple of 16
 *   d_sink  a 4-byte aligned device word; written only when a lane's
 *           folded data equals one fixed constant (so the loads cannot be
 *           optimised away; in practice it is never written) */
gclip_status gclip_ref_read(const void* d_src, int64_t bytes, uint32_t* d_sink, void* stream);

/* Copy [d_src, d_src + bytes) to d_dst: every vector is loaded (nontemporal)
 * and stored (ordinary stores, which were faster at every size tried) once,
 * one workgroup per 32 KB.  d_dst == d_src copies in place, the traffic of
 * the clip's scale pass; otherwise the two ranges must not overlap.
 *   d_src, d_dst  16-byte aligned (may be NULL when bytes == 0)
 *   bytes         >= 0, a multiple of 16 */
gclip_status gclip_ref_copy(void* d_dst, const void* d_src, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GCLIP_REF_H */
