/*
 * gclip.h -- C ABI of libgclip: global L2-norm gradient clipping on one
 * MI355X (gfx950) GPU.
 *
 * What the library computes (the three pages this work follows):
 *
 *   Grad clip lesson (unhomeschool.com, ru), section "Math": the global norm is
 *   the square root of the sum of g^2 over every element of every gradient
 *   tensor; when it exceeds max_norm every element is multiplied by
 *   max_norm / norm, otherwise the gradients pass unchanged.  Section "Two
 *   variants: Per-Tensor or Global": all gradients are treated as one vector
 *   and every tensor gets the same factor.
 *
 *   Gradient clipping glossary (paweldubiel.com), section "Mechanism and
 *   details": g is kept when ||g||_2 <= c and becomes c g / ||g||_2 when
 *   ||g||_2 > c, for a threshold c > 0; a NaN or infinite value calls for
 *   diagnosis and an error-if-nonfinite switch stops that update.  Section
 *   "Order changes the result": clip after the whole effective batch has been
 *   accumulated.
 *
 *   Backprop lesson (unhomeschool.com, vi), section "Accumulation across
 *   microbatches": gradients are summed with += over microbatches and then
 *   averaged by 1/n_microbatches before the optimizer step.  Here that
 *   average is the avg_factor a: the norm is that of a*g and the factor
 *   written back is a*coef.  Section "Cost of general frameworks": dispatch
 *   from C and every buffer allocated once at start-up -- the hot calls below
 *   allocate nothing and never synchronise.
 *
 * Conventions shared by every entry point:
 *   - Device pointers are HIP device addresses on the current device; host
 *     pointers are ordinary process memory.  `stream` is a hipStream_t
 *     (NULL = the default stream).
 *   - Every function returns a gclip_status.  Argument errors are detected on
 *     the host before anything is enqueued; nothing is thrown or aborted.
 *   - The hot calls (every call on an existing list or optimizer other than
 *     create, destroy, info and gclip_result_read) only enqueue kernels: they
 *     allocate nothing, copy nothing, set no memory with a fill and never
 *     block.  Every launch leaves the list's workspace as it found it, so a
 *     hot call may be captured into a HIP graph and the graph replayed.
 *     Calls on one list must not overlap in time (they share its workspace):
 *     keep them on one stream, or order the streams.
 *   - Data-dependent status (a NaN or Inf in the gradients) is asynchronous:
 *     it lands in the device result block and gclip_result_read turns it into
 *     GCLIP_ENONFINITE.
 */
#ifndef GCLIP_H
#define GCLIP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 1: the global clip; 2: adds AdamW on the clipped gradient, loss-scaled
 * steps, per-tensor norms and clipping, and the last microbatch's +=; 3: the
 * per-tensor clip without the stop switch in two kernels, with its device
 * status code GCLIP_DEVICE_WAIT_TIMEOUT and gclip_set_gather_wait. */
#define GCLIP_VERSION 3

/* Storage format of every element of a list (one format per list). */
typedef enum gclip_dtype {
  GCLIP_F32 = 0,  /* IEEE binary32 */
  GCLIP_F16 = 1,  /* IEEE binary16 */
  GCLIP_BF16 = 2  /* bfloat16: the top 16 bits of a binary32 */
} gclip_dtype;

typedef enum gclip_status {
  GCLIP_OK = 0,
  GCLIP_EINVAL = 1,     /* bad argument (NULL, negative size, overlap, misalignment, bad threshold) */
  GCLIP_EDTYPE = 2,     /* unknown dtype */
  GCLIP_ENOMEM = 3,     /* device allocation failed (gclip_list_create only) */
  GCLIP_EHIP = 4,       /* a HIP runtime call failed; gclip_last_hip_error() holds its code */
  GCLIP_ENONFINITE = 5, /* gclip_result_read: a NaN/Inf element was seen and the caller asked to stop */
  GCLIP_EDEVICE = 6,    /* gclip_result_read: the kernels reported a failure (result.status != 0) */
  GCLIP_ERANGE = 7      /* a buffer given to a query function is too small, or a list too large for
                           gclip_clip_noalloc_'s fixed scratch */
} gclip_status;

/* Which kernels gclip_clip_ uses (gclip_list_set_path). */
typedef enum gclip_path {
  GCLIP_PATH_AUTO = 0,  /* fused when its kernel fits on a compute unit, else split */
  GCLIP_PATH_FUSED = 1, /* one kernel: norm, grid-wide decision, scale; each workgroup's block
                           stays in registers and LDS between the two passes */
  GCLIP_PATH_SPLIT = 2  /* two kernels: partial sums with the final reduce folded into the last
                           workgroup, then the scale pass */
} gclip_path;

/* Opaque list handle: the device descriptor table of one gradient list plus
 * its small workspace (per-workgroup partial sums and two counters). */
typedef struct gclip_list gclip_list;

/* Result block, 64 bytes, written by the kernels into DEVICE memory that the
 * caller owns (allocate it once; any 8-byte-aligned device address). */
typedef struct gclip_result {
  double sumsq;       /* sum over every element of (a*g)^2, in binary64 */
  double norm;        /* sqrt(sumsq): the global norm before clipping */
  double scale;       /* factor multiplied into every element: a*coef; 1.0 when nothing was written */
  double max_norm;    /* threshold of the last decision */
  int32_t nonfinite;  /* 1 when some element is NaN or +-Inf */
  int32_t clipped;    /* 1 when norm > max_norm (NaN > c is false) */
  int32_t skipped;    /* 1 when nothing was written because nonfinite && error_if_nonfinite */
  int32_t decided;    /* 1 once a scale pass has made its decision; 0 after gclip_norm alone */
  int32_t status;     /* 0, or a device-side failure code (GCLIP_DEVICE_*) */
  int32_t handed_back; /* fused path: workgroups that stopped waiting at the grid-wide decision
                          (gclip_list_set_wait); their blocks were scaled from memory by others */
  int32_t reserved[2];
} gclip_result;

/* Device-side failure codes in gclip_result.status. */
enum {
  /* gclip_clip_per_tensor_, gclip_tensor_norms or gclip_accumulate_norm
   * (and the split path of gclip_accumulate_clip_): the workgroup that
   * gathers every tensor's sum into the result block waited longer than
   * gclip_set_gather_wait allows (10 s by default, so only under an extreme
   * device load) and gave up.  The list's figures in the result block are
   * not complete.  Without the stop switch every tensor's figures and its
   * scaling still are; with it nothing is written, and the per-tensor factors
   * in the figures are not meaningful.  A gclip_scale or gclip_adamw_step
   * that follows on the same block (the split path of gclip_accumulate_clip_
   * is one) then writes nothing: after gclip_accumulate_clip_ the buffer
   * holds the sums, unscaled.  gclip_result_read returns GCLIP_EDEVICE. */
  GCLIP_DEVICE_WAIT_TIMEOUT = 1
};

/* Summary of a list's descriptor table (gclip_list_info). */
typedef struct gclip_list_info_t {
  int64_t n_tensors;
  int64_t n_elements;      /* total elements over all tensors */
  int64_t n_bytes;         /* total bytes of gradient storage */
  int64_t n_segments;      /* 16-byte-aligned vector runs */
  int64_t n_vectors;       /* 16-byte vectors over all runs */
  int64_t n_scalars;       /* elements handled one by one (unaligned ends, tiny tensors) */
  int32_t n_workers;       /* workgroups of the launch: one per compute unit, or one for a list whose
                              vectors fit in one group (4,096 vectors) with at most one single element
                              per thread, which the fused path clips in one workgroup */
  int32_t worker_threads;  /* threads per workgroup */
  int32_t dtype;
  int32_t path;            /* gclip_path that gclip_clip_ will use */
  int64_t resident_vectors; /* vectors the fused kernel keeps on chip between its passes */
} gclip_list_info_t;

/* One entry of a plan description (gclip_plan_query): a run of elements of
 * one tensor, which is
 *   kind 0  part of a worker's block of 16-byte vectors (the blocks end the
 *           list; each is read by its worker in both summing passes, kept on
 *           chip by the fused kernel and written back by the same worker),
 *   kind 1  single elements of a worker (every pass),
 *   kind 2  part of a chunk of 16-byte vectors over the whole list, claimed
 *           at run time by any worker in the split scale pass (worker -1),
 *   kind 3  part of a sum chunk of the streamed region before the blocks
 *           (cut where the blocks begin), claimed at run time by any worker
 *           in the summing passes (worker -1),
 *   kind 4  part of a scale chunk of that streamed region, claimed at run
 *           time by any worker in the fused kernel's scale pass (worker -1).
 * The summing passes cover kinds 0, 1 and 3, the split scale pass kinds 1 and
 * 2, the fused scale pass kinds 0, 1 and 4. */
typedef struct gclip_plan_entry {
  int32_t worker;
  int32_t tensor;
  int64_t elem_begin;
  int64_t elem_count;
  int32_t kind;
  int32_t reserved;
} gclip_plan_entry;

/* Build the descriptor table of a gradient list on the current device.
 * (Grad clip lesson, section "The naive algorithm cannot work on a GPU": the
 * tensors have very different shapes, so one launch must cover all of them;
 * section "ANDREA's three-kernel pipeline": one block per chunk, hundreds of
 * blocks across all tensors, partial sums in a small scratch buffer.)
 *   d_ptrs[i]  device address of tensor i's first element (contiguous storage,
 *              aligned to the element size); may be NULL when numels[i] == 0
 *   numels[i]  element count of tensor i (>= 0)
 *   n_tensors  >= 0 (0 is an empty list: norm 0, nothing written)
 *   dtype      a gclip_dtype, the same for every tensor
 *   out        receives the handle
 * The caller keeps ownership of the gradient buffers: they must stay
 * allocated and must not move while the list exists.  Overlapping or
 * duplicated ranges are rejected with GCLIP_EINVAL (they would be counted and
 * scaled twice).  This call allocates device memory and synchronises. */
gclip_status gclip_list_create(void* const* d_ptrs, const int64_t* numels, int32_t n_tensors, int32_t dtype,
                               gclip_list** out);

/* Free a list's device table and workspace.  Synchronises.  NULL is a no-op. */
gclip_status gclip_list_destroy(gclip_list* list);

/* Fill *out with the shape of a list's descriptor table. */
gclip_status gclip_list_info(const gclip_list* list, gclip_list_info_t* out);

/* Choose the kernels gclip_clip_ uses for this list (a gclip_path).  FUSED
 * where its kernel cannot run returns GCLIP_EINVAL. */
gclip_status gclip_list_set_path(gclip_list* list, int32_t path);

/* The fused kernel is an ordinary launch, so its workgroups need not all be
 * resident at once (other work may hold some compute units).  A workgroup
 * that has waited `microseconds` at the grid-wide decision hands its block
 * back and exits; the workgroups that see the decision then read that block
 * again from memory and scale it.  The result is the same either way, only
 * slower; result.handed_back counts such workgroups.  0 <= microseconds <=
 * 60e6 (default 1000; 0 makes every workgroup but the deciding one hand its
 * block back, which tests that path).  Host-only setting, no GPU work. */
gclip_status gclip_list_set_wait(gclip_list* list, int64_t microseconds);

/* Norm pass: sum of squares of a*g over the whole list, reduced to one
 * binary64 scalar on the device (grad clip lesson, section "ANDREA's
 * three-kernel pipeline", kernels 1 and 2; section "Math", the norm).
 *   avg_factor  a > 0 and finite (1/n_microbatches; 1.0 for none)
 *   d_result    device result block; receives sumsq, norm, nonfinite and
 *               decided = 0
 * One kernel launch on `stream`; a fixed summation order makes the result
 * bit-identical from run to run.  A list must not be used by two calls that
 * are in flight at once (they share the workspace). */
gclip_status gclip_norm(gclip_list* list, double avg_factor, gclip_result* d_result, void* stream);

/* Scale pass (grad clip lesson, section "ANDREA's three-kernel pipeline",
 * kernel 3; glossary page, "Mechanism and details").  Reads d_result->sumsq
 * and d_result->nonfinite (as left by gclip_norm, or replaced by the caller,
 * e.g. after summing sumsq across ranks), then on the device:
 *   norm = sqrt(sumsq); coef = (norm > max_norm) ? max_norm / norm : 1;
 *   s = avg_factor * coef;
 *   if (nonfinite && error_if_nonfinite) or s == 1: write nothing;
 *   else every element g becomes g * s rounded to nearest-even in its format.
 *   max_norm     c > 0, not NaN; +inf means never clip
 *   avg_factor   the same a given to gclip_norm
 *   error_if_nonfinite  nonzero: a NaN/Inf element stops the update
 * Writes scale, clipped, skipped, max_norm and decided = 1 into d_result.
 * When d_result->status != 0 (the norm before it reported a failure, e.g.
 * GCLIP_DEVICE_WAIT_TIMEOUT, so sumsq and nonfinite are not this step's) it
 * decides nothing, writes no gradient and leaves d_result as it is; a block
 * the caller fills in must therefore hold status 0. */
gclip_status gclip_scale(gclip_list* list, double max_norm, double avg_factor, int32_t error_if_nonfinite,
                         gclip_result* d_result, void* stream);

/* The whole path in place: gclip_norm followed by gclip_scale, as one
 * kernel (GCLIP_PATH_FUSED) or two launches (GCLIP_PATH_SPLIT).
 * Same arguments, same result block, same bits as the two calls. */
gclip_status gclip_clip_(gclip_list* list, double max_norm, double avg_factor, int32_t error_if_nonfinite,
                         gclip_result* d_result, void* stream);

/* Copy the device result block to *h_out after the work queued on `stream`
 * has finished.  The only call that waits.  Returns GCLIP_EDEVICE when
 * h_out->status != 0, else GCLIP_ENONFINITE when h_out->nonfinite and
 * error_if_nonfinite, else GCLIP_OK. */
gclip_status gclip_result_read(const gclip_result* d_result, void* stream, gclip_result* h_out,
                               int32_t error_if_nonfinite);

/* ---------------------------------------------------------------------------
 * Optimizer step on the clipped gradient (AdamW).
 *
 * Grad clip lesson, section "Order matters: Pre-Adam": the clip runs before
 * AdamW updates its moments m, v and the weights, so the moments only see the
 * clipped gradient.  Backprop lesson, section "Optimizer state": AdamW keeps
 * m and v per weight; section "Signals & checkpoints": weights, m and v are
 * binary32.  Instead of writing the clipped gradient back and reading it
 * again, the optimizer reads the factor the clip decided from the result
 * block and multiplies each gradient element by it on load: the clip then
 * costs one read pass (gclip_norm) before the optimizer.
 *
 * The update is AdamW as published (decoupled weight decay; the moments of
 * Adam with bias correction), in binary32 arithmetic:
 *   g  = s * grad                     s: the factor of the clip decision
 *   m  = beta1 * m + (1 - beta1) * g
 *   v  = beta2 * v + (1 - beta2) * g * g
 *   p  = p * (1 - lr * wd) - (lr / (1 - beta1^t)) * m / (sqrt(v) / sqrt(1 - beta2^t) + eps)
 * where t = step (>= 1, this step included).
 * ------------------------------------------------------------------------- */

/* Opaque handle: the device table of four parallel tensor lists. */
typedef struct gclip_adamw gclip_adamw;

typedef struct gclip_adamw_hparams {
  double lr;            /* >= 0, finite */
  double beta1, beta2;  /* in [0, 1) */
  double eps;           /* > 0, finite */
  double weight_decay;  /* >= 0, finite (decoupled) */
  int64_t step;         /* >= 1: steps taken, this one included */
} gclip_adamw_hparams;

/* Build the table of one parameter list on the current device.
 *   d_params, d_exp_avg, d_exp_avg_sq  binary32 tensors (weights, m, v),
 *                                      aligned to 4 bytes
 *   d_grads     gradient tensors in grad_dtype (a gclip_dtype), aligned to
 *               the element size; the same list gclip_list_create was given
 *   numels[i]   element count of tensor i in all four lists (>= 0)
 * The caller keeps ownership of every buffer; they must stay allocated and
 * must not move while the handle exists.  Any overlap between two of the
 * 4 * n_tensors ranges is rejected with GCLIP_EINVAL.  Allocates device
 * memory and synchronises. */
gclip_status gclip_adamw_create(void* const* d_params, void* const* d_grads, void* const* d_exp_avg,
                                void* const* d_exp_avg_sq, const int64_t* numels, int32_t n_tensors,
                                int32_t grad_dtype, gclip_adamw** out);

/* Free a handle's device table.  Synchronises.  NULL is a no-op. */
gclip_status gclip_adamw_destroy(gclip_adamw* opt);

/* One optimizer step on `stream`.  Reads d_result->sumsq and nonfinite (as
 * gclip_norm left them over the same gradients, or as the caller replaced
 * them), decides as gclip_scale does and writes scale, clipped, skipped,
 * max_norm and decided = 1 into d_result; then, unless skipped (a NaN/Inf
 * gradient with error_if_nonfinite: weights and moments stay bitwise
 * unchanged), updates every weight and both moments with g = s * grad.  The
 * gradients are only read.  As gclip_scale, it takes no step and leaves
 * d_result as it is when d_result->status != 0.  One kernel launch, no
 * allocation, no sync. */
gclip_status gclip_adamw_step(gclip_adamw* opt, const gclip_adamw_hparams* hp, double max_norm, double avg_factor,
                              int32_t error_if_nonfinite, gclip_result* d_result, void* stream);

/* ---------------------------------------------------------------------------
 * Per-tensor norms and per-tensor clipping.
 *
 * Grad clip lesson, section "Two variants: Per-Tensor or Global": besides the
 * global clip (the whole list as one vector) the page describes clipping
 * every tensor on its own, by its own norm -- simple, but it changes the
 * tensors' relative sizes.  The per-tensor norms are also the diagnostic a
 * run wants when one tensor spikes.  Both calls cut the list into pieces
 * that each lie inside one tensor, sum each piece in one workgroup, and let
 * the last workgroup to finish sum each tensor's pieces in order (so the bits
 * do not depend on scheduling).
 * ------------------------------------------------------------------------- */

/* One tensor's figures, 32 bytes, in an array of n_tensors in DEVICE memory
 * that the caller owns (8-byte aligned). */
typedef struct gclip_tensor_result {
  double sumsq;       /* sum over the tensor of (a*g)^2 */
  double norm;        /* its square root */
  double scale;       /* factor written into the tensor; 1.0 when nothing was written */
  int32_t nonfinite;  /* 1 when the tensor holds a NaN/Inf element */
  int32_t clipped;    /* 1 when the tensor's norm exceeded max_norm (per-tensor clip) */
} gclip_tensor_result;

/* Norms of every tensor of the list, of a*g, into d_tensors[0 .. n_tensors),
 * and the list's norm into d_result (sumsq, norm, nonfinite; decided = 0),
 * so that gclip_scale can follow to finish a global clip with per-tensor
 * figures.  Writes no gradient.  Enqueues two kernels (partial sums per
 * piece; then one workgroup per tensor sums its pieces, and the list's
 * figures are gathered in the same launch, see GCLIP_DEVICE_WAIT_TIMEOUT;
 * only the second for a list with no element); no allocation, no
 * synchronisation.  Errors as gclip_norm, plus GCLIP_EINVAL for a NULL or
 * misaligned d_tensors when the list has tensors. */
gclip_status gclip_tensor_norms(gclip_list* list, double avg_factor, gclip_tensor_result* d_tensors,
                                gclip_result* d_result, void* stream);

/* Per-tensor clipping in place: tensor t is multiplied by a * (max_norm /
 * norm_t) when norm_t > max_norm, by a otherwise (nothing is written when
 * that factor is 1).  With error_if_nonfinite, one NaN/Inf anywhere in the
 * list stops the whole update: no tensor is written and d_result->skipped is
 * set.  d_tensors receives every tensor's figures; d_result the list's sumsq,
 * norm and nonfinite, clipped = 1 when any tensor was clipped, scale = 1.0
 * (the factors are per tensor).  Without error_if_nonfinite no tensor waits
 * for another, and two kernels run on `stream` (partial sums per piece; then
 * every piece decides for its own tensor and scales, and the list's figures
 * are gathered in the same launch, see GCLIP_DEVICE_WAIT_TIMEOUT); with it,
 * three (the partials; one workgroup per tensor for the decisions, gathered
 * with the stop decision; the scale).  No allocation, no synchronisation.
 * Errors as gclip_clip_. */
gclip_status gclip_clip_per_tensor_(gclip_list* list, double max_norm, double avg_factor,
                                    int32_t error_if_nonfinite, gclip_tensor_result* d_tensors,
                                    gclip_result* d_result, void* stream);

/* How long, in microseconds, the per-tensor calls let their gathering
 * workgroup wait for every tensor's sum before it reports
 * GCLIP_DEVICE_WAIT_TIMEOUT: for every list of the process, from the next
 * call on.  Default 10 s (a negative value restores it); at most 60 s, else
 * GCLIP_EINVAL.  Meant for tests of that failure path: a short wait makes it
 * happen without any fault. */
gclip_status gclip_set_gather_wait(int64_t microseconds);

/* ---------------------------------------------------------------------------
 * The norm pass fused into the last microbatch's +=.
 *
 * Backprop lesson, section "Accumulation across microbatches": the backward
 * pass of every microbatch adds its gradient into the gradient buffer (+=);
 * the glossary page, section "Order changes the result", clips once the last
 * contribution is in.  The last += reads the buffer and the contribution and
 * writes the buffer anyway, so it sums the squares of the values it writes:
 * the norm then needs no read pass of its own.
 * ------------------------------------------------------------------------- */

typedef struct gclip_contrib gclip_contrib;

/* Register the buffers of one microbatch's contribution to a list's
 * gradients: d_contrib[t] holds the list's numels[t] elements of its dtype,
 * at the same address modulo 16 bytes as the list's tensor t (as separately
 * allocated tensors are), overlapping no tensor of the list and no other
 * contribution tensor.  The caller keeps the buffers alive and unmoved while
 * the handle is used; they are only read.  Uploads one 8-byte offset per
 * tensor; allocates and synchronises (not a hot call).  GCLIP_EINVAL on a
 * NULL pointer, a misaligned address or an overlap. */
gclip_status gclip_contrib_create(const gclip_list* list, void* const* d_contrib, gclip_contrib** out);

/* Free a contribution handle's device table.  Synchronises.  NULL is a
 * no-op.  A handle belongs to the list it was registered for: destroy it
 * before that list. */
gclip_status gclip_contrib_destroy(gclip_contrib* contrib);

/* The last +=, fused with the norm pass: for every element of the list,
 * acc <- acc + g rounded once to the storage format (the format's own IEEE
 * addition) and written back; the norm of a * acc (the new values) goes into
 * d_result (sumsq, norm, nonfinite; decided = 0) and, when d_tensors is not
 * NULL, every tensor's figures into d_tensors (n_tensors entries, as for
 * gclip_tensor_norms).  gclip_scale can then finish the global clip, or
 * gclip_adamw_step the optimizer step.  contrib must have been registered
 * for this list.  Two kernels on `stream` (the += with partial sums per
 * piece; then one workgroup per tensor sums its pieces, and the list's
 * figures are gathered in the same launch, see GCLIP_DEVICE_WAIT_TIMEOUT);
 * no allocation, no synchronisation. */
gclip_status gclip_accumulate_norm(gclip_list* list, const gclip_contrib* contrib, double avg_factor,
                                   gclip_tensor_result* d_tensors, gclip_result* d_result, void* stream);

/* The last += and the global clip of a * acc: the sum is written whatever
 * the decision, and scaled when the clip (and the stop switch) say so.  On
 * the fused path one kernel, which keeps part of the sums on chip across the
 * decision and so writes them only once; on the split path
 * gclip_accumulate_norm followed by gclip_scale.  No allocation, no
 * synchronisation. */
gclip_status gclip_accumulate_clip_(gclip_list* list, const gclip_contrib* contrib, double max_norm,
                                    double avg_factor, int32_t error_if_nonfinite, gclip_result* d_result,
                                    void* stream);

/* ---------------------------------------------------------------------------
 * Loss-scaled steps (mixed precision).
 *
 * Glossary page, introduction and section "Order changes the result": with
 * loss scaling the order of unscaling and clipping matters -- unscale first,
 * so that the threshold applies to the gradients' true size.  Here the
 * unscaling is folded into the averaging factor: a = 1 / (n_microbatches * S)
 * with the loss scale S read from device memory when the kernels start, so
 * the norm is that of the unscaled, averaged gradient and the written factor
 * is a * coef.  A NaN/Inf element is found-inf: nothing is written (the stop
 * switch is always on) and the optimizer step is to be skipped.  After the
 * step the loss scale is updated on the device, by dynamic loss scaling as
 * published (the pages do not give the rule): found-inf multiplies S by
 * backoff_factor and restarts the count of clean steps; otherwise the count
 * grows, and every growth_interval clean steps S is multiplied by
 * growth_factor (unless that is not finite in binary32).
 * ------------------------------------------------------------------------- */

/* Loss-scale state, 16 bytes in DEVICE memory that the caller owns. */
typedef struct gclip_amp_state {
  float scale;             /* loss scale S > 0 (binary32) */
  int32_t growth_tracker;  /* clean steps since the scale last changed */
  int32_t found_inf;       /* 1 when the last step's gradients held a NaN/Inf */
  int32_t reserved;
} gclip_amp_state;

typedef struct gclip_amp_params {
  double growth_factor;     /* >= 1, finite */
  double backoff_factor;    /* in (0, 1] */
  int32_t growth_interval;  /* >= 1 */
  int32_t reserved;
} gclip_amp_params;

/* gclip_norm of the unscaled, averaged gradient: a = 1 / (n_microbatches * S)
 * with S = d_amp->scale.  n_microbatches > 0 and finite.  Does not update
 * d_amp (gclip_clip_amp_ or gclip_adamw_step_amp do, after the step). */
gclip_status gclip_norm_amp(gclip_list* list, double n_microbatches, const gclip_amp_state* d_amp,
                            gclip_result* d_result, void* stream);

/* gclip_clip_ with a = 1 / (n_microbatches * S) and error_if_nonfinite on,
 * then the loss-scale update of d_amp (found_inf, scale, growth_tracker).
 * On the fused path the update is made in the same launch, by the workgroup
 * that decides, once every workgroup has read S; on the split path by one
 * more single-thread kernel after the two.  No allocation, no sync. */
gclip_status gclip_clip_amp_(gclip_list* list, double max_norm, double n_microbatches, gclip_amp_state* d_amp,
                             const gclip_amp_params* amp, gclip_result* d_result, void* stream);

/* gclip_adamw_step with a = 1 / (n_microbatches * S) and error_if_nonfinite
 * on (found-inf: weights and moments stay unchanged), then the loss-scale
 * update (none when d_result->status != 0: no step was taken).  To follow
 * gclip_norm_amp over the same gradients and d_amp. */
gclip_status gclip_adamw_step_amp(gclip_adamw* opt, const gclip_adamw_hparams* hp, double max_norm,
                                  double n_microbatches, gclip_amp_state* d_amp, const gclip_amp_params* amp,
                                  gclip_result* d_result, void* stream);

/* ---------------------------------------------------------------------------
 * For callers that cannot allocate device memory: serving loops and
 * harnesses that forbid hipMalloc.
 * ------------------------------------------------------------------------- */

/* Bytes of the static device array, one per GPU, that holds the descriptor
 * table and workspace of gclip_clip_noalloc_. */
#define GCLIP_NOALLOC_SCRATCH_BYTES (4u << 20)

/* gclip_list_create + gclip_clip_ + gclip_list_destroy in one call that
 * allocates no device memory: the list's descriptor table and workspace go
 * into a static device array of GCLIP_NOALLOC_SCRATCH_BYTES that each GPU the
 * library runs on holds until the process ends.  Arguments as
 * gclip_list_create (d_ptrs, numels, n_tensors, dtype) and gclip_clip_
 * (max_norm, avg_factor, error_if_nonfinite, d_result, stream); the same
 * kernels run on the same table, so the result block and the gradients come
 * out bit for bit as from those calls.  Each call builds the table in host
 * memory and copies it into this GPU's array with one hipMemcpyAsync on
 * `stream` (from pageable memory: it returns once the copy is staged), then
 * enqueues the kernels; it never synchronises the device.
 * Limits and errors: a list whose table and workspace need more than
 * GCLIP_NOALLOC_SCRATCH_BYTES -- a list of more than about 20 GB, or fewer
 * bytes with very many tensors or many elements handled one by one (8 bytes
 * of table each) -- is rejected with GCLIP_ERANGE; argument errors as the
 * two calls; nothing is enqueued on any error.
 * Every call on one GPU shares its array, which keeps the last call's
 * contents (each call rewrites what it reads): calls that overlap in time on
 * one GPU -- on two streams, or from two host threads -- race, and the caller
 * must order them.  Not for HIP graph capture (the copy is from pageable
 * memory). */
gclip_status gclip_clip_noalloc_(void* const* d_ptrs, const int64_t* numels, int32_t n_tensors, int32_t dtype,
                                 double max_norm, double avg_factor, int32_t error_if_nonfinite,
                                 gclip_result* d_result, void* stream);

/* Describe, without touching any GPU, how a list would be split: the runs
 * of each worker, in the order the kernels visit them.  Addresses only need
 * their alignment (they are never dereferenced).
 *   n_workers, worker_threads  launch shape to plan for (> 0)
 *   out, cap                   array of cap entries (may be NULL when cap == 0)
 *   n_out                      receives the number of entries needed
 * Returns GCLIP_ERANGE when cap is too small (n_out is still set). */
gclip_status gclip_plan_query(const uint64_t* addrs, const int64_t* numels, int32_t n_tensors, int32_t dtype,
                              int32_t n_workers, int32_t worker_threads, gclip_plan_entry* out, int64_t cap,
                              int64_t* n_out);

/* Replay on the host, without any GPU, the address walk one kernel would
 * make over a list planned for n_workers workers (the kernels' own cursor
 * code, compiled for the host), for checking it on the CPU:
 *   mode 0  norm kernel, 1  scale kernel,
 *        2  fused kernel, first pass, 3  fused kernel, second pass,
 *        4  per-tensor kernels (out_worker is then the tensor a piece
 *           belongs to, not a worker),
 *        5  the contribution reads of the fused kernel with the += (first
 *           pass), 6  those of a block handed back, for a contribution
 *           tensor t placed at addrs[t] + 2^44 + t 2^34
 * Fills out_addr[i] (address of a 16-byte vector, or, with bit 63 set, of a
 * single element) and out_worker[i] for every lane access; accesses to
 * chunks, which any worker may claim at run time, carry worker -1.  n_out
 * receives the count.  GCLIP_ERANGE when cap is too
 * small; GCLIP_EINVAL when the lanes of a step disagree on the cursor. */
gclip_status gclip_plan_trace(const uint64_t* addrs, const int64_t* numels, int32_t n_tensors, int32_t dtype,
                              int32_t n_workers, int32_t mode, uint64_t* out_addr, int32_t* out_worker, int64_t cap,
                              int64_t* n_out);

/* A static string naming a status code. */
const char* gclip_status_string(int32_t status);

/* The hipError_t behind the last GCLIP_EHIP returned on this thread. */
int32_t gclip_last_hip_error(void);

/* GCLIP_VERSION of the built library. */
int32_t gclip_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GCLIP_H */
