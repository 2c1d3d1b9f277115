// gclip_host.hpp -- host-side declarations shared by the C ABI's source
// files (internal to libgclip): the kernel launchers, the launch shape, and
// the argument checks every hot call makes before it enqueues anything.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/gclip.h"
#include "gclip_plan.hpp"

namespace gclip {
int worker_threads();
uint64_t resident_cap_vectors();
ChunkShape chunk_shape();
hipError_t launch_norm(const DevPlan& p, int32_t dtype, AvgSrc avg, gclip_result* res, hipStream_t st);
hipError_t launch_scale(const DevPlan& p, int32_t dtype, double max_norm, AvgSrc avg, int err, gclip_result* res,
                        hipStream_t st);
hipError_t launch_fused(const DevPlan& p, int32_t dtype, double max_norm, AvgSrc avg, int err, gclip_result* res,
                        uint64_t wait_ticks, AmpUpdate amp, hipStream_t st);
hipError_t fused_capacity(int32_t dtype, int* blocks_per_cu);
hipError_t launch_tensor_clip_fused(const DevPlan& p, const TensorPlan& T, int32_t dtype, AvgSrc avg,
                                    double max_norm, int err, gclip_tensor_result* out, gclip_result* res,
                                    uint64_t wait_ticks, hipStream_t st);
hipError_t tensor_fused_capacity(int32_t dtype, int* blocks_per_cu);
hipError_t launch_adamw(const AdamPlan& plan, int32_t dtype, const AdamHp& h, double max_norm, AvgSrc avg, int err,
                        gclip_result* res, hipStream_t st);
hipError_t launch_amp_update(const gclip_result* res, gclip_amp_state* st, double growth, double backoff,
                             int32_t interval, hipStream_t s);
hipError_t launch_tensor_norm(const TensorPlan& T, int32_t dtype, AvgSrc avg, double max_norm, int clip, int err,
                              gclip_tensor_result* out, gclip_result* res, hipStream_t st);
hipError_t launch_tensor_scale(const TensorPlan& T, int32_t dtype, gclip_tensor_result* out,
                               const gclip_result* res, hipStream_t st);
hipError_t launch_tensor_clip(const TensorPlan& T, int32_t dtype, AvgSrc avg, double max_norm,
                              gclip_tensor_result* out, gclip_result* res, uint64_t wait_ticks, hipStream_t st);
hipError_t launch_accumulate_norm(const TensorPlan& T, int32_t dtype, const uint64_t* gdelta, AvgSrc avg,
                                  gclip_tensor_result* out, gclip_result* res, uint64_t wait_ticks, bool gather,
                                  hipStream_t st);
hipError_t launch_tensor_norms(const TensorPlan& T, int32_t dtype, AvgSrc avg, gclip_tensor_result* out,
                               gclip_result* res, uint64_t wait_ticks, bool gather, hipStream_t st);
hipError_t launch_tensor_decisions(const TensorPlan& T, int32_t dtype, AvgSrc avg, double max_norm, int err,
                                   gclip_tensor_result* out, gclip_result* res, uint64_t wait_ticks, bool gather,
                                   hipStream_t st);
hipError_t launch_accum_fused(const DevPlan& p, const AccSrc& A, int32_t dtype, double max_norm, AvgSrc avg,
                              int err, gclip_result* res, uint64_t wait_ticks, hipStream_t st);

// GCLIP_EHIP, keeping e for gclip_last_hip_error() on this thread.
gclip_status hip_fail(hipError_t e);

inline bool factor_ok(double a) { return std::isfinite(a) && a > 0.0; }
inline bool threshold_ok(double c) { return !std::isnan(c) && c > 0.0; }
inline bool result_ptr_ok(const gclip_result* r) { return r && reinterpret_cast<uintptr_t>(r) % 8 == 0; }

}  // namespace gclip
