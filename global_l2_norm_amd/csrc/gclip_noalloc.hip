// gclip_noalloc.hip -- gclip_clip_noalloc_: the clip of a list given by its
// device pointers and sizes, for callers that cannot allocate device memory.
//
// gclip_list_create allocates a device block for a list's descriptor table
// and its workspace (the partial sums, the decision word, the counters, the
// block states).  Here both go into `scratch` instead: a file-scope device
// array of GCLIP_NOALLOC_SCRATCH_BYTES that every GPU the library runs on
// holds until the process ends.  Each call builds the table on the host,
// copies it, together with the initial value of every workspace word that a
// launch expects (decision word undecided, counters and block states zero),
// into this device's copy of the array with one hipMemcpyAsync on the
// caller's stream, and launches the kernels gclip_clip_ would launch.  No
// hipMalloc, hipFree or other device allocation is made.  All calls on one
// GPU share its copy of the array: calls that overlap in time on one GPU
// (two streams, or two host threads) race, and the caller must order them.
#include <hip/hip_runtime.h>

#include <mutex>
#include <new>
#include <vector>

#include "../../include/gclip.h"
#include "gclip_host.hpp"
#include "gclip_plan.hpp"

// The table and workspace of gclip_clip_noalloc_.  In host code this name
// is a host-side stand-in, not a device address: host code only ever uses
// the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[GCLIP_NOALLOC_SCRATCH_BYTES];

namespace gclip {
namespace {

constexpr size_t kScratchBytes = (size_t)GCLIP_NOALLOC_SCRATCH_BYTES;

// How long a workgroup of the fused kernel waits at the grid-wide decision
// before it hands its block back (gclip_list_create's default).
constexpr uint64_t kWaitUs = 1000;

struct DeviceState {
  unsigned char* ptr = nullptr;  // this device's copy of scratch
  int32_t ncu = 0;
  uint64_t wait_ticks = 0;
  bool fused_ok[3] = {false, false, false};  // per dtype
  bool ready = false;
};
constexpr int kMaxDevices = 64;
DeviceState g_state[kMaxDevices];
std::mutex g_mu;

// Set-up, once per device, with that device current: the address of this
// device's copy of scratch, the launch shape and whether the fused kernel
// fits on a compute unit.
hipError_t device_state(int dev, const DeviceState** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState& st = g_state[dev];
  if (!st.ready) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    int ncu = 0, clk = 0;
    if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&clk, hipDeviceAttributeWallClockRate, dev)) != hipSuccess) return e;
    for (int32_t dt = 0; dt < 3; ++dt) {
      int bpc = 0;
      if ((e = fused_capacity(dt, &bpc)) != hipSuccess) return e;
      st.fused_ok[dt] = bpc >= 1 && clk > 0;
    }
    st.ptr = static_cast<unsigned char*>(p);
    st.ncu = ncu;
    st.wait_ticks = kWaitUs * (uint64_t)(clk > 0 ? clk : 0) / 1000;
    st.ready = true;
  }
  *out = &st;
  return hipSuccess;
}

}  // namespace
}  // namespace gclip

extern "C" gclip_status gclip_clip_noalloc_(void* const* d_ptrs, const int64_t* numels, int32_t n_tensors,
                                            int32_t dtype, double max_norm, double avg_factor,
                                            int32_t error_if_nonfinite, gclip_result* d_result, void* stream) {
  using namespace gclip;
  if (!dtype_valid(dtype)) return GCLIP_EDTYPE;
  if (n_tensors < 0 || (n_tensors > 0 && (!d_ptrs || !numels)) || !result_ptr_ok(d_result) ||
      !threshold_ok(max_norm) || !factor_ok(avg_factor))
    return GCLIP_EINVAL;
  const uint64_t* addrs = reinterpret_cast<const uint64_t*>(d_ptrs);
  try {
    {
      // every argument error is reported before any HIP call
      const int rc = plan_validate(addrs, numels, n_tensors, dtype, nullptr, nullptr, nullptr);
      if (rc != 0) return (gclip_status)rc;
    }
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return GCLIP_EINVAL;
    const DeviceState* ds = nullptr;
    if ((e = device_state(dev, &ds)) != hipSuccess) return hip_fail(e);
    // the table is built in host memory kept per thread, so that steady
    // calls reuse it
    thread_local HostPlan plan;
    thread_local std::vector<unsigned char> image;
    const int rc = plan_build_list(addrs, numels, n_tensors, dtype, ds->ncu, worker_threads(),
                                   resident_cap_vectors(), chunk_shape(), plan, nullptr);
    if (rc != 0) return (gclip_status)rc;
    const PlanLayout L = plan_layout(plan);
    if (L.bytes > kScratchBytes) return GCLIP_ERANGE;
    image.resize(L.header);
    plan_image(plan, L, image.data());
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // from pageable host memory: the call returns once the image is staged,
    // so the next call may rebuild it; the copy itself is ordered on s after
    // the work already queued there, which may still read the array
    if ((e = hipMemcpyAsync(ds->ptr, image.data(), L.header, hipMemcpyHostToDevice, s)) != hipSuccess)
      return hip_fail(e);
    const DevPlan D = plan_view(plan, L, ds->ptr);
    const AvgSrc avg{avg_factor, nullptr};
    const int err = error_if_nonfinite ? 1 : 0;
    if (ds->fused_ok[dtype]) {
      e = launch_fused(D, dtype, max_norm, avg, err, d_result, ds->wait_ticks, AmpUpdate{nullptr, 0.0, 0.0, 0}, s);
    } else {
      e = launch_norm(D, dtype, avg, d_result, s);
      if (e == hipSuccess) e = launch_scale(D, dtype, max_norm, avg, err, d_result, s);
    }
    return e == hipSuccess ? GCLIP_OK : hip_fail(e);
  } catch (const std::bad_alloc&) {
    return GCLIP_ENOMEM;
  }
}
