// gclip_api.cpp -- the C ABI of libgclip (declared in include/gclip.h):
// argument checking, the one-time allocation of a list's descriptor table
// and workspace, and dispatch of the kernels in gclip_kernels.hip.
//
// As on the backprop lesson page (unhomeschool.com vi, section "Cost of
// general frameworks"), dispatch happens at the C level and every buffer is
// allocated once at start-up: only gclip_list_create / gclip_list_destroy
// allocate or synchronise; the hot calls only enqueue kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "../../include/gclip.h"
#include "gclip_plan.hpp"

#include "gclip_host.hpp"

// How long a workgroup of the fused kernel waits at the grid-wide decision
// before it hands its block back.  On an idle device the last workgroup
// arrives some tens of microseconds after the first.
constexpr int64_t kDefaultWaitUs = 1000;
constexpr int64_t kMaxWaitUs = 60 * 1000 * 1000;
// How long the per-tensor clip's workgroup 0 waits for every tensor's sum
// (GCLIP_DEVICE_WAIT_TIMEOUT past it); gclip_set_gather_wait changes it.
constexpr int64_t kTensorGatherWaitUs = 10 * 1000 * 1000;
std::atomic<int64_t> g_gather_wait_us{kTensorGatherWaitUs};

struct gclip_list {
  gclip::HostPlan plan;
  gclip::DevPlan dev{};
  gclip::TensorHostPlan tplan;
  gclip::TensorPlan tdev{};
  gclip_tensor_result* tscratch = nullptr;  // per-tensor figures when the caller passes none
  std::vector<uint64_t> addrs;              // the tensors, as given
  std::vector<int64_t> numels;
  void* blob = nullptr;
  int device = 0;
  bool fused_ok = false;
  bool tensor_fused_ok = false;  // the one-launch per-tensor clip fits on a compute unit
  int32_t path = GCLIP_PATH_SPLIT;
  int64_t wait_us = kDefaultWaitUs;
  uint64_t clock_khz = 0;  // device wall clock
  uint64_t wait_ticks = 0;
};

// The per-tensor gathering wait (gclip_set_gather_wait) in wall-clock ticks.
uint64_t gather_wait_ticks(const gclip_list* list) {
  return (uint64_t)g_gather_wait_us.load(std::memory_order_relaxed) * list->clock_khz / 1000;
}

struct gclip_contrib {
  const gclip_list* list = nullptr;
  uint64_t* delta = nullptr;  // device: n_tensors byte offsets, contribution minus list tensor, then the same
                              // offset per segment and per single element of the list's plan
  gclip::AccSrc acc{};        // the per-segment and per-single-element tables
  int device = 0;
};

struct gclip_adamw {
  gclip::AdamPiece* pieces = nullptr;
  uint32_t npieces = 0;
  int32_t dtype = 0;
  int device = 0;
};

namespace {

thread_local int32_t g_last_hip = 0;

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

using gclip::factor_ok;
using gclip::hip_fail;
using gclip::result_ptr_ok;
using gclip::threshold_ok;

// Device check of a hot call (argument values are checked before this).
gclip_status check_device(const gclip_list* list) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev != list->device) return GCLIP_EINVAL;
  return GCLIP_OK;
}

// The pieces of an AdamW list (see AdamPiece): for each tensor, vector pieces
// of up to kAdamPieceElems elements when all four addresses allow 4-element
// accesses, then the last (< 4) elements as a scalar piece; otherwise scalar
// pieces throughout.
void adamw_pieces(const uint64_t* p, const uint64_t* g, const uint64_t* m, const uint64_t* v, const int64_t* numels,
                  int32_t n, uint64_t es, std::vector<gclip::AdamPiece>& out) {
  for (int32_t t = 0; t < n; ++t) {
    const uint64_t ne = (uint64_t)numels[t];
    const bool vec = p[t] % 16 == 0 && m[t] % 16 == 0 && v[t] % 16 == 0 && g[t] % (4 * es) == 0;
    uint64_t e = 0;
    auto push = [&](uint64_t cnt, uint32_t isvec) {
      out.push_back(gclip::AdamPiece{p[t] + e * 4, g[t] + e * es, m[t] + e * 4, v[t] + e * 4, (uint32_t)cnt, isvec});
      e += cnt;
    };
    if (vec) {
      while (ne - e >= 4) {
        const uint64_t left = (ne - e) / 4 * 4;
        push(left < gclip::kAdamPieceElems ? left : gclip::kAdamPieceElems, 1u);
      }
    }
    while (e < ne) {
      const uint64_t left = ne - e;
      push(left < gclip::kAdamPieceElems ? left : gclip::kAdamPieceElems, 0u);
    }
  }
}

bool unit_interval(double b) { return std::isfinite(b) && b >= 0.0 && b < 1.0; }

}  // namespace

gclip_status gclip::hip_fail(hipError_t e) {
  g_last_hip = (int32_t)e;
  return GCLIP_EHIP;
}

extern "C" {

int32_t gclip_version(void) { return GCLIP_VERSION; }

int32_t gclip_last_hip_error(void) { return g_last_hip; }

const char* gclip_status_string(int32_t status) {
  switch (status) {
    case GCLIP_OK: return "ok";
    case GCLIP_EINVAL: return "invalid argument";
    case GCLIP_EDTYPE: return "unknown dtype";
    case GCLIP_ENOMEM: return "device allocation failed";
    case GCLIP_EHIP: return "HIP runtime error";
    case GCLIP_ENONFINITE: return "non-finite gradient element";
    case GCLIP_EDEVICE: return "device-side failure";
    case GCLIP_ERANGE: return "size out of range (a query buffer too small, or a list too large for a fixed scratch)";
    default: return "unknown status";
  }
}

gclip_status gclip_plan_query(const uint64_t* addrs, const int64_t* numels, int32_t n_tensors, int32_t dtype,
                              int32_t n_workers, int32_t worker_threads, gclip_plan_entry* out, int64_t cap,
                              int64_t* n_out) {
  if (!n_out || cap < 0 || (cap > 0 && !out)) return GCLIP_EINVAL;
  try {
    gclip::HostPlan p;
    const int rc = gclip::plan_build(addrs, numels, n_tensors, dtype, n_workers, worker_threads,
                                     gclip::resident_cap_vectors(), gclip::chunk_shape(), p, nullptr);
    if (rc != 0) return (gclip_status)rc;
    int64_t k = 0;
    auto emit = [&](int32_t w, int32_t t, int64_t b, int64_t c, int32_t kind) {
      if (k < cap) out[k] = gclip_plan_entry{w, t, b, c, kind, 0};
      ++k;
    };
    // the runs of the vector space [lo, hi) as (tensor, elements) pieces
    auto emit_vectors = [&](int32_t w, uint64_t lo, uint64_t hi, int32_t kind) {
      if (lo >= hi) return;
      int64_t s = (int64_t)(std::upper_bound(p.seg_vbegin.begin(), p.seg_vbegin.end() - 1, lo) -
                            p.seg_vbegin.begin()) - 1;
      for (; s < p.nseg(); ++s) {
        const uint64_t sb = p.seg_vbegin[(size_t)s], se = p.seg_vbegin[(size_t)s + 1];
        if (sb >= hi) break;
        const uint64_t a = lo > sb ? lo : sb, b = hi < se ? hi : se;
        if (a >= b) continue;
        emit(w, p.seg_tensor[(size_t)s], p.seg_elem0[(size_t)s] + (int64_t)(a - sb) * p.vec_elems,
             (int64_t)(b - a) * p.vec_elems, kind);
      }
    };
    for (int32_t w = 0; w < n_workers; ++w) {
      const uint64_t b = p.sb + (uint64_t)w * p.rb;
      emit_vectors(w, b < p.nvec() ? b : p.nvec(), b + p.rb < p.nvec() ? b + p.rb : p.nvec(), 0);
      const uint64_t cb = p.wk_scbegin[(size_t)w], ce = p.wk_scbegin[(size_t)w + 1];
      for (uint64_t i = cb; i < ce;) {
        uint64_t j = i + 1;
        while (j < ce && p.sc_tensor[j] == p.sc_tensor[i] && p.sc_elem[j] == p.sc_elem[j - 1] + 1) ++j;
        emit(w, p.sc_tensor[i], p.sc_elem[i], (int64_t)(j - i), 1);
        i = j;
      }
    }
    for (uint64_t c = 0; c < p.nchunk(); ++c) emit_vectors(-1, p.spl_vb[c], p.spl_vb[c + 1], 2);
    for (uint64_t c = 0; c < p.nsum(); ++c) {
      const uint64_t b = gclip::sum_chunk_begin(p.cvs_even, p.cvs_odd, c);
      const uint64_t e = gclip::sum_chunk_begin(p.cvs_even, p.cvs_odd, c + 1);
      emit_vectors(-1, b, e < p.sb ? e : p.sb, 3);
    }
    for (uint64_t c = 0; c < p.nchunk_streamed(); ++c) emit_vectors(-1, p.fus_vb[c], p.fus_vb[c + 1], 4);
    *n_out = k;
    return k > cap ? GCLIP_ERANGE : GCLIP_OK;
  } catch (const std::bad_alloc&) {
    return GCLIP_ENOMEM;
  }
}

gclip_status gclip_list_create(void* const* d_ptrs, const int64_t* numels, int32_t n_tensors, int32_t dtype,
                               gclip_list** out) {
  if (!out) return GCLIP_EINVAL;
  *out = nullptr;
  if (!gclip::dtype_valid(dtype)) return GCLIP_EDTYPE;
  if (n_tensors < 0 || (n_tensors > 0 && (!d_ptrs || !numels))) return GCLIP_EINVAL;
  static_assert(sizeof(uint64_t) == sizeof(void*), "64-bit addresses");
  gclip_list* L = nullptr;
  try {
    {
      // every argument error is reported before any HIP call
      const int rc = gclip::plan_validate(reinterpret_cast<const uint64_t*>(d_ptrs), numels, n_tensors, dtype,
                                          nullptr, nullptr, nullptr);
      if (rc != 0) return (gclip_status)rc;
    }
    L = new gclip_list();
    hipError_t e = hipGetDevice(&L->device);
    if (e != hipSuccess) {
      delete L;
      return hip_fail(e);
    }
    int ncu = 0, clk = 0;
    if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, L->device)) != hipSuccess ||
        (e = hipDeviceGetAttribute(&clk, hipDeviceAttributeWallClockRate, L->device)) != hipSuccess) {
      delete L;
      return hip_fail(e);
    }
    int bpc = 0;
    if ((e = gclip::fused_capacity(dtype, &bpc)) != hipSuccess) {
      delete L;
      return hip_fail(e);
    }
    L->fused_ok = bpc >= 1 && clk > 0;
    if ((e = gclip::tensor_fused_capacity(dtype, &bpc)) != hipSuccess) {
      delete L;
      return hip_fail(e);
    }
    L->tensor_fused_ok = L->fused_ok && bpc >= 1;
    L->path = L->fused_ok ? GCLIP_PATH_FUSED : GCLIP_PATH_SPLIT;
    L->clock_khz = clk > 0 ? (uint64_t)clk : 0;
    L->wait_ticks = (uint64_t)L->wait_us * L->clock_khz / 1000;

    const uint64_t* addrs = reinterpret_cast<const uint64_t*>(d_ptrs);
    std::string why;
    const int rc = gclip::plan_build_list(addrs, numels, n_tensors, dtype, ncu, gclip::worker_threads(),
                                          gclip::resident_cap_vectors(), gclip::chunk_shape(), L->plan, &why);
    if (rc != 0) {
      delete L;
      return (gclip_status)rc;
    }
    if (gclip::tensor_plan_build(L->plan, gclip::kTensorPieceVectors, L->tplan) != 0) {
      delete L;
      return GCLIP_EINVAL;
    }
    const gclip::HostPlan& P = L->plan;
    const size_t ntp = L->tplan.pieces.size(), ntf = L->tplan.first.size();
    const gclip::PlanLayout PL = gclip::plan_layout(P);
    size_t off = PL.bytes;
    auto take = [&](size_t bytes) {
      const size_t at = off;
      off = round_up(off + (bytes ? bytes : 8), 256);
      return at;
    };
    const size_t ntt = (size_t)P.n_tensors, nwb = (size_t)P.nworkers + 1;
    const size_t o_tpc = take(ntp * sizeof(gclip::TPiece)), o_tfi = take(ntf * 4), o_tpa = take(ntp * 8),
                 o_tsc = take(ntt * sizeof(gclip_tensor_result)), o_tsum = take(ntt * 8), o_tsy = take(128),
                 o_trb = take(nwb * 4), o_trs = take(nwb * 4), o_tcn = take(ntt * 4), o_tfa = take(ntt * 8);
    if ((e = hipMalloc(&L->blob, off)) != hipSuccess) {
      delete L;
      g_last_hip = (int32_t)e;
      return GCLIP_ENOMEM;
    }
    unsigned char* b = static_cast<unsigned char*>(L->blob);
    auto up = [&](size_t o, const void* src, size_t bytes) -> hipError_t {
      if (bytes == 0) return hipSuccess;
      return hipMemcpy(b + o, src, bytes, hipMemcpyHostToDevice);
    };
    std::vector<unsigned char> image(PL.header);
    gclip::plan_image(P, PL, image.data());
    // every tensor's factor slot empty (see the one-launch per-tensor clip)
    const std::vector<uint64_t> no_factor(ntt, gclip::kUndecided);
    if ((e = hipMemset(L->blob, 0, off)) != hipSuccess || (e = up(0, image.data(), PL.header)) ||
        (e = up(o_tpc, L->tplan.pieces.data(), ntp * sizeof(gclip::TPiece))) ||
        (e = up(o_tfi, L->tplan.first.data(), ntf * 4)) || (e = up(o_trb, L->tplan.run_b.data(), nwb * 4)) ||
        (e = up(o_trs, L->tplan.res_b.data(), nwb * 4)) || (e = up(o_tfa, no_factor.data(), ntt * 8)) ||
        (e = hipDeviceSynchronize()) != hipSuccess) {
      (void)hipFree(L->blob);
      delete L;
      return hip_fail(e);
    }
    L->dev = gclip::plan_view(P, PL, b);
    const gclip::DevPlan& D = L->dev;
    gclip::TensorPlan& T = L->tdev;
    T.pieces = reinterpret_cast<const gclip::TPiece*>(b + o_tpc);
    T.first = reinterpret_cast<const uint32_t*>(b + o_tfi);
    T.sc_addr = D.sc_addr;
    T.partials = reinterpret_cast<double*>(b + o_tpa);
    T.tsum = reinterpret_cast<double*>(b + o_tsum);
    T.tsync = reinterpret_cast<uint32_t*>(b + o_tsy);
    T.npieces = (uint32_t)ntp;
    T.ntensors = (int32_t)P.n_tensors;
    T.nlive = 0;
    for (size_t k = 0; k + 1 < ntf; ++k) T.nlive += L->tplan.first[k] < L->tplan.first[k + 1] ? 1u : 0u;
    T.nt_store = D.nt_store;
    T.run_b = reinterpret_cast<const uint32_t*>(b + o_trb);
    T.res_b = reinterpret_cast<const uint32_t*>(b + o_trs);
    T.ps = L->tplan.ps;
    T.tcount = reinterpret_cast<uint32_t*>(b + o_tcn);
    T.tfac = reinterpret_cast<double*>(b + o_tfa);
    L->tscratch = reinterpret_cast<gclip_tensor_result*>(b + o_tsc);
    L->addrs.assign(addrs, addrs + n_tensors);
    L->numels.assign(numels, numels + n_tensors);
    *out = L;
    return GCLIP_OK;
  } catch (const std::bad_alloc&) {
    if (L) {
      if (L->blob) (void)hipFree(L->blob);
      delete L;
    }
    return GCLIP_ENOMEM;
  }
}

gclip_status gclip_list_destroy(gclip_list* list) {
  if (!list) return GCLIP_OK;
  hipError_t e = hipSuccess;
  if (list->blob) e = hipFree(list->blob);
  delete list;
  return e == hipSuccess ? GCLIP_OK : hip_fail(e);
}

gclip_status gclip_list_info(const gclip_list* list, gclip_list_info_t* out) {
  if (!list || !out) return GCLIP_EINVAL;
  const gclip::HostPlan& P = list->plan;
  std::memset(out, 0, sizeof(*out));
  out->n_tensors = P.n_tensors;
  out->n_elements = P.n_elements;
  out->n_bytes = P.n_bytes;
  out->n_segments = P.nseg();
  out->n_vectors = (int64_t)P.nvec();
  out->n_scalars = (int64_t)P.nsc();
  out->n_workers = P.nworkers;
  out->worker_threads = P.threads;
  out->dtype = P.dtype;
  out->path = list->path;
  // the fused kernel keeps every block on chip: the vectors from sb on
  const int64_t res = list->path == GCLIP_PATH_FUSED ? (int64_t)(P.nvec() - P.sb) : 0;
  out->resident_vectors = res;
  return GCLIP_OK;
}

gclip_status gclip_list_set_path(gclip_list* list, int32_t path) {
  if (!list) return GCLIP_EINVAL;
  switch (path) {
    case GCLIP_PATH_AUTO: list->path = list->fused_ok ? GCLIP_PATH_FUSED : GCLIP_PATH_SPLIT; return GCLIP_OK;
    case GCLIP_PATH_FUSED:
      if (!list->fused_ok) return GCLIP_EINVAL;
      list->path = GCLIP_PATH_FUSED;
      return GCLIP_OK;
    case GCLIP_PATH_SPLIT: list->path = GCLIP_PATH_SPLIT; return GCLIP_OK;
    default: return GCLIP_EINVAL;
  }
}

gclip_status gclip_list_set_wait(gclip_list* list, int64_t microseconds) {
  if (!list || microseconds < 0 || microseconds > kMaxWaitUs) return GCLIP_EINVAL;
  list->wait_us = microseconds;
  list->wait_ticks = (uint64_t)microseconds * list->clock_khz / 1000;
  return GCLIP_OK;
}

gclip_status gclip_norm(gclip_list* list, double avg_factor, gclip_result* d_result, void* stream) {
  if (!list || !result_ptr_ok(d_result) || !factor_ok(avg_factor)) return GCLIP_EINVAL;
  gclip_status st = check_device(list);
  if (st != GCLIP_OK) return st;
  const hipError_t e =
      gclip::launch_norm(list->dev, list->plan.dtype, gclip::AvgSrc{avg_factor, nullptr}, d_result,
                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GCLIP_OK : hip_fail(e);
}

gclip_status gclip_scale(gclip_list* list, double max_norm, double avg_factor, int32_t error_if_nonfinite,
                         gclip_result* d_result, void* stream) {
  if (!list || !result_ptr_ok(d_result) || !threshold_ok(max_norm) || !factor_ok(avg_factor)) return GCLIP_EINVAL;
  gclip_status st = check_device(list);
  if (st != GCLIP_OK) return st;
  const hipError_t e =
      gclip::launch_scale(list->dev, list->plan.dtype, max_norm, gclip::AvgSrc{avg_factor, nullptr},
                          error_if_nonfinite ? 1 : 0, d_result, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GCLIP_OK : hip_fail(e);
}

namespace {
// The path's kernels on an already validated list: fused, or norm then scale.
// A loss-scale update (amp.st != nullptr) is taken by the fused kernel's
// deciding workgroup, or by a kernel of its own after the split path's two.
hipError_t launch_clip(gclip_list* list, double max_norm, gclip::AvgSrc avg, int err, gclip_result* d_result,
                       hipStream_t s, gclip::AmpUpdate amp = gclip::AmpUpdate{nullptr, 0.0, 0.0, 0}) {
  if (list->path == GCLIP_PATH_FUSED) {
    return gclip::launch_fused(list->dev, list->plan.dtype, max_norm, avg, err, d_result, list->wait_ticks, amp,
                               s);
  }
  hipError_t e = gclip::launch_norm(list->dev, list->plan.dtype, avg, d_result, s);
  if (e == hipSuccess) e = gclip::launch_scale(list->dev, list->plan.dtype, max_norm, avg, err, d_result, s);
  if (e == hipSuccess && amp.st) e = gclip::launch_amp_update(d_result, amp.st, amp.growth, amp.backoff, amp.interval, s);
  return e;
}

bool tensor_out_ok(const gclip_list* list, const gclip_tensor_result* t) {
  if (list->plan.n_tensors == 0) return true;
  return t && reinterpret_cast<uintptr_t>(t) % 8 == 0;
}
bool amp_state_ptr_ok(const gclip_amp_state* a) { return a && reinterpret_cast<uintptr_t>(a) % 4 == 0; }
bool amp_params_ok(const gclip_amp_params* a) {
  return a && std::isfinite(a->growth_factor) && a->growth_factor >= 1.0 && std::isfinite(a->backoff_factor) &&
         a->backoff_factor > 0.0 && a->backoff_factor <= 1.0 && a->growth_interval >= 1;
}
}  // namespace

gclip_status gclip_clip_(gclip_list* list, double max_norm, double avg_factor, int32_t error_if_nonfinite,
                         gclip_result* d_result, void* stream) {
  if (!list || !result_ptr_ok(d_result) || !threshold_ok(max_norm) || !factor_ok(avg_factor)) return GCLIP_EINVAL;
  gclip_status st = check_device(list);
  if (st != GCLIP_OK) return st;
  const hipError_t e = launch_clip(list, max_norm, gclip::AvgSrc{avg_factor, nullptr}, error_if_nonfinite ? 1 : 0,
                                   d_result, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GCLIP_OK : hip_fail(e);
}

gclip_status gclip_tensor_norms(gclip_list* list, double avg_factor, gclip_tensor_result* d_tensors,
                                gclip_result* d_result, void* stream) {
  if (!list || !result_ptr_ok(d_result) || !factor_ok(avg_factor) || !tensor_out_ok(list, d_tensors))
    return GCLIP_EINVAL;
  gclip_status st = check_device(list);
  if (st != GCLIP_OK) return st;
  const hipError_t e = gclip::launch_tensor_norms(list->tdev, list->plan.dtype, gclip::AvgSrc{avg_factor, nullptr},
                                                  d_tensors, d_result, gather_wait_ticks(list), list->clock_khz > 0,
                                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GCLIP_OK : hip_fail(e);
}

gclip_status gclip_clip_per_tensor_(gclip_list* list, double max_norm, double avg_factor,
                                    int32_t error_if_nonfinite, gclip_tensor_result* d_tensors,
                                    gclip_result* d_result, void* stream) {
  if (!list || !result_ptr_ok(d_result) || !threshold_ok(max_norm) || !factor_ok(avg_factor) ||
      !tensor_out_ok(list, d_tensors))
    return GCLIP_EINVAL;
  gclip_status st = check_device(list);
  if (st != GCLIP_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const gclip::AvgSrc avg{avg_factor, nullptr};
  hipError_t e;
  if (list->path == GCLIP_PATH_FUSED && list->tensor_fused_ok) {
    e = gclip::launch_tensor_clip_fused(list->dev, list->tdev, list->plan.dtype, avg, max_norm,
                                        error_if_nonfinite ? 1 : 0, d_tensors, d_result, list->wait_ticks, s);
  } else if (!error_if_nonfinite && list->clock_khz > 0) {
    e = gclip::launch_tensor_clip(list->tdev, list->plan.dtype, avg, max_norm, d_tensors, d_result,
                                  gather_wait_ticks(list), s);
  } else {
    e = gclip::launch_tensor_decisions(list->tdev, list->plan.dtype, avg, max_norm, error_if_nonfinite ? 1 : 0,
                                       d_tensors, d_result, gather_wait_ticks(list), list->clock_khz > 0, s);
    if (e == hipSuccess) e = gclip::launch_tensor_scale(list->tdev, list->plan.dtype, d_tensors, d_result, s);
  }
  return e == hipSuccess ? GCLIP_OK : hip_fail(e);
}

gclip_status gclip_set_gather_wait(int64_t microseconds) {
  if (microseconds > kMaxWaitUs) return GCLIP_EINVAL;
  g_gather_wait_us.store(microseconds < 0 ? kTensorGatherWaitUs : microseconds, std::memory_order_relaxed);
  return GCLIP_OK;
}

gclip_status gclip_contrib_create(const gclip_list* list, void* const* d_contrib, gclip_contrib** out) {
  if (!out) return GCLIP_EINVAL;
  *out = nullptr;
  if (!list) return GCLIP_EINVAL;
  const size_t n = list->addrs.size();
  if (n > 0 && !d_contrib) return GCLIP_EINVAL;
  const uint64_t es = (uint64_t)gclip::dtype_bytes(list->plan.dtype);
  try {
    std::vector<uint64_t> delta(n, 0);
    std::vector<std::pair<uint64_t, uint64_t>> ranges;
    for (size_t t = 0; t < n; ++t) {
      const uint64_t a = list->addrs[t], g = reinterpret_cast<uint64_t>(d_contrib[t]);
      const uint64_t bytes = (uint64_t)list->numels[t] * es;
      if (bytes == 0) continue;
      if (g == 0 || g % es != 0 || (g - a) % 16 != 0 || g + bytes < g) return GCLIP_EINVAL;
      delta[t] = g - a;
      ranges.emplace_back(a, a + bytes);
      ranges.emplace_back(g, g + bytes);
    }
    std::sort(ranges.begin(), ranges.end());
    for (size_t i = 1; i < ranges.size(); ++i)
      if (ranges[i].first < ranges[i - 1].second) return GCLIP_EINVAL;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev != list->device) return GCLIP_EINVAL;
    // the same offsets per segment and per single element, for the fused kernel
    const gclip::HostPlan& P = list->plan;
    const size_t nseg = (size_t)P.nseg(), nsc = (size_t)P.nsc();
    for (size_t k = 0; k < nseg; ++k) delta.push_back(delta[(size_t)P.seg_tensor[k]]);
    for (size_t k = 0; k < nsc; ++k) delta.push_back(delta[(size_t)P.sc_tensor[k]]);
    gclip_contrib* C = new gclip_contrib();
    C->list = list;
    C->device = dev;
    if ((e = hipMalloc(&C->delta, (delta.empty() ? 1 : delta.size()) * 8)) != hipSuccess) {
      delete C;
      g_last_hip = (int32_t)e;
      return GCLIP_ENOMEM;
    }
    if (!delta.empty() &&
        (e = hipMemcpy(C->delta, delta.data(), delta.size() * 8, hipMemcpyHostToDevice)) != hipSuccess) {
      (void)hipFree(C->delta);
      delete C;
      return hip_fail(e);
    }
    C->acc.seg_gdelta = C->delta + n;
    C->acc.sc_gdelta = C->delta + n + nseg;
    *out = C;
    return GCLIP_OK;
  } catch (const std::bad_alloc&) {
    return GCLIP_ENOMEM;
  }
}

gclip_status gclip_contrib_destroy(gclip_contrib* contrib) {
  if (!contrib) return GCLIP_OK;
  const hipError_t e = contrib->delta ? hipFree(contrib->delta) : hipSuccess;
  delete contrib;
  return e == hipSuccess ? GCLIP_OK : hip_fail(e);
}

gclip_status gclip_accumulate_norm(gclip_list* list, const gclip_contrib* contrib, double avg_factor,
                                   gclip_tensor_result* d_tensors, gclip_result* d_result, void* stream) {
  if (!list || !contrib || contrib->list != list || !result_ptr_ok(d_result) || !factor_ok(avg_factor) ||
      (d_tensors && !tensor_out_ok(list, d_tensors)))
    return GCLIP_EINVAL;
  gclip_status st = check_device(list);
  if (st != GCLIP_OK) return st;
  const hipError_t e = gclip::launch_accumulate_norm(list->tdev, list->plan.dtype, contrib->delta,
                                                     gclip::AvgSrc{avg_factor, nullptr},
                                                     d_tensors ? d_tensors : list->tscratch, d_result,
                                                     gather_wait_ticks(list), list->clock_khz > 0,
                                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GCLIP_OK : hip_fail(e);
}

gclip_status gclip_accumulate_clip_(gclip_list* list, const gclip_contrib* contrib, double max_norm,
                                    double avg_factor, int32_t error_if_nonfinite, gclip_result* d_result,
                                    void* stream) {
  if (!list || !contrib || contrib->list != list || !result_ptr_ok(d_result) || !threshold_ok(max_norm) ||
      !factor_ok(avg_factor))
    return GCLIP_EINVAL;
  gclip_status st = check_device(list);
  if (st != GCLIP_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const gclip::AvgSrc avg{avg_factor, nullptr};
  const int err = error_if_nonfinite ? 1 : 0;
  hipError_t e;
  if (list->path == GCLIP_PATH_FUSED) {
    e = gclip::launch_accum_fused(list->dev, contrib->acc, list->plan.dtype, max_norm, avg, err, d_result,
                                  list->wait_ticks, s);
  } else {
    e = gclip::launch_accumulate_norm(list->tdev, list->plan.dtype, contrib->delta, avg, list->tscratch, d_result,
                                      gather_wait_ticks(list), list->clock_khz > 0, s);
    if (e == hipSuccess) e = gclip::launch_scale(list->dev, list->plan.dtype, max_norm, avg, err, d_result, s);
  }
  return e == hipSuccess ? GCLIP_OK : hip_fail(e);
}

gclip_status gclip_norm_amp(gclip_list* list, double n_microbatches, const gclip_amp_state* d_amp,
                            gclip_result* d_result, void* stream) {
  if (!list || !result_ptr_ok(d_result) || !factor_ok(n_microbatches) || !amp_state_ptr_ok(d_amp))
    return GCLIP_EINVAL;
  gclip_status st = check_device(list);
  if (st != GCLIP_OK) return st;
  const hipError_t e = gclip::launch_norm(list->dev, list->plan.dtype, gclip::AvgSrc{n_microbatches, &d_amp->scale},
                                          d_result, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GCLIP_OK : hip_fail(e);
}

gclip_status gclip_clip_amp_(gclip_list* list, double max_norm, double n_microbatches, gclip_amp_state* d_amp,
                             const gclip_amp_params* amp, gclip_result* d_result, void* stream) {
  if (!list || !result_ptr_ok(d_result) || !threshold_ok(max_norm) || !factor_ok(n_microbatches) ||
      !amp_state_ptr_ok(d_amp) || !amp_params_ok(amp))
    return GCLIP_EINVAL;
  gclip_status st = check_device(list);
  if (st != GCLIP_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = launch_clip(list, max_norm, gclip::AvgSrc{n_microbatches, &d_amp->scale}, 1, d_result, s,
                                   gclip::AmpUpdate{d_amp, amp->growth_factor, amp->backoff_factor,
                                                    amp->growth_interval});
  return e == hipSuccess ? GCLIP_OK : hip_fail(e);
}

gclip_status gclip_adamw_create(void* const* d_params, void* const* d_grads, void* const* d_exp_avg,
                                void* const* d_exp_avg_sq, const int64_t* numels, int32_t n_tensors,
                                int32_t grad_dtype, gclip_adamw** out) {
  if (!out) return GCLIP_EINVAL;
  *out = nullptr;
  if (!gclip::dtype_valid(grad_dtype)) return GCLIP_EDTYPE;
  if (n_tensors < 0 || (n_tensors > 0 && (!d_params || !d_grads || !d_exp_avg || !d_exp_avg_sq || !numels)))
    return GCLIP_EINVAL;
  const uint64_t es = (uint64_t)gclip::dtype_bytes(grad_dtype);
  const uint64_t* P = reinterpret_cast<const uint64_t*>(d_params);
  const uint64_t* G = reinterpret_cast<const uint64_t*>(d_grads);
  const uint64_t* M = reinterpret_cast<const uint64_t*>(d_exp_avg);
  const uint64_t* V = reinterpret_cast<const uint64_t*>(d_exp_avg_sq);
  gclip_adamw* A = nullptr;
  try {
    // every argument error is reported before any HIP call
    std::vector<std::pair<uint64_t, uint64_t>> ranges;
    for (int32_t t = 0; t < n_tensors; ++t) {
      if (numels[t] < 0) return GCLIP_EINVAL;
      if (numels[t] == 0) continue;
      if ((uint64_t)numels[t] > ((uint64_t)1 << 56)) return GCLIP_EINVAL;
      const uint64_t a[4] = {P[t], G[t], M[t], V[t]};
      const uint64_t size[4] = {4, es, 4, 4};
      for (int k = 0; k < 4; ++k) {
        if (a[k] == 0 || a[k] % size[k] != 0) return GCLIP_EINVAL;
        const uint64_t bytes = (uint64_t)numels[t] * size[k];
        if (a[k] + bytes < a[k]) return GCLIP_EINVAL;
        ranges.emplace_back(a[k], a[k] + bytes);
      }
    }
    std::sort(ranges.begin(), ranges.end());
    for (size_t i = 1; i < ranges.size(); ++i)
      if (ranges[i].first < ranges[i - 1].second) return GCLIP_EINVAL;
    std::vector<gclip::AdamPiece> pieces;
    adamw_pieces(P, G, M, V, numels, n_tensors, es, pieces);
    if (pieces.size() > 0x7fffffffull) return GCLIP_EINVAL;
    A = new gclip_adamw();
    A->dtype = grad_dtype;
    A->npieces = (uint32_t)pieces.size();
    hipError_t e = hipGetDevice(&A->device);
    if (e != hipSuccess) {
      delete A;
      return hip_fail(e);
    }
    const size_t bytes = pieces.size() * sizeof(gclip::AdamPiece);
    if (bytes > 0) {
      if ((e = hipMalloc(&A->pieces, bytes)) != hipSuccess) {
        delete A;
        g_last_hip = (int32_t)e;
        return GCLIP_ENOMEM;
      }
      if ((e = hipMemcpy(A->pieces, pieces.data(), bytes, hipMemcpyHostToDevice)) != hipSuccess) {
        (void)hipFree(A->pieces);
        delete A;
        return hip_fail(e);
      }
    }
    *out = A;
    return GCLIP_OK;
  } catch (const std::bad_alloc&) {
    if (A) {
      if (A->pieces) (void)hipFree(A->pieces);
      delete A;
    }
    return GCLIP_ENOMEM;
  }
}

gclip_status gclip_adamw_destroy(gclip_adamw* opt) {
  if (!opt) return GCLIP_OK;
  hipError_t e = hipSuccess;
  if (opt->pieces) e = hipFree(opt->pieces);
  delete opt;
  return e == hipSuccess ? GCLIP_OK : hip_fail(e);
}

namespace {
gclip_status adamw_step(gclip_adamw* opt, const gclip_adamw_hparams* hp, double max_norm, gclip::AvgSrc avg,
                        int32_t error_if_nonfinite, gclip_result* d_result, const gclip_amp_state* amp_state,
                        const gclip_amp_params* amp, void* stream) {
  if (!opt || !hp || !result_ptr_ok(d_result) || !threshold_ok(max_norm) || !factor_ok(avg.a)) return GCLIP_EINVAL;
  if (!std::isfinite(hp->lr) || hp->lr < 0.0 || !unit_interval(hp->beta1) || !unit_interval(hp->beta2) ||
      !std::isfinite(hp->eps) || hp->eps <= 0.0 || !std::isfinite(hp->weight_decay) || hp->weight_decay < 0.0 ||
      hp->step < 1)
    return GCLIP_EINVAL;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev != opt->device) return GCLIP_EINVAL;
  const double bc1 = 1.0 - std::pow(hp->beta1, (double)hp->step);
  const double bc2 = 1.0 - std::pow(hp->beta2, (double)hp->step);
  gclip::AdamHp h;
  h.step_size = (float)(hp->lr / bc1);
  h.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
  h.eps = (float)hp->eps;
  h.decay = (float)(1.0 - hp->lr * hp->weight_decay);
  h.b1 = (float)hp->beta1;
  h.omb1 = (float)(1.0 - hp->beta1);
  h.b2 = (float)hp->beta2;
  h.omb2 = (float)(1.0 - hp->beta2);
  gclip::AdamPlan plan{opt->pieces, opt->npieces};
  const hipStream_t s = static_cast<hipStream_t>(stream);
  e = gclip::launch_adamw(plan, opt->dtype, h, max_norm, avg, error_if_nonfinite ? 1 : 0, d_result, s);
  if (e == hipSuccess && amp)
    e = gclip::launch_amp_update(d_result, const_cast<gclip_amp_state*>(amp_state), amp->growth_factor,
                                 amp->backoff_factor, amp->growth_interval, s);
  return e == hipSuccess ? GCLIP_OK : hip_fail(e);
}
}  // namespace

gclip_status gclip_adamw_step(gclip_adamw* opt, const gclip_adamw_hparams* hp, double max_norm, double avg_factor,
                              int32_t error_if_nonfinite, gclip_result* d_result, void* stream) {
  return adamw_step(opt, hp, max_norm, gclip::AvgSrc{avg_factor, nullptr}, error_if_nonfinite, d_result, nullptr,
                    nullptr, stream);
}

gclip_status gclip_adamw_step_amp(gclip_adamw* opt, const gclip_adamw_hparams* hp, double max_norm,
                                  double n_microbatches, gclip_amp_state* d_amp, const gclip_amp_params* amp,
                                  gclip_result* d_result, void* stream) {
  if (!amp_state_ptr_ok(d_amp) || !amp_params_ok(amp)) return GCLIP_EINVAL;
  return adamw_step(opt, hp, max_norm, gclip::AvgSrc{n_microbatches, &d_amp->scale}, 1, d_result, d_amp, amp,
                    stream);
}

gclip_status gclip_result_read(const gclip_result* d_result, void* stream, gclip_result* h_out,
                               int32_t error_if_nonfinite) {
  if (!d_result || !h_out) return GCLIP_EINVAL;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(h_out, d_result, sizeof(gclip_result), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e);
  if (h_out->status != 0) return GCLIP_EDEVICE;
  if (h_out->nonfinite && error_if_nonfinite) return GCLIP_ENONFINITE;
  return GCLIP_OK;
}

}  // extern "C"
