// gclip_trace.cpp -- host replay of the kernels' address walk (no GPU).
//
// For a list and a worker count, replays the loops of gclip_kernels.hip with
// the same cursor code (gclip_cursor.hpp) and reports every address a lane
// would touch, so that a CPU test can check the walk before any kernel runs:
// each pass visits every vector and every single element exactly once, and
// nothing outside the tensors.
#include <cstdint>
#include <new>
#include <string>
#include <vector>

#include "../../include/gclip.h"
#include "gclip_cursor.hpp"
#include "gclip_plan.hpp"

namespace {

using namespace gclip;

constexpr uint64_t kElementTag = 1ull << 63;  // marks the address of a single element

struct Recorder {
  uint64_t* addr;
  int32_t* worker;
  int64_t cap, n = 0;
  bool uniform_ok = true;
  void put(int32_t w, uint64_t a) {
    if (n < cap) {
      addr[n] = a;
      worker[n] = w;
    }
    ++n;
  }
};

// One group of up to kUnroll steps for all kThreads lanes: every lane starts
// from the same cursor and, the cursor work being uniform, every lane must
// end on the same cursor.
void replay_group(const DevPlan& p, Cursor& cur, uint64_t vb, uint64_t ve, uint64_t j, uint64_t j1, int32_t w,
                  Recorder* rec) {
  uint64_t base = 0;
  const int kind = group_kind(cur, vb, ve, j, j1, base);
  if (kind != kGroupCross) {
    for (uint32_t t = 0; t < (uint32_t)kThreads; ++t)
      for (int u = 0; u < kUnroll; ++u) {
        const bool ok = kind == kGroupFull || tail_ok(vb, ve, j, j1, u, t);
        if (kind == kGroupFull && !tail_ok(vb, ve, j, j1, u, t) && rec) rec->uniform_ok = false;
        if (ok && rec) rec->put(w, base + ((uint64_t)u * kThreads + t) * kVecBytes);
      }
    return;
  }
  Cursor end{};
  for (uint32_t t = 0; t < (uint32_t)kThreads; ++t) {
    Cursor c = cur;
    uint64_t a[kUnroll];
    bool ok[kUnroll];
    cross_addrs(p, c, vb, ve, j, j1, t, a, ok);
    if (rec)
      for (int u = 0; u < kUnroll; ++u)
        if (ok[u]) rec->put(w, a[u]);
    if (t == 0) {
      end = c;
    } else if (c.s != end.s || c.beg != end.beg || c.end != end.end || c.addr != end.addr) {
      if (rec) rec->uniform_ok = false;
    }
  }
  cur = end;
}

void replay_groups(const DevPlan& p, Cursor& cur, uint64_t vb, uint64_t ve, uint64_t j0, uint64_t j1, int32_t w,
                   Recorder* rec) {
  for (uint64_t j = j0; j < j1; j += kUnroll) replay_group(p, cur, vb, ve, j, j1, w, rec);
}

}  // namespace

extern "C" gclip_status gclip_plan_trace(const uint64_t* addrs, const int64_t* numels, int32_t n_tensors,
                                         int32_t dtype, int32_t n_workers, int32_t mode, uint64_t* out_addr,
                                         int32_t* out_worker, int64_t cap, int64_t* n_out) {
  if (!n_out || cap < 0 || (cap > 0 && (!out_addr || !out_worker)) || mode < 0 || mode > 3)
    return GCLIP_EINVAL;
  try {
    HostPlan hp;
    const int rc = plan_build(addrs, numels, n_tensors, dtype, n_workers, kThreads, hp, nullptr);
    if (rc != 0) return (gclip_status)rc;
    DevPlan p{};
    p.seg_vbegin = hp.seg_vbegin.data();
    p.seg_addr = hp.seg_addr.data();
    p.wk_vbegin = hp.wk_vbegin.data();
    p.wk_seg = hp.wk_seg.data();
    p.wk_scbegin = hp.wk_scbegin.data();
    p.sc_addr = hp.sc_addr.data();
    p.nworkers = hp.nworkers;
    p.nseg = (int32_t)hp.nseg();
    Recorder rec{out_addr, out_worker, cap};
    for (int32_t w = 0; w < p.nworkers; ++w) {
      const uint64_t vb = p.wk_vbegin[w], ve = p.wk_vbegin[w + 1];
      if (vb < ve) {
        Cursor cur0;
        cursor_load(p, cur0, p.wk_seg[w]);
        if (mode <= 1) {  // k_grad_norm_partial / k_grad_scale
          Cursor cur = cur0;
          replay_groups(p, cur, vb, ve, 0, (ve - vb + kThreads - 1) / kThreads, w, &rec);
        } else {  // k_grad_clip_fused, phase 1 (mode 2) or phase 2 (mode 3)
          const FusedSplit fs = fused_split(vb, ve);
          Recorder* r1 = mode == 2 ? &rec : nullptr;
          Recorder* r2 = mode == 3 ? &rec : nullptr;
          const uint64_t jr = fs.js + fs.nreg, jl = jr + fs.nlds;
          Cursor cur = cur0;
          replay_groups(p, cur, vb, ve, 0, fs.js, w, r1);
          Cursor cur_reg = cur;
          cursor_seek(p, cur_reg, vb + fs.js * kThreads);
          cur = cur_reg;
          for (int g = 0; g < kRegSteps / kUnroll; ++g)
            if ((uint32_t)(g * kUnroll) < fs.nreg) replay_group(p, cur, vb, ve, fs.js + g * kUnroll, jr, w, r1);
          Cursor cur_lds = cur;
          cursor_seek(p, cur_lds, vb + jr * kThreads);
          cur = cur_lds;
          replay_groups(p, cur, vb, ve, jr, jl, w, r1);
          if (mode == 3) {
            cur = cur_reg;
            for (int g = 0; g < kRegSteps / kUnroll; ++g)
              if ((uint32_t)(g * kUnroll) < fs.nreg) replay_group(p, cur, vb, ve, fs.js + g * kUnroll, jr, w, r2);
            cur = cur_lds;
            replay_groups(p, cur, vb, ve, jr, jl, w, r2);
            cur = cur0;
            replay_groups(p, cur, vb, ve, 0, fs.js, w, r2);
          }
        }
      }
      for (uint64_t i = p.wk_scbegin[w]; i < p.wk_scbegin[w + 1]; ++i) rec.put(w, p.sc_addr[i] | kElementTag);
    }
    *n_out = rec.n;
    if (!rec.uniform_ok) return GCLIP_EINVAL;
    return rec.n > cap ? GCLIP_ERANGE : GCLIP_OK;
  } catch (const std::bad_alloc&) {
    return GCLIP_ENOMEM;
  }
}
