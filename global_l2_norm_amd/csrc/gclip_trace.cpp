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

namespace gclip {
ChunkShape chunk_shape();
}

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

// The contribution's addresses for one group (load_group_contrib's walk).
void replay_contrib_group(const DevPlan& p, const AccSrc& A, Cursor& cur, uint64_t vb, uint64_t ve, uint64_t j,
                          uint64_t j1, int32_t w, Recorder* rec) {
  uint64_t base = 0;
  const int kind = group_kind(cur, vb, ve, j, j1, base);
  if (kind != kGroupCross) {
    const uint64_t d = A.seg_gdelta[cur.s];
    for (uint32_t t = 0; t < (uint32_t)kThreads; ++t)
      for (int u = 0; u < kUnroll; ++u)
        if (kind == kGroupFull || tail_ok(vb, ve, j, j1, u, t))
          rec->put(w, base + d + ((uint64_t)u * kThreads + t) * kVecBytes);
    return;
  }
  Cursor end{};
  const uint64_t b0 = vb + j * kThreads;
  for (uint32_t t = 0; t < (uint32_t)kThreads; ++t) {
    Cursor c = cur;
    uint64_t d = A.seg_gdelta[c.s];
    for (int u = 0; u < kUnroll; ++u) {
      if (j + u >= j1) continue;
      const uint64_t b = b0 + (uint64_t)u * kThreads, v = b + t;
      const uint64_t a = step_addr_delta(p, A.seg_gdelta, c, d, b, ve, v);
      if (v < ve) rec->put(w, a);
    }
    if (t == 0) {
      end = c;
    } else if (c.s != end.s || c.beg != end.beg || c.end != end.end || c.addr != end.addr) {
      rec->uniform_ok = false;
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
  if (!n_out || cap < 0 || (cap > 0 && (!out_addr || !out_worker)) || mode < 0 || mode > 6)
    return GCLIP_EINVAL;
  try {
    HostPlan hp;
    const int rc =
        plan_build(addrs, numels, n_tensors, dtype, n_workers, kThreads, kResidentCap, chunk_shape(), hp, nullptr);
    if (rc != 0) return (gclip_status)rc;
    DevPlan p{};
    p.seg_vbegin = hp.seg_vbegin.data();
    p.seg_addr = hp.seg_addr.data();
    p.blk_seg = hp.blk_seg.data();
    p.spl_vb = hp.spl_vb.data();
    p.spl_seg = hp.spl_seg.data();
    p.fus_vb = hp.fus_vb.data();
    p.fus_seg = hp.fus_seg.data();
    p.sum_seg = hp.sum_seg.data();
    p.wk_scbegin = hp.wk_scbegin.data();
    p.sc_addr = hp.sc_addr.data();
    p.nvec = hp.nvec();
    p.rb = hp.rb;
    p.sb = hp.sb;
    p.nchunk = (uint32_t)hp.nchunk();
    p.nchs = (uint32_t)hp.nchunk_streamed();
    p.nsum = (uint32_t)hp.nsum();
    p.cvs = hp.cvs_even;
    p.sum_groups = hp.sum_groups;
    p.nworkers = hp.nworkers;
    p.nseg = (int32_t)hp.nseg();
    Recorder rec{out_addr, out_worker, cap};
    if (mode == 5 || mode == 6) {
      // a contribution at addrs[t] + D_t, D_t = 2^44 + t 2^34 (aligned like
      // the list's tensor); the per-segment and per-element offsets as the
      // library builds them
      std::vector<uint64_t> dseg((size_t)hp.nseg()), dsc((size_t)hp.nsc());
      auto off = [](int32_t t) { return (1ull << 44) + ((uint64_t)t << 34); };
      for (size_t k = 0; k < dseg.size(); ++k) dseg[k] = off(hp.seg_tensor[k]);
      for (size_t k = 0; k < dsc.size(); ++k) dsc[k] = off(hp.sc_tensor[k]);
      const AccSrc A{dseg.data(), dsc.data()};
      if (mode == 5) {  // k_accum_clip_fused, first pass: sum chunks, then each block and its single elements
        for (uint32_t c = 0; c < p.nsum; ++c) {
          const Range r = p.sum_groups ? sum_chunk_range<true>(p, c) : sum_chunk_range<false>(p, c);
          Cursor cg;
          cursor_load(p, cg, r.seg);
          for (uint64_t j = 0; j < range_steps(r); j += kUnroll)
            replay_contrib_group(p, A, cg, r.b, r.e, j, range_steps(r), -1, &rec);
        }
      }
      for (int32_t w = 0; w < p.nworkers; ++w) {
        const Range r = block_range(p, w);
        if (r.b < r.e) {
          Cursor c0;
          cursor_load(p, c0, r.seg);
          const BlockSplit bs = block_split(r);
          if (mode == 5) {  // LDS steps, then register steps, each from the block's start
            Cursor cg = c0;
            for (uint32_t k0 = 0; k0 < bs.nlds; k0 += kUnroll)
              replay_contrib_group(p, A, cg, r.b, r.e, bs.nreg + k0, bs.nsteps, w, &rec);
            cg = c0;
            for (int g = 0; g < kRegSteps / kUnroll; ++g)
              if ((uint32_t)(g * kUnroll) < bs.nreg) replay_contrib_group(p, A, cg, r.b, r.e, g * kUnroll, bs.nreg, w, &rec);
          } else {  // a block handed back: the whole block in one walk
            Cursor cg = c0;
            for (uint64_t j = 0; j < bs.nsteps; j += kUnroll)
              replay_contrib_group(p, A, cg, r.b, r.e, j, bs.nsteps, w, &rec);
          }
        }
        if (mode == 5)
          for (uint64_t i = p.wk_scbegin[w]; i < p.wk_scbegin[w + 1]; ++i)
            rec.put(w, (p.sc_addr[i] + A.sc_gdelta[i]) | kElementTag);
      }
      *n_out = rec.n;
      if (!rec.uniform_ok) return GCLIP_EINVAL;
      return rec.n > cap ? GCLIP_ERANGE : GCLIP_OK;
    }
    if (mode == 4) {  // k_tensor_partial and k_tensor_scale: one workgroup per piece
      TensorHostPlan tp;
      if (tensor_plan_build(hp, kTensorPieceVectors, tp) != 0) return GCLIP_EINVAL;
      for (const TPiece& pc : tp.pieces) {
        for (uint32_t j = 0; j < pc.nvec; j += kPieceGroup)
          for (uint32_t t = 0; t < (uint32_t)kThreads; ++t)
            for (int u = 0; u < kUnroll; ++u) {
              const uint32_t i = piece_index(j, u, t);
              if (i < pc.nvec) rec.put((int32_t)pc.tensor, pc.addr + (uint64_t)i * kVecBytes);
            }
        for (uint32_t i = 0; i < pc.sc_count; ++i)
          rec.put((int32_t)pc.tensor, hp.sc_addr[pc.sc_begin + i] | kElementTag);
      }
      for (int32_t t = 0; t < n_tensors; ++t)  // pieces in tensor order, as the final sums assume
        if (tp.first[(size_t)t] > tp.first[(size_t)t + 1]) return GCLIP_EINVAL;
      for (uint32_t k = 0; k < (uint32_t)tp.pieces.size(); ++k) {
        const uint32_t t = tp.pieces[k].tensor;
        if (k < tp.first[t] || k >= tp.first[t + 1]) return GCLIP_EINVAL;
      }
      *n_out = rec.n;
      return rec.n > cap ? GCLIP_ERANGE : GCLIP_OK;
    }
    // claimed chunks of a table: any worker, so reported as worker -1
    auto replay_chunks = [&](const uint64_t* vb, const uint32_t* seg, uint32_t nch) {
      for (uint32_t c = 0; c < nch; ++c) {
        const Range r = tab_chunk_range(vb, seg, c);
        Cursor cur;
        cursor_load(p, cur, r.seg);
        replay_groups(p, cur, r.b, r.e, 0, range_steps(r), -1, &rec);
      }
    };
    // the summing passes claim the sum chunks of the streamed region first
    if (mode == 0 || mode == 2) {
      for (uint32_t c = 0; c < p.nsum; ++c) {
        const Range r = p.sum_groups ? sum_chunk_range<true>(p, c) : sum_chunk_range<false>(p, c);
        Cursor cur;
        cursor_load(p, cur, r.seg);
        replay_groups(p, cur, r.b, r.e, 0, range_steps(r), -1, &rec);
      }
    }
    for (int32_t w = 0; w < p.nworkers; ++w) {
      const Range r = block_range(p, w);
      if (r.b < r.e && mode != 1) {
        Cursor cur;
        cursor_load(p, cur, r.seg);
        if (mode == 0) {  // k_grad_norm_partial: the block as streamed groups
          replay_groups(p, cur, r.b, r.e, 0, range_steps(r), w, &rec);
        } else {  // k_grad_clip_fused, either pass: register groups, then LDS groups
          const BlockSplit bs = block_split(r);
          for (int g = 0; g < kRegSteps / kUnroll; ++g)
            if ((uint32_t)(g * kUnroll) < bs.nreg) replay_group(p, cur, r.b, r.e, g * kUnroll, bs.nreg, w, &rec);
          replay_groups(p, cur, r.b, r.e, bs.nreg, bs.nsteps, w, &rec);
        }
      }
      for (uint64_t i = p.wk_scbegin[w]; i < p.wk_scbegin[w + 1]; ++i) rec.put(w, p.sc_addr[i] | kElementTag);
    }
    if (mode == 1) replay_chunks(p.spl_vb, p.spl_seg, p.nchunk);  // k_grad_scale
    if (mode == 3) replay_chunks(p.fus_vb, p.fus_seg, p.nchs);    // fused, second pass
    *n_out = rec.n;
    if (!rec.uniform_ok) return GCLIP_EINVAL;
    return rec.n > cap ? GCLIP_ERANGE : GCLIP_OK;
  } catch (const std::bad_alloc&) {
    return GCLIP_ENOMEM;
  }
}
