// gclip_cursor.hpp -- launch shape of the kernels and the address walk over a
// plan's vector segments.  Compiled for the GPU (the kernels) and for the
// host (gclip_plan_trace, which replays the kernels' walk so that tests can
// check it on the CPU: every vector visited once per pass, every address
// inside its tensor).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gclip_plan.hpp"

namespace gclip {

// Launch shape and on-chip residency (overridable at build time for sweeps).
#ifndef GCLIP_THREADS
#define GCLIP_THREADS 512
#endif
#ifndef GCLIP_UNROLL
#define GCLIP_UNROLL 8
#endif
#ifndef GCLIP_REG_STEPS
#define GCLIP_REG_STEPS 32
#endif
#ifndef GCLIP_LDS_STEPS
#define GCLIP_LDS_STEPS 19
#endif
constexpr int kThreads = GCLIP_THREADS;     // threads per workgroup (8 waves, two per SIMD)
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = GCLIP_UNROLL;       // vectors in flight per lane in the streamed loops
constexpr int kRegSteps = GCLIP_REG_STEPS;  // fused kernel: steps of kThreads vectors kept in VGPRs
constexpr int kLdsSteps = GCLIP_LDS_STEPS;  // fused kernel: steps kept in LDS (kThreads * 16 B each)
static_assert(kThreads % 64 == 0 && kThreads <= 1024, "whole waves, at most 1024 threads");
static_assert((size_t)kLdsSteps * kThreads * 16 + 1024 <= 160 * 1024, "LDS of one workgroup on gfx950");
static_assert(kRegSteps % kUnroll == 0, "register steps come in whole groups");

struct Cursor {
  uint32_t s;
  uint64_t beg, end, addr;
};

__host__ __device__ __forceinline__ void cursor_load(const DevPlan& p, Cursor& c, uint32_t s) {
  c.s = s;
  c.beg = p.seg_vbegin[s];
  c.end = p.seg_vbegin[s + 1];
  c.addr = p.seg_addr[s];
}

// Move the (workgroup-uniform) cursor forward to the segment holding vector v.
__host__ __device__ __forceinline__ void cursor_seek(const DevPlan& p, Cursor& c, uint64_t v) {
  while (v >= c.end && (int32_t)(c.s + 1) < p.nseg) cursor_load(p, c, c.s + 1);
}

// Byte address of vector v for a step that covers vectors [b, b + kThreads)
// cut at ve (b < ve).  Leaves the cursor on the segment holding the step's
// last vector.  The loop is uniform: it only runs when the step crosses the
// end of a segment.
__host__ __device__ __forceinline__ uint64_t step_addr(const DevPlan& p, Cursor& c, uint64_t b, uint64_t ve,
                                                       uint64_t v) {
  const uint64_t last = (b + kThreads < ve ? b + kThreads : ve) - 1;
  uint64_t a = c.addr + (v - c.beg) * kVecBytes;
  while (last >= c.end) {
    cursor_load(p, c, c.s + 1);
    if (v >= c.beg) a = c.addr + (v - c.beg) * kVecBytes;
  }
  return a;
}

// A uniform 64-bit value held in scalar registers (the compiler cannot always
// prove that cursor fields loaded with vector loads are uniform).
__host__ __device__ __forceinline__ uint64_t uniform64(uint64_t x) {
#ifdef __HIP_DEVICE_COMPILE__
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
#else
  return x;
#endif
}

// A group is the steps j .. j + kUnroll - 1 (capped at j1) of a worker's
// share [vb, ve).  Three kinds:
//   kGroupFull  inside the cursor's segment, every step whole: lane t's
//               vector u is at base + (u * kThreads + t) * 16, no predicates;
//   kGroupTail  inside the segment, but the share (or j1) ends in the group:
//               same addresses, vector u valid when tail_ok() says so;
//   kGroupCross crosses a segment end: addresses from cross_addrs().
// The first two leave the cursor where it is.
enum GroupKind { kGroupFull = 0, kGroupTail = 1, kGroupCross = 2 };

__host__ __device__ __forceinline__ int group_kind(const Cursor& cur, uint64_t vb, uint64_t ve, uint64_t j,
                                                   uint64_t j1, uint64_t& base) {
  const uint64_t b0 = vb + j * kThreads;
  const uint64_t jn = j + kUnroll < j1 ? j + kUnroll : j1;
  const uint64_t gend = vb + jn * kThreads < ve ? vb + jn * kThreads : ve;
  if (gend <= cur.end) {
    base = cur.addr + (b0 - cur.beg) * kVecBytes;
    return (j + kUnroll <= j1 && b0 + (uint64_t)kUnroll * kThreads <= ve) ? kGroupFull : kGroupTail;
  }
  return kGroupCross;
}

__host__ __device__ __forceinline__ bool tail_ok(uint64_t vb, uint64_t ve, uint64_t j, uint64_t j1, int u,
                                                 uint32_t t) {
  return (j + u < j1) && (vb + (j + u) * kThreads + t < ve);
}

// Per-lane addresses of a crossing group, walking the cursor step by step.
__host__ __device__ __forceinline__ void cross_addrs(const DevPlan& p, Cursor& cur, uint64_t vb, uint64_t ve,
                                                     uint64_t j, uint64_t j1, uint32_t t, uint64_t (&a)[kUnroll],
                                                     bool (&ok)[kUnroll]) {
  const uint64_t b0 = vb + j * kThreads;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    ok[u] = false;
    a[u] = 0;
    if (j + u < j1) {
      const uint64_t b = b0 + (uint64_t)u * kThreads, v = b + t;
      a[u] = step_addr(p, cur, b, ve, v);
      ok[u] = v < ve;
    }
  }
}

// How a worker's share splits in the fused kernel: streamed steps [0, js),
// register steps [js, js + nreg), LDS steps [js + nreg, nsteps).  js is a
// multiple of kUnroll (so every group starts at a multiple of kUnroll, as in
// the other kernels) and the resident part is at most kRegSteps + kLdsSteps.
struct FusedSplit {
  uint64_t nsteps, js;
  uint32_t nreg, nlds;
};

__host__ __device__ __forceinline__ FusedSplit fused_split(uint64_t vb, uint64_t ve) {
  FusedSplit f;
  f.nsteps = (ve - vb + kThreads - 1) / kThreads;
  const uint64_t cap = (uint64_t)(kRegSteps + kLdsSteps);
  const uint64_t over = f.nsteps > cap ? f.nsteps - cap : 0;
  f.js = (over + kUnroll - 1) / kUnroll * kUnroll;
  if (f.js > f.nsteps) f.js = f.nsteps;
  const uint64_t nres = f.nsteps - f.js;
  f.nreg = nres < (uint64_t)kRegSteps ? (uint32_t)nres : (uint32_t)kRegSteps;
  f.nlds = (uint32_t)(nres - f.nreg);
  return f;
}

}  // namespace gclip
