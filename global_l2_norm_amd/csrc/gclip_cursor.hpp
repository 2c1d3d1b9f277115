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

constexpr int kThreads = 512;           // threads per workgroup (8 waves, two per SIMD)
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 8;              // vectors in flight per lane in the streamed loops
constexpr int kRegSteps = 32;           // fused kernel: steps of kThreads vectors kept in VGPRs
constexpr int kLdsSteps = 19;           // fused kernel: steps kept in LDS (19 * 8 KB)

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

// How a worker's share splits in the fused kernel: streamed steps [0, js),
// register steps [js, js + nreg), LDS steps [js + nreg, nsteps).
struct FusedSplit {
  uint64_t nsteps, js;
  uint32_t nreg, nlds;
};

__host__ __device__ __forceinline__ FusedSplit fused_split(uint64_t vb, uint64_t ve) {
  FusedSplit f;
  f.nsteps = (ve - vb + kThreads - 1) / kThreads;
  const uint64_t cap = (uint64_t)(kRegSteps + kLdsSteps);
  const uint64_t nres = f.nsteps < cap ? f.nsteps : cap;
  f.js = f.nsteps - nres;
  f.nreg = nres < (uint64_t)kRegSteps ? (uint32_t)nres : (uint32_t)kRegSteps;
  f.nlds = (uint32_t)(nres - f.nreg);
  return f;
}

}  // namespace gclip
