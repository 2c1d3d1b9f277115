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
#ifndef GCLIP_NT_SUM
#define GCLIP_NT_SUM 1
#endif
#ifndef GCLIP_NT_SCALE
#define GCLIP_NT_SCALE 1
#endif
#ifndef GCLIP_REG_STEPS
#define GCLIP_REG_STEPS 40
#endif
#ifndef GCLIP_LDS_STEPS
#define GCLIP_LDS_STEPS 19
#endif
#ifndef GCLIP_SUM_CHUNKS_PER_WORKER
#define GCLIP_SUM_CHUNKS_PER_WORKER 1
#endif
#ifndef GCLIP_SCALE_MIN_STEPS
#define GCLIP_SCALE_MIN_STEPS 8
#endif
#ifndef GCLIP_SCALE_MAX_STEPS
#define GCLIP_SCALE_MAX_STEPS 8
#endif
#ifndef GCLIP_SCALE_GUIDE
#define GCLIP_SCALE_GUIDE 2
#endif

constexpr int kThreads = GCLIP_THREADS;     // threads per workgroup (8 waves, two per SIMD)
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = GCLIP_UNROLL;       // vectors in flight per lane in the streamed loops
constexpr int kRegSteps = GCLIP_REG_STEPS;  // fused kernel: steps of kThreads vectors kept in VGPRs
constexpr int kLdsSteps = GCLIP_LDS_STEPS;  // fused kernel: steps kept in LDS (kThreads * 16 B each)
constexpr int kScaleMinSteps = GCLIP_SCALE_MIN_STEPS;  // scale chunks: at least this many steps,
constexpr int kScaleMaxSteps = GCLIP_SCALE_MAX_STEPS;  // at most this many,
constexpr int kScaleGuide = GCLIP_SCALE_GUIDE;         // about (work left) / (kScaleGuide * workers)
constexpr int kSumChunksPerWorker = GCLIP_SUM_CHUNKS_PER_WORKER;  // sum chunks per worker (about)
// What the fused kernel keeps on chip per worker, and a chunk, in vectors.
constexpr uint64_t kResidentCap = (uint64_t)(kRegSteps + kLdsSteps) * kThreads;
constexpr uint64_t kGroupVectors = (uint64_t)kUnroll * kThreads;  // one group of kUnroll steps
static_assert(kThreads % 64 == 0 && kThreads <= 1024, "whole waves, at most 1024 threads");
static_assert((size_t)kLdsSteps * kThreads * 16 + (size_t)kThreads * 4 + 1024 <= 160 * 1024,
              "LDS of one workgroup on gfx950");
static_assert(kRegSteps % kUnroll == 0, "register steps come in whole groups");
static_assert(kScaleMinSteps % kUnroll == 0 && kScaleMaxSteps % kUnroll == 0 && kScaleMinSteps > 0 &&
                  kScaleMaxSteps >= kScaleMinSteps && kScaleGuide > 0,
              "scale chunks come in whole groups");

// Read of a descriptor table.  The tables never change while a kernel runs,
// so on the device they are read through the constant address space: with a
// workgroup-uniform index that is a scalar load, which the wave can wait for
// without draining its vector loads (those complete in order, so waiting on
// a vector load of the table would also wait for every gradient load issued
// before it).
template <typename T>
__host__ __device__ __forceinline__ T ld_table(const T* p, uint64_t i) {
#ifdef __HIP_DEVICE_COMPILE__
  return ((const __attribute__((address_space(4))) T*)p)[i];
#else
  return p[i];
#endif
}

// A workgroup-uniform 32-bit value moved to a scalar register.
__host__ __device__ __forceinline__ uint32_t uniform32(uint32_t x) {
#ifdef __HIP_DEVICE_COMPILE__
  return __builtin_amdgcn_readfirstlane(x);
#else
  return x;
#endif
}

struct Cursor {
  uint32_t s;
  uint64_t beg, end, addr;
};

__host__ __device__ __forceinline__ void cursor_load(const DevPlan& p, Cursor& c, uint32_t s) {
  c.s = s;
  c.beg = ld_table(p.seg_vbegin, s);
  c.end = ld_table(p.seg_vbegin, (uint64_t)s + 1);
  c.addr = ld_table(p.seg_addr, s);
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

// step_addr for a second list laid out like this one at an offset per
// segment (delta[s]): the address of vector v in that list.  d is the
// offset of the cursor's segment and moves with the cursor; each new
// segment's offset is read like the rest of the table (a scalar load on the
// device), so a crossing step waits for no vector load before its own.
__host__ __device__ __forceinline__ uint64_t step_addr_delta(const DevPlan& p, const uint64_t* delta, Cursor& c,
                                                             uint64_t& d, uint64_t b, uint64_t ve, uint64_t v) {
  const uint64_t last = (b + kThreads < ve ? b + kThreads : ve) - 1;
  uint64_t a = c.addr + d + (v - c.beg) * kVecBytes;
  while (last >= c.end) {
    cursor_load(p, c, c.s + 1);
    d = ld_table(delta, c.s);
    if (v >= c.beg) a = c.addr + d + (v - c.beg) * kVecBytes;
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
// run [vb, ve).  Three kinds:
//   kGroupFull  inside the cursor's segment, every step whole: lane t's
//               vector u is at base + (u * kThreads + t) * 16, no predicates;
//   kGroupTail  inside the segment, but the run (or j1) ends in the group:
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

// A run of the vector space [b, e) and the segment holding b.
struct Range {
  uint64_t b, e;
  uint32_t seg;
};

__host__ __device__ __forceinline__ Range block_range(const DevPlan& p, int32_t w) {
  Range r;
  r.b = p.sb + (uint64_t)w * p.rb;
  r.e = r.b + p.rb < p.nvec ? r.b + p.rb : p.nvec;
  if (r.b > r.e) r.b = r.e;
  r.seg = ld_table(p.blk_seg, (uint64_t)w);
  return r;
}

// Chunk c of a chunk table: [vb[c], vb[c + 1]) (scale chunks).
__host__ __device__ __forceinline__ Range tab_chunk_range(const uint64_t* vb, const uint32_t* seg, uint32_t c) {
  Range r;
  r.b = ld_table(vb, c);
  r.e = ld_table(vb, (uint64_t)c + 1);
  r.seg = ld_table(seg, c);
  return r;
}

// Sum chunk c (cut at sb).  TWO: a list of kNtStoreMinBytes or more, whose
// sum chunks alternate between two sizes (sum_groups); otherwise all are cvs
// vectors.  The kernels of such lists (NTS) take TWO, the others keep the
// one-size arithmetic.
template <bool TWO = false>
__host__ __device__ __forceinline__ Range sum_chunk_range(const DevPlan& p, uint32_t c) {
  Range r;
  if constexpr (TWO) {
    const uint64_t ce = (uint64_t)(p.sum_groups & 0xffffu) * kGroupVectors;
    const uint64_t co = (uint64_t)(p.sum_groups >> 16) * kGroupVectors;
    r.b = sum_chunk_begin(ce, co, c);
    const uint64_t e = r.b + ((c & 1u) ? co : ce);
    r.e = e < p.sb ? e : p.sb;
  } else {
    r.b = (uint64_t)c * p.cvs;
    r.e = r.b + p.cvs < p.sb ? r.b + p.cvs : p.sb;
  }
  r.seg = ld_table(p.sum_seg, c);
  return r;
}

__host__ __device__ __forceinline__ uint64_t range_steps(const Range& r) {
  return (r.e - r.b + kThreads - 1) / kThreads;
}

// How a block splits in the fused kernel: register steps [0, nreg), LDS
// steps [nreg, nsteps).  nreg is kRegSteps (a multiple of kUnroll) unless the
// block is shorter, so every group starts at a multiple of kUnroll.
struct BlockSplit {
  uint32_t nsteps, nreg, nlds;
};

__host__ __device__ __forceinline__ BlockSplit block_split(const Range& r) {
  BlockSplit f;
  f.nsteps = (uint32_t)range_steps(r);
  f.nreg = f.nsteps < (uint32_t)kRegSteps ? f.nsteps : (uint32_t)kRegSteps;
  f.nlds = f.nsteps - f.nreg;
  return f;
}

// Per-tensor pieces (TPiece): the group at vector j of a piece gives lane t
// its vectors j + u * kThreads + t, u < kUnroll, those below the piece's nvec.
constexpr uint32_t kPieceGroup = (uint32_t)kThreads * kUnroll;
__host__ __device__ __forceinline__ uint32_t piece_index(uint32_t j, int u, uint32_t t) {
  return j + (uint32_t)u * kThreads + t;
}

}  // namespace gclip
