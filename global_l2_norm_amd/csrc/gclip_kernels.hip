// gclip_kernels.hip -- gfx950 kernels of global L2-norm gradient clipping.
//
// The method (grad clip lesson, unhomeschool.com ru, sections "Math" and
// "ANDREA's three-kernel pipeline"): a partial sum of squares per chunk into
// a small scratch buffer, a final reduction of that buffer to one scalar and
// its square root, then -- only if norm > max_norm -- one pass multiplying
// every gradient element by max_norm / norm.  The averaging by
// 1/n_microbatches of the backprop lesson (unhomeschool.com vi, section
// "Accumulation across microbatches") is folded in as the factor a.
//
// MI355X design:
//   - one workgroup of kThreads per compute unit.  The list's 16-byte
//     vector space (gclip_plan.hpp) ends with one block per worker; the rest
//     is cut into chunks that the workers claim at run time from eight
//     pools, one per XCD, so that the XCDs that stream faster take more of
//     them -- in the summing pass as in the scaling pass.  Loads are dwordx4
//     with kUnroll vectors in flight per lane, the next group's loads issued
//     before the current group is used;
//   - each vector's squares are summed in fp32 and added into per-lane
//     binary64 accumulators (vec_sumsq states when a vector is summed again
//     in binary64), so the sum cannot overflow and is non-finite exactly when
//     some element is NaN or +-Inf;
//   - lane sums are reduced by an xor butterfly inside each wave into one
//     partial per chunk and wave (a slot of the chunk's own), and over the
//     workgroup into one partial per worker for its block; the last
//     workgroup to arrive (a two-level agent-scope ticket) sums all partials
//     in index order, so the bits of the norm do not depend on scheduling or
//     on which workgroup took which chunk, and both paths give the same
//     bits; cross-workgroup data moves only through agent-scope atomics (see
//     complete_stores);
//   - the fused kernel keeps each worker's block (up to kRegSteps +
//     kLdsSteps steps) in VGPRs and LDS across the grid-wide decision, so the
//     scale pass writes those bytes without reading them again from HBM; it
//     is an ordinary launch whose waits are bounded (a workgroup that waits
//     too long hands its block back to the others), so it cannot deadlock
//     when other work holds some compute units.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/gclip.h"
#include "gclip_cursor.hpp"
#include "gclip_plan.hpp"

namespace gclip {


typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Gradient memory is accessed through global-address-space pointers so that
// the loads are global_load (vector memory counter only), not flat loads,
// which would also be waited for by every scalar-load and LDS wait.
typedef __attribute__((address_space(1))) u32x4 g_u32x4;
typedef __attribute__((address_space(1))) uint32_t g_u32;
typedef __attribute__((address_space(1))) uint16_t g_u16;

// Gradient vectors are read once per pass with no reuse that a cache could
// catch (the Infinity Cache does not keep read data between the passes), so
// they are read with nontemporal loads, which stream through the caches
// without displacing other lines: a cold 369 MB read ran about 10% faster
// that way on MI355X.  Stores are ordinary for lists below kNtStoreMinBytes
// -- the 256 MB Infinity Cache then absorbs much of the write-back, and
// nontemporal stores made a 369 MB scale pass 18% slower -- and nontemporal
// for larger lists, whose writes only thrash it (3% faster at 2.6 GB).
// (The load kind of each pass can be chosen at build time.)
constexpr bool kNtSum = GCLIP_NT_SUM != 0;
constexpr bool kNtScale = GCLIP_NT_SCALE != 0;

template <bool NT>
__device__ __forceinline__ u32x4 ld_vec(const g_u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT>
__device__ __forceinline__ void st_vec(g_u32x4* p, u32x4 q) {
  if constexpr (NT) __builtin_nontemporal_store(q, p);
  else *p = q;
}
template <bool NT>
__device__ __forceinline__ u32x4 load_vec(uint64_t a) { return ld_vec<NT>(reinterpret_cast<const g_u32x4*>(a)); }
template <bool NT>
__device__ __forceinline__ void store_vec(uint64_t a, u32x4 q) { st_vec<NT>(reinterpret_cast<g_u32x4*>(a), q); }

// ---------------------------------------------------------------- element arithmetic
// Sum of the squares of one vector's elements, exact in binary64 for the
// fallback and within 7 * 2^-24 relative otherwise.  The common case sums the
// squares in fp32 (binary64 arithmetic on every element would cost more
// issue slots than the memory pass leaves), which is safe while the fp32 sum
// lies in [2^-100, 2^126): no square overflowed and an underflowed square
// (< 2^-126, at most 8 of them) is below 2^-24 of the sum.  Any other vector
// -- huge or tiny elements, NaN, Inf -- is summed again in binary64, where
// squares of every finite fp32/fp16/bf16 value are exact and cannot
// overflow; an all-zero vector is 0 exactly.  fp16 values can never leave
// the safe range (|x| <= 65504, squares of subnormals are normal fp32).
__device__ __forceinline__ double sumsq64_f32(const u32x4 q) {
  double d = 0.0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const double x = (double)__uint_as_float(q[c]);
    d = __builtin_fma(x, x, d);
  }
  return d;
}

__device__ __forceinline__ double sumsq64_bf16(const u32x4 q) {
  double d = 0.0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const double lo = (double)__uint_as_float(q[c] << 16), hi = (double)__uint_as_float(q[c] & 0xffff0000u);
    d = __builtin_fma(lo, lo, d);
    d = __builtin_fma(hi, hi, d);
  }
  return d;
}

__device__ __forceinline__ bool fp32_sum_safe(float s) { return s >= 0x1p-100f && s < 0x1p+126f; }

template <int DT>
__device__ __forceinline__ double vec_sumsq(const u32x4 q) {
  if constexpr (DT == GCLIP_F32) {
    const float x0 = __uint_as_float(q[0]), x1 = __uint_as_float(q[1]);
    const float x2 = __uint_as_float(q[2]), x3 = __uint_as_float(q[3]);
    float s = x0 * x0;
    s = __builtin_fmaf(x1, x1, s);
    s = __builtin_fmaf(x2, x2, s);
    s = __builtin_fmaf(x3, x3, s);
    if (__builtin_expect(fp32_sum_safe(s), 1)) return (double)s;
    if (((q[0] | q[1] | q[2] | q[3]) & 0x7fffffffu) == 0u) return 0.0;
    return sumsq64_f32(q);
  } else if constexpr (DT == GCLIP_F16) {
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(q[c] & 0xffffu));
      const float hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(q[c] >> 16));
      s = __builtin_fmaf(lo, lo, s);
      s = __builtin_fmaf(hi, hi, s);
    }
    return (double)s;
  } else {
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float lo = __uint_as_float(q[c] << 16), hi = __uint_as_float(q[c] & 0xffff0000u);
      s = __builtin_fmaf(lo, lo, s);
      s = __builtin_fmaf(hi, hi, s);
    }
    if (__builtin_expect(fp32_sum_safe(s), 1)) return (double)s;
    if (((q[0] | q[1] | q[2] | q[3]) & 0x7fff7fffu) == 0u) return 0.0;
    return sumsq64_bf16(q);
  }
}

template <int DT>
__device__ __forceinline__ double elem_square(uint32_t bits) {
  double x;
  if constexpr (DT == GCLIP_F32) {
    x = (double)__uint_as_float(bits);
  } else if constexpr (DT == GCLIP_F16) {
    x = (double)(float)__builtin_bit_cast(_Float16, (uint16_t)bits);
  } else {
    x = (double)__uint_as_float(bits << 16);
  }
  return x * x;
}

// g * s rounded to nearest-even in the storage format.  fp32 storage is
// multiplied in binary64 (one rounding of the binary64 product); the 16-bit
// formats multiply in fp32 by s rounded to fp32.
template <int DT>
__device__ __forceinline__ uint32_t scale_elem(uint32_t bits, double s64, float s32) {
  if constexpr (DT == GCLIP_F32) {
    return __float_as_uint((float)((double)__uint_as_float(bits) * s64));
  } else if constexpr (DT == GCLIP_F16) {
    const _Float16 h = (_Float16)((float)__builtin_bit_cast(_Float16, (uint16_t)bits) * s32);
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
  } else {
    const __bf16 h = (__bf16)(__uint_as_float(bits << 16) * s32);
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
  }
}

template <int DT>
__device__ __forceinline__ u32x4 scale_vec(u32x4 q, double s64, float s32) {
  u32x4 r;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t w = q[c];
    if constexpr (DT == GCLIP_F32) {
      r[c] = scale_elem<DT>(w, s64, s32);
    } else {
      r[c] = scale_elem<DT>(w & 0xffffu, s64, s32) | (scale_elem<DT>(w >> 16, s64, s32) << 16);
    }
  }
  return r;
}

template <int DT>
__device__ __forceinline__ uint32_t load_elem(uint64_t a) {
  if constexpr (DT == GCLIP_F32) return *reinterpret_cast<const g_u32*>(a);
  else return (uint32_t)*reinterpret_cast<const g_u16*>(a);
}

template <int DT>
__device__ __forceinline__ void store_elem(uint64_t a, uint32_t bits) {
  if constexpr (DT == GCLIP_F32) *reinterpret_cast<g_u32*>(a) = bits;
  else *reinterpret_cast<g_u16*>(a) = (uint16_t)bits;
}

// A lane's total: its per-slot accumulators in slot order, then its single elements.
__device__ __forceinline__ double lane_total(const double (&acc)[kUnroll], double accs) {
  double t = acc[0];
#pragma unroll
  for (int u = 1; u < kUnroll; ++u) t += acc[u];
  return t + accs;
}

// ---------------------------------------------------------------- group loads and stores
// Load the vectors of one group into q (zeros where a lane has no vector).
template <bool NT>
__device__ __forceinline__ void load_group(const DevPlan& p, Cursor& cur, uint64_t vb, uint64_t ve, uint64_t j,
                                           uint64_t j1, u32x4 (&q)[kUnroll]) {
  const uint32_t t = threadIdx.x;
  uint64_t base = 0;
  const int kind = group_kind(cur, vb, ve, j, j1, base);
  if (kind == kGroupFull) {
    const g_u32x4* g = reinterpret_cast<const g_u32x4*>(uniform64(base));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) q[u] = ld_vec<NT>(&g[u * kThreads + t]);
  } else if (kind == kGroupTail) {
    const g_u32x4* g = reinterpret_cast<const g_u32x4*>(uniform64(base));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      q[u] = tail_ok(vb, ve, j, j1, u, t) ? ld_vec<NT>(&g[u * kThreads + t]) : u32x4{0u, 0u, 0u, 0u};
  } else {
    // crossing group: walk the cursor step by step (the same walk as
    // cross_addrs), each load issued as soon as its address is known
    const uint64_t b0 = vb + j * kThreads;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      q[u] = u32x4{0u, 0u, 0u, 0u};
      if (j + u < j1) {
        const uint64_t b = b0 + (uint64_t)u * kThreads, v = b + t;
        const uint64_t a = step_addr(p, cur, b, ve, v);
        if (v < ve) q[u] = load_vec<NT>(a);
      }
    }
  }
}

// Store f(vector u) for every vector of one group (the addresses of the
// group are recomputed exactly as load_group computed them).
template <bool NT, typename F>
__device__ __forceinline__ void store_group(const DevPlan& p, Cursor& cur, uint64_t vb, uint64_t ve, uint64_t j,
                                            uint64_t j1, F&& f) {
  const uint32_t t = threadIdx.x;
  uint64_t base = 0;
  const int kind = group_kind(cur, vb, ve, j, j1, base);
  if (kind == kGroupFull) {
    g_u32x4* g = reinterpret_cast<g_u32x4*>(uniform64(base));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) st_vec<NT>(&g[u * kThreads + t], f(u));
  } else if (kind == kGroupTail) {
    g_u32x4* g = reinterpret_cast<g_u32x4*>(uniform64(base));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (tail_ok(vb, ve, j, j1, u, t)) st_vec<NT>(&g[u * kThreads + t], f(u));
  } else {
    const uint64_t b0 = vb + j * kThreads;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (j + u < j1) {
        const uint64_t b = b0 + (uint64_t)u * kThreads, v = b + t;
        const uint64_t a = step_addr(p, cur, b, ve, v);
        if (v < ve) store_vec<NT>(a, f(u));
      }
    }
  }
}

// ---------------------------------------------------------------- norm and scale passes
// Steps [j0, j1) of the run [vb, ve), accumulating into acc.  Step j always
// adds into acc[j % kUnroll] (groups start at multiples of kUnroll in every
// kernel), so every kernel adds the same values in the same order.  The next
// group's loads are issued before the current group is summed, so a lane
// always has a full group of loads in flight.
template <int DT>
__device__ __forceinline__ void norm_steps(const DevPlan& p, Cursor& cur, uint64_t vb, uint64_t ve, uint64_t j0,
                                           uint64_t j1, double (&acc)[kUnroll]) {
  if (j0 >= j1) return;
  u32x4 q[kUnroll];
  load_group<kNtSum>(p, cur, vb, ve, j0, j1, q);
  for (uint64_t j = j0; j < j1; j += kUnroll) {
    u32x4 q2[kUnroll];
    if (j + kUnroll < j1) {
      load_group<kNtSum>(p, cur, vb, ve, j + kUnroll, j1, q2);
    } else {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) q2[u] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc[u] += vec_sumsq<DT>(q[u]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) q[u] = q2[u];
  }
}

template <int DT>
__device__ __forceinline__ double norm_scalars(const DevPlan& p, int w) {
  double s = 0.0;
  const uint64_t b = ld_table(p.wk_scbegin, (uint64_t)w), e = ld_table(p.wk_scbegin, (uint64_t)w + 1);
  for (uint64_t i = b + threadIdx.x; i < e; i += kThreads) s += elem_square<DT>(load_elem<DT>(p.sc_addr[i]));
  return s;
}

// Steps [j0, j1) of the run [vb, ve): read, multiply, write back.  A group's
// loads are all issued before its first store.
template <int DT>
__device__ __forceinline__ void scale_steps(const DevPlan& p, Cursor& cur, uint64_t vb, uint64_t ve, uint64_t j0,
                                            uint64_t j1, double s64, float s32) {
  for (uint64_t j = j0; j < j1; j += kUnroll) {
    u32x4 q[kUnroll];
    Cursor c2 = cur;
    load_group<kNtScale>(p, cur, vb, ve, j, j1, q);
    store_group<false>(p, c2, vb, ve, j, j1, [&](int u) { return scale_vec<DT>(q[u], s64, s32); });
  }
}

template <int DT>
__device__ __forceinline__ void scale_scalars(const DevPlan& p, int w, double s64, float s32) {
  const uint64_t b = ld_table(p.wk_scbegin, (uint64_t)w), e = ld_table(p.wk_scbegin, (uint64_t)w + 1);
  for (uint64_t i = b + threadIdx.x; i < e; i += kThreads) {
    const uint64_t a = p.sc_addr[i];
    store_elem<DT>(a, scale_elem<DT>(load_elem<DT>(a), s64, s32));
  }
}

// ---------------------------------------------------------------- counters in the workspace
// Cross-workgroup data (partials, the decision, the counters) is written and
// read only with agent-scope atomics, which go to the device-coherent level
// of the memory system.
__device__ __forceinline__ uint32_t atomic_ld(const uint32_t* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_st(uint32_t* a, uint32_t v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t atomic_add(uint32_t* a, uint32_t v) {
  return __hip_atomic_fetch_add(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double atomic_ld(const double* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_st(double* a, double v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Words of line 0 of sync.
constexpr int kEpochWord = 0, kSkipWord = 1, kHandedWord = 2;

__device__ __forceinline__ uint32_t* sum_pools(const DevPlan& p) { return p.sync + kSyncLineWords; }
__device__ __forceinline__ uint32_t* scale_pools(const DevPlan& p) { return p.sync + (1 + kPools) * kSyncLineWords; }
__device__ __forceinline__ uint32_t* arrival_tickets(const DevPlan& p) {
  return p.sync + (1 + 2 * kPools) * kSyncLineWords;
}
__device__ __forceinline__ uint32_t* finish_tickets(const DevPlan& p) {
  return p.sync + (2 + 3 * kPools) * kSyncLineWords;
}

// Waiting for this workgroup's stores to complete before its next atomic is
// issued orders them for every reader, so no agent-scope fence is needed: on
// gfx950 such a fence writes back and invalidates the whole L2 of the XCD,
// which costs ~18 us when 256 workgroups do it at the end of a pass.
__device__ __forceinline__ void complete_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Ticket over every workgroup of a launch, in two levels: workgroup w counts
// in the line of its group w % kPools (its XCD: workgroups are dealt to the
// XCDs in turn), the last of each group counts in the top line.  No counter
// takes more than ~nworkers / kPools atomics at once.  True in exactly one
// workgroup, the last to take the ticket.  The counter a workgroup completes
// is reset by it for the next launch.  Thread 0 only; its stores must be
// complete (complete_stores) before the call.
__device__ __forceinline__ bool take_ticket(uint32_t* lines, int32_t nworkers) {
  const uint32_t g = blockIdx.x % (uint32_t)kPools;
  const uint32_t members = ((uint32_t)nworkers - g + kPools - 1) / kPools;
  const uint32_t groups = nworkers < kPools ? (uint32_t)nworkers : (uint32_t)kPools;
  uint32_t* mine = lines + g * kSyncLineWords;
  uint32_t* top = lines + kPools * kSyncLineWords;
  if (atomic_add(mine, 1u) != members - 1u) return false;
  atomic_st(mine, 0u);
  if (atomic_add(top, 1u) != groups - 1u) return false;
  atomic_st(top, 0u);
  return true;
}

// ---------------------------------------------------------------- chunk claiming
// Workgroup w takes chunk w first, without any claim; chunks nworkers ..
// nch - 1 are claimed at run time from kPools pools, the one of the
// workgroup's own XCD first.  Pool q holds chunks nworkers + q, nworkers + q
// + kPools, ...; a claim is a ticket drawn on a pool's counter.
constexpr uint32_t kNone = 0xffffffffu;

struct Claimer {
  uint32_t* pools;
  uint32_t base;   // first claimed chunk (nworkers)
  uint32_t ndyn;   // claimed chunks
  uint32_t pool;   // pool drawn from
  bool dry;        // every pool found empty
};

__device__ __forceinline__ Claimer make_claimer(uint32_t* pools, const DevPlan& p, uint32_t nch) {
  const uint32_t base = (uint32_t)p.nworkers;
  const uint32_t ndyn = nch > base ? nch - base : 0u;
  return Claimer{pools, base, ndyn, blockIdx.x % (uint32_t)kPools, ndyn == 0u};
}

__device__ __forceinline__ uint32_t pool_size(const Claimer& cl, uint32_t q) {
  return q < cl.ndyn ? (cl.ndyn - q + kPools - 1) / kPools : 0u;
}

// A claim is taken in two steps: the ticket is drawn before a chunk streams
// and turned into a chunk after it, so waiting for the counter's reply
// overlaps the chunk's loads instead of draining them.  Thread 0 only.
__device__ __forceinline__ uint32_t claim_issue(const Claimer& cl) {
  return cl.dry ? 0u : atomic_add(&cl.pools[cl.pool * kSyncLineWords], 1u);
}

// The chunk of ticket tk (drawn on pool cl.pool), or, when that pool is
// empty, a chunk of another pool: every pool's counter is read at once and a
// pool that still has chunks is claimed from, until a claim succeeds or all
// are empty (kNone).  Counters only grow during a launch, so a pool found
// empty stays empty, and a failed claim leaves its pool empty: the loop ends
// within kPools failures.
__device__ __forceinline__ uint32_t claim_resolve(Claimer& cl, uint32_t tk) {
  if (cl.dry) return kNone;
  if (tk < pool_size(cl, cl.pool)) return cl.base + cl.pool + tk * (uint32_t)kPools;
  for (int round = 0; round <= kPools; ++round) {
    // the first pool after cl.pool, in circular order, that still has chunks
    uint32_t pick = kNone, best = kPools;
#pragma unroll
    for (int q = 0; q < kPools; ++q) {
      const uint32_t cnt = atomic_ld(&cl.pools[q * kSyncLineWords]);
      const uint32_t dist = ((uint32_t)q + 2u * kPools - cl.pool - 1u) % (uint32_t)kPools;
      if (cnt < pool_size(cl, (uint32_t)q) && dist < best) {
        best = dist;
        pick = (uint32_t)q;
      }
    }
    if (pick == kNone) break;
    cl.pool = pick;
    const uint32_t k2 = atomic_add(&cl.pools[pick * kSyncLineWords], 1u);
    if (k2 < pool_size(cl, pick)) return cl.base + pick + k2 * (uint32_t)kPools;
  }
  cl.dry = true;
  return kNone;
}

__device__ __forceinline__ void reset_pools(uint32_t* pools) {
  for (int q = 0; q < kPools; ++q) atomic_st(&pools[q * kSyncLineWords], 0u);
}

// Claims run two chunks ahead: the chunk after next is claimed while the
// current one streams and is handed over at the per-chunk barrier through
// LDS slot i % 2 (a slot is rewritten only two barriers after it was read).
struct ClaimSlots {
  uint32_t claim[2];
};

// The chunk loops below draw the ticket for the chunk after next when a
// chunk starts, before its later groups are loaded, and resolve it after the
// chunk's last group has been waited for: loads and atomics complete in
// order, so by then the ticket's reply is in and resolving it costs no wait.
// Only then is the next chunk's first group loaded, so it stays in flight
// across the chunk's barrier.  (Resolving after that load made the wave wait
// for it too: every chunk ended with nothing in flight.)  At the start, the
// ticket for the second chunk is drawn before the first chunk's first group
// is loaded and resolved after it.

// Sum every sum chunk of the streamed region [0, sb) that this workgroup
// takes.  Each wave reduces its lanes' sums over a chunk to one value and
// stores it in the chunk's own slot, partials[c * kWaves + wave], so the
// final sum does not depend on which workgroup took the chunk; the only
// barrier per chunk hands the next claim to every wave.
template <int DT>
__device__ __forceinline__ void norm_chunks(const DevPlan& p, ClaimSlots& sl) {
  const uint32_t nch = p.nsum;
  if (blockIdx.x >= nch) return;  // then no chunk is left to claim either
  const uint32_t t = threadIdx.x, lane = t & 63u, wave = t >> 6;
  Claimer cl = make_claimer(sum_pools(p), p, nch);
  uint32_t c = blockIdx.x, cn;
  Cursor cur;
  u32x4 q[kUnroll];
  {
    uint32_t tk = 0;
    if (t == 0) tk = claim_issue(cl);
    const Range r = sum_chunk_range(p, c);
    cursor_load(p, cur, r.seg);
    load_group<kNtSum>(p, cur, r.b, r.e, 0, range_steps(r), q);
    if (t == 0) sl.claim[1] = claim_resolve(cl, tk);
    __syncthreads();
    cn = uniform32(sl.claim[1]);
  }
  for (uint32_t i = 0; c != kNone; ++i) {
    const Range r = sum_chunk_range(p, c);
    const uint64_t ns = range_steps(r);
    uint32_t tk = 0;
    if (t == 0 && cn != kNone) tk = claim_issue(cl);
    double acc[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc[u] = 0.0;
    for (uint64_t j = 0; j + kUnroll < ns; j += kUnroll) {
      u32x4 q2[kUnroll];
      load_group<kNtSum>(p, cur, r.b, r.e, j + kUnroll, ns, q2);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc[u] += vec_sumsq<DT>(q[u]);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) q[u] = q2[u];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc[u] += vec_sumsq<DT>(q[u]);
    const uint32_t par = i & 1u;
    if (t == 0) sl.claim[par] = cn != kNone ? claim_resolve(cl, tk) : kNone;
    Cursor curn;
    if (cn != kNone) {
      const Range rn = sum_chunk_range(p, cn);
      cursor_load(p, curn, rn.seg);
      load_group<kNtSum>(p, curn, rn.b, rn.e, 0, range_steps(rn), q);
    }
    double v = lane_total(acc, 0.0);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) atomic_st(&p.partials[(size_t)c * kWaves + wave], v);
    __syncthreads();
    c = cn;
    cn = uniform32(sl.claim[par]);
    cur = curn;
  }
}

// Scale in place every chunk of the table (vb, seg, nch) that this workgroup
// takes.  A chunk's last group is scaled into registers before the ticket is
// resolved, and stored after it.
template <int DT, bool NTS>
__device__ __forceinline__ void scale_chunks(const DevPlan& p, ClaimSlots& sl, const uint64_t* vb,
                                             const uint32_t* seg, uint32_t nch, double s64, float s32) {
  if (blockIdx.x >= nch) return;  // then no chunk is left to claim either
  const uint32_t t = threadIdx.x;
  Claimer cl = make_claimer(scale_pools(p), p, nch);
  uint32_t c = blockIdx.x, cn;
  Cursor cur;
  u32x4 q[kUnroll];
  {
    uint32_t tk = 0;
    if (t == 0) tk = claim_issue(cl);
    const Range r = tab_chunk_range(vb, seg, c);
    cursor_load(p, cur, r.seg);
    load_group<kNtScale>(p, cur, r.b, r.e, 0, range_steps(r), q);
    if (t == 0) sl.claim[1] = claim_resolve(cl, tk);
    __syncthreads();
    cn = uniform32(sl.claim[1]);
  }
  for (uint32_t i = 0; c != kNone; ++i) {
    const Range r = tab_chunk_range(vb, seg, c);
    const uint64_t ns = range_steps(r);
    uint32_t tk = 0;
    if (t == 0 && cn != kNone) tk = claim_issue(cl);
    Cursor cst;
    cursor_load(p, cst, r.seg);
    uint64_t j = 0;
    for (; j + kUnroll < ns; j += kUnroll) {
      u32x4 q2[kUnroll];
      load_group<kNtScale>(p, cur, r.b, r.e, j + kUnroll, ns, q2);
      store_group<NTS>(p, cst, r.b, r.e, j, ns, [&](int u) { return scale_vec<DT>(q[u], s64, s32); });
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) q[u] = q2[u];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) q[u] = scale_vec<DT>(q[u], s64, s32);
    const uint32_t par = i & 1u;
    if (t == 0) sl.claim[par] = cn != kNone ? claim_resolve(cl, tk) : kNone;
    store_group<NTS>(p, cst, r.b, r.e, j, ns, [&](int u) { return q[u]; });
    Cursor curn;
    if (cn != kNone) {
      u32x4 q2[kUnroll];
      const Range rn = tab_chunk_range(vb, seg, cn);
      cursor_load(p, curn, rn.seg);
      load_group<kNtScale>(p, curn, rn.b, rn.e, 0, range_steps(rn), q2);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) q[u] = q2[u];
    }
    __syncthreads();
    c = cn;
    cn = uniform32(sl.claim[par]);
    cur = curn;
  }
}

// ---------------------------------------------------------------- reductions and the decision
// Sum of v over the workgroup, the same bits in every thread.  Butterfly
// inside each wave (a + b == b + a, so every lane holds the same sum), then
// the wave sums in wave order.
__device__ __forceinline__ double wg_sum(double v, double* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // red may still be read by a previous call
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  double t = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) t += red[i];
  return t;
}

// Partials: one per wave per sum chunk, then one per worker.
__device__ __forceinline__ uint32_t npartials(const DevPlan& p) {
  return p.nsum * (uint32_t)kWaves + (uint32_t)p.nworkers;
}
__device__ __forceinline__ double* worker_partial(const DevPlan& p, int w) {
  return p.partials + (size_t)p.nsum * kWaves + w;
}

// Sum of all partials in index order (lane i takes i, i + kThreads, ...).
__device__ __forceinline__ double partials_sum(const DevPlan& p, double* red) {
  double v = 0.0;
  const uint32_t n = npartials(p);
  for (uint32_t i = threadIdx.x; i < n; i += kThreads) v += atomic_ld(&p.partials[i]);
  return wg_sum(v, red);
}

// After the last workgroup has summed the partials it overwrites them with
// NaN, so a partial that was somehow read before it was written could only
// ever show up as a NaN norm, never as a plausible wrong one.
__device__ __forceinline__ void poison_partials(const DevPlan& p) {
  const uint32_t n = npartials(p);
  for (uint32_t i = threadIdx.x; i < n; i += kThreads) atomic_st(&p.partials[i], __builtin_nan(""));
}

struct Decision {
  double s;
  int clipped, skip;
};

// Grad clip lesson "Math" / glossary "Mechanism and details": unchanged when
// norm <= c, factor c / norm when norm > c; times the averaging factor a.
__device__ __forceinline__ Decision decide(double sumsq, int nonfinite, double max_norm, double avg, int err) {
  Decision d;
  const double norm = sqrt(sumsq);
  d.clipped = norm > max_norm ? 1 : 0;
  const double coef = d.clipped ? max_norm / norm : 1.0;
  d.skip = (nonfinite && err) ? 1 : 0;
  d.s = avg * coef;
  return d;
}

// The averaging factor: given by the host, or 1 / (n * S) with the loss
// scale S read from device memory (loss-scaled steps).
__device__ __forceinline__ double avg_value(const AvgSrc& s) {
  return s.scale ? 1.0 / (s.a * (double)*s.scale) : s.a;
}

// The flag of a NaN/Inf element: the raw sum of squares is not finite.  An
// averaging factor that is not finite and positive (only possible when it
// comes from a loss scale that is not) counts as one too, so that nothing
// is written.
__device__ __forceinline__ int nonfinite_of(double S, double avg) {
  return (__builtin_isfinite(S) && __builtin_isfinite(avg) && avg > 0.0) ? 0 : 1;
}

__device__ __forceinline__ void write_norm(gclip_result* res, double S, double avg) {
  const double sumsq = (avg * avg) * S;
  res->sumsq = sumsq;
  res->norm = sqrt(sumsq);
  res->nonfinite = nonfinite_of(S, avg);
}

__device__ __forceinline__ void write_decision(gclip_result* res, const Decision& d, double max_norm) {
  const bool wrote = !(d.skip || d.s == 1.0);
  res->scale = wrote ? d.s : 1.0;
  res->clipped = d.clipped;
  res->skipped = d.skip;
  res->max_norm = max_norm;
  res->decided = 1;
}

// Arrival after the summing pass: true in the last workgroup (all threads).
// The caller's partials must already be stored.
__device__ __forceinline__ bool arrive(const DevPlan& p, int* flag) {
  if (threadIdx.x == 0) {
    complete_stores();
    *flag = take_ticket(arrival_tickets(p), p.nworkers) ? 1 : 0;
  }
  __syncthreads();
  return *flag != 0;
}

// Blocks handed back by the fused kernel.  Worker w's state word is kHeld
// while w holds its block (or has written it), kHanded once w has stopped
// waiting at the decision and left its block unscaled in memory, kTaken once
// another workgroup has taken it over.  Line 0's kHandedWord counts the
// hand-backs.
constexpr uint32_t kHeld = 0u, kHanded = 2u, kTaken = 3u;

struct HandSlots {
  uint32_t n;
  uint32_t list[kThreads];
};

// Take over every block handed back so far and scale it from memory, with
// the worker's single elements (whole workgroup).
template <int DT>
__device__ __forceinline__ void take_handed_blocks(const DevPlan& p, HandSlots& hs, double s64, float s32) {
  for (uint32_t base = 0; base < (uint32_t)p.nworkers; base += kThreads) {
    if (threadIdx.x == 0) hs.n = 0;
    __syncthreads();
    const uint32_t i = base + threadIdx.x;
    if (i < (uint32_t)p.nworkers && atomic_ld(&p.bstate[i]) == kHanded) {
      uint32_t expected = kHanded;
      if (__hip_atomic_compare_exchange_strong(&p.bstate[i], &expected, kTaken, __ATOMIC_RELAXED,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
        hs.list[atomicAdd(&hs.n, 1u)] = i;
    }
    __syncthreads();
    const uint32_t n = hs.n;
    for (uint32_t k = 0; k < n; ++k) {
      const int v = (int)hs.list[k];
      const Range r = block_range(p, v);
      if (r.b < r.e) {
        Cursor cur;
        cursor_load(p, cur, r.seg);
        scale_steps<DT>(p, cur, r.b, r.e, 0, range_steps(r), s64, s32);
      }
      scale_scalars<DT>(p, v, s64, s32);
    }
    __syncthreads();
  }
}

// Second ticket, at the very end.  The last workgroup to finish -- every
// other one has then left the pools and the block states alone -- resets the
// scale pools and, after a fused launch, scales whatever blocks are still
// handed back (the decision is published before the deciding workgroup
// finishes, so it is known here), clears their states and records how many
// workers handed their block back.
template <int DT>
__device__ __forceinline__ void finish(const DevPlan& p, gclip_result* res, bool fused, HandSlots& hs, int* flag) {
  __syncthreads();
  if (threadIdx.x == 0) {
    complete_stores();
    *flag = take_ticket(finish_tickets(p), p.nworkers) ? 1 : 0;
  }
  __syncthreads();
  if (*flag == 0) return;
  if (fused) {
    const uint32_t handed = atomic_ld(&p.sync[kHandedWord]);
    if (handed != 0u) {
      const double s = atomic_ld(&p.bcast[0]);
      const uint32_t skip = atomic_ld(&p.sync[kSkipWord]);
      if (skip == 0u && s != 1.0) take_handed_blocks<DT>(p, hs, s, (float)s);
      __syncthreads();
      for (uint32_t i = threadIdx.x; i < (uint32_t)p.nworkers; i += kThreads) atomic_st(&p.bstate[i], kHeld);
    }
    if (threadIdx.x == 0) {
      res->handed_back = (int32_t)handed;
      atomic_st(&p.sync[kHandedWord], 0u);
    }
  }
  if (threadIdx.x == 0) reset_pools(scale_pools(p));
}

// ---------------------------------------------------------------- kernels
// Kernels 1 and 2 of the pages' pipeline.  Partial sums of squares: the
// chunks of the streamed region this workgroup claims (one partial per chunk
// and wave), then worker w's block and single elements (one partial per
// worker); the last workgroup to arrive sums every partial in index order.
// The fused kernel adds the same values in the same order, so both paths
// give the same bits.
template <int DT>
__global__ __launch_bounds__(kThreads) void k_grad_norm_partial(DevPlan p, AvgSrc avs, gclip_result* res) {
  const double avg = avg_value(avs);
  __shared__ double red[kWaves];
  __shared__ ClaimSlots sl;
  __shared__ int flag;
  const int w = blockIdx.x;
  norm_chunks<DT>(p, sl);
  double acc[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) acc[u] = 0.0;
  const Range r = block_range(p, w);
  if (r.b < r.e) {
    Cursor cur;
    cursor_load(p, cur, r.seg);
    norm_steps<DT>(p, cur, r.b, r.e, 0, range_steps(r), acc);
  }
  const double part = wg_sum(lane_total(acc, norm_scalars<DT>(p, w)), red);
  if (threadIdx.x == 0) atomic_st(worker_partial(p, w), part);
  if (arrive(p, &flag)) {
    const double S = partials_sum(p, red);
    poison_partials(p);
    if (threadIdx.x == 0) {
      reset_pools(sum_pools(p));
      write_norm(res, S, avg);
      res->scale = 1.0;
      res->clipped = 0;
      res->skipped = 0;
      res->decided = 0;
      res->status = 0;
      res->handed_back = 0;
    }
  }
}

// Kernel 3: the decision from the device result block, then g <- g * s over
// the chunks each workgroup claims, or no write at all.
template <int DT, bool NTS>
__global__ __launch_bounds__(kThreads) void k_grad_scale(DevPlan p, double max_norm, AvgSrc avs, int err,
                                                         gclip_result* res) {
  const double avg = avg_value(avs);
  __shared__ ClaimSlots sl;
  __shared__ HandSlots hs;
  __shared__ int flag;
  const int w = blockIdx.x;
  const Decision d = decide(res->sumsq, res->nonfinite, max_norm, avg, err);
  if (w == 0 && threadIdx.x == 0) write_decision(res, d, max_norm);
  if (!(d.skip || d.s == 1.0)) {
    const double s64 = d.s;
    const float s32 = (float)d.s;
    scale_chunks<DT, NTS>(p, sl, p.spl_vb, p.spl_seg, p.nchunk, s64, s32);
    scale_scalars<DT>(p, w, s64, s32);
  }
  finish<DT>(p, res, false, hs, &flag);
}

// Phase 2 of the fused kernel: the block straight from VGPRs and LDS, then
// the scale chunks of the streamed region this workgroup claims.
template <int DT, bool NTS>
__device__ __forceinline__ void write_block_and_chunks(const DevPlan& p, ClaimSlots& sl, const Range& r,
                                                       const BlockSplit& bs, const u32x4 (&keep)[kRegSteps],
                                                       const u32x4* keep_lds, double s64, float s32) {
  const uint32_t t = threadIdx.x;
  if (r.b < r.e) {
    Cursor cur;
    cursor_load(p, cur, r.seg);
#pragma unroll
    for (int g = 0; g < kRegSteps / kUnroll; ++g) {
      if ((uint32_t)(g * kUnroll) < bs.nreg)
        store_group<NTS>(p, cur, r.b, r.e, g * kUnroll, bs.nreg,
                         [&](int u) { return scale_vec<DT>(keep[g * kUnroll + u], s64, s32); });
    }
    for (uint32_t k0 = 0; k0 < bs.nlds; k0 += kUnroll)
      store_group<NTS>(p, cur, r.b, r.e, bs.nreg + k0, bs.nsteps,
                       [&](int u) { return scale_vec<DT>(keep_lds[(k0 + u) * kThreads + t], s64, s32); });
  }
  scale_chunks<DT, NTS>(p, sl, p.fus_vb, p.fus_seg, p.nchs, s64, s32);
}

// The whole path in one launch.  Phase 1 sums the chunks of the streamed
// region the workgroup claims, then reads its block into VGPRs and LDS; the
// last workgroup to arrive reduces the partials and decides; phase 2 writes
// the block straight from VGPRs/LDS, then reads, scales and writes the
// chunks of the streamed region it claims.  The launch does not need every
// workgroup resident at once: a workgroup that has waited wait_ticks
// (wall-clock ticks) for the decision hands its block back and exits,
// freeing its compute unit for the workgroups still to run, and the
// workgroups that do see the decision -- in the end the last one to finish
// -- scale the handed-back blocks from memory.
template <int DT, bool NTS>
__global__ __launch_bounds__(kThreads, 1) void k_grad_clip_fused(DevPlan p, double max_norm, AvgSrc avs, int err,
                                                                 gclip_result* res, uint32_t epoch,
                                                                 uint64_t wait_ticks) {
  const double avg = avg_value(avs);
  __shared__ u32x4 keep_lds[kLdsSteps * kThreads];
  __shared__ double red[kWaves];
  __shared__ ClaimSlots sl;
  __shared__ HandSlots hs;
  __shared__ int flag;
  __shared__ int gave_up;
  __shared__ int handed;
  __shared__ double bc_s;
  __shared__ int bc_skip;
  const int w = blockIdx.x;
  const uint32_t t = threadIdx.x;

  norm_chunks<DT>(p, sl);
  double acc[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) acc[u] = 0.0;
  const Range r = block_range(p, w);
  const BlockSplit bs = block_split(r);
  u32x4 keep[kRegSteps];
  if (r.b < r.e) {
    Cursor cur;
    cursor_load(p, cur, r.seg);
    // register steps: issue every load first, then accumulate in step order
#pragma unroll
    for (int g = 0; g < kRegSteps / kUnroll; ++g) {
      u32x4 q[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) q[u] = u32x4{0u, 0u, 0u, 0u};
      if ((uint32_t)(g * kUnroll) < bs.nreg) load_group<kNtSum>(p, cur, r.b, r.e, g * kUnroll, bs.nreg, q);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) keep[g * kUnroll + u] = q[u];
    }
#pragma unroll
    for (int k = 0; k < kRegSteps; ++k)
      if ((uint32_t)k < bs.nreg) acc[k % kUnroll] += vec_sumsq<DT>(keep[k]);
    for (uint32_t k0 = 0; k0 < bs.nlds; k0 += kUnroll) {
      u32x4 q[kUnroll];
      load_group<kNtSum>(p, cur, r.b, r.e, bs.nreg + k0, bs.nsteps, q);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (k0 + u < bs.nlds) {
          acc[u] += vec_sumsq<DT>(q[u]);
          keep_lds[(k0 + u) * kThreads + t] = q[u];
        }
      }
    }
  }
  const double part = wg_sum(lane_total(acc, norm_scalars<DT>(p, w)), red);
  if (t == 0) atomic_st(worker_partial(p, w), part);

  // grid-wide decision: the last workgroup to arrive reduces and releases
  if (t == 0) gave_up = 0;
  if (arrive(p, &flag)) {
    const double S = partials_sum(p, red);
    poison_partials(p);
    if (t == 0) {
      const double sumsq = (avg * avg) * S;
      const Decision d = decide(sumsq, nonfinite_of(S, avg), max_norm, avg, err);
      write_norm(res, S, avg);
      write_decision(res, d, max_norm);
      res->status = 0;
      bc_s = d.s;
      bc_skip = d.skip;
      reset_pools(sum_pools(p));
      atomic_st(&p.bcast[0], d.s);
      atomic_st(&p.sync[kSkipWord], (uint32_t)d.skip);
      complete_stores();
      atomic_st(&p.sync[kEpochWord], epoch);
    }
  } else if (t == 0) {
    const uint64_t t0 = wall_clock64();
    while (atomic_ld(&p.sync[kEpochWord]) != epoch) {
      __builtin_amdgcn_s_sleep(2);
      if (wall_clock64() - t0 > wait_ticks) {
        // hand the block back: its state is visible before the count
        atomic_st(&p.bstate[w], kHanded);
        complete_stores();
        atomic_add(&p.sync[kHandedWord], 1u);
        gave_up = 1;
        break;
      }
    }
    if (!gave_up) {
      bc_s = atomic_ld(&p.bcast[0]);
      bc_skip = (int)atomic_ld(&p.sync[kSkipWord]);
    }
  }
  __syncthreads();
  const double s64 = bc_s;
  if (!gave_up && !bc_skip && s64 != 1.0) {
    const float s32 = (float)s64;
    write_block_and_chunks<DT, NTS>(p, sl, r, bs, keep, keep_lds, s64, s32);
    scale_scalars<DT>(p, w, s64, s32);
    if (t == 0) handed = (int)atomic_ld(&p.sync[kHandedWord]);
    __syncthreads();
    if (handed) take_handed_blocks<DT>(p, hs, s64, s32);
  }
  finish<DT>(p, res, true, hs, &flag);
}

// ---------------------------------------------------------------- per-tensor norms and clipping
// Grad clip lesson, "Two variants: Per-Tensor or Global": every tensor by its
// own norm, in the three kernels of the lesson's pipeline.  k_tensor_partial:
// one workgroup per piece (a run of one tensor, TPiece), kUnroll vectors in
// flight per lane, one partial per piece, plain stores and no atomics (a
// returning atomic per workgroup held each workgroup's slot for a round trip
// to the device-coherent level, and the pieces of one large tensor queued on
// its counter).  k_tensor_decide: one workgroup stages the partials in LDS,
// every lane loading many at once, sums each tensor's pieces in piece order
// and takes the decisions.  k_tensor_scale: one workgroup per piece.  Every
// sum is taken in a fixed order, so the bits do not depend on scheduling.

template <int DT>
__device__ __forceinline__ double piece_sumsq(const TensorPlan& T, const TPiece& pc) {
  const uint32_t t = threadIdx.x;
  double acc[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) acc[u] = 0.0;
  const g_u32x4* base = reinterpret_cast<const g_u32x4*>(uniform64(pc.addr));
  const uint32_t nvec = uniform32(pc.nvec);
  for (uint32_t j = 0; j < nvec; j += kPieceGroup) {
    u32x4 q[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t i = piece_index(j, u, t);
      q[u] = i < nvec ? ld_vec<kNtSum>(base + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc[u] += vec_sumsq<DT>(q[u]);
  }
  double s = 0.0;
  for (uint32_t i = t; i < pc.sc_count; i += kThreads) s += elem_square<DT>(load_elem<DT>(T.sc_addr[pc.sc_begin + i]));
  return lane_total(acc, s);
}

template <int DT, bool NTS>
__device__ __forceinline__ void piece_scale(const TensorPlan& T, const TPiece& pc, double s64, float s32) {
  const uint32_t t = threadIdx.x;
  g_u32x4* base = reinterpret_cast<g_u32x4*>(uniform64(pc.addr));
  const uint32_t nvec = uniform32(pc.nvec);
  for (uint32_t j = 0; j < nvec; j += kPieceGroup) {
    u32x4 q[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t i = piece_index(j, u, t);
      if (i < nvec) q[u] = ld_vec<kNtScale>(base + i);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t i = piece_index(j, u, t);
      if (i < nvec) st_vec<NTS>(base + i, scale_vec<DT>(q[u], s64, s32));
    }
  }
  for (uint32_t i = t; i < pc.sc_count; i += kThreads) {
    const uint64_t a = T.sc_addr[pc.sc_begin + i];
    store_elem<DT>(a, scale_elem<DT>(load_elem<DT>(a), s64, s32));
  }
}

constexpr int kStage = 12288;  // partials staged in LDS at once by k_tensor_decide (96 KB + 48 KB of owners)
constexpr int kStageBatch = 16;  // loads in flight per lane while staging

template <int DT>
__global__ __launch_bounds__(kThreads) void k_tensor_partial(TensorPlan T) {
  __shared__ double red[kWaves];
  const TPiece pc = ld_table(T.pieces, blockIdx.x);
  const double part = wg_sum(piece_sumsq<DT>(T, pc), red);
  if (threadIdx.x == 0) T.partials[blockIdx.x] = part;
}

// One workgroup.  Every tensor's figures and, for the per-tensor clip (clip
// != 0), its decision; then the list's result block.  With the stop switch,
// a NaN/Inf in any tensor stops the whole update.
//
// The partials are staged in LDS in windows of kStage, with the tensor of
// each piece.  A segmented sum in two levels, in a fixed order: lane i sums
// the staged pieces [i C, (i + 1) C) in order, cut where a tensor starts,
// and leaves each fragment's sum in place at the fragment's first piece;
// then the lane that owns tensor k (k % kThreads) adds the tensor's
// fragments in order -- the one at its first piece in the window and one at
// every chunk start inside it.  A lane keeps its first tensor's running sum
// in a register and any further tensor's in out[k].
__device__ __forceinline__ double tensor_in_window(const double* stage, uint32_t C, uint32_t lo, uint32_t hi) {
  double S = stage[lo];
  for (uint32_t j = (lo / C + 1) * C; j < hi; j += C) S += stage[j];
  return S;
}

__global__ __launch_bounds__(kThreads) void k_tensor_decide(TensorPlan T, AvgSrc avs, double max_norm, int clip,
                                                            int err, gclip_tensor_result* out, gclip_result* res) {
  __shared__ double stage[kStage];
  __shared__ uint32_t owner[kStage];
  __shared__ double red[kWaves];
  const double avg = avg_value(avs);
  const uint32_t t = threadIdx.x;
  const int32_t k0 = (int32_t)t;  // this lane's first tensor
  const bool has0 = k0 < T.ntensors;
  const uint32_t b0 = has0 ? T.first[k0] : 0u, e0 = has0 ? T.first[k0 + 1] : 0u;
  double S0 = 0.0;
  for (int32_t k = k0 + kThreads; k < T.ntensors; k += kThreads) out[k].sumsq = 0.0;  // further tensors' sums
  for (uint32_t w0 = 0; w0 < T.npieces; w0 += kStage) {
    const uint32_t wn = T.npieces - w0 < (uint32_t)kStage ? T.npieces - w0 : (uint32_t)kStage;
    __syncthreads();  // the previous window is no longer read
    for (uint32_t i0 = 0; i0 < wn; i0 += (uint32_t)(kThreads * kStageBatch)) {
      double v[kStageBatch];
      uint32_t o[kStageBatch];
#pragma unroll
      for (int u = 0; u < kStageBatch; ++u) {
        const uint32_t i = i0 + (uint32_t)u * kThreads + t;
        v[u] = i < wn ? T.partials[w0 + i] : 0.0;
        o[u] = i < wn ? T.pieces[w0 + i].tensor : 0u;
      }
#pragma unroll
      for (int u = 0; u < kStageBatch; ++u) {
        const uint32_t i = i0 + (uint32_t)u * kThreads + t;
        if (i < wn) {
          stage[i] = v[u];
          owner[i] = o[u];
        }
      }
    }
    __syncthreads();
    // level 1: this lane's chunk, cut where a tensor starts
    const uint32_t C = (wn + kThreads - 1) / kThreads;
    {
      const uint32_t cb = t * C, ce = cb + C < wn ? cb + C : wn;
      if (cb < ce) {
        uint32_t start = cb;
        double acc = stage[cb];
        for (uint32_t i = cb + 1; i < ce; ++i) {
          const double v = stage[i];
          if (owner[i] != owner[i - 1]) {
            stage[start] = acc;
            start = i;
            acc = v;
          } else {
            acc += v;
          }
        }
        stage[start] = acc;
      }
    }
    __syncthreads();
    // level 2: each tensor's fragments in this window
    const uint32_t wend = w0 + wn;
    if (has0) {
      const uint32_t lo = b0 > w0 ? b0 : w0, hi = e0 < wend ? e0 : wend;
      if (lo < hi) S0 += tensor_in_window(stage, C, lo - w0, hi - w0);
    }
    for (int32_t k = k0 + kThreads; k < T.ntensors; k += kThreads) {
      const uint32_t b = T.first[k], e = T.first[k + 1];
      const uint32_t lo = b > w0 ? b : w0, hi = e < wend ? e : wend;
      if (lo < hi) out[k].sumsq += tensor_in_window(stage, C, lo - w0, hi - w0);
    }
  }
  double mine = 0.0;
  int nf_mine = 0;
  double sumsq0 = 0.0;
  int nf0 = 0;
  if (has0) {
    sumsq0 = (avg * avg) * S0;
    nf0 = nonfinite_of(S0, avg);
    out[k0].sumsq = sumsq0;
    out[k0].norm = sqrt(sumsq0);
    out[k0].nonfinite = nf0;
    mine = S0;
    nf_mine = nf0;
  }
  for (int32_t k = k0 + kThreads; k < T.ntensors; k += kThreads) {
    const double S = out[k].sumsq;
    const double sumsq = (avg * avg) * S;
    const int nf = nonfinite_of(S, avg);
    out[k].sumsq = sumsq;
    out[k].norm = sqrt(sumsq);
    out[k].nonfinite = nf;
    mine += S;
    nf_mine |= nf;
  }
  const double S = wg_sum(mine, red);
  const int nf_any = __syncthreads_or(nf_mine);
  const int skip = (clip && err && nf_any) ? 1 : 0;
  int clipped_mine = 0;
  for (int32_t k = k0; k < T.ntensors; k += kThreads) {
    const double sumsq = k == k0 ? sumsq0 : out[k].sumsq;
    const int nf = k == k0 ? nf0 : out[k].nonfinite;
    if (clip) {
      const Decision d = decide(sumsq, nf, max_norm, avg, err);
      out[k].scale = (skip || d.s == 1.0) ? 1.0 : d.s;
      out[k].clipped = d.clipped;
      clipped_mine |= d.clipped;
    } else {
      out[k].scale = 1.0;
      out[k].clipped = 0;
    }
  }
  const int clipped_any = __syncthreads_or(clipped_mine);
  // the partials have all been read: overwrite them with NaN, so that a
  // partial read before it is written could only show up as a NaN norm
  for (uint32_t i = t; i < T.npieces; i += kThreads) T.partials[i] = __builtin_nan("");
  if (t == 0) {
    write_norm(res, S, avg);
    res->nonfinite = nf_any | res->nonfinite;
    res->scale = 1.0;
    res->clipped = clipped_any;
    res->skipped = skip;
    if (clip) res->max_norm = max_norm;
    res->decided = clip ? 1 : 0;
    res->status = 0;
    res->handed_back = 0;
  }
}

// Every piece multiplied by its tensor's factor (nothing written where that
// factor is 1).  Grid: npieces.
template <int DT, bool NTS>
__global__ __launch_bounds__(kThreads) void k_tensor_scale(TensorPlan T, const gclip_tensor_result* out) {
  const TPiece pc = ld_table(T.pieces, blockIdx.x);
  const double s64 = out[uniform32(pc.tensor)].scale;
  if (s64 == 1.0) return;
  piece_scale<DT, NTS>(T, pc, s64, (float)s64);
}

// ---------------------------------------------------------------- the last microbatch's += with the norm
// Backprop lesson, "Accumulation across microbatches": acc += g, rounded once
// to the storage format.  The 16-bit formats add in fp32 and round to the
// format: fp32 has at least 2p + 2 bits for both (p = 11, 8), so the two
// roundings agree with the format's own correctly rounded addition.  The
// squares of the values written are summed as in the norm pass, one partial
// per piece; k_tensor_decide then reduces them.
template <int DT>
__device__ __forceinline__ uint32_t add_elem(uint32_t a, uint32_t g) {
  if constexpr (DT == GCLIP_F32) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(g));
  } else if constexpr (DT == GCLIP_F16) {
    const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)a) + (float)__builtin_bit_cast(_Float16, (uint16_t)g);
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)s);
  } else {
    const float s = __uint_as_float(a << 16) + __uint_as_float(g << 16);
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)s);
  }
}

template <int DT>
__device__ __forceinline__ u32x4 add_vec(u32x4 a, u32x4 g) {
  u32x4 r;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if constexpr (DT == GCLIP_F32) {
      r[c] = add_elem<DT>(a[c], g[c]);
    } else {
      r[c] = add_elem<DT>(a[c] & 0xffffu, g[c] & 0xffffu) | (add_elem<DT>(a[c] >> 16, g[c] >> 16) << 16);
    }
  }
  return r;
}

// One workgroup per piece; gdelta[t] is the byte offset from tensor t of the
// list to tensor t of the contribution (same alignment, so the same vector
// layout).
template <int DT, bool NTS>
__global__ __launch_bounds__(kThreads) void k_accum_partial(TensorPlan T, const uint64_t* gdelta) {
  __shared__ double red[kWaves];
  const TPiece pc = ld_table(T.pieces, blockIdx.x);
  const uint64_t d = ld_table(gdelta, (uint64_t)uniform32(pc.tensor));
  const uint32_t t = threadIdx.x;
  double acc[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) acc[u] = 0.0;
  g_u32x4* base = reinterpret_cast<g_u32x4*>(uniform64(pc.addr));
  const g_u32x4* gbase = reinterpret_cast<const g_u32x4*>(uniform64(pc.addr + d));
  const uint32_t nvec = uniform32(pc.nvec);
  for (uint32_t j = 0; j < nvec; j += kPieceGroup) {
    u32x4 q[kUnroll], h[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t i = piece_index(j, u, t);
      const bool ok = i < nvec;
      q[u] = ok ? ld_vec<kNtSum>(base + i) : u32x4{0u, 0u, 0u, 0u};
      h[u] = ok ? ld_vec<kNtSum>(gbase + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t i = piece_index(j, u, t);
      const u32x4 n = add_vec<DT>(q[u], h[u]);
      if (i < nvec) st_vec<NTS>(base + i, n);
      acc[u] += vec_sumsq<DT>(n);
    }
  }
  double s = 0.0;
  for (uint32_t i = t; i < pc.sc_count; i += kThreads) {
    const uint64_t a = T.sc_addr[pc.sc_begin + i];
    const uint32_t v = add_elem<DT>(load_elem<DT>(a), load_elem<DT>(a + d));
    store_elem<DT>(a, v);
    s += elem_square<DT>(v);
  }
  const double part = wg_sum(lane_total(acc, s), red);
  if (t == 0) T.partials[blockIdx.x] = part;
}

// ---------------------------------------------------------------- AdamW on the clipped gradient
// Grad clip lesson, "Order matters: Pre-Adam": the optimizer's moments see
// the clipped gradient.  Each workgroup updates one piece of one tensor: the
// weights p and moments m, v (binary32) from the gradient times the factor s
// of the clip decision, which is read from the result block -- the clipped
// gradient itself is never written.
typedef __attribute__((address_space(1))) float g_f32;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) u32x2 g_u32x2;

template <int DT>
__device__ __forceinline__ float grad_value(uint32_t bits) {
  if constexpr (DT == GCLIP_F32) return __uint_as_float(bits);
  else if constexpr (DT == GCLIP_F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
  else return __uint_as_float(bits << 16);
}

// Four consecutive gradient values from a 4-element-aligned address.
template <int DT>
__device__ __forceinline__ void load_grad4(uint64_t a, float (&g)[4]) {
  if constexpr (DT == GCLIP_F32) {
    const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const g_u32x4*>(a));
#pragma unroll
    for (int k = 0; k < 4; ++k) g[k] = __uint_as_float(q[k]);
  } else {
    const u32x2 q = __builtin_nontemporal_load(reinterpret_cast<const g_u32x2*>(a));
    g[0] = grad_value<DT>(q[0] & 0xffffu);
    g[1] = grad_value<DT>(q[0] >> 16);
    g[2] = grad_value<DT>(q[1] & 0xffffu);
    g[3] = grad_value<DT>(q[1] >> 16);
  }
}

__device__ __forceinline__ void adamw_elem(float& p, float& m, float& v, float g, const AdamHp& h) {
  m = h.b1 * m + h.omb1 * g;
  v = h.b2 * v + h.omb2 * (g * g);
  const float denom = sqrtf(v) * h.inv_sqrt_bc2 + h.eps;
  p = p * h.decay - h.step_size * (m / denom);
}

#ifndef GCLIP_ADAM_UNROLL
#define GCLIP_ADAM_UNROLL 4
#endif
#ifndef GCLIP_ADAM_NT_STORE
#define GCLIP_ADAM_NT_STORE 0
#endif
constexpr int kAdamUnroll = GCLIP_ADAM_UNROLL;
constexpr bool kAdamNtStore = GCLIP_ADAM_NT_STORE != 0;
#ifndef GCLIP_ADAM_NT_LOAD
#define GCLIP_ADAM_NT_LOAD 1
#endif
constexpr bool kAdamNtLoad = GCLIP_ADAM_NT_LOAD != 0;

template <int DT>
__global__ __launch_bounds__(kAdamThreads) void k_adamw_clip(AdamPlan P, AdamHp h, double max_norm, AvgSrc avs,
                                                             int err, gclip_result* res) {
  const double avg = avg_value(avs);
  const Decision d = decide(res->sumsq, res->nonfinite, max_norm, avg, err);
  if (blockIdx.x == 0 && threadIdx.x == 0) write_decision(res, d, max_norm);
  if (d.skip || blockIdx.x >= P.npieces) return;
  const float s = (float)d.s;
  const AdamPiece pc = ld_table(P.pieces, blockIdx.x);
  constexpr uint32_t es = DT == GCLIP_F32 ? 4u : 2u;
  if (pc.vec) {
    // kAdamUnroll iterations at a time: every load first, then the math, then the stores
    constexpr uint32_t stride = kAdamThreads * 4u;
    for (uint32_t i0 = threadIdx.x * 4u; i0 < pc.count; i0 += stride * kAdamUnroll) {
      u32x4 p4[kAdamUnroll], m4[kAdamUnroll], v4[kAdamUnroll];
      float g[kAdamUnroll][4];
#pragma unroll
      for (int u = 0; u < kAdamUnroll; ++u) {
        const uint32_t i = i0 + (uint32_t)u * stride;
        if (i < pc.count) {
          p4[u] = ld_vec<kAdamNtLoad>(reinterpret_cast<const g_u32x4*>(pc.p + (uint64_t)i * 4u));
          m4[u] = ld_vec<kAdamNtLoad>(reinterpret_cast<const g_u32x4*>(pc.m + (uint64_t)i * 4u));
          v4[u] = ld_vec<kAdamNtLoad>(reinterpret_cast<const g_u32x4*>(pc.v + (uint64_t)i * 4u));
          load_grad4<DT>(pc.g + (uint64_t)i * es, g[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < kAdamUnroll; ++u) {
        const uint32_t i = i0 + (uint32_t)u * stride;
        if (i < pc.count) {
          u32x4 po, mo, vo;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            float pk = __uint_as_float(p4[u][k]), mk = __uint_as_float(m4[u][k]), vk = __uint_as_float(v4[u][k]);
            adamw_elem(pk, mk, vk, g[u][k] * s, h);
            po[k] = __float_as_uint(pk);
            mo[k] = __float_as_uint(mk);
            vo[k] = __float_as_uint(vk);
          }
          st_vec<kAdamNtStore>(reinterpret_cast<g_u32x4*>(pc.p + (uint64_t)i * 4u), po);
          st_vec<kAdamNtStore>(reinterpret_cast<g_u32x4*>(pc.m + (uint64_t)i * 4u), mo);
          st_vec<kAdamNtStore>(reinterpret_cast<g_u32x4*>(pc.v + (uint64_t)i * 4u), vo);
        }
      }
    }
  } else {
    for (uint32_t i = threadIdx.x; i < pc.count; i += kAdamThreads) {
      g_f32* pp = reinterpret_cast<g_f32*>(pc.p + (uint64_t)i * 4u);
      g_f32* mp = reinterpret_cast<g_f32*>(pc.m + (uint64_t)i * 4u);
      g_f32* vp = reinterpret_cast<g_f32*>(pc.v + (uint64_t)i * 4u);
      float pk = *pp, mk = *mp, vk = *vp;
      const float g = grad_value<DT>(load_elem<DT>(pc.g + (uint64_t)i * es));
      adamw_elem(pk, mk, vk, g * s, h);
      *pp = pk;
      *mp = mk;
      *vp = vk;
    }
  }
}

// ---------------------------------------------------------------- host launchers
int worker_threads() { return kThreads; }
uint64_t resident_cap_vectors() { return kResidentCap; }
ChunkShape chunk_shape() {
  ChunkShape c;
  c.group_vectors = kGroupVectors;
  c.sum_chunks_per_worker = (uint32_t)kSumChunksPerWorker;
  c.scale_min_vectors = (uint64_t)kScaleMinSteps * kThreads;
  c.scale_max_vectors = (uint64_t)kScaleMaxSteps * kThreads;
  c.scale_guide = (uint32_t)kScaleGuide;
  return c;
}

hipError_t launch_norm(const DevPlan& p, int32_t dtype, AvgSrc avg, gclip_result* res, hipStream_t st) {
  const dim3 grid((unsigned)p.nworkers), block(kThreads);
  switch (dtype) {
    case GCLIP_F32: hipLaunchKernelGGL(k_grad_norm_partial<GCLIP_F32>, grid, block, 0, st, p, avg, res); break;
    case GCLIP_F16: hipLaunchKernelGGL(k_grad_norm_partial<GCLIP_F16>, grid, block, 0, st, p, avg, res); break;
    default: hipLaunchKernelGGL(k_grad_norm_partial<GCLIP_BF16>, grid, block, 0, st, p, avg, res); break;
  }
  return hipGetLastError();
}

// Kernel of dtype DT with ordinary (NTS false) or nontemporal stores.
template <bool NTS>
const void* scale_kernel(int32_t dtype) {
  return dtype == GCLIP_F32   ? (const void*)k_grad_scale<GCLIP_F32, NTS>
         : dtype == GCLIP_F16 ? (const void*)k_grad_scale<GCLIP_F16, NTS>
                              : (const void*)k_grad_scale<GCLIP_BF16, NTS>;
}
template <bool NTS>
const void* fused_kernel(int32_t dtype) {
  return dtype == GCLIP_F32   ? (const void*)k_grad_clip_fused<GCLIP_F32, NTS>
         : dtype == GCLIP_F16 ? (const void*)k_grad_clip_fused<GCLIP_F16, NTS>
                              : (const void*)k_grad_clip_fused<GCLIP_BF16, NTS>;
}

hipError_t launch_scale(const DevPlan& p, int32_t dtype, double max_norm, AvgSrc avg, int err, gclip_result* res,
                        hipStream_t st) {
  DevPlan pc = p;
  void* args[] = {&pc, &max_norm, &avg, &err, &res};
  const void* fn = p.nt_store ? scale_kernel<true>(dtype) : scale_kernel<false>(dtype);
  return hipLaunchKernel(fn, dim3((unsigned)p.nworkers), dim3(kThreads), args, 0, st);
}

hipError_t launch_fused(const DevPlan& p, int32_t dtype, double max_norm, AvgSrc avg, int err, gclip_result* res,
                        uint32_t epoch, uint64_t wait_ticks, hipStream_t st) {
  DevPlan pc = p;
  void* args[] = {&pc, &max_norm, &avg, &err, &res, &epoch, &wait_ticks};
  const void* fn = p.nt_store ? fused_kernel<true>(dtype) : fused_kernel<false>(dtype);
  return hipLaunchKernel(fn, dim3((unsigned)p.nworkers), dim3(kThreads), args, 0, st);
}

hipError_t launch_tensor_norm(const TensorPlan& T, int32_t dtype, AvgSrc avg, double max_norm, int clip, int err,
                              gclip_tensor_result* out, gclip_result* res, hipStream_t st) {
  if (T.npieces > 0) {
    const dim3 grid(T.npieces), block(kThreads);
    switch (dtype) {
      case GCLIP_F32: hipLaunchKernelGGL(k_tensor_partial<GCLIP_F32>, grid, block, 0, st, T); break;
      case GCLIP_F16: hipLaunchKernelGGL(k_tensor_partial<GCLIP_F16>, grid, block, 0, st, T); break;
      default: hipLaunchKernelGGL(k_tensor_partial<GCLIP_BF16>, grid, block, 0, st, T); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_tensor_decide, dim3(1), dim3(kThreads), 0, st, T, avg, max_norm, clip, err, out, res);
  return hipGetLastError();
}

template <bool NTS>
const void* tensor_scale_kernel(int32_t dtype) {
  return dtype == GCLIP_F32   ? (const void*)k_tensor_scale<GCLIP_F32, NTS>
         : dtype == GCLIP_F16 ? (const void*)k_tensor_scale<GCLIP_F16, NTS>
                              : (const void*)k_tensor_scale<GCLIP_BF16, NTS>;
}

hipError_t launch_tensor_scale(const TensorPlan& T, int32_t dtype, const gclip_tensor_result* out, hipStream_t st) {
  if (T.npieces == 0) return hipSuccess;
  TensorPlan tc = T;
  void* args[] = {&tc, &out};
  const void* fn = T.nt_store ? tensor_scale_kernel<true>(dtype) : tensor_scale_kernel<false>(dtype);
  return hipLaunchKernel(fn, dim3(T.npieces), dim3(kThreads), args, 0, st);
}

template <bool NTS>
const void* accum_kernel(int32_t dtype) {
  return dtype == GCLIP_F32   ? (const void*)k_accum_partial<GCLIP_F32, NTS>
         : dtype == GCLIP_F16 ? (const void*)k_accum_partial<GCLIP_F16, NTS>
                              : (const void*)k_accum_partial<GCLIP_BF16, NTS>;
}

hipError_t launch_accumulate_norm(const TensorPlan& T, int32_t dtype, const uint64_t* gdelta, AvgSrc avg,
                                  gclip_tensor_result* out, gclip_result* res, hipStream_t st) {
  if (T.npieces > 0) {
    TensorPlan tc = T;
    void* args[] = {&tc, &gdelta};
    const void* fn = T.nt_store ? accum_kernel<true>(dtype) : accum_kernel<false>(dtype);
    const hipError_t e = hipLaunchKernel(fn, dim3(T.npieces), dim3(kThreads), args, 0, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_tensor_decide, dim3(1), dim3(kThreads), 0, st, T, avg, 0.0, 0, 0, out, res);
  return hipGetLastError();
}

hipError_t launch_adamw(const AdamPlan& plan, int32_t dtype, const AdamHp& h, double max_norm, AvgSrc avg, int err,
                        gclip_result* res, hipStream_t st) {
  const dim3 grid(plan.npieces > 0 ? plan.npieces : 1u), block(kAdamThreads);
  switch (dtype) {
    case GCLIP_F32: hipLaunchKernelGGL(k_adamw_clip<GCLIP_F32>, grid, block, 0, st, plan, h, max_norm, avg, err, res); break;
    case GCLIP_F16: hipLaunchKernelGGL(k_adamw_clip<GCLIP_F16>, grid, block, 0, st, plan, h, max_norm, avg, err, res); break;
    default: hipLaunchKernelGGL(k_adamw_clip<GCLIP_BF16>, grid, block, 0, st, plan, h, max_norm, avg, err, res); break;
  }
  return hipGetLastError();
}

// The loss scale after a step (dynamic loss scaling as published by
// Micikevicius et al.): found-inf multiplies it by backoff and restarts the
// count of clean steps; a clean step counts, and the interval-th one
// multiplies the scale by growth unless that is not finite in binary32.
// One thread; the step's kernels ran before it on the same stream.
__global__ void k_amp_update(const gclip_result* res, gclip_amp_state* st, double growth, double backoff,
                             int32_t interval) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  const int32_t inf = res->nonfinite ? 1 : 0;
  st->found_inf = inf;
  if (inf) {
    st->scale = (float)((double)st->scale * backoff);
    st->growth_tracker = 0;
    return;
  }
  const int32_t clean = st->growth_tracker + 1;
  if (clean == interval) {
    const float grown = (float)((double)st->scale * growth);
    if (__builtin_isfinite(grown)) st->scale = grown;
    st->growth_tracker = 0;
  } else {
    st->growth_tracker = clean;
  }
}

hipError_t launch_amp_update(const gclip_result* res, gclip_amp_state* st, double growth, double backoff,
                             int32_t interval, hipStream_t s) {
  hipLaunchKernelGGL(k_amp_update, dim3(1), dim3(64), 0, s, res, st, growth, backoff, interval);
  return hipGetLastError();
}

// Workgroups of the fused kernel that fit on one compute unit at once (the
// smaller of its two store variants).
hipError_t fused_capacity(int32_t dtype, int* blocks_per_cu) {
  int a = 0, b = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, fused_kernel<false>(dtype), kThreads, 0);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, fused_kernel<true>(dtype), kThreads, 0);
  *blocks_per_cu = a < b ? a : b;
  return e;
}

}  // namespace gclip
