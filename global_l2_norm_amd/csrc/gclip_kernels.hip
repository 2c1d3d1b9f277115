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
//   - one workgroup of kThreads per compute unit.  For the sum of squares,
//     worker w reads a fixed part of the list's 16-byte vector space
//     (gclip_plan.hpp): an equal share of the streamed region and its block
//     at the end of the space.  For scaling, which needs no partial sums, the
//     workers claim chunks at run time from eight pools, one per XCD, so that
//     the XCDs that stream faster take more of them.  Loads are dwordx4 with
//     kUnroll vectors in flight per lane, the next group's loads issued
//     before the current group is used;
//   - each vector's squares are summed in fp32 and added into per-lane
//     binary64 accumulators (vec_sumsq states when a vector is summed again
//     in binary64), so the sum cannot overflow and is non-finite exactly when
//     some element is NaN or +-Inf;
//   - lane sums are reduced by an xor butterfly inside each wave and in wave
//     order through LDS into one partial per worker; the partials are summed
//     in index order by whichever workgroup arrives last (an agent-scope
//     ticket), so the bits of the norm do not depend on scheduling and both
//     paths give the same bits; cross-workgroup data moves only through
//     agent-scope atomics (see complete_stores);
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

constexpr uint32_t kSpinLimit = 1u << 26;  // bounded wait at the grid barrier

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
// that way on MI355X.  Stores stay ordinary: next to nontemporal loads,
// nontemporal stores made the read-modify-write passes markedly slower.  (Both kinds of load can be
// chosen per pass at build time.)
constexpr bool kNtSum = GCLIP_NT_SUM != 0;
constexpr bool kNtScale = GCLIP_NT_SCALE != 0;

template <bool NT>
__device__ __forceinline__ u32x4 ld_vec(const g_u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
__device__ __forceinline__ void st_vec(g_u32x4* p, u32x4 q) { *p = q; }
template <bool NT>
__device__ __forceinline__ u32x4 load_vec(uint64_t a) { return ld_vec<NT>(reinterpret_cast<const g_u32x4*>(a)); }
__device__ __forceinline__ void store_vec(uint64_t a, u32x4 q) { st_vec(reinterpret_cast<g_u32x4*>(a), q); }

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
template <typename F>
__device__ __forceinline__ void store_group(const DevPlan& p, Cursor& cur, uint64_t vb, uint64_t ve, uint64_t j,
                                            uint64_t j1, F&& f) {
  const uint32_t t = threadIdx.x;
  uint64_t base = 0;
  const int kind = group_kind(cur, vb, ve, j, j1, base);
  if (kind == kGroupFull) {
    g_u32x4* g = reinterpret_cast<g_u32x4*>(uniform64(base));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) st_vec(&g[u * kThreads + t], f(u));
  } else if (kind == kGroupTail) {
    g_u32x4* g = reinterpret_cast<g_u32x4*>(uniform64(base));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (tail_ok(vb, ve, j, j1, u, t)) st_vec(&g[u * kThreads + t], f(u));
  } else {
    const uint64_t b0 = vb + j * kThreads;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (j + u < j1) {
        const uint64_t b = b0 + (uint64_t)u * kThreads, v = b + t;
        const uint64_t a = step_addr(p, cur, b, ve, v);
        if (v < ve) store_vec(a, f(u));
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
  const uint64_t b = p.wk_scbegin[w], e = p.wk_scbegin[w + 1];
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
    store_group(p, c2, vb, ve, j, j1, [&](int u) { return scale_vec<DT>(q[u], s64, s32); });
  }
}

template <int DT>
__device__ __forceinline__ void scale_scalars(const DevPlan& p, int w, double s64, float s32) {
  const uint64_t b = p.wk_scbegin[w], e = p.wk_scbegin[w + 1];
  for (uint64_t i = b + threadIdx.x; i < e; i += kThreads) {
    const uint64_t a = p.sc_addr[i];
    store_elem<DT>(a, scale_elem<DT>(load_elem<DT>(a), s64, s32));
  }
}

// ---------------------------------------------------------------- chunk claiming
constexpr uint32_t kNone = 0xffffffffu;

// Chunk c lives in pool c % kPools; pool q holds chunks q, q + kPools, ...
// below nch.
__device__ __forceinline__ uint32_t pool_size(uint32_t nch, uint32_t q) {
  return q < nch ? (nch - q + kPools - 1) / kPools : 0u;
}

// Claim state of one workgroup, kept by its thread 0: the pool it draws from
// (its own XCD's first) and how many pools it has found empty.
struct Claimer {
  uint32_t pool, dry;
};

// The next chunk for this workgroup, or kNone once every pool is empty.
// Thread 0 only.  Each pool's counter only grows during a launch, so a pool
// found empty stays empty.
__device__ __forceinline__ uint32_t claim(uint32_t* pools, uint32_t nch, Claimer& cl) {
  while (cl.dry < (uint32_t)kPools) {
    const uint32_t q = cl.pool;
    const uint32_t k = __hip_atomic_fetch_add(&pools[q * kSyncLineWords], 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    if (k < pool_size(nch, q)) return q + k * (uint32_t)kPools;
    cl.pool = (q + 1) % (uint32_t)kPools;
    ++cl.dry;
  }
  return kNone;
}

__device__ __forceinline__ uint32_t* scale_pools(const DevPlan& p) { return p.sync + kSyncLineWords; }

__device__ __forceinline__ void reset_pools(uint32_t* pools) {
  for (int q = 0; q < kPools; ++q)
    __hip_atomic_store(&pools[q * kSyncLineWords], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Claims run two chunks ahead: the chunk after next is claimed while the
// current one streams and is handed over at the per-chunk barrier through
// LDS slot i % 2 (a slot is rewritten only two barriers after it was read).
struct ClaimSlots {
  uint32_t claim[2];
};

// Scale in place every chunk below nch that this workgroup claims, each cut
// at `end`.  The next chunk's first group is loaded before the current
// chunk's last stores.
template <int DT>
__device__ __forceinline__ void scale_chunks(const DevPlan& p, ClaimSlots& sl, uint32_t nch, uint64_t end,
                                             double s64, float s32) {
  const uint32_t t = threadIdx.x;
  uint32_t* pools = scale_pools(p);
  Claimer cl{blockIdx.x % (uint32_t)kPools, 0u};
  if (t == 0) {
    sl.claim[0] = claim(pools, nch, cl);
    sl.claim[1] = claim(pools, nch, cl);
  }
  __syncthreads();
  uint32_t c = sl.claim[0], cn = sl.claim[1];
  __syncthreads();
  Cursor cur;
  u32x4 q[kUnroll];
  if (c != kNone) {
    const Range r = chunk_range(p, c, end);
    cursor_load(p, cur, r.seg);
    load_group<kNtScale>(p, cur, r.b, r.e, 0, range_steps(r), q);
  }
  for (uint32_t i = 0; c != kNone; ++i) {
    uint32_t cnn = kNone;
    if (t == 0) cnn = claim(pools, nch, cl);
    const Range r = chunk_range(p, c, end);
    const uint64_t ns = range_steps(r);
    Cursor cst;
    cursor_load(p, cst, r.seg);
    Cursor curn = cur;
    for (uint64_t j = 0; j < ns; j += kUnroll) {
      u32x4 q2[kUnroll];
      if (j + kUnroll < ns) {
        load_group<kNtScale>(p, cur, r.b, r.e, j + kUnroll, ns, q2);
      } else if (cn != kNone) {
        const Range rn = chunk_range(p, cn, end);
        cursor_load(p, curn, rn.seg);
        load_group<kNtScale>(p, curn, rn.b, rn.e, 0, range_steps(rn), q2);
      } else {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) q2[u] = u32x4{0u, 0u, 0u, 0u};
      }
      store_group(p, cst, r.b, r.e, j, ns, [&](int u) { return scale_vec<DT>(q[u], s64, s32); });
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) q[u] = q2[u];
    }
    const uint32_t par = i & 1u;
    if (t == 0) sl.claim[par] = cnn;
    __syncthreads();
    c = cn;
    cn = sl.claim[par];
    cur = curn;
  }
}

// Chunks that cover [0, end).
__device__ __forceinline__ uint32_t chunks_below(const DevPlan& p, uint64_t end) {
  return (uint32_t)((end + p.cv - 1) / p.cv);
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

// Sum of the workers' partials in index order (lane i takes i, i + kThreads, ...).
__device__ __forceinline__ double partials_sum(const DevPlan& p, double* red) {
  double v = 0.0;
  const uint32_t n = (uint32_t)p.nworkers;
  for (uint32_t i = threadIdx.x; i < n; i += kThreads)
    v += __hip_atomic_load(&p.partials[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return wg_sum(v, red);
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

__device__ __forceinline__ void write_norm(gclip_result* res, double S, double avg) {
  const double sumsq = (avg * avg) * S;
  res->sumsq = sumsq;
  res->norm = sqrt(sumsq);
  res->nonfinite = __builtin_isfinite(S) ? 0 : 1;
}

__device__ __forceinline__ void write_decision(gclip_result* res, const Decision& d, double max_norm) {
  const bool wrote = !(d.skip || d.s == 1.0);
  res->scale = wrote ? d.s : 1.0;
  res->clipped = d.clipped;
  res->skipped = d.skip;
  res->max_norm = max_norm;
  res->decided = 1;
}

// Cross-workgroup data (partials, the decision, the counters) is written and
// read only with agent-scope atomics, which go to the device-coherent level
// of the memory system.  Waiting for those stores to complete before the
// next atomic is issued orders them for every reader, so no agent-scope
// fence is needed: on gfx950 such a fence writes back and invalidates the
// whole L2 of the XCD, which costs ~18 us when 256 workgroups do it at the
// end of a pass.
__device__ __forceinline__ void complete_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Ticket: returns true in the last workgroup to arrive (all threads).  The
// caller's partials must already be stored (agent-scope atomics).
__device__ __forceinline__ bool arrive(const DevPlan& p, int* flag) {
  if (threadIdx.x == 0) {
    complete_stores();
    const uint32_t prev = __hip_atomic_fetch_add(&p.sync[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = (prev == (uint32_t)p.nworkers - 1u) ? 1 : 0;
  }
  __syncthreads();
  return *flag != 0;
}

// Blocks handed back by the fused kernel.  Worker w's state word is kHeld
// while w holds its block (or has written it), kHanded once w has stopped
// waiting at the decision and left its block unscaled in memory, kTaken once
// another workgroup has taken it over.  sync[3] counts the hand-backs.
constexpr uint32_t kHeld = 0u, kHanded = 2u, kTaken = 3u;

struct HandSlots {
  uint32_t n;
  uint32_t list[kThreads];
};

// Take over every block handed back so far and scale it from memory, with
// the worker's single elements (whole workgroup).
template <int DT>
__device__ void take_handed_blocks(const DevPlan& p, HandSlots& hs, double s64, float s32) {
  for (uint32_t base = 0; base < (uint32_t)p.nworkers; base += kThreads) {
    if (threadIdx.x == 0) hs.n = 0;
    __syncthreads();
    const uint32_t i = base + threadIdx.x;
    if (i < (uint32_t)p.nworkers &&
        __hip_atomic_load(&p.bstate[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == kHanded) {
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
__device__ void finish(const DevPlan& p, gclip_result* res, bool fused, HandSlots& hs, int* flag) {
  __syncthreads();
  if (threadIdx.x == 0) {
    complete_stores();
    const uint32_t prev = __hip_atomic_fetch_add(&p.sync[4], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = (prev == (uint32_t)p.nworkers - 1u) ? 1 : 0;
  }
  __syncthreads();
  if (*flag == 0) return;
  if (fused) {
    const uint32_t handed = __hip_atomic_load(&p.sync[3], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (handed != 0u) {
      const double s = __hip_atomic_load(&p.bcast[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t skip = __hip_atomic_load(&p.sync[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (skip == 0u && s != 1.0) take_handed_blocks<DT>(p, hs, s, (float)s);
      __syncthreads();
      for (uint32_t i = threadIdx.x; i < (uint32_t)p.nworkers; i += kThreads)
        __hip_atomic_store(&p.bstate[i], kHeld, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (threadIdx.x == 0) {
      res->handed_back = (int32_t)handed;
      __hip_atomic_store(&p.sync[3], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (threadIdx.x == 0) {
    reset_pools(scale_pools(p));
    __hip_atomic_store(&p.sync[4], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// After the last workgroup has summed the partials it overwrites them with
// NaN, so a partial that was somehow read before it was written could only
// ever show up as a NaN norm, never as a plausible wrong one.
__device__ __forceinline__ void poison_partials(const DevPlan& p) {
  const uint32_t n = (uint32_t)p.nworkers;
  for (uint32_t i = threadIdx.x; i < n; i += kThreads)
    __hip_atomic_store(&p.partials[i], __builtin_nan(""), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- kernels
// Worker w's partial sum of squares: its streamed share, then its block, then
// its single elements, reduced over the workgroup.  The fused kernel adds the
// same values in the same order, so both paths give the same bits.
template <int DT>
__device__ __forceinline__ void norm_share(const DevPlan& p, int w, double (&acc)[kUnroll]) {
  const Range sh = share_range(p, w);
  if (sh.b < sh.e) {
    Cursor cur;
    cursor_load(p, cur, sh.seg);
    norm_steps<DT>(p, cur, sh.b, sh.e, 0, range_steps(sh), acc);
  }
}

// Kernels 1 and 2 of the pages' pipeline: one partial sum of squares per
// worker, with the final reduction folded into the last workgroup to arrive.
template <int DT>
__global__ __launch_bounds__(kThreads) void k_grad_norm_partial(DevPlan p, double avg, gclip_result* res) {
  __shared__ double red[kWaves];
  __shared__ int flag;
  const int w = blockIdx.x;
  double acc[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) acc[u] = 0.0;
  norm_share<DT>(p, w, acc);
  const Range r = block_range(p, w);
  if (r.b < r.e) {
    Cursor cur;
    cursor_load(p, cur, r.seg);
    norm_steps<DT>(p, cur, r.b, r.e, 0, range_steps(r), acc);
  }
  const double part = wg_sum(lane_total(acc, norm_scalars<DT>(p, w)), red);
  if (threadIdx.x == 0) __hip_atomic_store(&p.partials[w], part, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (arrive(p, &flag)) {
    const double S = partials_sum(p, red);
    poison_partials(p);
    if (threadIdx.x == 0) {
      write_norm(res, S, avg);
      res->scale = 1.0;
      res->clipped = 0;
      res->skipped = 0;
      res->decided = 0;
      res->status = 0;
      res->handed_back = 0;
      __hip_atomic_store(&p.sync[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Kernel 3: the decision from the device result block, then g <- g * s over
// the chunks each workgroup claims, or no write at all.
template <int DT>
__global__ __launch_bounds__(kThreads) void k_grad_scale(DevPlan p, double max_norm, double avg, int err,
                                                         gclip_result* res) {
  __shared__ ClaimSlots sl;
  __shared__ HandSlots hs;
  __shared__ int flag;
  const int w = blockIdx.x;
  const Decision d = decide(res->sumsq, res->nonfinite, max_norm, avg, err);
  if (w == 0 && threadIdx.x == 0) write_decision(res, d, max_norm);
  if (!(d.skip || d.s == 1.0)) {
    const double s64 = d.s;
    const float s32 = (float)d.s;
    scale_chunks<DT>(p, sl, p.nchunk, p.nvec, s64, s32);
    scale_scalars<DT>(p, w, s64, s32);
  }
  finish<DT>(p, res, false, hs, &flag);
}

// The whole path in one launch.  Phase 1 streams the worker's share and
// reads its block into VGPRs and LDS; the last workgroup to arrive reduces
// the partials and decides; phase 2 writes the block straight from
// VGPRs/LDS, then reads, scales and writes the chunks of the streamed region
// it claims.  The launch does not need every workgroup resident at once: a
// workgroup that has waited wait_ticks (wall-clock ticks) for the decision
// hands its block back and exits, freeing its compute unit for the
// workgroups still to run, and the workgroups that do see the decision --
// in the end the last one to finish -- scale the handed-back blocks from
// memory.
template <int DT>
__global__ __launch_bounds__(kThreads, 1) void k_grad_clip_fused(DevPlan p, double max_norm, double avg, int err,
                                                                 gclip_result* res, uint32_t epoch,
                                                                 uint64_t wait_ticks) {
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

  double acc[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) acc[u] = 0.0;
  norm_share<DT>(p, w, acc);
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
  if (t == 0) __hip_atomic_store(&p.partials[w], part, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // grid-wide decision: the last workgroup to arrive reduces and releases
  if (t == 0) gave_up = 0;
  if (arrive(p, &flag)) {
    const double S = partials_sum(p, red);
    poison_partials(p);
    if (t == 0) {
      const double sumsq = (avg * avg) * S;
      const int nonfinite = __builtin_isfinite(S) ? 0 : 1;
      const Decision d = decide(sumsq, nonfinite, max_norm, avg, err);
      write_norm(res, S, avg);
      write_decision(res, d, max_norm);
      res->status = 0;
      bc_s = d.s;
      bc_skip = d.skip;
      __hip_atomic_store(&p.bcast[0], d.s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.sync[2], (uint32_t)d.skip, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.sync[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      complete_stores();
      __hip_atomic_store(&p.sync[1], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else if (t == 0) {
    const uint64_t t0 = wall_clock64();
    while (__hip_atomic_load(&p.sync[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
      __builtin_amdgcn_s_sleep(2);
      if (wall_clock64() - t0 > wait_ticks) {
        // hand the block back: its state is visible before the count
        __hip_atomic_store(&p.bstate[w], kHanded, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        complete_stores();
        __hip_atomic_fetch_add(&p.sync[3], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        gave_up = 1;
        break;
      }
    }
    if (!gave_up) {
      bc_s = __hip_atomic_load(&p.bcast[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      bc_skip = (int)__hip_atomic_load(&p.sync[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  const double s64 = bc_s;
  if (!gave_up && !bc_skip && s64 != 1.0) {
    const float s32 = (float)s64;
    if (r.b < r.e) {
      Cursor cur;
      cursor_load(p, cur, r.seg);
#pragma unroll
      for (int g = 0; g < kRegSteps / kUnroll; ++g) {
        if ((uint32_t)(g * kUnroll) < bs.nreg)
          store_group(p, cur, r.b, r.e, g * kUnroll, bs.nreg,
                      [&](int u) { return scale_vec<DT>(keep[g * kUnroll + u], s64, s32); });
      }
      for (uint32_t k0 = 0; k0 < bs.nlds; k0 += kUnroll)
        store_group(p, cur, r.b, r.e, bs.nreg + k0, bs.nsteps,
                    [&](int u) { return scale_vec<DT>(keep_lds[(k0 + u) * kThreads + t], s64, s32); });
    }
    scale_chunks<DT>(p, sl, chunks_below(p, p.sb), p.sb, s64, s32);
    scale_scalars<DT>(p, w, s64, s32);
    if (t == 0) handed = (int)__hip_atomic_load(&p.sync[3], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (handed) take_handed_blocks<DT>(p, hs, s64, s32);
  }
  finish<DT>(p, res, true, hs, &flag);
}

// ---------------------------------------------------------------- host launchers
int worker_threads() { return kThreads; }
uint64_t resident_cap_vectors() { return kResidentCap; }
uint64_t chunk_vectors() { return kChunkVectors; }

hipError_t launch_norm(const DevPlan& p, int32_t dtype, double avg, gclip_result* res, hipStream_t st) {
  const dim3 grid((unsigned)p.nworkers), block(kThreads);
  switch (dtype) {
    case GCLIP_F32: hipLaunchKernelGGL(k_grad_norm_partial<GCLIP_F32>, grid, block, 0, st, p, avg, res); break;
    case GCLIP_F16: hipLaunchKernelGGL(k_grad_norm_partial<GCLIP_F16>, grid, block, 0, st, p, avg, res); break;
    default: hipLaunchKernelGGL(k_grad_norm_partial<GCLIP_BF16>, grid, block, 0, st, p, avg, res); break;
  }
  return hipGetLastError();
}

hipError_t launch_scale(const DevPlan& p, int32_t dtype, double max_norm, double avg, int err, gclip_result* res,
                        hipStream_t st) {
  const dim3 grid((unsigned)p.nworkers), block(kThreads);
  switch (dtype) {
    case GCLIP_F32: hipLaunchKernelGGL(k_grad_scale<GCLIP_F32>, grid, block, 0, st, p, max_norm, avg, err, res); break;
    case GCLIP_F16: hipLaunchKernelGGL(k_grad_scale<GCLIP_F16>, grid, block, 0, st, p, max_norm, avg, err, res); break;
    default: hipLaunchKernelGGL(k_grad_scale<GCLIP_BF16>, grid, block, 0, st, p, max_norm, avg, err, res); break;
  }
  return hipGetLastError();
}

hipError_t launch_fused(const DevPlan& p, int32_t dtype, double max_norm, double avg, int err, gclip_result* res,
                        uint32_t epoch, uint64_t wait_ticks, hipStream_t st) {
  const dim3 grid((unsigned)p.nworkers), block(kThreads);
  switch (dtype) {
    case GCLIP_F32:
      hipLaunchKernelGGL(k_grad_clip_fused<GCLIP_F32>, grid, block, 0, st, p, max_norm, avg, err, res, epoch,
                         wait_ticks);
      break;
    case GCLIP_F16:
      hipLaunchKernelGGL(k_grad_clip_fused<GCLIP_F16>, grid, block, 0, st, p, max_norm, avg, err, res, epoch,
                         wait_ticks);
      break;
    default:
      hipLaunchKernelGGL(k_grad_clip_fused<GCLIP_BF16>, grid, block, 0, st, p, max_norm, avg, err, res, epoch,
                         wait_ticks);
      break;
  }
  return hipGetLastError();
}

// Workgroups of the fused kernel that fit on one compute unit at once.
hipError_t fused_capacity(int32_t dtype, int* blocks_per_cu) {
  const void* fn = dtype == GCLIP_F32   ? (const void*)k_grad_clip_fused<GCLIP_F32>
                   : dtype == GCLIP_F16 ? (const void*)k_grad_clip_fused<GCLIP_F16>
                                        : (const void*)k_grad_clip_fused<GCLIP_BF16>;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, kThreads, 0);
}

}  // namespace gclip
