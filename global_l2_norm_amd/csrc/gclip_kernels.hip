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
//   - one workgroup of kThreads per compute unit; worker w owns an equal
//     share of the list's 16-byte vector space (gclip_plan.hpp), read with
//     dwordx4 loads, kUnroll vectors in flight per lane;
//   - squares are accumulated per lane in binary64: the square of an fp32,
//     fp16 or bf16 value is exact there and the sum cannot overflow, so the
//     sum is non-finite exactly when some element is NaN or +-Inf;
//   - lane sums are reduced by an xor butterfly inside each wave and in wave
//     order through LDS; per-worker partials are summed in worker order by
//     whichever workgroup arrives last (an agent-scope ticket), so the bits
//     of the norm do not depend on scheduling; cross-workgroup data moves
//     only through agent-scope atomics (see complete_stores);
//   - the fused kernel (cooperative launch, all workgroups resident) keeps
//     the last kRegSteps + kLdsSteps steps of each worker's share in VGPRs and
//     LDS across the grid-wide decision, so the scale pass writes those bytes
//     without reading them again from HBM.
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

__device__ __forceinline__ u32x4 load_vec(uint64_t a) { return *reinterpret_cast<const g_u32x4*>(a); }
__device__ __forceinline__ void store_vec(uint64_t a, u32x4 q) { *reinterpret_cast<g_u32x4*>(a) = q; }

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

// ---------------------------------------------------------------- reductions
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

// A lane's total: its per-slot accumulators in slot order, then its single elements.
__device__ __forceinline__ double lane_total(const double (&acc)[kUnroll], double accs) {
  double t = acc[0];
#pragma unroll
  for (int u = 1; u < kUnroll; ++u) t += acc[u];
  return t + accs;
}

// Sum of the workers' partials in worker order (lane i takes i, i + kThreads, ...).
__device__ __forceinline__ double partials_sum(const DevPlan& p, double* red) {
  double v = 0.0;
  for (int i = threadIdx.x; i < p.nworkers; i += kThreads)
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

// ---------------------------------------------------------------- group loads and stores
// Load the vectors of one group into q (zeros where a lane has no vector).
__device__ __forceinline__ void load_group(const DevPlan& p, Cursor& cur, uint64_t vb, uint64_t ve, uint64_t j,
                                           uint64_t j1, u32x4 (&q)[kUnroll]) {
  const uint32_t t = threadIdx.x;
  uint64_t base = 0;
  const int kind = group_kind(cur, vb, ve, j, j1, base);
  if (kind == kGroupFull) {
    const g_u32x4* g = reinterpret_cast<const g_u32x4*>(uniform64(base));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) q[u] = g[u * kThreads + t];
  } else if (kind == kGroupTail) {
    const g_u32x4* g = reinterpret_cast<const g_u32x4*>(uniform64(base));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      q[u] = tail_ok(vb, ve, j, j1, u, t) ? g[u * kThreads + t] : u32x4{0u, 0u, 0u, 0u};
  } else {
    uint64_t a[kUnroll];
    bool ok[kUnroll];
    cross_addrs(p, cur, vb, ve, j, j1, t, a, ok);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) q[u] = ok[u] ? load_vec(a[u]) : u32x4{0u, 0u, 0u, 0u};
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
    for (int u = 0; u < kUnroll; ++u) g[u * kThreads + t] = f(u);
  } else if (kind == kGroupTail) {
    g_u32x4* g = reinterpret_cast<g_u32x4*>(uniform64(base));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (tail_ok(vb, ve, j, j1, u, t)) g[u * kThreads + t] = f(u);
  } else {
    uint64_t a[kUnroll];
    bool ok[kUnroll];
    cross_addrs(p, cur, vb, ve, j, j1, t, a, ok);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (ok[u]) store_vec(a[u], f(u));
  }
}

// ---------------------------------------------------------------- norm and scale passes
// Streamed steps [j0, j1) of a worker's share, accumulating into acc.
// Step j of a share always adds into acc[j % kUnroll]: groups start at
// multiples of kUnroll in every kernel, so the norm kernel and the fused
// kernel add the same values in the same order.
template <int DT>
__device__ __forceinline__ void norm_steps(const DevPlan& p, Cursor& cur, uint64_t vb, uint64_t ve, uint64_t j0,
                                           uint64_t j1, double (&acc)[kUnroll]) {
  for (uint64_t j = j0; j < j1; j += kUnroll) {
    u32x4 q[kUnroll];
    load_group(p, cur, vb, ve, j, j1, q);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc[u] += vec_sumsq<DT>(q[u]);
  }
}

template <int DT>
__device__ __forceinline__ double norm_scalars(const DevPlan& p, int w) {
  double s = 0.0;
  const uint64_t b = p.wk_scbegin[w], e = p.wk_scbegin[w + 1];
  for (uint64_t i = b + threadIdx.x; i < e; i += kThreads) s += elem_square<DT>(load_elem<DT>(p.sc_addr[i]));
  return s;
}

// Streamed steps [j0, j1): read, multiply, write back.  The group's loads are
// all issued before its first store.
template <int DT>
__device__ __forceinline__ void scale_steps(const DevPlan& p, Cursor& cur, uint64_t vb, uint64_t ve, uint64_t j0,
                                            uint64_t j1, double s64, float s32) {
  for (uint64_t j = j0; j < j1; j += kUnroll) {
    u32x4 q[kUnroll];
    Cursor c2 = cur;
    load_group(p, cur, vb, ve, j, j1, q);
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

// Cross-workgroup data (per-workgroup partials, the decision, the counters)
// is written and read only with agent-scope atomics, which go to the
// device-coherent level of the memory system.  Waiting for those stores to
// complete before the next atomic is issued orders them for every reader, so
// no agent-scope fence is needed: on gfx950 such a fence writes back and
// invalidates the whole L2 of the XCD, which costs ~18 us when 256
// workgroups do it at the end of a pass.
__device__ __forceinline__ void complete_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Ticket: returns true in the last workgroup to arrive (all threads).
__device__ __forceinline__ bool arrive(const DevPlan& p, int w, double part, int* flag) {
  if (threadIdx.x == 0) {
    __hip_atomic_store(&p.partials[w], part, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    complete_stores();
    const uint32_t prev = __hip_atomic_fetch_add(&p.sync[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = (prev == (uint32_t)p.nworkers - 1u) ? 1 : 0;
  }
  __syncthreads();
  return *flag != 0;
}

// After the last workgroup has summed the partials it overwrites them with
// NaN, so a partial that was somehow read before it was written could only
// ever show up as a NaN norm, never as a plausible wrong one.
__device__ __forceinline__ void poison_partials(const DevPlan& p) {
  for (int i = threadIdx.x; i < p.nworkers; i += kThreads)
    __hip_atomic_store(&p.partials[i], __builtin_nan(""), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- kernels
// Kernels 1 and 2 of the pages' pipeline: partial sums of squares, with the
// final reduction folded into the last workgroup to arrive.
template <int DT>
__global__ __launch_bounds__(kThreads) void k_grad_norm_partial(DevPlan p, double avg, gclip_result* res) {
  __shared__ double red[kWaves];
  __shared__ int flag;
  const int w = blockIdx.x;
  const uint64_t vb = p.wk_vbegin[w], ve = p.wk_vbegin[w + 1];
  double acc[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) acc[u] = 0.0;
  if (vb < ve) {
    Cursor cur;
    cursor_load(p, cur, p.wk_seg[w]);
    norm_steps<DT>(p, cur, vb, ve, 0, (ve - vb + kThreads - 1) / kThreads, acc);
  }
  const double part = wg_sum(lane_total(acc, norm_scalars<DT>(p, w)), red);
  if (arrive(p, w, part, &flag)) {
    const double S = partials_sum(p, red);
    poison_partials(p);
    if (threadIdx.x == 0) {
      write_norm(res, S, avg);
      res->scale = 1.0;
      res->clipped = 0;
      res->skipped = 0;
      res->decided = 0;
      res->status = 0;
      __hip_atomic_store(&p.sync[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Kernel 3: the decision from the device result block, then g <- g * s, or
// an immediate exit without a single write.
template <int DT>
__global__ __launch_bounds__(kThreads) void k_grad_scale(DevPlan p, double max_norm, double avg, int err,
                                                         gclip_result* res) {
  const int w = blockIdx.x;
  const Decision d = decide(res->sumsq, res->nonfinite, max_norm, avg, err);
  if (w == 0 && threadIdx.x == 0) write_decision(res, d, max_norm);
  if (d.skip || d.s == 1.0) return;
  const double s64 = d.s;
  const float s32 = (float)d.s;
  const uint64_t vb = p.wk_vbegin[w], ve = p.wk_vbegin[w + 1];
  if (vb < ve) {
    Cursor cur;
    cursor_load(p, cur, p.wk_seg[w]);
    scale_steps<DT>(p, cur, vb, ve, 0, (ve - vb + kThreads - 1) / kThreads, s64, s32);
  }
  scale_scalars<DT>(p, w, s64, s32);
}

// The whole path in one cooperative launch.  Phase 1 reads the worker's
// share once (the last resident steps into VGPRs and LDS), the last workgroup
// to arrive reduces the partials and decides, and phase 2 scales: resident
// steps are written straight from VGPRs/LDS, the rest is read again.
template <int DT>
__global__ __launch_bounds__(kThreads, 1) void k_grad_clip_fused(DevPlan p, double max_norm, double avg, int err,
                                                                 gclip_result* res, uint32_t epoch) {
  __shared__ u32x4 keep_lds[kLdsSteps * kThreads];
  __shared__ double red[kWaves];
  __shared__ int flag;
  __shared__ int timed_out;
  __shared__ double bc_s;
  __shared__ int bc_skip;
  const int w = blockIdx.x;
  const uint32_t t = threadIdx.x;
  const uint64_t vb = p.wk_vbegin[w], ve = p.wk_vbegin[w + 1];
  const FusedSplit fs = fused_split(vb, ve);
  const uint64_t js = fs.js;      // streamed steps [0, js)
  const uint32_t nreg = fs.nreg;  // register steps [js, js + nreg)
  const uint32_t nlds = fs.nlds;  // LDS steps [js + nreg, nsteps)

  double acc[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) acc[u] = 0.0;
  u32x4 keep[kRegSteps];
  Cursor cur0, cur_reg, cur_lds;
  if (vb < ve) {
    cursor_load(p, cur0, p.wk_seg[w]);
    Cursor cur = cur0;
    norm_steps<DT>(p, cur, vb, ve, 0, js, acc);
    cur_reg = cur;
    cursor_seek(p, cur_reg, vb + js * kThreads);
    cur = cur_reg;
    // register steps: issue every load first, then accumulate in step order
#pragma unroll
    for (int g = 0; g < kRegSteps / kUnroll; ++g) {
      u32x4 q[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) q[u] = u32x4{0u, 0u, 0u, 0u};
      if ((uint32_t)(g * kUnroll) < nreg) load_group(p, cur, vb, ve, js + g * kUnroll, js + nreg, q);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) keep[g * kUnroll + u] = q[u];
    }
#pragma unroll
    for (int k = 0; k < kRegSteps; ++k)
      if ((uint32_t)k < nreg) acc[k % kUnroll] += vec_sumsq<DT>(keep[k]);
    cur_lds = cur;
    cursor_seek(p, cur_lds, vb + (js + nreg) * kThreads);
    cur = cur_lds;
    for (uint32_t k0 = 0; k0 < nlds; k0 += kUnroll) {
      u32x4 q[kUnroll];
      load_group(p, cur, vb, ve, js + nreg + k0, js + nreg + nlds, q);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (k0 + u < nlds) {
          acc[u] += vec_sumsq<DT>(q[u]);
          keep_lds[(k0 + u) * kThreads + t] = q[u];
        }
      }
    }
  }
  const double part = wg_sum(lane_total(acc, norm_scalars<DT>(p, w)), red);

  // grid-wide decision: the last workgroup to arrive reduces and releases
  if (t == 0) timed_out = 0;
  if (arrive(p, w, part, &flag)) {
    const double S = partials_sum(p, red);
    poison_partials(p);
    if (t == 0) {
      const double sumsq = (avg * avg) * S;
      const int nonfinite = __builtin_isfinite(S) ? 0 : 1;
      const Decision d = decide(sumsq, nonfinite, max_norm, avg, err);
      write_norm(res, S, avg);
      write_decision(res, d, max_norm);
      bc_s = d.s;
      bc_skip = d.skip;
      __hip_atomic_store(&p.bcast[0], d.s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.sync[2], (uint32_t)d.skip, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.sync[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      complete_stores();
      __hip_atomic_store(&p.sync[1], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else if (t == 0) {
    uint32_t spins = 0;
    while (__hip_atomic_load(&p.sync[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kSpinLimit) {
        timed_out = 1;
        break;
      }
    }
    bc_s = __hip_atomic_load(&p.bcast[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bc_skip = (int)__hip_atomic_load(&p.sync[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const double s64 = bc_s;
  if (!timed_out && !bc_skip && s64 != 1.0) {
    const float s32 = (float)s64;
    if (vb < ve) {
      Cursor cur = cur_reg;
#pragma unroll
      for (int g = 0; g < kRegSteps / kUnroll; ++g) {
        if ((uint32_t)(g * kUnroll) < nreg)
          store_group(p, cur, vb, ve, js + g * kUnroll, js + nreg,
                      [&](int u) { return scale_vec<DT>(keep[g * kUnroll + u], s64, s32); });
      }
      cur = cur_lds;
      for (uint32_t k0 = 0; k0 < nlds; k0 += kUnroll)
        store_group(p, cur, vb, ve, js + nreg + k0, js + nreg + nlds,
                    [&](int u) { return scale_vec<DT>(keep_lds[(k0 + u) * kThreads + t], s64, s32); });
      cur = cur0;
      scale_steps<DT>(p, cur, vb, ve, 0, js, s64, s32);
    }
    scale_scalars<DT>(p, w, s64, s32);
  }

  // Second ticket: the last workgroup to finish records whether any
  // workgroup gave up waiting at the barrier (then its share was not scaled).
  __syncthreads();
  if (t == 0) {
    if (timed_out) __hip_atomic_fetch_or(&p.sync[3], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    complete_stores();
    const uint32_t prev = __hip_atomic_fetch_add(&p.sync[4], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == (uint32_t)p.nworkers - 1u) {
      const uint32_t lost = __hip_atomic_exchange(&p.sync[3], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      res->status = lost ? 1 : 0;
      __hip_atomic_store(&p.sync[4], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------- host launchers
int worker_threads() { return kThreads; }
int64_t fused_resident_vectors_per_worker() { return (int64_t)(kRegSteps + kLdsSteps) * kThreads; }

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
                        uint32_t epoch, hipStream_t st) {
  DevPlan pc = p;
  void* args[] = {&pc, &max_norm, &avg, &err, &res, &epoch};
  const void* fn = dtype == GCLIP_F32   ? (const void*)k_grad_clip_fused<GCLIP_F32>
                   : dtype == GCLIP_F16 ? (const void*)k_grad_clip_fused<GCLIP_F16>
                                        : (const void*)k_grad_clip_fused<GCLIP_BF16>;
  return hipLaunchCooperativeKernel(fn, dim3((unsigned)p.nworkers), dim3(kThreads), args, 0, st);
}

// Workgroups of the fused kernel that fit on the device at once.
hipError_t fused_capacity(int32_t dtype, int* blocks_per_cu) {
  const void* fn = dtype == GCLIP_F32   ? (const void*)k_grad_clip_fused<GCLIP_F32>
                   : dtype == GCLIP_F16 ? (const void*)k_grad_clip_fused<GCLIP_F16>
                                        : (const void*)k_grad_clip_fused<GCLIP_BF16>;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, kThreads, 0);
}

}  // namespace gclip
