// gclip_device.hpp -- device code shared by the kernels of libgclip: 16-byte
// vector loads and stores, the element arithmetic of the three storage
// formats (sum of squares, the scaled value, rounding), the workgroup sum,
// the agent-scope atomics and the clip decision.
#pragma once

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

// Device-scope vector accesses, for data that one workgroup writes and
// another, on any XCD, reads later in the same launch.  Each XCD has an L2
// of its own that ordinary stores only reach (it is written back to memory
// at the end of the kernel), so such data is stored with the device-scope
// bit (sc1: written through to memory) and loaded with it, the encoding of
// agent-scope atomic accesses; the reader takes an agent-scope acquire
// before its loads, since a line it shares with other data may sit in its
// own caches.  The 16-byte forms go through a buffer resource, whose
// base must be the same in every lane: a group's base address; a vector at
// an address of its own takes two agent-scope 8-byte accesses instead.
constexpr int kAuxNt = 2;    // cache policy bits of the buffer builtins: nt
constexpr int kAuxSc1 = 16;  // sc1
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer: 32-bit data format, no swizzle
__device__ __forceinline__ __amdgpu_buffer_rsrc_t group_rsrc(uint64_t base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
template <bool NT>
__device__ __forceinline__ u32x4 ld_vec_dev(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kAuxSc1 | (NT ? kAuxNt : 0));
}
template <bool NT>
__device__ __forceinline__ void st_vec_dev(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 q) {
  __builtin_amdgcn_raw_buffer_store_b128(q, r, (int)off, 0, kAuxSc1 | (NT ? kAuxNt : 0));
}
__device__ __forceinline__ u32x4 load_vec_dev(uint64_t a) {
  const uint64_t* p = reinterpret_cast<const uint64_t*>(a);
  const uint64_t lo = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi = __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
}
__device__ __forceinline__ void store_vec_dev(uint64_t a, u32x4 q) {
  uint64_t* p = reinterpret_cast<uint64_t*>(a);
  __hip_atomic_store(p, (uint64_t)q[0] | ((uint64_t)q[1] << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(p + 1, (uint64_t)q[2] | ((uint64_t)q[3] << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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

// acc + g rounded once to the storage format (the last microbatch's +=).
// The 16-bit formats add in fp32 and round to the format: fp32 has at least
// 2p + 2 bits for both (p = 11, 8), so the two roundings agree with the
// format's own correctly rounded addition.
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

// ---------------------------------------------------------------- agent-scope atomics
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
__device__ __forceinline__ uint64_t atomic_ld(const uint64_t* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_st(uint64_t* a, uint64_t v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_st(double* a, double v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waiting for this workgroup's stores to complete before its next atomic is
// issued orders them for every reader of agent-scope atomics, so no
// agent-scope fence is needed for those: on gfx950 such a fence writes back
// and invalidates the whole L2 of the XCD, which costs ~18 us when 256
// workgroups do it at the end of a pass.  It does not publish plain stores
// to other XCDs: those stay in the L2 of the writer's XCD (each XCD has its
// own) until it writes them back, so plain data that another workgroup reads
// in the same launch needs the memory model's agent-scope release and
// acquire.
__device__ __forceinline__ void complete_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// The reader's side of that: once a wait on another workgroup's flag or
// ticket has ended, an agent-scope acquire before reading what the flag
// guards.  The compiler may then move no later load above the flag's load,
// and the hardware serves none of them from a stale cache line: on gfx950
// it is one buffer_inv sc1, which invalidates the compute unit's vector L1
// and its XCD's L2 lines that may be stale.  Taken once per workgroup per
// wait, never inside a loop over the data.
__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// ---------------------------------------------------------------- workgroup sum and the decision
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

// A tensor's figures from its raw sum, as the per-tensor clip writes them
// without the stop switch; returns whether it is clipped.
__device__ __forceinline__ int tensor_figures(gclip_tensor_result* o, double S, double avg, double max_norm) {
  const double sumsq = (avg * avg) * S;
  const int nf = nonfinite_of(S, avg);
  const Decision d = decide(sumsq, nf, max_norm, avg, 0);
  o->sumsq = sumsq;
  o->norm = sqrt(sumsq);
  o->nonfinite = nf;
  o->scale = d.s == 1.0 ? 1.0 : d.s;
  o->clipped = d.clipped;
  return d.clipped;
}

// The loss scale after a step (dynamic loss scaling as published by
// Micikevicius et al.): found-inf multiplies it by backoff and restarts the
// count of clean steps; a clean step counts, and the interval-th one
// multiplies the scale by growth unless that is not finite in binary32.
// One thread, once every kernel that reads the scale for this step has read
// it.
__device__ __forceinline__ void amp_update(gclip_amp_state* st, int found_inf, const AmpUpdate& u) {
  st->found_inf = found_inf ? 1 : 0;
  if (found_inf) {
    st->scale = (float)((double)st->scale * u.backoff);
    st->growth_tracker = 0;
    return;
  }
  const int32_t clean = st->growth_tracker + 1;
  if (clean == u.interval) {
    const float grown = (float)((double)st->scale * u.growth);
    if (__builtin_isfinite(grown)) st->scale = grown;
    st->growth_tracker = 0;
  } else {
    st->growth_tracker = clean;
  }
}

}  // namespace gclip
