// gclip_adamw.hip -- gfx950 kernels that follow the clip decision: the AdamW
// step on the clipped gradient, and the loss-scale update of loss-scaled
// steps.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/gclip.h"
#include "gclip_cursor.hpp"
#include "gclip_device.hpp"
#include "gclip_plan.hpp"

namespace gclip {

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
// The moments are written with nontemporal stores and the weights with
// ordinary ones: measured on MI355X, that mix ran 8% faster than ordinary
// stores throughout, and nontemporal stores throughout were slower than
// either (the Infinity Cache absorbs a third of the writes, not all three).
#ifndef GCLIP_ADAM_NT_STORE_MOMENTS
#define GCLIP_ADAM_NT_STORE_MOMENTS 1
#endif
constexpr bool kAdamNtStoreMoments = GCLIP_ADAM_NT_STORE_MOMENTS != 0;
#ifndef GCLIP_ADAM_NT_LOAD
#define GCLIP_ADAM_NT_LOAD 1
#endif
constexpr bool kAdamNtLoad = GCLIP_ADAM_NT_LOAD != 0;

template <int DT>
__global__ __launch_bounds__(kAdamThreads) void k_adamw_clip(AdamPlan P, AdamHp h, double max_norm, AvgSrc avs,
                                                             int err, gclip_result* res) {
  // a result block that reports a failure (a gathering wait gave up) holds
  // no norm of this step: no decision, no update
  if (res->status != 0) return;
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
          st_vec<kAdamNtStoreMoments>(reinterpret_cast<g_u32x4*>(pc.m + (uint64_t)i * 4u), mo);
          st_vec<kAdamNtStoreMoments>(reinterpret_cast<g_u32x4*>(pc.v + (uint64_t)i * 4u), vo);
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

// The loss-scale update as a kernel of its own (one thread), after the
// step's kernels that read the scale.  No update when the result block
// reports a failure: that step was neither taken nor found non-finite.
__global__ void k_amp_update(const gclip_result* res, gclip_amp_state* st, double growth, double backoff,
                             int32_t interval) {
  if (blockIdx.x != 0 || threadIdx.x != 0 || res->status != 0) return;
  amp_update(st, res->nonfinite, AmpUpdate{st, growth, backoff, interval});
}

hipError_t launch_amp_update(const gclip_result* res, gclip_amp_state* st, double growth, double backoff,
                             int32_t interval, hipStream_t s) {
  hipLaunchKernelGGL(k_amp_update, dim3(1), dim3(64), 0, s, res, st, growth, backoff, interval);
  return hipGetLastError();
}

}  // namespace gclip
