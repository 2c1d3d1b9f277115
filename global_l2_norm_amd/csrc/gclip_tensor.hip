// gclip_tensor.hip -- gfx950 kernels that work per tensor: per-tensor norms
// and per-tensor clipping, and the last microbatch's += fused with the norm
// pass.  Both walk the list's per-tensor pieces (TPiece, gclip_plan.hpp).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/gclip.h"
#include "gclip_cursor.hpp"
#include "gclip_device.hpp"
#include "gclip_plan.hpp"

namespace gclip {

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
// Without the stop switch the clip takes two kernels instead of three
// (k_tensor_clip below).

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

// A piece read, scaled and written back kScaleBatch vectors per lane at a
// time: on MI355X a one-workgroup-per-piece in-place pass ran fastest with
// few loads per lane before their stores (2: 170 us for the 120M fp32
// list's per-tensor clip, 8: 175 us), the many resident workgroups keeping
// enough loads in flight.
constexpr int kScaleBatch = 2;
static_assert(kUnroll % kScaleBatch == 0, "whole batches per group");

template <int DT, bool NTS>
__device__ __forceinline__ void piece_scale(const TensorPlan& T, const TPiece& pc, double s64, float s32) {
  const uint32_t t = threadIdx.x;
  g_u32x4* base = reinterpret_cast<g_u32x4*>(uniform64(pc.addr));
  const uint32_t nvec = uniform32(pc.nvec);
  for (uint32_t j = 0; j < nvec; j += kPieceGroup) {
#pragma unroll
    for (int b = 0; b < kUnroll; b += kScaleBatch) {
      u32x4 q[kScaleBatch];
#pragma unroll
      for (int u = 0; u < kScaleBatch; ++u) {
        const uint32_t i = piece_index(j, b + u, t);
        if (i < nvec) q[u] = ld_vec<kNtScale>(base + i);
      }
#pragma unroll
      for (int u = 0; u < kScaleBatch; ++u) {
        const uint32_t i = piece_index(j, b + u, t);
        if (i < nvec) st_vec<NTS>(base + i, scale_vec<DT>(q[u], s64, s32));
      }
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
// factor is 1, nor at all when the result block reports a failure -- a
// gathering wait that gave up has not taken the stop switch's decision -- or
// that the stop switch stopped the update, when workgroup 0 sets every
// tensor's factor in the figures to 1).  Grid: npieces.
template <int DT, bool NTS>
__global__ __launch_bounds__(kThreads) void k_tensor_scale(TensorPlan T, gclip_tensor_result* out,
                                                           const gclip_result* res) {
  if (res->status != 0) return;
  if (res->skipped) {
    if (blockIdx.x == 0)
      for (int32_t j = (int32_t)threadIdx.x; j < T.ntensors; j += kThreads) out[j].scale = 1.0;
    return;
  }
  const TPiece pc = ld_table(T.pieces, blockIdx.x);
  const double s64 = out[uniform32(pc.tensor)].scale;
  if (s64 == 1.0) return;
  piece_scale<DT, NTS>(T, pc, s64, (float)s64);
}

// ---------------------------------------------------------------- per-tensor clip in two kernels
// Without the stop switch no tensor's decision depends on any other tensor,
// so the decision needs no kernel of its own: after k_tensor_partial, every
// workgroup of k_tensor_clip sums the partials of its own piece's tensor --
// lane i takes pieces i, i + kThreads, ... of the tensor, then the
// workgroup sum, the same order in every workgroup of the tensor, so they
// agree on the bits -- decides and scales its piece.  The workgroup of a
// tensor's first piece writes the tensor's figures and publishes its raw sum
// with an agent-scope atomic store, then counts it (an add whose result is
// not waited for).  Workgroup 0, after its own piece, waits until every
// tensor with elements has been counted and writes the list's result block
// from the sums in tensor order; then it clears the count for the next
// call.  No other workgroup waits for anything, so the launch finishes
// whatever the residency; workgroup 0's wait is bounded by wall-clock time
// and, past it, the result block reports GCLIP_DEVICE_WAIT_TIMEOUT (every
// count of the launch still arrives before the launch ends, so taking them
// back leaves the count at zero for the next call).  The figures of tensors
// without elements (no piece) are written by workgroup 0 before it waits.
__device__ __forceinline__ double tensor_sum(const TensorPlan& T, uint32_t b, uint32_t e, double* red) {
  double v = 0.0;
  for (uint32_t i = b + threadIdx.x; i < e; i += kThreads) v += T.partials[i];
  return wg_sum(v, red);
}

template <int DT, bool NTS>
__global__ __launch_bounds__(kThreads) void k_tensor_clip(TensorPlan T, AvgSrc avs, double max_norm,
                                                          gclip_tensor_result* out, gclip_result* res,
                                                          uint64_t wait_ticks) {
  __shared__ double red[kWaves];
  __shared__ int in_time;
  const double avg = avg_value(avs);
  const uint32_t t = threadIdx.x;
  if (blockIdx.x < T.npieces) {
    const TPiece pc = ld_table(T.pieces, blockIdx.x);
    const uint32_t k = uniform32(pc.tensor);
    const uint32_t b = ld_table(T.first, (uint64_t)k), e = ld_table(T.first, (uint64_t)k + 1);
    const double S = tensor_sum(T, b, e, red);
    const Decision d = decide((avg * avg) * S, nonfinite_of(S, avg), max_norm, avg, 0);
    if (blockIdx.x == b && t == 0) {
      tensor_figures(&out[k], S, avg, max_norm);
      atomic_st(&T.tsum[k], S);
      complete_stores();
      (void)atomic_add(T.tsync, 1u);
    }
    if (d.s != 1.0) piece_scale<DT, NTS>(T, pc, d.s, (float)d.s);
  }
  if (blockIdx.x != 0) return;
  // tensors without elements have no piece: their figures, before the wait
  for (int32_t k = (int32_t)t; k < T.ntensors; k += kThreads)
    if (ld_table(T.first, (uint64_t)k) == ld_table(T.first, (uint64_t)k + 1)) tensor_figures(&out[k], 0.0, avg, max_norm);
  if (t == 0) {
    in_time = 1;
    const uint64_t t0 = wall_clock64();
    while (atomic_ld(T.tsync) != T.nlive) {
      __builtin_amdgcn_s_sleep(2);
      if (wall_clock64() - t0 > wait_ticks) {
        in_time = 0;
        break;
      }
    }
    if (in_time) acquire_agent();  // every counted tensor stored its sum before its count
  }
  __syncthreads();
  if (!in_time) {
    if (t == 0) {
      res->status = GCLIP_DEVICE_WAIT_TIMEOUT;
      (void)atomic_add(T.tsync, 0u - T.nlive);
    }
    return;
  }
  double v = 0.0;
  int nf_mine = 0, clipped_mine = 0;
  for (int32_t k = (int32_t)t; k < T.ntensors; k += kThreads) {
    const bool live = ld_table(T.first, (uint64_t)k) < ld_table(T.first, (uint64_t)k + 1);
    const double S = live ? atomic_ld(&T.tsum[k]) : 0.0;
    v += S;
    nf_mine |= nonfinite_of(S, avg);
    clipped_mine |= decide((avg * avg) * S, nonfinite_of(S, avg), max_norm, avg, 0).clipped;
  }
  const double S = wg_sum(v, red);
  const int nf_any = __syncthreads_or(nf_mine);
  const int clipped_any = __syncthreads_or(clipped_mine);
  if (t == 0) {
    write_norm(res, S, avg);
    res->nonfinite = nf_any | res->nonfinite;
    res->scale = 1.0;
    res->clipped = clipped_any;
    res->skipped = 0;
    res->max_norm = max_norm;
    res->decided = 1;
    res->status = 0;
    res->handed_back = 0;
    atomic_st(T.tsync, 0u);  // every count of this launch has arrived
  }
}

// The per-tensor reduction after k_tensor_partial or k_accum_partial: one
// workgroup per tensor (one when there is none).  Workgroup k sums tensor k's
// partials (the order of k_tensor_clip), writes its figures -- with clip != 0
// also its decision -- and publishes its raw sum as k_tensor_clip's first
// pieces do; workgroup 0 gathers the list's figures the same way, under the
// same bounded wait, and takes the stop decision (a NaN/Inf anywhere with the
// switch on): it records it in the result block only, and k_tensor_scale,
// the next launch, then writes nothing and sets every tensor's factor in the
// figures to 1 -- overwriting them here could race with the tensors' own
// writes, which sit in other XCDs' L2 until the launch ends.  Last, it
// overwrites the partials with NaN: every workgroup has read its tensor's
// partials before it counted.
__global__ __launch_bounds__(kThreads) void k_tensor_gather(TensorPlan T, AvgSrc avs, double max_norm, int clip,
                                                            int err, gclip_tensor_result* out, gclip_result* res,
                                                            uint64_t wait_ticks) {
  __shared__ double red[kWaves];
  __shared__ int in_time;
  const double avg = avg_value(avs);
  const uint32_t t = threadIdx.x;
  const uint32_t k = blockIdx.x;
  if ((int32_t)k < T.ntensors) {
    const uint32_t b = ld_table(T.first, (uint64_t)k), e = ld_table(T.first, (uint64_t)k + 1);
    const double S = b < e ? tensor_sum(T, b, e, red) : 0.0;
    if (t == 0) {
      if (clip) {
        tensor_figures(&out[k], S, avg, max_norm);
      } else {
        const double sumsq = (avg * avg) * S;
        out[k].sumsq = sumsq;
        out[k].norm = sqrt(sumsq);
        out[k].nonfinite = nonfinite_of(S, avg);
        out[k].scale = 1.0;
        out[k].clipped = 0;
      }
      if (b < e) {
        atomic_st(&T.tsum[k], S);
        complete_stores();
        (void)atomic_add(T.tsync, 1u);
      }
    }
  }
  if (k != 0) return;
  if (t == 0) {
    in_time = 1;
    const uint64_t t0 = wall_clock64();
    while (atomic_ld(T.tsync) != T.nlive) {
      __builtin_amdgcn_s_sleep(2);
      if (wall_clock64() - t0 > wait_ticks) {
        in_time = 0;
        break;
      }
    }
    if (in_time) acquire_agent();  // every counted tensor stored its sum before its count
  }
  __syncthreads();
  if (!in_time) {
    if (t == 0) {
      res->status = GCLIP_DEVICE_WAIT_TIMEOUT;
      (void)atomic_add(T.tsync, 0u - T.nlive);
    }
    return;
  }
  double v = 0.0;
  int nf_mine = 0, clipped_mine = 0;
  for (int32_t j = (int32_t)t; j < T.ntensors; j += kThreads) {
    const bool live = ld_table(T.first, (uint64_t)j) < ld_table(T.first, (uint64_t)j + 1);
    const double S = live ? atomic_ld(&T.tsum[j]) : 0.0;
    v += S;
    nf_mine |= nonfinite_of(S, avg);
    if (clip) clipped_mine |= decide((avg * avg) * S, nonfinite_of(S, avg), max_norm, avg, err).clipped;
  }
  const double S = wg_sum(v, red);
  const int nf_any = __syncthreads_or(nf_mine);
  const int clipped_any = __syncthreads_or(clipped_mine);
  const int skip = (clip && err && nf_any) ? 1 : 0;
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
    atomic_st(T.tsync, 0u);  // every count of this launch has arrived
  }
}

// ---------------------------------------------------------------- the last microbatch's += with the norm
// Backprop lesson, "Accumulation across microbatches": acc += g, rounded once
// to the storage format.  The 16-bit formats add in fp32 and round to the
// format: fp32 has at least 2p + 2 bits for both (p = 11, 8), so the two
// roundings agree with the format's own correctly rounded addition.  The
// squares of the values written are summed as in the norm pass, one partial
// per piece; k_tensor_decide then reduces them.
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

// ---------------------------------------------------------------- host launchers
// One partial per piece (nothing when the list has no piece).
hipError_t launch_tensor_partial(const TensorPlan& T, int32_t dtype, hipStream_t st) {
  if (T.npieces == 0) return hipSuccess;
  const dim3 grid(T.npieces), block(kThreads);
  switch (dtype) {
    case GCLIP_F32: hipLaunchKernelGGL(k_tensor_partial<GCLIP_F32>, grid, block, 0, st, T); break;
    case GCLIP_F16: hipLaunchKernelGGL(k_tensor_partial<GCLIP_F16>, grid, block, 0, st, T); break;
    default: hipLaunchKernelGGL(k_tensor_partial<GCLIP_BF16>, grid, block, 0, st, T); break;
  }
  return hipGetLastError();
}

hipError_t launch_tensor_norm(const TensorPlan& T, int32_t dtype, AvgSrc avg, double max_norm, int clip, int err,
                              gclip_tensor_result* out, gclip_result* res, hipStream_t st) {
  const hipError_t e = launch_tensor_partial(T, dtype, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_tensor_decide, dim3(1), dim3(kThreads), 0, st, T, avg, max_norm, clip, err, out, res);
  return hipGetLastError();
}

hipError_t launch_tensor_gather(const TensorPlan& T, AvgSrc avg, double max_norm, int clip, int err,
                                gclip_tensor_result* out, gclip_result* res, uint64_t wait_ticks, hipStream_t st);

// The per-tensor clip's partials and every decision: gathered in one
// workgroup per tensor, or in k_tensor_decide without a wall clock to bound
// the gathering wait.  k_tensor_scale follows.
hipError_t launch_tensor_decisions(const TensorPlan& T, int32_t dtype, AvgSrc avg, double max_norm, int err,
                                   gclip_tensor_result* out, gclip_result* res, uint64_t wait_ticks, bool gather,
                                   hipStream_t st) {
  if (!gather) return launch_tensor_norm(T, dtype, avg, max_norm, 1, err, out, res, st);
  const hipError_t e = launch_tensor_partial(T, dtype, st);
  if (e != hipSuccess) return e;
  return launch_tensor_gather(T, avg, max_norm, 1, err, out, res, wait_ticks, st);
}

hipError_t launch_tensor_gather(const TensorPlan& T, AvgSrc avg, double max_norm, int clip, int err,
                                gclip_tensor_result* out, gclip_result* res, uint64_t wait_ticks, hipStream_t st) {
  hipLaunchKernelGGL(k_tensor_gather, dim3(T.ntensors > 0 ? (uint32_t)T.ntensors : 1u), dim3(kThreads), 0, st, T,
                     avg, max_norm, clip, err, out, res, wait_ticks);
  return hipGetLastError();
}

// Per-tensor norms alone: the partials, then the per-tensor reduction --
// gathered in one workgroup per tensor when the device has a wall clock to
// bound the gathering wait (wait_ticks != 0), else in k_tensor_decide.
hipError_t launch_tensor_norms(const TensorPlan& T, int32_t dtype, AvgSrc avg, gclip_tensor_result* out,
                               gclip_result* res, uint64_t wait_ticks, bool gather, hipStream_t st) {
  if (!gather) return launch_tensor_norm(T, dtype, avg, 0.0, 0, 0, out, res, st);
  const hipError_t e = launch_tensor_partial(T, dtype, st);
  if (e != hipSuccess) return e;
  return launch_tensor_gather(T, avg, 0.0, 0, 0, out, res, wait_ticks, st);
}

template <bool NTS>
const void* tensor_scale_kernel(int32_t dtype) {
  return dtype == GCLIP_F32   ? (const void*)k_tensor_scale<GCLIP_F32, NTS>
         : dtype == GCLIP_F16 ? (const void*)k_tensor_scale<GCLIP_F16, NTS>
                              : (const void*)k_tensor_scale<GCLIP_BF16, NTS>;
}

hipError_t launch_tensor_scale(const TensorPlan& T, int32_t dtype, gclip_tensor_result* out,
                               const gclip_result* res, hipStream_t st) {
  if (T.npieces == 0) return hipSuccess;
  TensorPlan tc = T;
  void* args[] = {&tc, &out, &res};
  const void* fn = T.nt_store ? tensor_scale_kernel<true>(dtype) : tensor_scale_kernel<false>(dtype);
  return hipLaunchKernel(fn, dim3(T.npieces), dim3(kThreads), args, 0, st);
}

template <bool NTS>
const void* tensor_clip_kernel(int32_t dtype) {
  return dtype == GCLIP_F32   ? (const void*)k_tensor_clip<GCLIP_F32, NTS>
         : dtype == GCLIP_F16 ? (const void*)k_tensor_clip<GCLIP_F16, NTS>
                              : (const void*)k_tensor_clip<GCLIP_BF16, NTS>;
}

// The per-tensor clip without the stop switch: k_tensor_partial, then
// k_tensor_clip (one workgroup per piece; one workgroup when there is none).
hipError_t launch_tensor_clip(const TensorPlan& T, int32_t dtype, AvgSrc avg, double max_norm,
                              gclip_tensor_result* out, gclip_result* res, uint64_t wait_ticks, hipStream_t st) {
  if (T.npieces > 0) {
    TensorPlan tc = T;
    void* args[] = {&tc};
    const void* fn = dtype == GCLIP_F32   ? (const void*)k_tensor_partial<GCLIP_F32>
                     : dtype == GCLIP_F16 ? (const void*)k_tensor_partial<GCLIP_F16>
                                          : (const void*)k_tensor_partial<GCLIP_BF16>;
    const hipError_t e = hipLaunchKernel(fn, dim3(T.npieces), dim3(kThreads), args, 0, st);
    if (e != hipSuccess) return e;
  }
  TensorPlan tc = T;
  void* args[] = {&tc, &avg, &max_norm, &out, &res, &wait_ticks};
  const void* fn = T.nt_store ? tensor_clip_kernel<true>(dtype) : tensor_clip_kernel<false>(dtype);
  return hipLaunchKernel(fn, dim3(T.npieces > 0 ? T.npieces : 1u), dim3(kThreads), args, 0, st);
}

template <bool NTS>
const void* accum_kernel(int32_t dtype) {
  return dtype == GCLIP_F32   ? (const void*)k_accum_partial<GCLIP_F32, NTS>
         : dtype == GCLIP_F16 ? (const void*)k_accum_partial<GCLIP_F16, NTS>
                              : (const void*)k_accum_partial<GCLIP_BF16, NTS>;
}

hipError_t launch_accumulate_norm(const TensorPlan& T, int32_t dtype, const uint64_t* gdelta, AvgSrc avg,
                                  gclip_tensor_result* out, gclip_result* res, uint64_t wait_ticks, bool gather,
                                  hipStream_t st) {
  if (T.npieces > 0) {
    TensorPlan tc = T;
    void* args[] = {&tc, &gdelta};
    const void* fn = T.nt_store ? accum_kernel<true>(dtype) : accum_kernel<false>(dtype);
    const hipError_t e = hipLaunchKernel(fn, dim3(T.npieces), dim3(kThreads), args, 0, st);
    if (e != hipSuccess) return e;
  }
  if (gather) return launch_tensor_gather(T, avg, 0.0, 0, 0, out, res, wait_ticks, st);
  hipLaunchKernelGGL(k_tensor_decide, dim3(1), dim3(kThreads), 0, st, T, avg, 0.0, 0, 0, out, res);
  return hipGetLastError();
}

}  // namespace gclip
