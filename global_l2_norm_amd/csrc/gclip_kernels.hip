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
//     is cut into chunks: each worker takes two without a claim, and the
//     rest are claimed at run time from one counter, so that the XCDs that
//     stream faster take more of them.  Loads are dwordx4
//     with kUnroll vectors in flight per lane, the next group's loads issued
//     before the current group is used;
//   - each vector's squares are summed in fp32 and added into per-lane
//     binary64 accumulators (vec_sumsq states when a vector is summed again
//     in binary64), so the sum cannot overflow and is non-finite exactly when
//     some element is NaN or +-Inf;
//   - lane sums are reduced by an xor butterfly inside each wave, and the
//     waves' sums in wave order into one partial per chunk (a slot of the
//     chunk's own) and one per worker for its block; the last
//     workgroup to arrive (a two-level agent-scope ticket) sums all partials
//     in index order, so the bits of the norm do not depend on scheduling or
//     on which workgroup took which chunk, and both paths give the same
//     bits; cross-workgroup data moves only through agent-scope atomics (see
//     complete_stores) and, for the += kernel's sums, device-scope vector
//     stores and loads (ld_vec_dev); the += kernel's single elements are
//     rescaled by the workgroup that wrote them, except when a block is
//     handed back, which passes them on with an agent-scope release and
//     acquire;
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
#include "gclip_device.hpp"
#include "gclip_plan.hpp"
#ifdef GCLIP_PHASE_STAMPS
#include "../../include/gclip_stamps.h"
#include "gclip_host.hpp"
#endif

namespace gclip {

// Phase timeline, in a separate build only (-DGCLIP_PHASE_STAMPS, see
// include/gclip_stamps.h): thread 0 of each workgroup of the fused kernel
// stores the wall clock at the kernel's phase boundaries.  In the library
// itself the stamps compile to nothing.
#ifdef GCLIP_PHASE_STAMPS
__device__ uint64_t g_phase_stamps[GCLIP_STAMP_WORKERS * GCLIP_STAMP_POINTS];
#define GCLIP_STAMP(k)                                                                  \
  do {                                                                                  \
    if (threadIdx.x == 0 && blockIdx.x < GCLIP_STAMP_WORKERS)                           \
      ::gclip::g_phase_stamps[blockIdx.x * GCLIP_STAMP_POINTS + (k)] = wall_clock64(); \
  } while (0)
#else
#define GCLIP_STAMP(k) \
  do {                 \
  } while (0)
#endif

// ---------------------------------------------------------------- group loads and stores
// Load the vectors of one group into q (zeros where a lane has no vector);
// DEV: with device-scope loads (data another XCD wrote in this launch).
template <bool NT, bool DEV = false>
__device__ __forceinline__ void load_group(const DevPlan& p, Cursor& cur, uint64_t vb, uint64_t ve, uint64_t j,
                                           uint64_t j1, u32x4 (&q)[kUnroll]) {
  const uint32_t t = threadIdx.x;
  uint64_t base = 0;
  const int kind = group_kind(cur, vb, ve, j, j1, base);
  if (DEV && kind != kGroupCross) {
    const __amdgpu_buffer_rsrc_t rs = group_rsrc(uniform64(base), (uint32_t)kGroupVectors * kVecBytes);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      q[u] = kind == kGroupFull || tail_ok(vb, ve, j, j1, u, t)
                 ? ld_vec_dev<NT>(rs, ((uint32_t)u * kThreads + t) * kVecBytes)
                 : u32x4{0u, 0u, 0u, 0u};
  } else if (kind == kGroupFull) {
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
        if (v < ve) q[u] = DEV ? load_vec_dev(a) : load_vec<NT>(a);
      }
    }
  }
}

// Store f(vector u) for every vector of one group (the addresses of the
// group are recomputed exactly as load_group computed them); DEV: with
// device-scope stores (data another XCD reads in this launch).
template <bool NT, bool DEV = false, typename F>
__device__ __forceinline__ void store_group(const DevPlan& p, Cursor& cur, uint64_t vb, uint64_t ve, uint64_t j,
                                            uint64_t j1, F&& f) {
  const uint32_t t = threadIdx.x;
  uint64_t base = 0;
  const int kind = group_kind(cur, vb, ve, j, j1, base);
  if (DEV && kind != kGroupCross) {
    const __amdgpu_buffer_rsrc_t rs = group_rsrc(uniform64(base), (uint32_t)kGroupVectors * kVecBytes);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (kind == kGroupFull || tail_ok(vb, ve, j, j1, u, t))
        st_vec_dev<NT>(rs, ((uint32_t)u * kThreads + t) * kVecBytes, f(u));
  } else if (kind == kGroupFull) {
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
        if (v < ve) {
          if constexpr (DEV) {
            store_vec_dev(a, f(u));
          } else {
            store_vec<NT>(a, f(u));
          }
        }
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

// Steps [j0, j1) of the run [vb, ve): read (DEV: with device-scope loads),
// multiply, write back.  A group's loads are all issued before its first
// store.
template <int DT, bool DEV = false>
__device__ __forceinline__ void scale_steps(const DevPlan& p, Cursor& cur, uint64_t vb, uint64_t ve, uint64_t j0,
                                            uint64_t j1, double s64, float s32) {
  for (uint64_t j = j0; j < j1; j += kUnroll) {
    u32x4 q[kUnroll];
    Cursor c2 = cur;
    load_group<kNtScale, DEV>(p, cur, vb, ve, j, j1, q);
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

// ---------------------------------------------------------------- the last += in the same launch
// Backprop lesson, "Accumulation across microbatches": with a contribution
// (AccSrc), every vector of the list is read together with the contribution
// laid out like it, and the sum acc + g (add_vec) takes the vector's place.

// The contribution's vectors for one group (the walk of load_group, on the
// caller's own cursor): at the list's addresses plus the offset of the
// segment that holds each vector.
template <bool NT>
__device__ __forceinline__ void load_group_contrib(const DevPlan& p, const AccSrc& A, Cursor& cur, uint64_t vb,
                                                   uint64_t ve, uint64_t j, uint64_t j1, u32x4 (&h)[kUnroll]) {
  const uint32_t t = threadIdx.x;
  uint64_t base = 0;
  const int kind = group_kind(cur, vb, ve, j, j1, base);
  if (kind != kGroupCross) {
    const uint64_t d = ld_table(A.seg_gdelta, (uint64_t)uniform32(cur.s));
    const g_u32x4* g = reinterpret_cast<const g_u32x4*>(uniform64(base + d));
    if (kind == kGroupFull) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) h[u] = ld_vec<NT>(&g[u * kThreads + t]);
    } else {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        h[u] = tail_ok(vb, ve, j, j1, u, t) ? ld_vec<NT>(&g[u * kThreads + t]) : u32x4{0u, 0u, 0u, 0u};
    }
  } else {
    const uint64_t b0 = vb + j * kThreads;
    uint64_t d = ld_table(A.seg_gdelta, (uint64_t)uniform32(cur.s));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      h[u] = u32x4{0u, 0u, 0u, 0u};
      if (j + u < j1) {
        const uint64_t b = b0 + (uint64_t)u * kThreads, v = b + t;
        const uint64_t a = step_addr_delta(p, A.seg_gdelta, cur, d, b, ve, v);
        if (v < ve) h[u] = load_vec<NT>(a);
      }
    }
  }
}

// Worker w's single elements: acc + g written back; returns the sum of the
// new values' squares.
template <int DT>
__device__ __forceinline__ double accum_scalars(const DevPlan& p, const AccSrc& A, int w) {
  double s = 0.0;
  const uint64_t b = ld_table(p.wk_scbegin, (uint64_t)w), e = ld_table(p.wk_scbegin, (uint64_t)w + 1);
  for (uint64_t i = b + threadIdx.x; i < e; i += kThreads) {
    const uint64_t a = p.sc_addr[i];
    const uint32_t v = add_elem<DT>(load_elem<DT>(a), load_elem<DT>(a + A.sc_gdelta[i]));
    store_elem<DT>(a, v);
    s += elem_square<DT>(v);
  }
  return s;
}

// Steps [j0, j1) of the run [vb, ve): acc + g, times s when `scale`, written
// back (a block handed back before it was written).
template <int DT>
__device__ __forceinline__ void accum_scale_steps(const DevPlan& p, const AccSrc& A, Cursor& cur, uint64_t vb,
                                                  uint64_t ve, uint64_t j0, uint64_t j1, double s64, float s32,
                                                  bool scale) {
  Cursor cg = cur;
  for (uint64_t j = j0; j < j1; j += kUnroll) {
    u32x4 q[kUnroll], h[kUnroll];
    Cursor cs = cur;
    load_group<kNtScale>(p, cur, vb, ve, j, j1, q);
    load_group_contrib<kNtScale>(p, A, cg, vb, ve, j, j1, h);
    store_group<false>(p, cs, vb, ve, j, j1, [&](int u) {
      const u32x4 n = add_vec<DT>(q[u], h[u]);
      return scale ? scale_vec<DT>(n, s64, s32) : n;
    });
  }
}

// ---------------------------------------------------------------- counters in the workspace
// Word of line 0 of sync.
constexpr int kHandedWord = 0;

__device__ __forceinline__ uint32_t* sum_claims(const DevPlan& p) { return p.sync + kSyncLineWords; }
__device__ __forceinline__ uint32_t* scale_claims(const DevPlan& p) { return p.sync + 2 * kSyncLineWords; }
__device__ __forceinline__ uint32_t* arrival_tickets(const DevPlan& p) { return p.sync + 3 * kSyncLineWords; }
__device__ __forceinline__ uint32_t* finish_tickets(const DevPlan& p) {
  return p.sync + (4 + kTicketGroups) * kSyncLineWords;
}

// Ticket over every workgroup of a launch, in two levels: workgroup w counts
// in the line of its group w % kTicketGroups (its XCD: workgroups are dealt
// to the XCDs in turn), the last of each group counts in the top line.  No
// counter takes more than ~nworkers / kTicketGroups atomics at once.  True in exactly one
// workgroup, the last to take the ticket.  The counter a workgroup completes
// is reset by it for the next launch.  Thread 0 only; its stores must be
// complete (complete_stores) before the call.
__device__ __forceinline__ bool take_ticket(uint32_t* lines, int32_t nworkers) {
  const uint32_t g = blockIdx.x % (uint32_t)kTicketGroups;
  const uint32_t members = ((uint32_t)nworkers - g + kTicketGroups - 1) / kTicketGroups;
  const uint32_t groups = nworkers < kTicketGroups ? (uint32_t)nworkers : (uint32_t)kTicketGroups;
  uint32_t* mine = lines + g * kSyncLineWords;
  uint32_t* top = lines + kTicketGroups * kSyncLineWords;
  if (atomic_add(mine, 1u) != members - 1u) return false;
  atomic_st(mine, 0u);
  if (atomic_add(top, 1u) != groups - 1u) return false;
  atomic_st(top, 0u);
  return true;
}

// ---------------------------------------------------------------- chunk claiming
// Workgroup w takes chunks w and nworkers + w without any claim; chunks
// 2 nworkers .. nch - 1 are claimed at run time in index order, a claim
// being a ticket drawn on one counter, so that the workgroups that stream
// faster take more of them.  Every claim is then one atomic, whose reply
// comes back while a chunk streams.  (With one pool per XCD, a workgroup
// whose own pool was empty had to read every pool's counter before it could
// claim again: two round trips that no chunk hid, taken just as the last
// chunks ran out; on the 2.6 GB list the pass ran 4.5 % slower.)  The two
// chunks taken without a claim keep the first tickets, which every
// workgroup draws at once, off the start of the pass: drawn there and waited
// for at once, they queued on the counter for up to 3 us.
constexpr uint32_t kNone = 0xffffffffu;

struct Claimer {
  uint32_t* counter;
  uint32_t base;  // first claimed chunk: 2 nworkers
  uint32_t ndyn;  // claimed chunks
};

__device__ __forceinline__ Claimer make_claimer(uint32_t* counter, const DevPlan& p, uint32_t nch) {
  const uint32_t base = 2u * (uint32_t)p.nworkers;
  return Claimer{counter, base, nch > base ? nch - base : 0u};
}

// The chunk workgroup w takes second, without a claim (kNone if none).
__device__ __forceinline__ uint32_t second_chunk(const DevPlan& p, uint32_t nch, uint32_t w) {
  const uint32_t c = (uint32_t)p.nworkers + w;
  return c < nch ? c : kNone;
}

// A claim is taken in two steps: the ticket is drawn before a chunk streams
// and turned into a chunk after it, so waiting for the counter's reply
// overlaps the chunk's loads instead of draining them.  Thread 0 only.
// Tickets are drawn only while claims succeed, so the counter stays below
// ndyn + nworkers.
__device__ __forceinline__ uint32_t claim_issue(const Claimer& cl) {
  return cl.ndyn == 0u ? kNone : atomic_add(cl.counter, 1u);
}

__device__ __forceinline__ uint32_t claim_resolve(const Claimer& cl, uint32_t tk) {
  return tk < cl.ndyn ? cl.base + tk : kNone;
}

// Claims run two chunks ahead: the chunk after next is claimed while the
// current one streams and is handed over at the per-chunk barrier through
// LDS slot i % 2 (a slot is rewritten only two barriers after it was read).
struct ClaimSlots {
  uint32_t claim[2];
  double wsum[2][kWaves];  // each wave's sum of the current chunk (by chunk parity)
};

// The chunk loops below draw the ticket for the chunk after next when a
// chunk starts, before its later groups are loaded, and resolve it after the
// chunk's last group has been waited for: loads and atomics complete in
// order, so by then the ticket's reply is in and resolving it costs no wait.
// Only then is the next chunk's first group loaded, so it stays in flight
// across the chunk's barrier.  (Resolving after that load made the wave wait
// for it too: every chunk ended with nothing in flight.)  The first two
// chunks need no claim, so the first ticket is drawn as the first chunk
// starts, for the third.

// A sum chunk's partial: its waves' sums added in wave order.
__device__ __forceinline__ double chunk_total(const double (&ws)[kWaves]) {
  double s = ws[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) s += ws[k];
  return s;
}

// Sum every sum chunk of the streamed region [0, sb) that this workgroup
// takes.  Each wave reduces its lanes' sums over a chunk to one value; at
// the chunk's barrier (the only one, which also hands the next claim to
// every wave) thread 0 adds the waves' values in wave order into the chunk's
// own slot, partials[c], so the final sum does not depend on which workgroup
// took the chunk.
template <int DT, bool TWO>
__device__ __forceinline__ void norm_chunks(const DevPlan& p, ClaimSlots& sl) {
  const uint32_t nch = p.nsum;
  if (blockIdx.x >= nch) return;  // then no chunk is left to claim either
  const uint32_t t = threadIdx.x, lane = t & 63u, wave = t >> 6;
  const Claimer cl = make_claimer(sum_claims(p), p, nch);
  uint32_t c = blockIdx.x, cn = second_chunk(p, nch, blockIdx.x);
  Cursor cur;
  u32x4 q[kUnroll];
  {
    const Range r = sum_chunk_range<TWO>(p, c);
    cursor_load(p, cur, r.seg);
    load_group<kNtSum>(p, cur, r.b, r.e, 0, range_steps(r), q);
  }
  for (uint32_t i = 0; c != kNone; ++i) {
    const Range r = sum_chunk_range<TWO>(p, c);
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
      const Range rn = sum_chunk_range<TWO>(p, cn);
      cursor_load(p, curn, rn.seg);
      load_group<kNtSum>(p, curn, rn.b, rn.e, 0, range_steps(rn), q);
    }
    double v = lane_total(acc, 0.0);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) sl.wsum[par][wave] = v;
    __syncthreads();
    if (t == 0) atomic_st(&p.partials[c], chunk_total(sl.wsum[par]));
    c = cn;
    cn = uniform32(sl.claim[par]);
    cur = curn;
  }
}

// The last round of a pass's claimed chunks (the last nworkers of them) is
// written with nontemporal stores even where the pass writes ordinary ones:
// the launch then ends with fewer dirty lines in the L2s to write back.
// Measured on MI355X (two runs on two boxes): -1.5 to -3.2 us on the +=
// list, 0 to -1.6 us on the 184 MB fp16 list, within +-0.3 us elsewhere;
// two or four rounds were slower.
#ifndef GCLIP_LATE_NT_ROUNDS
#define GCLIP_LATE_NT_ROUNDS 1
#endif
constexpr uint32_t kLateNtRounds = GCLIP_LATE_NT_ROUNDS;

// Scale in place every chunk of the table (vb, seg, nch) that this workgroup
// takes (DEV: read with device-scope loads).  A chunk's last group is scaled
// into registers before the ticket is resolved, and stored after it.
template <int DT, bool NTS, bool DEV = false>
__device__ __forceinline__ void scale_chunks(const DevPlan& p, ClaimSlots& sl, const uint64_t* vb,
                                             const uint32_t* seg, uint32_t nch, double s64, float s32) {
  if (blockIdx.x >= nch) return;  // then no chunk is left to claim either
  const uint32_t t = threadIdx.x;
  const Claimer cl = make_claimer(scale_claims(p), p, nch);
  uint32_t c = blockIdx.x, cn = second_chunk(p, nch, blockIdx.x);
  Cursor cur;
  u32x4 q[kUnroll];
  {
    const Range r = tab_chunk_range(vb, seg, c);
    cursor_load(p, cur, r.seg);
    load_group<kNtScale, DEV>(p, cur, r.b, r.e, 0, range_steps(r), q);
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
      load_group<kNtScale, DEV>(p, cur, r.b, r.e, j + kUnroll, ns, q2);
      store_group<NTS>(p, cst, r.b, r.e, j, ns, [&](int u) { return scale_vec<DT>(q[u], s64, s32); });
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) q[u] = q2[u];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) q[u] = scale_vec<DT>(q[u], s64, s32);
    const uint32_t par = i & 1u;
    if (t == 0) sl.claim[par] = cn != kNone ? claim_resolve(cl, tk) : kNone;
    if (!NTS && kLateNtRounds > 0 && c + kLateNtRounds * (uint32_t)p.nworkers >= nch) {
      store_group<true>(p, cst, r.b, r.e, j, ns, [&](int u) { return q[u]; });
    } else {
      store_group<NTS>(p, cst, r.b, r.e, j, ns, [&](int u) { return q[u]; });
    }
    Cursor curn;
    if (cn != kNone) {
      u32x4 q2[kUnroll];
      const Range rn = tab_chunk_range(vb, seg, cn);
      cursor_load(p, curn, rn.seg);
      load_group<kNtScale, DEV>(p, curn, rn.b, rn.e, 0, range_steps(rn), q2);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) q[u] = q2[u];
    }
    __syncthreads();
    c = cn;
    cn = uniform32(sl.claim[par]);
    cur = curn;
  }
}

// The sum chunks this workgroup takes, with the +=: every group is read
// with its contribution (both one group ahead), added, written back with
// device-scope stores (after the decision any workgroup may rescale them)
// and summed, one partial per chunk as in norm_chunks.
template <int DT, bool NTS>
__device__ __forceinline__ void accum_chunks(const DevPlan& p, const AccSrc& A, ClaimSlots& sl) {
  const uint32_t nch = p.nsum;
  if (blockIdx.x >= nch) return;  // then no chunk is left to claim either
  const uint32_t t = threadIdx.x, lane = t & 63u, wave = t >> 6;
  const Claimer cl = make_claimer(sum_claims(p), p, nch);
  uint32_t c = blockIdx.x, cn = second_chunk(p, nch, blockIdx.x);
  Cursor cur, cg;
  u32x4 q[kUnroll], h[kUnroll];
  {
    const Range r = sum_chunk_range<NTS>(p, c);
    cursor_load(p, cur, r.seg);
    cg = cur;
    load_group<kNtSum>(p, cur, r.b, r.e, 0, range_steps(r), q);
    load_group_contrib<kNtSum>(p, A, cg, r.b, r.e, 0, range_steps(r), h);
  }
  for (uint32_t i = 0; c != kNone; ++i) {
    const Range r = sum_chunk_range<NTS>(p, c);
    const uint64_t ns = range_steps(r);
    uint32_t tk = 0;
    if (t == 0 && cn != kNone) tk = claim_issue(cl);
    Cursor cst;
    cursor_load(p, cst, r.seg);
    double acc[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc[u] = 0.0;
    uint64_t j = 0;
    for (; j + kUnroll < ns; j += kUnroll) {
      u32x4 q2[kUnroll], h2[kUnroll];
      load_group<kNtSum>(p, cur, r.b, r.e, j + kUnroll, ns, q2);
      load_group_contrib<kNtSum>(p, A, cg, r.b, r.e, j + kUnroll, ns, h2);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) q[u] = add_vec<DT>(q[u], h[u]);
      store_group<NTS, true>(p, cst, r.b, r.e, j, ns, [&](int u) { return q[u]; });
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc[u] += vec_sumsq<DT>(q[u]);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        q[u] = q2[u];
        h[u] = h2[u];
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) q[u] = add_vec<DT>(q[u], h[u]);
    store_group<NTS, true>(p, cst, r.b, r.e, j, ns, [&](int u) { return q[u]; });
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc[u] += vec_sumsq<DT>(q[u]);
    const uint32_t par = i & 1u;
    if (t == 0) sl.claim[par] = cn != kNone ? claim_resolve(cl, tk) : kNone;
    Cursor curn, cgn;
    if (cn != kNone) {
      const Range rn = sum_chunk_range<NTS>(p, cn);
      cursor_load(p, curn, rn.seg);
      cgn = curn;
      load_group<kNtSum>(p, curn, rn.b, rn.e, 0, range_steps(rn), q);
      load_group_contrib<kNtSum>(p, A, cgn, rn.b, rn.e, 0, range_steps(rn), h);
    }
    double v = lane_total(acc, 0.0);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) sl.wsum[par][wave] = v;
    __syncthreads();
    if (t == 0) atomic_st(&p.partials[c], chunk_total(sl.wsum[par]));
    c = cn;
    cn = uniform32(sl.claim[par]);
    cur = curn;
    cg = cgn;
  }
}

// ---------------------------------------------------------------- reductions and the decision
// Partials: one per sum chunk, then one per worker.
__device__ __forceinline__ uint32_t npartials(const DevPlan& p) {
  return p.nsum + (uint32_t)p.nworkers;
}
__device__ __forceinline__ double* worker_partial(const DevPlan& p, int w) {
  return p.partials + (size_t)p.nsum + w;
}

// Sum of all partials in index order (lane i takes i, i + kThreads, ...).
// A lane issues the loads of kPartialBatch partials before it adds any, so
// the sum waits for one round trip per batch, not one per partial (it is on
// the path to the grid-wide decision); adding 0.0 for the slots past the end
// leaves the sum's bits as they are.
constexpr int kPartialBatch = 8;
__device__ __forceinline__ double partials_sum(const DevPlan& p, double* red) {
  double v = 0.0;
  const uint32_t n = npartials(p);
  for (uint32_t i0 = threadIdx.x; i0 < n; i0 += kThreads * kPartialBatch) {
    double x[kPartialBatch];
#pragma unroll
    for (int k = 0; k < kPartialBatch; ++k) {
      const uint32_t i = i0 + (uint32_t)k * kThreads;
      x[k] = i < n ? atomic_ld(&p.partials[i]) : 0.0;
    }
#pragma unroll
    for (int k = 0; k < kPartialBatch; ++k) v += x[k];
  }
  return wg_sum(v, red);
}

// After the last workgroup has summed the partials it overwrites them with
// NaN, so a partial that was somehow read before it was written could only
// ever show up as a NaN norm, never as a plausible wrong one.
__device__ __forceinline__ void poison_partials(const DevPlan& p) {
  const uint32_t n = npartials(p);
  for (uint32_t i = threadIdx.x; i < n; i += kThreads) atomic_st(&p.partials[i], __builtin_nan(""));
}

// Arrival after the summing pass: true in the last workgroup (all threads).
// The caller's partials must already be stored.
__device__ __forceinline__ bool arrive(const DevPlan& p, int* flag) {
  if (threadIdx.x == 0) {
    complete_stores();
    *flag = take_ticket(arrival_tickets(p), p.nworkers) ? 1 : 0;
    if (*flag) acquire_agent();  // before the partials are read
  }
  __syncthreads();
  return *flag != 0;
}

// Blocks handed back by the fused kernel.  Worker w's state word is kHeld
// while w holds its block (or has written it), kHanded once w has stopped
// waiting at the decision and left its block -- and its own chunk (the first
// scale chunk; with the +=, its sum chunk) -- unscaled in memory, kTaken once
// another workgroup has taken it over.  Line 0's kHandedWord counts the
// hand-backs.
constexpr uint32_t kHeld = 0u, kHanded = 2u, kTaken = 3u;

struct HandSlots {
  uint32_t n;
  uint32_t list[kThreads];
};

// Take over every block handed back so far and scale it from memory, with
// the worker's single elements and its own chunks of the streamed region (no
// other workgroup scales them: the two scale chunks workgroup w takes
// without a claim) -- the whole workgroup.  With the += (ACC) the block was
// never written: it is read with its contribution, added and written --
// times s only when `scale` (the sum is written whatever the decision); the
// single elements and the chunks already hold their sums, and are scaled
// only when `scale` (the chunks' sums, which any workgroup may have written,
// read with device-scope loads).
template <int DT, bool ACC = false>
__device__ __forceinline__ void take_handed_blocks(const DevPlan& p, HandSlots& hs, double s64, float s32,
                                                   const AccSrc& A = AccSrc{}, bool scale = true) {
  for (uint32_t base = 0; base < (uint32_t)p.nworkers; base += kThreads) {
    if (threadIdx.x == 0) hs.n = 0;
    __syncthreads();
    const uint32_t i = base + threadIdx.x;
    if (i < (uint32_t)p.nworkers && atomic_ld(&p.bstate[i]) == kHanded) {
      // with the +=, acquire: the giver released its sums with the state
      constexpr int kTakeOrder = ACC ? __ATOMIC_ACQUIRE : __ATOMIC_RELAXED;
      uint32_t expected = kHanded;
      if (__hip_atomic_compare_exchange_strong(&p.bstate[i], &expected, kTaken, kTakeOrder, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT))
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
        if constexpr (ACC) {
          accum_scale_steps<DT>(p, A, cur, r.b, r.e, 0, range_steps(r), s64, s32, scale);
        } else {
          scale_steps<DT>(p, cur, r.b, r.e, 0, range_steps(r), s64, s32);
        }
      }
      if (ACC && !scale) continue;
      scale_scalars<DT>(p, v, s64, s32);
      for (uint32_t k = 0; k < 2; ++k) {
        const uint32_t own = (uint32_t)v + k * (uint32_t)p.nworkers;
        if (own >= p.nchs) break;
        const Range c = tab_chunk_range(p.fus_vb, p.fus_seg, own);
        Cursor cur;
        cursor_load(p, cur, c.seg);
        scale_steps<DT, ACC>(p, cur, c.b, c.e, 0, range_steps(c), s64, s32);
      }
    }
    __syncthreads();
  }
}

// Second ticket, at the very end.  The last workgroup to finish -- every
// other one has then left the claim counter and the block states alone --
// resets the scale pass's claim counter and, after a fused launch, scales
// whatever blocks are still handed back (the decision is published before
// the deciding workgroup finishes, so it is known here), clears their
// states and records how many workers handed their block back.
template <int DT, bool ACC = false>
__device__ __forceinline__ void finish(const DevPlan& p, gclip_result* res, bool fused, HandSlots& hs, int* flag,
                                       const AccSrc& A = AccSrc{}) {
  __syncthreads();
  if (threadIdx.x == 0) {
    complete_stores();
    *flag = take_ticket(finish_tickets(p), p.nworkers) ? 1 : 0;
    if (*flag) acquire_agent();  // before the hand-back count, the decision and the states are read
  }
  __syncthreads();
  if (*flag == 0) return;
  if (fused) {
    const uint32_t handed = atomic_ld(&p.sync[kHandedWord]);
    if (handed != 0u) {
      // the deciding workgroup published before it took its finish ticket
      const uint64_t dw = atomic_ld(&p.bcast[0]);
      const bool skip = dw == kDecidedSkip || dw == kUndecided;
      const double s = skip ? 1.0 : __builtin_bit_cast(double, dw);
      if constexpr (ACC) {
        take_handed_blocks<DT, true>(p, hs, s, (float)s, A, !skip && s != 1.0);
      } else {
        if (!skip && s != 1.0) take_handed_blocks<DT>(p, hs, s, (float)s);
      }
      __syncthreads();
      for (uint32_t i = threadIdx.x; i < (uint32_t)p.nworkers; i += kThreads) atomic_st(&p.bstate[i], kHeld);
    }
    if (threadIdx.x == 0) {
      res->handed_back = (int32_t)handed;
      atomic_st(&p.sync[kHandedWord], 0u);
      // every workgroup has left its wait for the decision: the next launch
      // (a replayed graph's too) starts from an undecided word
      atomic_st(&p.bcast[0], kUndecided);
    }
  }
  if (threadIdx.x == 0) atomic_st(scale_claims(p), 0u);
}

// ---------------------------------------------------------------- kernels
// Kernels 1 and 2 of the pages' pipeline.  Partial sums of squares: the
// chunks of the streamed region this workgroup claims (one partial per chunk
// and wave), then worker w's block and single elements (one partial per
// worker); the last workgroup to arrive sums every partial in index order.
// The fused kernel adds the same values in the same order, so both paths
// give the same bits.
template <int DT, bool TWO>
__global__ __launch_bounds__(kThreads) void k_grad_norm_partial(DevPlan p, AvgSrc avs, gclip_result* res) {
  const double avg = avg_value(avs);
  __shared__ double red[kWaves];
  __shared__ ClaimSlots sl;
  __shared__ int flag;
  const int w = blockIdx.x;
  norm_chunks<DT, TWO>(p, sl);
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
      atomic_st(sum_claims(p), 0u);
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
// the chunks each workgroup claims, or no write at all.  A block whose status
// reports a failure (a gathering wait before this pass gave up, so sumsq and
// nonfinite are not this call's) is left as it is and nothing is written:
// deciding from it could scale by a stale norm, or miss a NaN the stop switch
// would have caught.
template <int DT, bool NTS>
__global__ __launch_bounds__(kThreads) void k_grad_scale(DevPlan p, double max_norm, AvgSrc avs, int err,
                                                         gclip_result* res) {
  const double avg = avg_value(avs);
  __shared__ ClaimSlots sl;
  __shared__ HandSlots hs;
  __shared__ int flag;
  const int w = blockIdx.x;
  const bool failed = res->status != 0;
  const Decision d = decide(res->sumsq, res->nonfinite, max_norm, avg, err);
  if (w == 0 && threadIdx.x == 0 && !failed) write_decision(res, d, max_norm);
  if (!failed && !(d.skip || d.s == 1.0)) {
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
  GCLIP_STAMP(GCLIP_STAMP_BLOCK_WRITTEN);
  scale_chunks<DT, NTS>(p, sl, p.fus_vb, p.fus_seg, p.nchs, s64, s32);
  GCLIP_STAMP(GCLIP_STAMP_CHUNKS_SCALED);
}

// With the += (ACC): the block's sums, scaled when `scale`, and -- only then
// -- the scale chunks of the streamed region it claims (which hold sums
// already, written by any workgroup: read with device-scope loads).
template <int DT, bool NTS>
__device__ __forceinline__ void write_block_sums(const DevPlan& p, ClaimSlots& sl, const Range& r,
                                                 const BlockSplit& bs, const u32x4 (&keep)[kRegSteps],
                                                 const u32x4* keep_lds, double s64, float s32, bool scale) {
  const uint32_t t = threadIdx.x;
  if (r.b < r.e) {
    Cursor cur;
    cursor_load(p, cur, r.seg);
#pragma unroll
    for (int g = 0; g < kRegSteps / kUnroll; ++g) {
      if ((uint32_t)(g * kUnroll) < bs.nreg)
        store_group<NTS>(p, cur, r.b, r.e, g * kUnroll, bs.nreg, [&](int u) {
          return scale ? scale_vec<DT>(keep[g * kUnroll + u], s64, s32) : keep[g * kUnroll + u];
        });
    }
    for (uint32_t k0 = 0; k0 < bs.nlds; k0 += kUnroll)
      store_group<NTS>(p, cur, r.b, r.e, bs.nreg + k0, bs.nsteps, [&](int u) {
        const u32x4 n = keep_lds[(k0 + u) * kThreads + t];
        return scale ? scale_vec<DT>(n, s64, s32) : n;
      });
  }
  GCLIP_STAMP(GCLIP_STAMP_BLOCK_WRITTEN);
  if (scale) scale_chunks<DT, NTS, true>(p, sl, p.fus_vb, p.fus_seg, p.nchs, s64, s32);
  GCLIP_STAMP(GCLIP_STAMP_CHUNKS_SCALED);
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
//
// With the last microbatch's contribution (ACC), phase 1 adds it as it reads:
// the workgroup's sum chunk of the streamed region is written back as sums at
// once (device-scope stores), the block is kept as sums on chip (its LDS
// steps are read first, one group of both lists ahead, while the registers
// that will hold the rest are still free), and phase 2 writes the block's
// sums -- scaled, unless the decision writes nothing, when they are written
// as they are -- so the block is written once; then, when the decision
// scales, it rescales the scale chunks of the streamed region it claims, as
// the plain clip scales them, with device-scope loads.
template <int DT, bool NTS, bool ACC>
__device__ __forceinline__ void clip_fused(const DevPlan& p, const AccSrc& A, double max_norm, AvgSrc avs, int err,
                                           gclip_result* res, uint64_t wait_ticks, const AmpUpdate& amp) {
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
  GCLIP_STAMP(GCLIP_STAMP_START);

  if constexpr (ACC) {
    accum_chunks<DT, NTS>(p, A, sl);
  } else {
    norm_chunks<DT, NTS>(p, sl);
  }
  GCLIP_STAMP(GCLIP_STAMP_CHUNKS_SUMMED);
  double acc[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) acc[u] = 0.0;
  const Range r = block_range(p, w);
  const BlockSplit bs = block_split(r);
  u32x4 keep[kRegSteps];
  if (ACC && r.b < r.e) {
    Cursor c0;
    cursor_load(p, c0, r.seg);
    {  // LDS steps, the next group's loads (both lists) in flight while one is added
      Cursor cur = c0, cg = c0;
      u32x4 q[kUnroll], h[kUnroll];
      if (bs.nlds > 0) {
        load_group<kNtSum>(p, cur, r.b, r.e, bs.nreg, bs.nsteps, q);
        load_group_contrib<kNtSum>(p, A, cg, r.b, r.e, bs.nreg, bs.nsteps, h);
      }
      for (uint32_t k0 = 0; k0 < bs.nlds; k0 += kUnroll) {
        const bool more = k0 + kUnroll < bs.nlds;
        u32x4 q2[kUnroll], h2[kUnroll];
        if (more) {
          load_group<kNtSum>(p, cur, r.b, r.e, bs.nreg + k0 + kUnroll, bs.nsteps, q2);
          load_group_contrib<kNtSum>(p, A, cg, r.b, r.e, bs.nreg + k0 + kUnroll, bs.nsteps, h2);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          if (k0 + u < bs.nlds) {
            const u32x4 n = add_vec<DT>(q[u], h[u]);
            acc[u] += vec_sumsq<DT>(n);
            keep_lds[(k0 + u) * kThreads + t] = n;
          }
        }
        if (more) {
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            q[u] = q2[u];
            h[u] = h2[u];
          }
        }
      }
    }
    {  // register steps: every load of the list first, then the contribution group by group
      Cursor cur = c0;
#pragma unroll
      for (int g = 0; g < kRegSteps / kUnroll; ++g) {
        u32x4 q[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) q[u] = u32x4{0u, 0u, 0u, 0u};
        if ((uint32_t)(g * kUnroll) < bs.nreg) load_group<kNtSum>(p, cur, r.b, r.e, g * kUnroll, bs.nreg, q);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) keep[g * kUnroll + u] = q[u];
      }
      Cursor cg = c0;
#pragma unroll
      for (int g = 0; g < kRegSteps / kUnroll; ++g) {
        if ((uint32_t)(g * kUnroll) < bs.nreg) {
          u32x4 h[kUnroll];
          load_group_contrib<kNtSum>(p, A, cg, r.b, r.e, g * kUnroll, bs.nreg, h);
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) keep[g * kUnroll + u] = add_vec<DT>(keep[g * kUnroll + u], h[u]);
        }
      }
#pragma unroll
      for (int k = 0; k < kRegSteps; ++k)
        if ((uint32_t)k < bs.nreg) acc[k % kUnroll] += vec_sumsq<DT>(keep[k]);
    }
  } else if (!ACC && r.b < r.e) {
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
  GCLIP_STAMP(GCLIP_STAMP_BLOCK_READ);
  double sc = 0.0;
  if constexpr (ACC) {
    sc = accum_scalars<DT>(p, A, w);
  } else {
    sc = norm_scalars<DT>(p, w);
  }
  const double part = wg_sum(lane_total(acc, sc), red);
  if (t == 0) atomic_st(worker_partial(p, w), part);

  // grid-wide decision: the last workgroup to arrive reduces and releases.
  // With the +=, the sums of the streamed region were stored with
  // device-scope stores, every wave's completed before the arrival ticket,
  // and whoever rescales them after the decision loads them with
  // device-scope loads.  The single elements were stored with ordinary
  // stores: phase 2 rescales only this workgroup's own, which a barrier makes
  // visible to it, and only a hand-back passes them to another workgroup,
  // with an agent-scope release (the state word) and acquire (the taker's
  // compare-and-swap).
  if constexpr (ACC) {
    complete_stores();
    __syncthreads();
  }
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
      // the decision is published by value: the word is the flag, so the
      // workgroups waiting for it need no ordering against any other store
      atomic_st(&p.bcast[0], d.skip ? kDecidedSkip : __builtin_bit_cast(uint64_t, d.s));
      atomic_st(sum_claims(p), 0u);
      // every workgroup has arrived, so each has read the loss scale it uses:
      // the state can move on to the next step's
      if (amp.st) amp_update(amp.st, nonfinite_of(S, avg), amp);
    }
  } else if (t == 0) {
    const uint64_t t0 = wall_clock64();
    uint64_t dw;
    while ((dw = atomic_ld(&p.bcast[0])) == kUndecided) {
      __builtin_amdgcn_s_sleep(2);
      if (wall_clock64() - t0 > wait_ticks) {
        // hand the block back: its state is visible before the count (with
        // the +=, released: the taker rescales this workgroup's sums)
        if constexpr (ACC) {
          __hip_atomic_store(&p.bstate[w], kHanded, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          atomic_st(&p.bstate[w], kHanded);
        }
        complete_stores();
        atomic_add(&p.sync[kHandedWord], 1u);
        gave_up = 1;
        break;
      }
    }
    if (!gave_up) {
      bc_skip = dw == kDecidedSkip ? 1 : 0;
      bc_s = bc_skip ? 1.0 : __builtin_bit_cast(double, dw);
      // with the +=, phase 2 loads sums that other workgroups stored: an
      // agent-scope acquire first, so that no copy of their lines that this
      // XCD's caches took earlier (a line shared with a single element or a
      // block) is read in their place
      if constexpr (ACC) acquire_agent();
    }
  }
  __syncthreads();
  if (!gave_up) GCLIP_STAMP(GCLIP_STAMP_DECISION_SEEN);
  const double s64 = bc_s;
  if constexpr (ACC) {
    if (!gave_up) {
      const bool scale = !bc_skip && s64 != 1.0;
      const float s32 = (float)s64;
      write_block_sums<DT, NTS>(p, sl, r, bs, keep, keep_lds, s64, s32, scale);
      if (scale) scale_scalars<DT>(p, w, s64, s32);
      if (t == 0) handed = (int)atomic_ld(&p.sync[kHandedWord]);
      __syncthreads();
      if (handed) take_handed_blocks<DT, true>(p, hs, s64, s32, A, scale);
    }
  } else {
    if (!gave_up && !bc_skip && s64 != 1.0) {
      const float s32 = (float)s64;
      write_block_and_chunks<DT, NTS>(p, sl, r, bs, keep, keep_lds, s64, s32);
      scale_scalars<DT>(p, w, s64, s32);
      if (t == 0) handed = (int)atomic_ld(&p.sync[kHandedWord]);
      __syncthreads();
      if (handed) take_handed_blocks<DT>(p, hs, s64, s32);
    }
  }
  finish<DT, ACC>(p, res, true, hs, &flag, A);
  GCLIP_STAMP(GCLIP_STAMP_END);
}

template <int DT, bool NTS>
__global__ __launch_bounds__(kThreads, 1) void k_grad_clip_fused(DevPlan p, double max_norm, AvgSrc avs, int err,
                                                                 gclip_result* res, uint64_t wait_ticks,
                                                                 AmpUpdate amp) {
  clip_fused<DT, NTS, false>(p, AccSrc{nullptr, nullptr}, max_norm, avs, err, res, wait_ticks, amp);
}

// The last microbatch's += and the clip in one launch.
template <int DT, bool NTS>
__global__ __launch_bounds__(kThreads, 1) void k_accum_clip_fused(DevPlan p, AccSrc A, double max_norm, AvgSrc avs,
                                                                  int err, gclip_result* res,
                                                                  uint64_t wait_ticks) {
  clip_fused<DT, NTS, true>(p, A, max_norm, avs, err, res, wait_ticks, AmpUpdate{nullptr, 0.0, 0.0, 0});
}

// ---------------------------------------------------------------- a list of one group, one workgroup
// A plan with one_group set has a single worker whose block is the whole
// vector space (one group of steps) and at most one single element per
// lane.  One workgroup then takes the whole clip: the group's loads, its
// sum, the decision and -- only if it writes -- the scaled group from the
// same registers.  It adds the same values in the same order as the grid
// kernels do on this plan (the block's steps into acc[j % kUnroll], the
// single elements per lane, wg_sum into the worker's partial), and the
// partial is the norm's sum as it is: the grid kernels' last workgroup adds
// the one partial to zeros, which leaves its bits as they are.  So the bits
// are those of both paths, without a ticket, an atomic or a wait.
template <int DT>
__global__ __launch_bounds__(kThreads) void k_grad_clip_small(DevPlan p, double max_norm, AvgSrc avs, int err,
                                                              gclip_result* res, AmpUpdate amp) {
  const double avg = avg_value(avs);
  __shared__ double red[kWaves];
  __shared__ double bc_s;
  __shared__ int bc_write;
  const Range r = block_range(p, 0);
  const uint64_t ns = range_steps(r);
  Cursor cur;
  u32x4 q[kUnroll];
  double acc[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    q[u] = u32x4{0u, 0u, 0u, 0u};
    acc[u] = 0.0;
  }
  if (ns > 0) {
    cursor_load(p, cur, r.seg);
    Cursor c0 = cur;
    load_group<kNtSum>(p, c0, r.b, r.e, 0, ns, q);
  }
  const double sc = norm_scalars<DT>(p, 0);
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    if ((uint64_t)u < ns) acc[u] += vec_sumsq<DT>(q[u]);
  const double S = wg_sum(lane_total(acc, sc), red);
  if (threadIdx.x == 0) {
    const Decision d = decide((avg * avg) * S, nonfinite_of(S, avg), max_norm, avg, err);
    write_norm(res, S, avg);
    write_decision(res, d, max_norm);
    res->status = 0;
    res->handed_back = 0;
    if (amp.st) amp_update(amp.st, nonfinite_of(S, avg), amp);
    bc_s = d.s;
    bc_write = !(d.skip || d.s == 1.0);
  }
  __syncthreads();
  if (!bc_write) return;
  const double s64 = bc_s;
  const float s32 = (float)s64;
  if (ns > 0) store_group<false>(p, cur, r.b, r.e, 0, ns, [&](int u) { return scale_vec<DT>(q[u], s64, s32); });
  scale_scalars<DT>(p, 0, s64, s32);
}

// ---------------------------------------------------------------- per-tensor clip in one launch
// Grad clip lesson, "Two variants: Per-Tensor or Global": every tensor by its
// own norm, in one launch that keeps part of the list on chip across the
// decisions, as clip_fused does for the global norm.  It walks the list's
// per-tensor pieces (TPiece: a run of one tensor, at most one group of
// vectors, the tensor's single elements on its first piece).  Worker w:
//   phase 1 -- sums its run of streamed pieces [run_b[w], run_b[w + 1]),
//     then loads its resident pieces (the last pieces of the list, at most
//     kTensorResidentPieces) into VGPRs and LDS and sums them.  Each piece's
//     partial is taken exactly as k_tensor_partial takes it: per lane the
//     piece's vectors and single elements, per wave an xor butterfly, then
//     the waves in wave order (the wave sums wait in LDS, so a piece costs
//     no barrier).  It then counts the pieces of every tensor it summed on
//     the tensor's counter; the workgroup that completes a tensor sums its
//     partials in k_tensor_clip's order, stores its figures, raw sum and
//     factor, and clears the counter.  Then the arrival ticket: the last
//     workgroup gathers the list's figures as k_tensor_clip's workgroup 0
//     does, and publishes the decision word (kDecidedSkip when the stop
//     switch meets a NaN/Inf).  So every figure and every written bit is the
//     two-kernel path's;
//   phase 2 -- writes its resident pieces scaled by their tensors' factors
//     (nothing where a factor is 1), then scales streamed pieces as one-piece
//     chunks: pieces w and nworkers + w without a claim, the rest claimed.
// A tensor's factor is read by value: its slot holds kUndecided until the
// tensor's completer stores the factor (before its arrival ticket, so before
// the decision), and the last workgroup to finish empties it again.  Waits
// are bounded as in clip_fused: a workgroup that waits too long for the
// decision hands its resident pieces and its two unclaimed streamed pieces
// back, and the workgroups that see the decision -- in the end the last one
// to finish -- scale those from memory.
static_assert(kTensorPieceVectors <= kGroupVectors, "a piece is at most one group");
static_assert(kTensorRegPieces * kUnroll == kRegSteps, "the register pieces fill the register steps");
static_assert(kTensorLdsPieces * kUnroll <= kLdsSteps, "the LDS pieces fit the LDS steps");
constexpr uint32_t kPieceSlots = 64;      // piece partials waiting in LDS for their waves' sum
constexpr int kTensorBatch = 8;           // completed tensors summed at once
constexpr uint32_t kFactorMissWord = 1;   // line 0 of sync: factors never seen (the launch then fails)

// The piece's vectors into q (one group; lane t holds vector u kThreads + t).
template <bool NT>
__device__ __forceinline__ void load_piece(const TPiece& pc, u32x4 (&q)[kUnroll]) {
  const g_u32x4* base = reinterpret_cast<const g_u32x4*>(uniform64(pc.addr));
  const uint32_t nvec = uniform32(pc.nvec);
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t i = piece_index(0, u, threadIdx.x);
    q[u] = i < nvec ? ld_vec<NT>(base + i) : u32x4{0u, 0u, 0u, 0u};
  }
}

// One lane's share of a piece's sum of squares, as piece_sumsq takes it.
template <int DT>
__device__ __forceinline__ double piece_lane_sum(const TensorPlan& T, const TPiece& pc, const u32x4 (&q)[kUnroll]) {
  double acc[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    acc[u] = 0.0;
    acc[u] += vec_sumsq<DT>(q[u]);
  }
  double s = 0.0;
  const uint32_t nsc = uniform32(pc.sc_count), sc0 = uniform32(pc.sc_begin);
  for (uint32_t i = threadIdx.x; i < nsc; i += kThreads) s += elem_square<DT>(load_elem<DT>(T.sc_addr[sc0 + i]));
  return lane_total(acc, s);
}

// The wave's sum of v (an xor butterfly, as wg_sum takes it) into slot[wave].
__device__ __forceinline__ void wave_sum_to(double v, double* slot) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  if ((threadIdx.x & 63) == 0) slot[threadIdx.x >> 6] = v;
}

// The partials of pieces [base, base + n): each slot's wave sums added in
// wave order (as wg_sum adds them), stored by lanes of wave 0.
__device__ __forceinline__ void flush_partials(const TensorPlan& T, double (*pred)[kWaves], uint32_t base, uint32_t n) {
  __syncthreads();
  if (threadIdx.x < n) {
    double s = pred[threadIdx.x][0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) s += pred[threadIdx.x][k];
    atomic_st(&T.partials[base + threadIdx.x], s);
  }
  __syncthreads();
}

// A tensor's figures, every field with an agent-scope store.
__device__ __forceinline__ void store_figures(gclip_tensor_result* dst, const gclip_tensor_result& o) {
  atomic_st(&dst->sumsq, o.sumsq);
  atomic_st(&dst->norm, o.norm);
  atomic_st(&dst->scale, o.scale);
  atomic_st(reinterpret_cast<uint32_t*>(&dst->nonfinite), (uint32_t)o.nonfinite);
  atomic_st(reinterpret_cast<uint32_t*>(&dst->clipped), (uint32_t)o.clipped);
}

// A tensor's factor slot, read once (the read is issued with a piece's loads).
__device__ __forceinline__ uint64_t factor_bits(const TensorPlan& T, uint32_t k) {
  return atomic_ld(reinterpret_cast<const uint64_t*>(&T.tfac[k]));
}

// A tensor's factor by value (see above), from bits already read; 1.0 --
// nothing written -- and a counted miss if it does not show within
// kFactorWaitTicks (about a second of the device's wall clock), which cannot
// happen unless a store is lost.
constexpr uint64_t kFactorWaitTicks = 1ull << 27;
__device__ __forceinline__ double tensor_factor(const DevPlan& p, const TensorPlan& T, uint32_t k, uint64_t b) {
  const uint64_t* slot = reinterpret_cast<const uint64_t*>(&T.tfac[k]);
  if (b == kUndecided) {
    const uint64_t t0 = wall_clock64();
    while ((b = atomic_ld(slot)) == kUndecided) {
      __builtin_amdgcn_s_sleep(1);
      if (wall_clock64() - t0 > kFactorWaitTicks) {
        if (threadIdx.x == 0) (void)atomic_add(&p.sync[kFactorMissWord], 1u);
        return 1.0;
      }
    }
  }
  return __builtin_bit_cast(double, b);
}

// A piece scaled from memory (a handed-back piece): every vector, then its
// single elements.
template <int DT, bool NTS>
__device__ __forceinline__ void scale_piece_mem(const TensorPlan& T, const TPiece& pc, double s64, float s32) {
  u32x4 q[kUnroll];
  load_piece<kNtScale>(pc, q);
  g_u32x4* base = reinterpret_cast<g_u32x4*>(uniform64(pc.addr));
  const uint32_t nvec = uniform32(pc.nvec);
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t i = piece_index(0, u, threadIdx.x);
    if (i < nvec) st_vec<NTS>(base + i, scale_vec<DT>(q[u], s64, s32));
  }
  const uint32_t nsc = uniform32(pc.sc_count), sc0 = uniform32(pc.sc_begin);
  for (uint32_t i = threadIdx.x; i < nsc; i += kThreads) {
    const uint64_t a = T.sc_addr[sc0 + i];
    store_elem<DT>(a, scale_elem<DT>(load_elem<DT>(a), s64, s32));
  }
}

// Piece c scaled by its tensor's factor, from memory, when that is not 1.
template <int DT, bool NTS>
__device__ __forceinline__ void scale_piece_by_tensor(const DevPlan& p, const TensorPlan& T, uint32_t c) {
  const TPiece pc = ld_table(T.pieces, c);
  const uint32_t k = uniform32(pc.tensor);
  const double f = tensor_factor(p, T, k, factor_bits(T, k));
  if (f != 1.0) scale_piece_mem<DT, NTS>(T, pc, f, (float)f);
}

// Take over every handed-back worker's pieces and scale them from memory:
// its resident pieces and the two streamed pieces it takes without a claim.
template <int DT, bool NTS>
__device__ __forceinline__ void take_handed_pieces(const DevPlan& p, const TensorPlan& T, HandSlots& hs) {
  const uint32_t nw = (uint32_t)p.nworkers;
  for (uint32_t base = 0; base < nw; base += kThreads) {
    if (threadIdx.x == 0) hs.n = 0;
    __syncthreads();
    const uint32_t i = base + threadIdx.x;
    if (i < nw && atomic_ld(&p.bstate[i]) == kHanded) {
      uint32_t expected = kHanded;
      if (__hip_atomic_compare_exchange_strong(&p.bstate[i], &expected, kTaken, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT))
        hs.list[atomicAdd(&hs.n, 1u)] = i;
    }
    __syncthreads();
    const uint32_t n = hs.n;
    for (uint32_t k = 0; k < n; ++k) {
      const uint32_t v = hs.list[k];
      const uint32_t ra = T.ps + ld_table(T.res_b, (uint64_t)v), rz = T.ps + ld_table(T.res_b, (uint64_t)v + 1);
      for (uint32_t c = ra; c < rz; ++c) scale_piece_by_tensor<DT, NTS>(p, T, c);
      for (uint32_t c = v; c < T.ps && c < v + 2u * nw; c += nw) scale_piece_by_tensor<DT, NTS>(p, T, c);
    }
    __syncthreads();
  }
}

template <int DT, bool NTS>
__global__ __launch_bounds__(kThreads, 1) void k_tensor_clip_fused(DevPlan p, TensorPlan T, AvgSrc avs,
                                                                   double max_norm, int err,
                                                                   gclip_tensor_result* out, gclip_result* res,
                                                                   uint64_t wait_ticks) {
  const double avg = avg_value(avs);
  __shared__ u32x4 keep_lds[kTensorLdsPieces * kUnroll * kThreads];
  __shared__ double pred[kPieceSlots][kWaves];
  __shared__ double red[kWaves];
  __shared__ uint32_t done[kPieceSlots];
  __shared__ uint32_t ndone;
  __shared__ ClaimSlots sl;
  __shared__ HandSlots hs;
  __shared__ int flag;
  __shared__ int gave_up;
  __shared__ int skip_all;
  const uint32_t w = blockIdx.x, t = threadIdx.x;
  const uint32_t nw = (uint32_t)p.nworkers;
  GCLIP_STAMP(GCLIP_STAMP_START);

  // ---- phase 1: the streamed run, then the resident pieces: data one piece
  // ahead, descriptors two (a piece's loads need its descriptor's address,
  // a scalar load).  Resident piece k goes to LDS for k < kTensorLdsPieces --
  // first, while the registers are free -- and to VGPRs after.
  const uint32_t rb = ld_table(T.run_b, (uint64_t)w), re = ld_table(T.run_b, (uint64_t)w + 1);
  const uint32_t ra = T.ps + ld_table(T.res_b, (uint64_t)w), rz = T.ps + ld_table(T.res_b, (uint64_t)w + 1);
  const uint32_t ns = re - rb, nr = rz - ra, m = ns + nr;
  // piece i of the two runs
  auto run_piece = [&](uint32_t i) { return i < ns ? rb + i : ra + (i - ns); };
  u32x4 q[kUnroll];
  TPiece pc{}, pcn{};
  if (m > 0) {
    pc = ld_table(T.pieces, run_piece(0));
    load_piece<kNtSum>(pc, q);
  }
  if (m > 1) pcn = ld_table(T.pieces, run_piece(1));
  {
    uint32_t nslot = 0;
    for (uint32_t i = 0; i < ns; ++i) {
      u32x4 q2[kUnroll];
      TPiece pcnn{};
      const bool more = i + 1 < m;
      if (i + 2 < m) pcnn = ld_table(T.pieces, run_piece(i + 2));
      if (more) load_piece<kNtSum>(pcn, q2);
      wave_sum_to(piece_lane_sum<DT>(T, pc, q), pred[nslot]);
      if (++nslot == kPieceSlots) {
        flush_partials(T, pred, rb + i + 1 - nslot, nslot);
        nslot = 0;
      }
      if (more) {
        pc = pcn;
        pcn = pcnn;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) q[u] = q2[u];
      }
    }
    if (nslot) flush_partials(T, pred, re - nslot, nslot);
  }
  GCLIP_STAMP(GCLIP_STAMP_CHUNKS_SUMMED);
  u32x4 keep[kTensorRegPieces * kUnroll];
#pragma unroll
  for (int k = 0; k < kTensorResidentPieces; ++k) {
    if ((uint32_t)k < nr) {
      u32x4 q2[kUnroll];
      TPiece pcnn{};
      const bool more = (uint32_t)k + 1 < nr;
      if ((uint32_t)k + 2 < nr) pcnn = ld_table(T.pieces, ra + (uint32_t)k + 2);
      if (more) load_piece<kNtSum>(pcn, q2);
      wave_sum_to(piece_lane_sum<DT>(T, pc, q), pred[k]);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (k < kTensorLdsPieces) {
          keep_lds[(k * kUnroll + u) * kThreads + t] = q[u];
        } else {
          keep[(k >= kTensorLdsPieces ? k - kTensorLdsPieces : 0) * kUnroll + u] = q[u];
        }
      }
      if (more) {
        pc = pcn;
        pcn = pcnn;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) q[u] = q2[u];
      }
    }
  }
  if (nr) flush_partials(T, pred, ra, nr);
  GCLIP_STAMP(GCLIP_STAMP_BLOCK_READ);

  // ---- phase 1: count the pieces of every tensor summed here; complete tensors
  // The two runs are taken kPieceSlots pieces at a time, a lane per piece; a
  // run's pieces of one tensor form a segment, counted on the tensor's
  // counter by the lane of its first piece (segments end where the run or
  // the tensor does: pieces are in tensor order).  A window holds at most
  // kPieceSlots segment starts, so at most kPieceSlots completions.
  if (t == 0) complete_stores();  // the partials (wave 0's stores) before the counts
  {
    const uint32_t m = ns + nr;
    for (uint32_t w0 = 0; w0 < m; w0 += kPieceSlots) {
      if (t == 0) ndone = 0;
      __syncthreads();
      const uint32_t i = w0 + t;
      if (t < kPieceSlots && i < m) {
        const uint32_t c = i < ns ? rb + i : ra + (i - ns);
        const uint32_t run_end = i < ns ? re : rz;
        const uint32_t k = T.pieces[c].tensor;
        const uint32_t b = T.first[k], f = T.first[k + 1];
        if (i == 0 || i == ns || c == b) {
          const uint32_t e = f < run_end ? f : run_end;
          if (atomic_add(&T.tcount[k], e - c) + (e - c) == f - b) done[atomicAdd(&ndone, 1u)] = k;
        }
      }
      __syncthreads();
      const uint32_t nd = ndone;
      if (nd == 0) continue;
      if (t == 0) acquire_agent();  // every piece of these tensors stored its partial before its count
      __syncthreads();
      // kTensorBatch tensors at a time, their partials' loads all in flight:
      // lane t sums partials b + t, b + t + kThreads, ... of each (the order of
      // k_tensor_clip), then the waves in wave order
      for (uint32_t d0 = 0; d0 < nd; d0 += kTensorBatch) {
        uint32_t tb[kTensorBatch], te[kTensorBatch], rounds = 0;
#pragma unroll
        for (int j = 0; j < kTensorBatch; ++j) {
          tb[j] = te[j] = 0;
          if (d0 + (uint32_t)j < nd) {
            const uint32_t k = done[d0 + j];
            tb[j] = T.first[k];
            te[j] = T.first[k + 1];
            const uint32_t r = (te[j] - tb[j] + kThreads - 1) / kThreads;
            rounds = r > rounds ? r : rounds;
          }
        }
        double v[kTensorBatch];
#pragma unroll
        for (int j = 0; j < kTensorBatch; ++j) v[j] = 0.0;
        for (uint32_t r = 0; r < rounds; ++r) {
          double x[kTensorBatch];
#pragma unroll
          for (int j = 0; j < kTensorBatch; ++j) {
            const uint32_t pi = tb[j] + r * kThreads + t;
            x[j] = pi < te[j] ? atomic_ld(&T.partials[pi]) : 0.0;
          }
#pragma unroll
          for (int j = 0; j < kTensorBatch; ++j) v[j] += x[j];
        }
#pragma unroll
        for (int j = 0; j < kTensorBatch; ++j)
          if (d0 + (uint32_t)j < nd) wave_sum_to(v[j], pred[j]);
        __syncthreads();
        if (t < kTensorBatch && d0 + t < nd) {
          const uint32_t k = done[d0 + t];
          double S = pred[t][0];
#pragma unroll
          for (int j = 1; j < kWaves; ++j) S += pred[t][j];
          gclip_tensor_result o;
          tensor_figures(&o, S, avg, max_norm);
          const Decision dd = decide((avg * avg) * S, nonfinite_of(S, avg), max_norm, avg, 0);
          // every figure with agent-scope stores: the last workgroup may
          // overwrite the factor (the stop switch), from another XCD
          store_figures(&out[k], o);
          atomic_st(&T.tsum[k], S);
          atomic_st(reinterpret_cast<uint64_t*>(&T.tfac[k]), __builtin_bit_cast(uint64_t, dd.s));
          atomic_st(&T.tcount[k], 0u);  // every piece of k has been counted
        }
        __syncthreads();
      }
    }
  }

  GCLIP_STAMP(GCLIP_STAMP_TENSORS_DONE);

  // ---- the grid-wide decision: the last workgroup gathers the list's figures
  if (t == 0) gave_up = 0;
  if (arrive(p, &flag)) {
    double v = 0.0;
    int nf_mine = 0, clipped_mine = 0;
    for (int32_t j = (int32_t)t; j < T.ntensors; j += kThreads) {
      // the raw sum is loaded with the table entries, not after them (an
      // empty tensor's slot holds no sum and is not used)
      const double Sr = atomic_ld(&T.tsum[j]);
      const bool live = ld_table(T.first, (uint64_t)j) < ld_table(T.first, (uint64_t)j + 1);
      const double S = live ? Sr : 0.0;
      v += S;
      nf_mine |= nonfinite_of(S, avg);
      clipped_mine |= decide((avg * avg) * S, nonfinite_of(S, avg), max_norm, avg, err).clipped;
      if (!live) {
        gclip_tensor_result o;
        tensor_figures(&o, 0.0, avg, max_norm);
        store_figures(&out[j], o);
      }
    }
    const double S = wg_sum(v, red);
    const int nf_any = __syncthreads_or(nf_mine);
    const int clipped_any = __syncthreads_or(clipped_mine);
    const int skip = (err && nf_any) ? 1 : 0;
    if (skip) {
      // the stop switch: no tensor is written, every factor in the figures is 1
      for (int32_t j = (int32_t)t; j < T.ntensors; j += kThreads) atomic_st(&out[j].scale, 1.0);
    }
    if (t == 0) {
      write_norm(res, S, avg);
      res->nonfinite = nf_any | res->nonfinite;
      res->scale = 1.0;
      res->clipped = clipped_any;
      res->skipped = skip;
      res->max_norm = max_norm;
      res->decided = 1;
      atomic_st(reinterpret_cast<uint32_t*>(&res->status), 0u);
      skip_all = skip;
      // published by value, as in clip_fused: no workgroup reads the figures
      // or the result block after it, so no store here need complete first
      atomic_st(&p.bcast[0], skip ? kDecidedSkip : __builtin_bit_cast(uint64_t, 1.0));
    }
  } else if (t == 0) {
    const uint64_t t0 = wall_clock64();
    uint64_t dw;
    while ((dw = atomic_ld(&p.bcast[0])) == kUndecided) {
      __builtin_amdgcn_s_sleep(2);
      if (wall_clock64() - t0 > wait_ticks) {
        atomic_st(&p.bstate[w], kHanded);
        complete_stores();
        atomic_add(&p.sync[kHandedWord], 1u);
        gave_up = 1;
        break;
      }
    }
    if (!gave_up) skip_all = dw == kDecidedSkip ? 1 : 0;
  }
  __syncthreads();
  if (!gave_up) GCLIP_STAMP(GCLIP_STAMP_DECISION_SEEN);

  // ---- phase 2: the resident pieces, then claimed streamed pieces
  if (!gave_up && !skip_all) {
    uint64_t fb[kTensorResidentPieces];
#pragma unroll
    for (int k = 0; k < kTensorResidentPieces; ++k)
      fb[k] = (uint32_t)k < nr ? factor_bits(T, uniform32(ld_table(T.pieces, ra + (uint32_t)k).tensor)) : 0;
#pragma unroll
    for (int k = 0; k < kTensorResidentPieces; ++k) {
      if ((uint32_t)k < nr) {
        const TPiece pc = ld_table(T.pieces, ra + (uint32_t)k);
        const double f = tensor_factor(p, T, uniform32(pc.tensor), fb[k]);
        if (f != 1.0) {
          const float f32 = (float)f;
          g_u32x4* base = reinterpret_cast<g_u32x4*>(uniform64(pc.addr));
          const uint32_t nvec = uniform32(pc.nvec);
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            const uint32_t i = piece_index(0, u, t);
            if (i < nvec) {
              const u32x4 x = k < kTensorLdsPieces ? keep_lds[(k * kUnroll + u) * kThreads + t]
                                                   : keep[(k >= kTensorLdsPieces ? k - kTensorLdsPieces : 0) * kUnroll + u];
              st_vec<NTS>(base + i, scale_vec<DT>(x, f, f32));
            }
          }
          const uint32_t nsc = uniform32(pc.sc_count), sc0 = uniform32(pc.sc_begin);
          for (uint32_t i = t; i < nsc; i += kThreads) {
            const uint64_t a = T.sc_addr[sc0 + i];
            store_elem<DT>(a, scale_elem<DT>(load_elem<DT>(a), f, f32));
          }
        }
      }
    }
    GCLIP_STAMP(GCLIP_STAMP_BLOCK_WRITTEN);
    // streamed pieces: one-piece chunks, the next one loaded while this one is written
    const uint32_t nch = T.ps;
    if (w < nch) {
      const Claimer cl = make_claimer(scale_claims(p), p, nch);
      uint32_t c = w, cn = second_chunk(p, nch, w);
      u32x4 q[kUnroll];
      TPiece pc = ld_table(T.pieces, c);
      load_piece<kNtScale>(pc, q);
      uint64_t fb = factor_bits(T, uniform32(pc.tensor));
      for (uint32_t i = 0; c != kNone; ++i) {
        uint32_t tk = 0;
        if (t == 0 && cn != kNone) tk = claim_issue(cl);
        const double f = tensor_factor(p, T, uniform32(pc.tensor), fb);
        const uint32_t par = i & 1u;
        if (t == 0) sl.claim[par] = cn != kNone ? claim_resolve(cl, tk) : kNone;
        if (f != 1.0) {
          const float f32 = (float)f;
          g_u32x4* base = reinterpret_cast<g_u32x4*>(uniform64(pc.addr));
          const uint32_t nvec = uniform32(pc.nvec);
          // the last round of pieces with nontemporal stores, as in scale_chunks
          if (!NTS && kLateNtRounds > 0 && c + kLateNtRounds * nw >= nch) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
              const uint32_t vi = piece_index(0, u, t);
              if (vi < nvec) st_vec<true>(base + vi, scale_vec<DT>(q[u], f, f32));
            }
          } else {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
              const uint32_t vi = piece_index(0, u, t);
              if (vi < nvec) st_vec<NTS>(base + vi, scale_vec<DT>(q[u], f, f32));
            }
          }
          const uint32_t nsc = uniform32(pc.sc_count), sc0 = uniform32(pc.sc_begin);
          for (uint32_t vi = t; vi < nsc; vi += kThreads) {
            const uint64_t a = T.sc_addr[sc0 + vi];
            store_elem<DT>(a, scale_elem<DT>(load_elem<DT>(a), f, f32));
          }
        }
        if (cn != kNone) {
          pc = ld_table(T.pieces, cn);
          load_piece<kNtScale>(pc, q);
          fb = factor_bits(T, uniform32(pc.tensor));
        }
        __syncthreads();
        c = cn;
        cn = uniform32(sl.claim[par]);
      }
    }
    GCLIP_STAMP(GCLIP_STAMP_CHUNKS_SCALED);
    if (t == 0) flag = (int)atomic_ld(&p.sync[kHandedWord]);
    __syncthreads();
    if (flag) take_handed_pieces<DT, NTS>(p, T, hs);
  }

  // ---- finish: the last workgroup takes what is still handed back and resets the workspace
  __syncthreads();
  if (t == 0) {
    complete_stores();
    flag = take_ticket(finish_tickets(p), p.nworkers) ? 1 : 0;
    if (flag) acquire_agent();  // before the hand-back count, the decision and the states are read
  }
  __syncthreads();
  GCLIP_STAMP(GCLIP_STAMP_END);
  if (flag == 0) return;
  const uint32_t handed = atomic_ld(&p.sync[kHandedWord]);
  if (handed != 0u) {
    if (atomic_ld(&p.bcast[0]) != kDecidedSkip) take_handed_pieces<DT, NTS>(p, T, hs);
    __syncthreads();
    for (uint32_t i = t; i < nw; i += kThreads) atomic_st(&p.bstate[i], kHeld);
  }
  __syncthreads();
  for (int32_t j = (int32_t)t; j < T.ntensors; j += kThreads)
    atomic_st(reinterpret_cast<uint64_t*>(&T.tfac[j]), kUndecided);
  if (t == 0) {
    res->handed_back = (int32_t)handed;
    atomic_st(&p.sync[kHandedWord], 0u);
    if (atomic_ld(&p.sync[kFactorMissWord]) != 0u) {
      atomic_st(reinterpret_cast<uint32_t*>(&res->status), (uint32_t)GCLIP_DEVICE_WAIT_TIMEOUT);
      atomic_st(&p.sync[kFactorMissWord], 0u);
    }
    atomic_st(&p.bcast[0], kUndecided);
    atomic_st(scale_claims(p), 0u);
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
  if (p.nt_store) {
    switch (dtype) {
      case GCLIP_F32: hipLaunchKernelGGL((k_grad_norm_partial<GCLIP_F32, true>), grid, block, 0, st, p, avg, res); break;
      case GCLIP_F16: hipLaunchKernelGGL((k_grad_norm_partial<GCLIP_F16, true>), grid, block, 0, st, p, avg, res); break;
      default: hipLaunchKernelGGL((k_grad_norm_partial<GCLIP_BF16, true>), grid, block, 0, st, p, avg, res); break;
    }
  } else {
    switch (dtype) {
      case GCLIP_F32: hipLaunchKernelGGL((k_grad_norm_partial<GCLIP_F32, false>), grid, block, 0, st, p, avg, res); break;
      case GCLIP_F16: hipLaunchKernelGGL((k_grad_norm_partial<GCLIP_F16, false>), grid, block, 0, st, p, avg, res); break;
      default: hipLaunchKernelGGL((k_grad_norm_partial<GCLIP_BF16, false>), grid, block, 0, st, p, avg, res); break;
    }
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

template <bool NTS>
const void* accum_fused_kernel(int32_t dtype) {
  return dtype == GCLIP_F32   ? (const void*)k_accum_clip_fused<GCLIP_F32, NTS>
         : dtype == GCLIP_F16 ? (const void*)k_accum_clip_fused<GCLIP_F16, NTS>
                              : (const void*)k_accum_clip_fused<GCLIP_BF16, NTS>;
}

hipError_t launch_accum_fused(const DevPlan& p, const AccSrc& A, int32_t dtype, double max_norm, AvgSrc avg,
                              int err, gclip_result* res, uint64_t wait_ticks, hipStream_t st) {
  DevPlan pc = p;
  AccSrc ac = A;
  void* args[] = {&pc, &ac, &max_norm, &avg, &err, &res, &wait_ticks};
  const void* fn = p.nt_store ? accum_fused_kernel<true>(dtype) : accum_fused_kernel<false>(dtype);
  return hipLaunchKernel(fn, dim3((unsigned)p.nworkers), dim3(kThreads), args, 0, st);
}

hipError_t launch_fused(const DevPlan& p, int32_t dtype, double max_norm, AvgSrc avg, int err, gclip_result* res,
                        uint64_t wait_ticks, AmpUpdate amp, hipStream_t st) {
  DevPlan pc = p;
  if (p.one_group) {
    void* args[] = {&pc, &max_norm, &avg, &err, &res, &amp};
    const void* fn = dtype == GCLIP_F32   ? (const void*)k_grad_clip_small<GCLIP_F32>
                     : dtype == GCLIP_F16 ? (const void*)k_grad_clip_small<GCLIP_F16>
                                          : (const void*)k_grad_clip_small<GCLIP_BF16>;
    return hipLaunchKernel(fn, dim3(1), dim3(kThreads), args, 0, st);
  }
  void* args[] = {&pc, &max_norm, &avg, &err, &res, &wait_ticks, &amp};
  const void* fn = p.nt_store ? fused_kernel<true>(dtype) : fused_kernel<false>(dtype);
  return hipLaunchKernel(fn, dim3((unsigned)p.nworkers), dim3(kThreads), args, 0, st);
}

template <bool NTS>
const void* tensor_fused_kernel(int32_t dtype) {
  return dtype == GCLIP_F32   ? (const void*)k_tensor_clip_fused<GCLIP_F32, NTS>
         : dtype == GCLIP_F16 ? (const void*)k_tensor_clip_fused<GCLIP_F16, NTS>
                              : (const void*)k_tensor_clip_fused<GCLIP_BF16, NTS>;
}

hipError_t launch_tensor_clip_fused(const DevPlan& p, const TensorPlan& T, int32_t dtype, AvgSrc avg,
                                    double max_norm, int err, gclip_tensor_result* out, gclip_result* res,
                                    uint64_t wait_ticks, hipStream_t st) {
  DevPlan pc = p;
  TensorPlan tc = T;
  void* args[] = {&pc, &tc, &avg, &max_norm, &err, &out, &res, &wait_ticks};
  const void* fn = p.nt_store ? tensor_fused_kernel<true>(dtype) : tensor_fused_kernel<false>(dtype);
  return hipLaunchKernel(fn, dim3((unsigned)p.nworkers), dim3(kThreads), args, 0, st);
}

// Workgroups of the one-launch per-tensor clip that fit on one compute unit.
hipError_t tensor_fused_capacity(int32_t dtype, int* blocks_per_cu) {
  int lo = 1 << 30;
  for (const void* fn : {tensor_fused_kernel<false>(dtype), tensor_fused_kernel<true>(dtype)}) {
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kThreads, 0);
    if (e != hipSuccess) return e;
    lo = n < lo ? n : lo;
  }
  *blocks_per_cu = lo;
  return hipSuccess;
}

// Workgroups of the fused kernels that fit on one compute unit at once (the
// smallest over the store variants, with and without the +=).
hipError_t fused_capacity(int32_t dtype, int* blocks_per_cu) {
  const void* fns[] = {fused_kernel<false>(dtype), fused_kernel<true>(dtype), accum_fused_kernel<false>(dtype),
                       accum_fused_kernel<true>(dtype)};
  int lo = 1 << 30;
  for (const void* fn : fns) {
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kThreads, 0);
    if (e != hipSuccess) return e;
    lo = n < lo ? n : lo;
  }
  *blocks_per_cu = lo;
  return hipSuccess;
}

}  // namespace gclip

#ifdef GCLIP_PHASE_STAMPS
extern "C" gclip_status gclip_phase_stamps(uint64_t* host, int32_t n_workers, int64_t* ticks_per_s) {
  if (!host || !ticks_per_s || n_workers < 0 || n_workers > GCLIP_STAMP_WORKERS) return GCLIP_EINVAL;
  int dev = 0, khz = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  if (e == hipSuccess)
    e = hipMemcpyFromSymbol(host, HIP_SYMBOL(gclip::g_phase_stamps),
                            (size_t)n_workers * GCLIP_STAMP_POINTS * sizeof(uint64_t), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return gclip::hip_fail(e);
  *ticks_per_s = (int64_t)khz * 1000;
  return GCLIP_OK;
}
#endif
