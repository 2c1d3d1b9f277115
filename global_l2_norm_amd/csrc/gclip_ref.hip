// gclip_ref.hip -- the attainable-bandwidth reference kernels of
// include/gclip_ref.h: a plain streaming read and a plain copy (in place
// when the two addresses are equal), each in the launch shape that streamed
// fastest on MI355X among those tried (one workgroup per piece, against
// persistent workgroups with static or interleaved shares, at 256 to 1024
// lanes and 4 to 24 vectors in flight per lane).  They do nothing but move
// the bytes, so their rates bound what the clip's two passes can reach:
// the read pass of the norm and the read + write pass of the scale.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/gclip.h"
#include "../../include/gclip_ref.h"
#include "gclip_device.hpp"
#include "gclip_host.hpp"

namespace gclip {

constexpr int kRefThreads = 512;
constexpr int kReadUnroll = 16;  // vectors in flight per lane: one piece is 16 x 512 x 16 B = 128 KB
constexpr int kCopyUnroll = 4;   // 32 KB pieces: a workgroup's loads (nontemporal), then its stores (ordinary)
constexpr uint32_t kSinkMagic = 0x9e3779b9u;

// Every lane folds its vectors into one word; the word is stored only when
// it equals kSinkMagic, so the loads cannot be dropped and the store
// practically never happens.
__global__ __launch_bounds__(kRefThreads) void k_ref_read(const g_u32x4* src, uint64_t nvec, uint32_t* sink) {
  const uint64_t base = (uint64_t)blockIdx.x * (kReadUnroll * kRefThreads);
  u32x4 q[kReadUnroll];
#pragma unroll
  for (int u = 0; u < kReadUnroll; ++u) {
    const uint64_t v = base + (uint64_t)u * kRefThreads + threadIdx.x;
    q[u] = v < nvec ? ld_vec<true>(src + v) : u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < kReadUnroll; ++u) x ^= q[u][0] ^ q[u][1] ^ q[u][2] ^ q[u][3];
  if (x == kSinkMagic) *sink = x;
}

__global__ __launch_bounds__(kRefThreads) void k_ref_copy(g_u32x4* dst, const g_u32x4* src, uint64_t nvec) {
  const uint64_t base = (uint64_t)blockIdx.x * (kCopyUnroll * kRefThreads);
  u32x4 q[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const uint64_t v = base + (uint64_t)u * kRefThreads + threadIdx.x;
    if (v < nvec) q[u] = ld_vec<true>(src + v);
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const uint64_t v = base + (uint64_t)u * kRefThreads + threadIdx.x;
    if (v < nvec) st_vec<false>(dst + v, q[u]);
  }
}

namespace {

bool span_ok(const void* p, int64_t bytes) {
  return bytes >= 0 && bytes % 16 == 0 && (bytes == 0 || (p && reinterpret_cast<uintptr_t>(p) % 16 == 0));
}

// One workgroup per piece of `per` vectors; at most 2^31 - 1 workgroups.
bool grid_of(uint64_t nvec, uint64_t per, unsigned* grid) {
  const uint64_t g = (nvec + per - 1) / per;
  if (g > 0x7fffffffull) return false;
  *grid = (unsigned)g;
  return true;
}

}  // namespace
}  // namespace gclip

extern "C" gclip_status gclip_ref_read(const void* d_src, int64_t bytes, uint32_t* d_sink, void* stream) {
  using namespace gclip;
  if (!span_ok(d_src, bytes) || !d_sink || reinterpret_cast<uintptr_t>(d_sink) % 4 != 0) return GCLIP_EINVAL;
  const uint64_t nvec = (uint64_t)bytes / 16;
  unsigned grid = 0;
  if (!grid_of(nvec, (uint64_t)kReadUnroll * kRefThreads, &grid)) return GCLIP_EINVAL;
  if (grid == 0) return GCLIP_OK;
  hipLaunchKernelGGL(k_ref_read, dim3(grid), dim3(kRefThreads), 0, static_cast<hipStream_t>(stream),
                     reinterpret_cast<const g_u32x4*>(reinterpret_cast<uintptr_t>(d_src)), nvec, d_sink);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? GCLIP_OK : hip_fail(e);
}

extern "C" gclip_status gclip_ref_copy(void* d_dst, const void* d_src, int64_t bytes, void* stream) {
  using namespace gclip;
  if (!span_ok(d_src, bytes) || !span_ok(d_dst, bytes)) return GCLIP_EINVAL;
  const uint64_t s = reinterpret_cast<uint64_t>(d_src), d = reinterpret_cast<uint64_t>(d_dst);
  if (s != d && bytes > 0 && s < d + (uint64_t)bytes && d < s + (uint64_t)bytes) return GCLIP_EINVAL;
  const uint64_t nvec = (uint64_t)bytes / 16;
  unsigned grid = 0;
  if (!grid_of(nvec, (uint64_t)kCopyUnroll * kRefThreads, &grid)) return GCLIP_EINVAL;
  if (grid == 0) return GCLIP_OK;
  hipLaunchKernelGGL(k_ref_copy, dim3(grid), dim3(kRefThreads), 0, static_cast<hipStream_t>(stream),
                     reinterpret_cast<g_u32x4*>(reinterpret_cast<uintptr_t>(d_dst)),
                     reinterpret_cast<const g_u32x4*>(reinterpret_cast<uintptr_t>(d_src)), nvec);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? GCLIP_OK : hip_fail(e);
}
