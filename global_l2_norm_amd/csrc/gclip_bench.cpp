// gclip_bench.cpp -- native timing driver for libgclip's C ABI.
//
//   gclip_bench --data FILE [--mode clip|split|norm|scale|all] [--reps N] [--warmup W]
//               [--no-flush] [--drain-us U] [--calibrate-bytes B]
//
// FILE is a synthetic gradient set written by `python -m synth.dump`.  Each
// tensor gets its own hipMalloc, as a framework's allocator would give it.
// Every rep restores the gradients from a pristine device copy and, unless
// --no-flush, reads a 2 GiB buffer so that no cache holds them, then times
// one call with HIP events on the call's stream.  The restore's writes are
// given --drain-us microseconds (default 2000) after it completes to drain
// from the caches to HBM before the flush, so they do not spill into the
// timed call.  --calibrate-bytes also
// runs a plain copy kernel of that many bytes (for scaling PMC counters).
// Prints one JSON line per mode.  Only the public ABI is used; torch is not
// involved, so the process holds a single HIP runtime.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <chrono>
#include <vector>

#include "../../include/gclip.h"

#define HIP_OK(x)                                                                       \
  do {                                                                                  \
    hipError_t e_ = (x);                                                                \
    if (e_ != hipSuccess) {                                                             \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      exit(3);                                                                          \
    }                                                                                   \
  } while (0)

namespace {

constexpr size_t kFlushBytes = size_t(2) << 30;

__global__ void k_flush_read(const uint4* __restrict__ p, size_t n, unsigned* __restrict__ sink) {
  unsigned acc = 0;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;  // keeps the loads alive
}

__global__ void k_calib_copy(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

struct Set {
  int dtype = 0, err = 0;
  double max_norm = 1.0, avg = 1.0;
  std::vector<int64_t> numel;
  std::vector<std::vector<unsigned char>> host;
};

bool read_set(const char* path, Set& s) {
  FILE* f = fopen(path, "rb");
  if (!f) return false;
  char magic[8];
  uint32_t hdr[4];
  double dd[2];
  bool ok = fread(magic, 1, 8, f) == 8 && memcmp(magic, "GCLIPSET", 8) == 0 && fread(hdr, 4, 4, f) == 4 &&
            fread(dd, 8, 2, f) == 2 && hdr[0] == 1;
  if (ok) {
    s.dtype = (int)hdr[1];
    s.err = (int)hdr[3];
    s.max_norm = dd[0];
    s.avg = dd[1];
    s.numel.resize(hdr[2]);
    ok = fread(s.numel.data(), 8, hdr[2], f) == hdr[2];
    const size_t es = s.dtype == 0 ? 4 : 2;
    for (size_t t = 0; ok && t < s.numel.size(); ++t) {
      s.host.emplace_back((size_t)s.numel[t] * es);
      ok = fread(s.host.back().data(), 1, s.host.back().size(), f) == s.host.back().size();
    }
  }
  fclose(f);
  return ok;
}

void die(const char* what, gclip_status st) {
  fprintf(stderr, "%s: %s (hip %d)\n", what, gclip_status_string(st), gclip_last_hip_error());
  exit(4);
}

}  // namespace

int main(int argc, char** argv) {
  const char* data = nullptr;
  std::string mode = "all";
  int reps = 50, warmup = 5;
  bool flush = true;
  long drain_us = 2000;
  size_t calib = 0;
  for (int i = 1; i < argc; ++i) {
    std::string a = argv[i];
    if (a == "--data" && i + 1 < argc) data = argv[++i];
    else if (a == "--mode" && i + 1 < argc) mode = argv[++i];
    else if (a == "--reps" && i + 1 < argc) reps = atoi(argv[++i]);
    else if (a == "--warmup" && i + 1 < argc) warmup = atoi(argv[++i]);
    else if (a == "--no-flush") flush = false;
    else if (a == "--drain-us" && i + 1 < argc) drain_us = atol(argv[++i]);
    else if (a == "--calibrate-bytes" && i + 1 < argc) calib = strtoull(argv[++i], nullptr, 10);
    else {
      fprintf(stderr, "usage: %s --data FILE [--mode clip|split|norm|scale|all] [--reps N] [--warmup W] "
                      "[--no-flush] [--drain-us U] [--calibrate-bytes B]\n", argv[0]);
      return 2;
    }
  }
  if (!data || reps < 1 || warmup < 0) {
    fprintf(stderr, "--data FILE is required and --reps must be positive\n");
    return 2;
  }
  Set s;
  if (!read_set(data, s)) {
    fprintf(stderr, "cannot read gradient set %s\n", data);
    return 2;
  }
  const size_t es = s.dtype == 0 ? 4 : 2;
  const size_t n = s.numel.size();
  int64_t total = 0;
  std::vector<void*> d(n, nullptr), pristine(n, nullptr);
  for (size_t t = 0; t < n; ++t) {
    total += s.numel[t];
    const size_t b = (size_t)s.numel[t] * es;
    if (b == 0) continue;
    HIP_OK(hipMalloc(&d[t], b));
    HIP_OK(hipMalloc(&pristine[t], b));
    HIP_OK(hipMemcpy(pristine[t], s.host[t].data(), b, hipMemcpyHostToDevice));
  }
  void* fl = nullptr;
  unsigned* sink = nullptr;
  HIP_OK(hipMalloc(&fl, kFlushBytes));
  HIP_OK(hipMemset(fl, 1, kFlushBytes));
  HIP_OK(hipMalloc(&sink, 1 << 16));
  gclip_result* res = nullptr;
  HIP_OK(hipMalloc(&res, sizeof(gclip_result)));
  HIP_OK(hipMemset(res, 0, sizeof(gclip_result)));
  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  hipEvent_t e0, e1;
  HIP_OK(hipEventCreate(&e0));
  HIP_OK(hipEventCreate(&e1));

  gclip_list* L = nullptr;
  gclip_status rc = gclip_list_create(d.data(), s.numel.data(), (int32_t)n, s.dtype, &L);
  if (rc != GCLIP_OK) die("gclip_list_create", rc);
  gclip_list_info_t info;
  gclip_list_info(L, &info);

  auto restore = [&]() {
    for (size_t t = 0; t < n; ++t)
      if (d[t]) HIP_OK(hipMemcpyAsync(d[t], pristine[t], (size_t)s.numel[t] * es, hipMemcpyDeviceToDevice, st));
    if (drain_us > 0) {
      HIP_OK(hipStreamSynchronize(st));
      std::this_thread::sleep_for(std::chrono::microseconds(drain_us));
    }
    if (flush) k_flush_read<<<4096, 256, 0, st>>>((const uint4*)fl, kFlushBytes / 16, sink);
  };

  if (calib) {
    void *a = nullptr, *b = nullptr;
    HIP_OK(hipMalloc(&a, calib));
    HIP_OK(hipMalloc(&b, calib));
    HIP_OK(hipMemset(a, 3, calib));
    float best = 1e30f;
    for (int r = 0; r < 3; ++r) {
      k_flush_read<<<4096, 256, 0, st>>>((const uint4*)fl, kFlushBytes / 16, sink);
      HIP_OK(hipEventRecord(e0, st));
      k_calib_copy<<<4096, 256, 0, st>>>((const uint4*)a, (uint4*)b, calib / 16);
      HIP_OK(hipEventRecord(e1, st));
      HIP_OK(hipEventSynchronize(e1));
      float ms;
      HIP_OK(hipEventElapsedTime(&ms, e0, e1));
      best = std::min(best, ms);
    }
    printf("{\"calibration_copy_bytes\": %zu, \"best_us\": %.2f, \"GBps_read_plus_write\": %.1f}\n", calib,
           best * 1e3, 2.0 * calib / (best * 1e-3) / 1e9);
    HIP_OK(hipFree(a));
    HIP_OK(hipFree(b));
  }

  std::vector<std::string> modes;
  if (mode == "all") modes = {"clip", "split", "norm", "scale"};
  else modes = {mode};
  for (const std::string& m : modes) {
    if (m == "split") rc = gclip_list_set_path(L, GCLIP_PATH_SPLIT);
    else rc = gclip_list_set_path(L, GCLIP_PATH_AUTO);
    if (rc != GCLIP_OK) die("gclip_list_set_path", rc);
    std::vector<float> us;
    for (int r = 0; r < warmup + reps; ++r) {
      restore();
      if (m == "scale") {
        rc = gclip_norm(L, s.avg, res, st);
        if (rc != GCLIP_OK) die("gclip_norm", rc);
      }
      HIP_OK(hipEventRecord(e0, st));
      if (m == "norm") rc = gclip_norm(L, s.avg, res, st);
      else if (m == "scale") rc = gclip_scale(L, s.max_norm, s.avg, s.err, res, st);
      else rc = gclip_clip_(L, s.max_norm, s.avg, s.err, res, st);
      if (rc != GCLIP_OK) die(m.c_str(), rc);
      HIP_OK(hipEventRecord(e1, st));
      HIP_OK(hipEventSynchronize(e1));
      float ms;
      HIP_OK(hipEventElapsedTime(&ms, e0, e1));
      if (r >= warmup) us.push_back(ms * 1e3f);
    }
    gclip_result h;
    const gclip_status rs = gclip_result_read(res, st, &h, s.err);
    const bool wrote = (m != "norm") && !(h.skipped || h.scale == 1.0);
    const double bytes = (double)total * es * (m == "norm" ? 1.0 : (m == "scale" ? (wrote ? 2.0 : 0.0) : (wrote ? 3.0 : 1.0)));
    std::vector<float> so = us;
    std::sort(so.begin(), so.end());
    double mean = 0;
    for (float x : us) mean += x;
    mean /= us.size();
    printf("{\"mode\": \"%s\", \"path\": \"%s\", \"reps\": %d, \"mean_us\": %.2f, \"median_us\": %.2f, "
           "\"min_us\": %.2f, \"alg_bytes\": %.0f, \"GBps\": %.1f, \"pct_hbm_peak\": %.2f, \"norm\": %.9g, "
           "\"scale\": %.9g, \"status\": %d, \"device_status\": %d, \"workers\": %d, \"resident_bytes\": %lld, "
           "\"flush\": %s, \"drain_us\": %ld}\n",
           m.c_str(), (m == "split" || info.path == GCLIP_PATH_SPLIT) ? "split" : "fused", reps, mean,
           so[so.size() / 2], so[0], bytes, bytes / (mean * 1e-6) / 1e9, bytes / (mean * 1e-6) / 1e9 / 8000.0 * 100.0,
           h.norm, h.scale, (int)rs, h.status, info.n_workers, (long long)info.resident_vectors * 16,
           flush ? "true" : "false", drain_us);
    fflush(stdout);
  }
  gclip_list_destroy(L);
  for (size_t t = 0; t < n; ++t) {
    if (d[t]) HIP_OK(hipFree(d[t]));
    if (pristine[t]) HIP_OK(hipFree(pristine[t]));
  }
  HIP_OK(hipFree(fl));
  HIP_OK(hipFree(sink));
  HIP_OK(hipFree(res));
  HIP_OK(hipStreamDestroy(st));
  return 0;
}
