// gclip_plan.hpp -- descriptor table of a gradient list (host side) and its
// device view.  Internal to libgclip.
//
// One launch must cover tensors of very different shapes (grad clip lesson,
// unhomeschool.com ru, section "The naive algorithm cannot work on a GPU":
// [8449 x 768] next to [768]), with one block per chunk and hundreds of blocks
// across all tensors (section "ANDREA's three-kernel pipeline").  Here the
// table is built once per list:
//   - each tensor's 16-byte-aligned body becomes a "segment" of 16-byte
//     vectors; the segments are laid end to end into one vector space;
//   - the unaligned head and tail elements of each tensor, and every element
//     of a tensor whose aligned body is shorter than kMinSegVectors, go to a
//     list of single elements ("scalars");
//   - worker w (one workgroup) owns an equal share of the vector space and an
//     equal share of the scalar list, so every worker moves the same bytes
//     whatever the tensor sizes.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace gclip {

constexpr int kVecBytes = 16;
constexpr int64_t kMinSegVectors = 64;  // aligned bodies shorter than 1 KB are handled element by element

inline int dtype_bytes(int32_t dtype) { return dtype == 0 ? 4 : 2; }
inline bool dtype_valid(int32_t dtype) { return dtype == 0 || dtype == 1 || dtype == 2; }

struct HostPlan {
  int32_t dtype = 0;
  int esize = 4;
  int vec_elems = 4;
  int32_t nworkers = 0;
  int32_t threads = 0;
  int64_t n_tensors = 0;
  int64_t n_elements = 0;
  int64_t n_bytes = 0;
  std::vector<uint64_t> seg_vbegin;  // nseg + 1 prefix offsets in the vector space
  std::vector<uint64_t> seg_addr;    // nseg: address of the segment's first vector
  std::vector<int32_t> seg_tensor;   // nseg
  std::vector<int64_t> seg_elem0;    // nseg: element index of the segment start in its tensor
  std::vector<uint64_t> wk_vbegin;   // nworkers + 1
  std::vector<uint32_t> wk_seg;      // nworkers: segment holding wk_vbegin[w]
  std::vector<uint64_t> sc_addr;     // nsc: address of each single element
  std::vector<int32_t> sc_tensor;    // nsc
  std::vector<int64_t> sc_elem;      // nsc
  std::vector<uint64_t> wk_scbegin;  // nworkers + 1

  int64_t nseg() const { return (int64_t)seg_addr.size(); }
  uint64_t nvec() const { return seg_vbegin.empty() ? 0 : seg_vbegin.back(); }
  uint64_t nsc() const { return (uint64_t)sc_addr.size(); }
};

// Check a list: sizes >= 0, addresses non-NULL and aligned to the element
// size, no two tensors overlapping.  Returns 0 or a gclip_status code.
int plan_validate(const uint64_t* addrs, const int64_t* numels, int32_t n, int32_t dtype, std::string* why,
                  int64_t* n_elements, int64_t* n_bytes);

// Validate a list and build its plan.  Returns a gclip_status code (0 = OK)
// and, on failure, a short reason in *why.
int plan_build(const uint64_t* addrs, const int64_t* numels, int32_t n, int32_t dtype, int32_t nworkers,
               int32_t threads, HostPlan& out, std::string* why);

// Device view of a plan plus the list's workspace (all device addresses).
struct DevPlan {
  const uint64_t* seg_vbegin;
  const uint64_t* seg_addr;
  const uint64_t* wk_vbegin;
  const uint32_t* wk_seg;
  const uint64_t* wk_scbegin;
  const uint64_t* sc_addr;
  double* partials;   // nworkers partial sums of g^2 (binary64)
  double* bcast;      // [0]: factor decided inside the fused kernel
  uint32_t* sync;     // [0] arrival ticket, [1] epoch released by the last arrival, [2] skip flag,
                      // [3] barrier-timeout flag, [4] finish ticket (fused kernel)
  int32_t nworkers;
  int32_t nseg;
};

}  // namespace gclip
