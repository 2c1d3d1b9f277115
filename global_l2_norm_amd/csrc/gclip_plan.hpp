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
//     list of single elements ("scalars"), shared out equally by worker;
//   - the vector space ends with one "block" of rb vectors per worker
//     (workgroup): what the fused kernel keeps on chip between its passes;
//   - the rest, the streamed region [0, sb), is cut into chunks; each
//     worker takes two without a claim, the rest are claimed at run time, so
//     that the XCDs that stream faster take more of them: "sum chunks" for the summing passes (cvs vectors
//     each; in lists of kNtStoreMinBytes or more two sizes in turn, see HostPlan::cvs_even) (a
//     sum chunk's partial goes to a slot of its own, so the content and
//     order of the final sum do not depend on which worker took which
//     chunk), and "scale chunks" for the fused kernel's scale pass.  The
//     split scale kernel cuts the whole space [0, nvec) into scale chunks.
//     Scale chunks can shrink as the work left shrinks (guided scheduling);
//     the default keeps them at one size, which measured as fast.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/gclip.h"

namespace gclip {

constexpr int kVecBytes = 16;
constexpr int64_t kMinSegVectors = 64;  // aligned bodies shorter than 1 KB are handled element by element

inline int dtype_bytes(int32_t dtype) { return dtype == 0 ? 4 : 2; }

// Start of sum chunk c when the chunks alternate between ce vectors (even c)
// and co vectors (odd c).  (constexpr: host and device code alike.)
constexpr uint64_t sum_chunk_begin(uint64_t ce, uint64_t co, uint64_t c) {
  return (c >> 1) * (ce + co) + ((c & 1u) ? ce : 0u);
}
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
  uint64_t rb = 0;                   // vectors per block: worker w's is [sb + w rb, sb + (w + 1) rb) cut at nvec
  uint64_t sb = 0;                   // end of the streamed region, start of the blocks
  uint64_t cvs_even = 0;             // vectors per sum chunk: chunks of cvs_even (even index) and cvs_odd (odd
  uint64_t cvs_odd = 0;              // index) in turn from 0, cut at sb (sum_chunk_begin); equal unless the list
                                     // is of kNtStoreMinBytes or more
  uint32_t sum_groups = 0;           // in such a list, both sizes in groups: cvs_even | cvs_odd << 16
  std::vector<uint32_t> blk_seg;     // nworkers: segment holding each block's first vector
  std::vector<uint64_t> spl_vb;      // nchunk + 1: scale chunk c of the split kernel is [spl_vb[c], spl_vb[c + 1])
  std::vector<uint32_t> spl_seg;     // nchunk: segment holding each of those chunks' first vector
  std::vector<uint64_t> fus_vb;      // nchs + 1: scale chunks of the fused kernel, over [0, sb)
  std::vector<uint32_t> fus_seg;     // nchs
  std::vector<uint32_t> sum_seg;     // nsum: segment holding each sum chunk's first vector
  std::vector<uint64_t> sc_addr;     // nsc: address of each single element
  std::vector<int32_t> sc_tensor;    // nsc
  std::vector<int64_t> sc_elem;      // nsc
  std::vector<uint64_t> wk_scbegin;  // nworkers + 1
  bool one_group = false;            // one worker, and the whole list is one group of vectors plus at most
                                     // one single element per lane (see plan_build_list)

  int64_t nseg() const { return (int64_t)seg_addr.size(); }
  uint64_t nvec() const { return seg_vbegin.empty() ? 0 : seg_vbegin.back(); }
  uint64_t nsc() const { return (uint64_t)sc_addr.size(); }
  uint64_t nchunk() const { return (uint64_t)spl_seg.size(); }           // split scale chunks (whole space)
  uint64_t nchunk_streamed() const { return (uint64_t)fus_seg.size(); }  // fused scale chunks (below sb)
  uint64_t nsum() const { return (uint64_t)sum_seg.size(); }  // sum chunks (below sb)
};

// Check a list: sizes >= 0, addresses non-NULL and aligned to the element
// size, no two tensors overlapping.  Returns 0 or a gclip_status code.
int plan_validate(const uint64_t* addrs, const int64_t* numels, int32_t n, int32_t dtype, std::string* why,
                  int64_t* n_elements, int64_t* n_bytes);

// Validate a list and build its plan for nworkers workgroups of `threads`
// lanes: blocks of at most resident_cap vectors, and sum and scale chunks
// as `shape` says.
// Returns a gclip_status code (0 = OK) and, on failure, a reason in *why.
struct ChunkShape {
  uint64_t group_vectors;          // chunks are whole groups of steps
  uint32_t sum_chunks_per_worker;  // sum chunks: about this many per worker
  uint64_t scale_min_vectors;      // scale chunks: between these sizes, ...
  uint64_t scale_max_vectors;
  uint32_t scale_guide;            // ... about (work left) / (scale_guide * nworkers) each
};

int plan_build(const uint64_t* addrs, const int64_t* numels, int32_t n, int32_t dtype, int32_t nworkers,
               int32_t threads, uint64_t resident_cap, const ChunkShape& shape, HostPlan& out, std::string* why);

// The plan of a list on a device of ncu compute units: one worker per
// compute unit, unless the whole list is one group of vectors and at most
// one single element per lane -- then a single worker, so that one
// workgroup can take the whole clip with no grid-wide decision (its launch
// and round trips, not its bytes, set the time of such a list).
int plan_build_list(const uint64_t* addrs, const int64_t* numels, int32_t n, int32_t dtype, int32_t ncu,
                    int32_t threads, uint64_t resident_cap, const ChunkShape& shape, HostPlan& out,
                    std::string* why);

// The fused kernel's decision word (bcast[0]): the bits of the factor s, or
// one of two signalling-NaN patterns.  Arithmetic never yields a signalling
// NaN, and s is finite whenever it is written, so no factor collides with
// them.  The word holds kUndecided from the list's creation on and again
// after every launch (its last workgroup resets it).
constexpr uint64_t kUndecided = 0x7ff4000000000001ull;
constexpr uint64_t kDecidedSkip = 0x7ff4000000000002ull;

// Device view of a plan plus the list's workspace (all device addresses).
// sync holds 128-byte lines of counters (one line per counter group, so that
// the XCDs do not share lines):
//   line 0                           count of handed-back blocks (word 0); tensor factors the
//                                    one-launch per-tensor clip never saw (word 1)
//   line 1                           claim counter of the summing passes
//   line 2                           claim counter of the scaling passes
//   lines 3 .. 3 + kTicketGroups     arrival tickets: one per XCD group, then the top one
//   lines 4 + kTicketGroups ..       finish tickets: one per XCD group, then the top one
constexpr int kTicketGroups = 8;
constexpr int64_t kNtStoreMinBytes = (int64_t)1 << 30;
constexpr int kSyncLineWords = 32;  // 128 bytes
constexpr int kSyncWords = kSyncLineWords * (5 + 2 * kTicketGroups);

struct DevPlan {
  const uint64_t* seg_vbegin;
  const uint64_t* seg_addr;
  const uint32_t* blk_seg;
  const uint64_t* spl_vb;
  const uint32_t* spl_seg;
  const uint64_t* fus_vb;
  const uint32_t* fus_seg;
  const uint32_t* sum_seg;
  const uint64_t* wk_scbegin;
  const uint64_t* sc_addr;
  double* partials;   // nsum sum-chunk partials, then nworkers worker partials (block + single elements)
  uint64_t* bcast;    // [0]: the decision of the fused kernel, published by value (kUndecided between launches)
  uint32_t* sync;     // kSyncWords counters (see above)
  uint32_t* bstate;   // nworkers: whether each block was handed back by the fused kernel
  uint64_t nvec, rb, sb, cvs;  // cvs: the sum chunks' size when it is one (lists under kNtStoreMinBytes)
  uint32_t nchunk;    // split scale chunks over [0, nvec)
  uint32_t nchs;      // fused scale chunks over the streamed region [0, sb)
  uint32_t nsum;      // sum chunks over the streamed region [0, sb)
  uint32_t nt_store;  // 1: the scale passes write with nontemporal stores (lists of kNtStoreMinBytes or more)
  uint32_t one_group; // 1: HostPlan::one_group
  int32_t nworkers;
  int32_t nseg;
  uint32_t sum_groups;  // HostPlan::sum_groups (lists of kNtStoreMinBytes or more)
};

// Where a plan's tables and workspace lie in one device allocation (byte
// offsets, each 256-byte aligned).  [0, header) holds the tables and the
// workspace words that must hold their initial value when a launch starts
// (the decision word, the counters, the block states); the partials follow,
// up to `bytes`, and need no initial value (every launch writes each one
// before it is read).
struct PlanLayout {
  size_t segv, sega, blk, splv, spls, fusv, fuss, sum, wksc, sca, bc, sync, bst, part;
  size_t header;
  size_t bytes;
};

// The layout of plan p.
PlanLayout plan_layout(const HostPlan& p);

// The host image of [0, L.header): every table, the decision word undecided,
// counters and block states zero.  img must hold L.header bytes.
void plan_image(const HostPlan& p, const PlanLayout& L, unsigned char* img);

// The device view of plan p laid out by L at device address base.
DevPlan plan_view(const HostPlan& p, const PlanLayout& L, unsigned char* base);

// The averaging factor of a call: a itself, or, for a loss-scaled step,
// 1 / (a * S) with a = n_microbatches and the binary32 loss scale S read from
// device memory when the kernel starts.
struct AvgSrc {
  double a;
  const float* scale;
};

// The loss-scale update of a loss-scaled step, when the kernel that decides
// also updates the state (st == nullptr: no update).
struct AmpUpdate {
  gclip_amp_state* st;
  double growth, backoff;
  int32_t interval;
};

// A microbatch's contribution laid out like a list: the contribution to
// vector v of segment s is at (address of v) + seg_gdelta[s], the one to
// single element i at sc_addr[i] + sc_gdelta[i].
struct AccSrc {
  const uint64_t* seg_gdelta;  // nseg
  const uint64_t* sc_gdelta;   // nsc
};

// ---------------------------------------------------------------- AdamW on the clipped gradient
// One piece of the optimizer's work: elements [0, count) of one tensor in the
// four parallel lists, from the given addresses.  vec != 0 when the weights
// and both moments are 16-byte aligned there, the gradient is aligned to 4
// elements and count is a multiple of 4: a lane then moves 4 elements per
// access.
struct AdamPiece {
  uint64_t p, g, m, v;
  uint32_t count, vec;
};

#ifndef GCLIP_ADAM_PIECE
#define GCLIP_ADAM_PIECE 4096
#endif
#ifndef GCLIP_ADAM_THREADS
#define GCLIP_ADAM_THREADS 256
#endif
constexpr int kAdamThreads = GCLIP_ADAM_THREADS;
constexpr uint32_t kAdamPieceElems = GCLIP_ADAM_PIECE;

struct AdamPlan {
  const AdamPiece* pieces;
  uint32_t npieces;
};

// Per-tensor work (per-tensor norms and per-tensor clipping): the list cut
// into pieces that each lie inside one tensor, so that one workgroup's sum
// belongs to one tensor.  A piece is nvec 16-byte vectors from addr (a run
// of its tensor's vector segment) and, on the tensor's first piece only, the
// tensor's single elements sc_addr[sc_begin .. sc_begin + sc_count) of the
// list's plan.  Pieces are in tensor order; tensor t owns pieces
// first[t] .. first[t + 1] - 1 (none when it is empty).
struct TPiece {
  uint64_t addr;
  uint32_t nvec, tensor;
  uint32_t sc_begin, sc_count;
  uint32_t pad[2];
};
static_assert(sizeof(TPiece) == 32, "one piece is one 32-byte scalar load");

#ifndef GCLIP_TENSOR_PIECE_VECTORS
#define GCLIP_TENSOR_PIECE_VECTORS 4096
#endif
constexpr uint32_t kTensorPieceVectors = GCLIP_TENSOR_PIECE_VECTORS;

// The one-launch per-tensor clip keeps up to kTensorResidentPieces pieces
// per worker on chip across the decisions: kTensorRegPieces in VGPRs (one
// piece is at most one group, kUnroll steps of kThreads vectors) and the rest
// in LDS.
constexpr int kTensorRegPieces = 5;
constexpr int kTensorLdsPieces = 2;
constexpr int kTensorResidentPieces = kTensorRegPieces + kTensorLdsPieces;

struct TensorHostPlan {
  std::vector<TPiece> pieces;
  std::vector<uint32_t> first;  // n_tensors + 1
  // The one-launch per-tensor clip over nworkers workers: the last
  // nres = min(npieces, nworkers * kTensorResidentPieces) pieces are kept on
  // chip, worker w holding [ps + res_b[w], ps + res_b[w + 1]); the streamed
  // pieces [0, ps) are summed in runs [run_b[w], run_b[w + 1]) and scaled as
  // claimed one-piece chunks.
  uint32_t ps = 0;
  std::vector<uint32_t> run_b;  // nworkers + 1
  std::vector<uint32_t> res_b;  // nworkers + 1
};

// Cut a list's plan into per-tensor pieces of at most piece_vectors vectors,
// and share them out over the plan's workers for the one-launch per-tensor
// clip.  Returns a gclip_status code (0 = OK).
int tensor_plan_build(const HostPlan& p, uint32_t piece_vectors, TensorHostPlan& out);

struct TensorPlan {
  const TPiece* pieces;
  const uint32_t* first;
  const uint64_t* sc_addr;
  double* partials;  // one per piece
  double* tsum;      // one per tensor: raw sums published by k_tensor_clip
  uint32_t* tsync;   // [0]: tensors counted by k_tensor_clip (zero between calls)
  uint32_t npieces;
  int32_t ntensors;
  uint32_t nlive;    // tensors with at least one piece
  uint32_t nt_store;
  // the one-launch per-tensor clip (TensorHostPlan's run_b, res_b, ps)
  const uint32_t* run_b;
  const uint32_t* res_b;
  uint32_t ps;
  uint32_t* tcount;  // n_tensors: pieces summed so far (zero between calls)
  double* tfac;      // n_tensors: each tensor's factor, stored by the workgroup that completes it
};

// Per-step constants, rounded to binary32 from binary64 on the host.
struct AdamHp {
  float step_size;     // lr / (1 - beta1^t)
  float inv_sqrt_bc2;  // 1 / sqrt(1 - beta2^t)
  float eps;
  float decay;         // 1 - lr * wd
  float b1, omb1;      // beta1, 1 - beta1
  float b2, omb2;      // beta2, 1 - beta2
};

}  // namespace gclip
