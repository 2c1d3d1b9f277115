// gclip_plan.cpp -- host construction of a gradient list's descriptor table.
// Pure C++: no HIP call, so it can be exercised without a GPU.
#include "gclip_plan.hpp"

#include <algorithm>
#include <cstring>
#include <utility>

namespace gclip {

namespace {

// Balanced split of [0, total) into n parts: part w starts at w*q + min(w, r).
uint64_t share_begin(uint64_t total, int32_t n, int32_t w) {
  const uint64_t q = total / (uint64_t)n, r = total % (uint64_t)n;
  return (uint64_t)w * q + std::min<uint64_t>((uint64_t)w, r);
}

// Guided schedule over [0, total): each chunk about (work left) /
// (guide * nworkers), in whole groups, between min_v and max_v vectors.
// Returns the chunk starts plus total.
std::vector<uint64_t> guided_chunks(uint64_t total, int32_t nworkers, uint64_t group, uint64_t min_v, uint64_t max_v,
                                    uint32_t guide) {
  std::vector<uint64_t> vb{0};
  uint64_t b = 0;
  while (b < total) {
    const uint64_t left = total - b, div = (uint64_t)guide * (uint64_t)nworkers;
    uint64_t n = (left + div - 1) / div;
    n = (n + group - 1) / group * group;
    if (n < min_v) n = min_v;
    if (n > max_v) n = max_v;
    b = left > n ? b + n : total;
    vb.push_back(b);
  }
  return vb;
}

}  // namespace

// How much larger the even XCDs' sum chunks are than the odd XCDs' in a list
// of kNtStoreMinBytes or more.  Measured on MI355X, 1.3B bf16 list: 1,154.5
// against 1,164.2 us.  (Under 1 GiB the same split gained nothing beyond the
// spread between runs, and the two-size arithmetic cost the += kernel 2 us,
// so smaller lists keep one size and the kernels' one-size arithmetic.)
constexpr double kSumXcdSkew = 0.07;

int plan_validate(const uint64_t* addrs, const int64_t* numels, int32_t n, int32_t dtype, std::string* why,
                  int64_t* n_elements, int64_t* n_bytes) {
  auto fail = [&](int code, const char* msg) {
    if (why) *why = msg;
    return code;
  };
  if (!dtype_valid(dtype)) return fail(2, "unknown dtype");
  if (n < 0) return fail(1, "negative tensor count");
  if (n > 0 && (!addrs || !numels)) return fail(1, "NULL address or size array");
  const int esize = dtype_bytes(dtype);
  std::vector<std::pair<uint64_t, uint64_t>> ranges;
  ranges.reserve((size_t)n);
  const uint64_t kMaxElems = (uint64_t)1 << 56;
  int64_t ne_total = 0, nb_total = 0;
  for (int32_t t = 0; t < n; ++t) {
    if (numels[t] < 0) return fail(1, "negative element count");
    if (numels[t] == 0) continue;
    if ((uint64_t)numels[t] > kMaxElems) return fail(1, "tensor too large");
    if (addrs[t] == 0) return fail(1, "NULL tensor address");
    if (addrs[t] % (uint64_t)esize != 0) return fail(1, "tensor address not aligned to its element size");
    const uint64_t bytes = (uint64_t)numels[t] * (uint64_t)esize;
    if (addrs[t] + bytes < addrs[t]) return fail(1, "tensor range wraps the address space");
    ranges.emplace_back(addrs[t], addrs[t] + bytes);
    ne_total += numels[t];
    nb_total += (int64_t)bytes;
  }
  std::sort(ranges.begin(), ranges.end());
  for (size_t i = 1; i < ranges.size(); ++i)
    if (ranges[i].first < ranges[i - 1].second) return fail(1, "tensors overlap or repeat");
  if (n_elements) *n_elements = ne_total;
  if (n_bytes) *n_bytes = nb_total;
  return 0;
}

int plan_build(const uint64_t* addrs, const int64_t* numels, int32_t n, int32_t dtype, int32_t nworkers,
               int32_t threads, uint64_t resident_cap, const ChunkShape& shape, HostPlan& out, std::string* why) {
  const int rc = plan_validate(addrs, numels, n, dtype, why, nullptr, nullptr);
  if (rc != 0) return rc;
  const uint64_t group_vectors = shape.group_vectors;
  if (nworkers <= 0 || threads <= 0 || group_vectors == 0 || shape.sum_chunks_per_worker == 0 ||
      shape.scale_guide == 0 || shape.scale_min_vectors == 0 || shape.scale_min_vectors % group_vectors != 0 ||
      shape.scale_max_vectors < shape.scale_min_vectors || shape.scale_max_vectors % group_vectors != 0) {
    if (why) *why = "non-positive launch shape";
    return 1;
  }
  HostPlan p;
  p.dtype = dtype;
  p.esize = dtype_bytes(dtype);
  p.vec_elems = kVecBytes / p.esize;
  p.nworkers = nworkers;
  p.threads = threads;
  p.n_tensors = n;
  plan_validate(addrs, numels, n, dtype, nullptr, &p.n_elements, &p.n_bytes);

  // segments and scalars, in list order
  p.seg_vbegin.push_back(0);
  for (int32_t t = 0; t < n; ++t) {
    const int64_t ne = numels[t];
    if (ne == 0) continue;
    const uint64_t a = addrs[t];
    int64_t head = (int64_t)(((uint64_t)kVecBytes - a % kVecBytes) % kVecBytes) / p.esize;
    if (head > ne) head = ne;
    const int64_t body = (ne - head) / p.vec_elems;
    auto add_scalars = [&](int64_t b, int64_t e) {
      for (int64_t i = b; i < e; ++i) {
        p.sc_addr.push_back(a + (uint64_t)i * (uint64_t)p.esize);
        p.sc_tensor.push_back(t);
        p.sc_elem.push_back(i);
      }
    };
    if (body < kMinSegVectors) {
      add_scalars(0, ne);
      continue;
    }
    add_scalars(0, head);
    p.seg_addr.push_back(a + (uint64_t)head * (uint64_t)p.esize);
    p.seg_tensor.push_back(t);
    p.seg_elem0.push_back(head);
    p.seg_vbegin.push_back(p.seg_vbegin.back() + (uint64_t)body);
    add_scalars(head + body * p.vec_elems, ne);
  }

  // blocks at the end, chunks over the whole space
  const uint64_t nv = p.nvec(), ns = p.nsc();
  const uint64_t even = (nv + (uint64_t)nworkers - 1) / (uint64_t)nworkers;
  p.rb = even < resident_cap ? even : resident_cap;
  p.sb = nv > (uint64_t)nworkers * p.rb ? nv - (uint64_t)nworkers * p.rb : 0;
  // sum chunks: about sum_chunks_per_worker per worker, in whole groups of
  // steps (each chunk boundary costs the streaming loop a partial drain, so
  // fewer, larger chunks are faster as long as the workers stay balanced).
  // In a list of kNtStoreMinBytes or more the chunks alternate between two
  // sizes: chunk c is summed first by worker c mod nworkers, on XCD
  // c mod kTicketGroups (workgroups are dealt to the XCDs in turn), and on
  // MI355X the odd-numbered XCDs stream that pass 6-10 % slower, so with an
  // even worker count the even chunks are larger by kSumXcdSkew.
  {
    const uint64_t want = (uint64_t)nworkers * shape.sum_chunks_per_worker;
    const uint64_t per = (p.sb + want - 1) / want;
    uint64_t g = (per + group_vectors - 1) / group_vectors;
    if (g == 0) g = 1;
    uint64_t ge = g, go = g;
    if (p.n_bytes >= kNtStoreMinBytes && nworkers % 2 == 0) {
      const uint64_t pair = (2 * per + group_vectors - 1) / group_vectors;
      ge = (uint64_t)((double)pair * (1.0 + kSumXcdSkew) / 2.0 + 0.5);
      if (ge >= pair) ge = pair - 1;
      if (ge == 0) ge = 1;
      go = pair > ge ? pair - ge : 1;
    }
    if (p.n_bytes >= kNtStoreMinBytes && (ge > 0xffffu || go > 0xffffu)) {
      if (why) *why = "sum chunks too large";  // above 4 GiB each: a list far beyond a device's memory
      return 1;
    }
    p.cvs_even = ge * group_vectors;
    p.cvs_odd = go * group_vectors;
    if (p.n_bytes >= kNtStoreMinBytes) p.sum_groups = (uint32_t)ge | (uint32_t)go << 16;
  }
  p.spl_vb = guided_chunks(nv, nworkers, group_vectors, shape.scale_min_vectors, shape.scale_max_vectors,
                           shape.scale_guide);
  p.fus_vb = guided_chunks(p.sb, nworkers, group_vectors, shape.scale_min_vectors, shape.scale_max_vectors,
                           shape.scale_guide);
  if (p.spl_vb.size() > 0xffffffffull / 64 || p.fus_vb.size() > 0xffffffffull / 64) {
    if (why) *why = "too many chunks";
    return 1;
  }
  // segment holding vector v (v < nv): last segment whose start is <= v
  auto seg_of = [&](uint64_t v) -> uint32_t {
    return (uint32_t)((std::upper_bound(p.seg_vbegin.begin(), p.seg_vbegin.end() - 1, v) - p.seg_vbegin.begin()) - 1);
  };
  p.blk_seg.assign((size_t)nworkers, 0);
  for (int32_t w = 0; w < nworkers; ++w) {
    const uint64_t b = p.sb + (uint64_t)w * p.rb;
    if (b < nv) p.blk_seg[(size_t)w] = seg_of(b);
  }
  p.spl_seg.resize(p.spl_vb.size() - 1);
  for (size_t c = 0; c < p.spl_seg.size(); ++c) p.spl_seg[c] = seg_of(p.spl_vb[c]);
  p.fus_seg.resize(p.fus_vb.size() - 1);
  for (size_t c = 0; c < p.fus_seg.size(); ++c) p.fus_seg[c] = seg_of(p.fus_vb[c]);
  uint64_t nsum = 0;
  if (p.sb > 0) {
    nsum = 2 * (p.sb / (p.cvs_even + p.cvs_odd));
    while (sum_chunk_begin(p.cvs_even, p.cvs_odd, nsum) < p.sb) ++nsum;
  }
  if (nsum > 0xffffffffull / 64) {
    if (why) *why = "too many chunks";
    return 1;
  }
  p.sum_seg.resize((size_t)nsum);
  for (uint64_t c = 0; c < nsum; ++c) p.sum_seg[(size_t)c] = seg_of(sum_chunk_begin(p.cvs_even, p.cvs_odd, c));
  p.wk_scbegin.resize((size_t)nworkers + 1);
  for (int32_t w = 0; w <= nworkers; ++w) p.wk_scbegin[(size_t)w] = share_begin(ns, nworkers, w);
  out = std::move(p);
  return 0;
}

PlanLayout plan_layout(const HostPlan& p) {
  const size_t nseg = (size_t)p.nseg(), nw = (size_t)p.nworkers, nsc = (size_t)p.nsc(), nch = (size_t)p.nchunk();
  const size_t nchs = (size_t)p.nchunk_streamed(), nsum = (size_t)p.nsum();
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = (off + (bytes ? bytes : 8) + 255) / 256 * 256;
    return at;
  };
  PlanLayout L;
  L.segv = take((nseg + 1) * 8);
  L.sega = take(nseg * 8);
  L.blk = take(nw * 4);
  L.splv = take((nch + 1) * 8);
  L.spls = take(nch * 4);
  L.fusv = take((nchs + 1) * 8);
  L.fuss = take(nchs * 4);
  L.sum = take(nsum * 4);
  L.wksc = take((nw + 1) * 8);
  L.sca = take(nsc * 8);
  L.bc = take(8);
  L.sync = take((size_t)kSyncWords * 4);
  L.bst = take(nw * 4);
  L.header = off;
  L.part = take((nsum + nw) * 8);
  L.bytes = off;
  return L;
}

void plan_image(const HostPlan& p, const PlanLayout& L, unsigned char* img) {
  std::memset(img, 0, L.header);
  auto put = [&](size_t o, const void* src, size_t bytes) {
    if (bytes) std::memcpy(img + o, src, bytes);
  };
  const size_t nseg = (size_t)p.nseg(), nw = (size_t)p.nworkers, nsc = (size_t)p.nsc(), nch = (size_t)p.nchunk();
  const size_t nchs = (size_t)p.nchunk_streamed(), nsum = (size_t)p.nsum();
  put(L.segv, p.seg_vbegin.data(), (nseg + 1) * 8);
  put(L.sega, p.seg_addr.data(), nseg * 8);
  put(L.blk, p.blk_seg.data(), nw * 4);
  put(L.splv, p.spl_vb.data(), (nch + 1) * 8);
  put(L.spls, p.spl_seg.data(), nch * 4);
  put(L.fusv, p.fus_vb.data(), (nchs + 1) * 8);
  put(L.fuss, p.fus_seg.data(), nchs * 4);
  put(L.sum, p.sum_seg.data(), nsum * 4);
  put(L.wksc, p.wk_scbegin.data(), (nw + 1) * 8);
  put(L.sca, p.sc_addr.data(), nsc * 8);
  put(L.bc, &kUndecided, 8);
}

DevPlan plan_view(const HostPlan& p, const PlanLayout& L, unsigned char* b) {
  DevPlan D{};
  D.seg_vbegin = reinterpret_cast<const uint64_t*>(b + L.segv);
  D.seg_addr = reinterpret_cast<const uint64_t*>(b + L.sega);
  D.blk_seg = reinterpret_cast<const uint32_t*>(b + L.blk);
  D.spl_vb = reinterpret_cast<const uint64_t*>(b + L.splv);
  D.spl_seg = reinterpret_cast<const uint32_t*>(b + L.spls);
  D.fus_vb = reinterpret_cast<const uint64_t*>(b + L.fusv);
  D.fus_seg = reinterpret_cast<const uint32_t*>(b + L.fuss);
  D.sum_seg = reinterpret_cast<const uint32_t*>(b + L.sum);
  D.wk_scbegin = reinterpret_cast<const uint64_t*>(b + L.wksc);
  D.sc_addr = reinterpret_cast<const uint64_t*>(b + L.sca);
  D.partials = reinterpret_cast<double*>(b + L.part);
  D.bcast = reinterpret_cast<uint64_t*>(b + L.bc);
  D.sync = reinterpret_cast<uint32_t*>(b + L.sync);
  D.bstate = reinterpret_cast<uint32_t*>(b + L.bst);
  D.nvec = p.nvec();
  D.rb = p.rb;
  D.sb = p.sb;
  D.cvs = p.cvs_even;
  D.sum_groups = p.sum_groups;
  D.nchunk = (uint32_t)p.nchunk();
  D.nchs = (uint32_t)p.nchunk_streamed();
  D.nsum = (uint32_t)p.nsum();
  D.nt_store = p.n_bytes >= kNtStoreMinBytes ? 1u : 0u;
  D.one_group = p.one_group ? 1u : 0u;
  D.nworkers = p.nworkers;
  D.nseg = (int32_t)p.nseg();
  return D;
}

int plan_build_list(const uint64_t* addrs, const int64_t* numels, int32_t n, int32_t dtype, int32_t ncu,
                    int32_t threads, uint64_t resident_cap, const ChunkShape& shape, HostPlan& out,
                    std::string* why) {
  int rc = plan_build(addrs, numels, n, dtype, ncu, threads, resident_cap, shape, out, why);
  if (rc != 0) return rc;
  auto fits = [&](const HostPlan& p) {
    return p.nvec() <= shape.group_vectors && p.nsc() <= (uint64_t)threads;
  };
  if (ncu > 1 && fits(out)) rc = plan_build(addrs, numels, n, dtype, 1, threads, resident_cap, shape, out, why);
  if (rc == 0) out.one_group = out.nworkers == 1 && out.sb == 0 && fits(out);
  return rc;
}

int tensor_plan_build(const HostPlan& p, uint32_t piece_vectors, TensorHostPlan& out) {
  if (piece_vectors == 0) return 1;
  out.pieces.clear();
  out.first.assign((size_t)p.n_tensors + 1, 0);
  if (p.nsc() > 0xffffffffull) return 1;
  size_t s = 0, c = 0;  // next segment, next single element (both in tensor order)
  for (int64_t t = 0; t < p.n_tensors; ++t) {
    out.first[(size_t)t] = (uint32_t)out.pieces.size();
    const size_t c0 = c;
    while (c < p.sc_tensor.size() && p.sc_tensor[c] == (int32_t)t) ++c;
    const uint32_t nsc = (uint32_t)(c - c0);
    bool first = true;
    auto push = [&](uint64_t addr, uint32_t nvec) {
      out.pieces.push_back(TPiece{addr, nvec, (uint32_t)t, first ? (uint32_t)c0 : 0u, first ? nsc : 0u, {0u, 0u}});
      first = false;
    };
    if (s < p.seg_tensor.size() && p.seg_tensor[s] == (int32_t)t) {
      const uint64_t nv = p.seg_vbegin[s + 1] - p.seg_vbegin[s];
      for (uint64_t v = 0; v < nv; v += piece_vectors) {
        const uint64_t k = nv - v < piece_vectors ? nv - v : piece_vectors;
        push(p.seg_addr[s] + v * kVecBytes, (uint32_t)k);
      }
      ++s;
    }
    if (first && nsc > 0) push(0, 0);
    if (out.pieces.size() > 0x7fffffffull) return 1;
  }
  out.first[(size_t)p.n_tensors] = (uint32_t)out.pieces.size();
  const uint64_t np = out.pieces.size(), nw = (uint64_t)(p.nworkers > 0 ? p.nworkers : 1);
  const uint64_t nres = np < nw * (uint64_t)kTensorResidentPieces ? np : nw * (uint64_t)kTensorResidentPieces;
  out.ps = (uint32_t)(np - nres);
  out.run_b.resize((size_t)nw + 1);
  out.res_b.resize((size_t)nw + 1);
  // both shared out by piece count: with one piece in flight a short piece
  // costs about a round trip, nearly what a whole one does, so balancing by
  // bytes loads the workers that get the short pieces (measured: 57 ms
  // instead of 1.1 ms on a list that ends with 4,096 one-element tensors)
  for (uint64_t w = 0; w <= nw; ++w) {
    out.run_b[(size_t)w] = (uint32_t)share_begin(out.ps, (int32_t)nw, (int32_t)w);
    out.res_b[(size_t)w] = (uint32_t)share_begin(nres, (int32_t)nw, (int32_t)w);
  }
  return 0;
}

}  // namespace gclip
