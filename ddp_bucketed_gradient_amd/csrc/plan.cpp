// plan.cpp -- bucket plan, variable locators, device segment tables and the
// staged workspace size. Everything here decides which bytes the kernels
// touch; the state machine that schedules them is in core.cpp. Page citations
// use the short names defined in core.hpp.
#include "core.hpp"

#include <algorithm>
#include <utility>

namespace ddpb {

static int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

Plan make_plan(const std::vector<int64_t>& numel, int64_t elem_size, int64_t cap_bytes, int32_t R,
               const std::vector<int32_t>* order) {
  Plan p;
  p.P = static_cast<int32_t>(numel.size());
  p.R = R;
  p.cap_bytes = cap_bytes;
  p.elem_size = elem_size;
  p.numel = numel;

  // [Li] "Gradient Bucketing" / [C30] "bucket_cap_mb 不是张量切分器": walk the
  // parameters last to first, add each whole tensor, close the bucket once its
  // size reaches or exceeds the cap; the last, partly filled bucket is kept.
  std::vector<int32_t> cur;
  int64_t size = 0;
  for (int32_t i = 0; i < p.P; ++i) {
    const int32_t v = order ? (*order)[i] : p.P - 1 - i;
    cur.push_back(v);
    size += numel[v] * elem_size;
    if (size >= cap_bytes) {
      p.members.push_back(std::move(cur));
      cur.clear();
      size = 0;
    }
  }
  if (!cur.empty()) p.members.push_back(std::move(cur));

  // [C30] "Variable 到 Bucket": variable -> (bucket, intra-bucket index,
  // offset, length); members sit back to back in insertion order.
  const int32_t B = p.B();
  p.loc.assign(p.P, Locator{-1, -1, 0, 0});
  p.bucket_elems.assign(B, 0);
  p.flat_base.assign(B, 0);
  int64_t base = 0;
  for (int32_t b = 0; b < B; ++b) {
    int64_t off = 0;
    for (size_t i = 0; i < p.members[b].size(); ++i) {
      const int32_t v = p.members[b][i];
      p.loc[v] = Locator{b, static_cast<int32_t>(i), off, numel[v]};
      off += numel[v];
    }
    p.bucket_elems[b] = off;
    p.flat_base[b] = base;
    base += round_up(off, kFlatAlignElems);
  }
  p.flat_elems = base;

  // Device work table: every member cut into segments of <= kSegElems.
  p.seg_first.assign(B + 1, 0);
  for (int32_t b = 0; b < B; ++b) {
    p.seg_first[b] = static_cast<int32_t>(p.segs.size());
    for (int32_t v : p.members[b]) {
      const Locator& L = p.loc[v];
      for (int64_t s = 0; s < numel[v]; s += kSegElems) {
        Segment g;
        g.var = v;
        g.start = s;
        g.len = std::min(kSegElems, numel[v] - s);
        g.boff = L.offset + s;
        g.flags = (g.start % 4 == 0 ? kSegVecStart : 0) | (g.boff % 4 == 0 ? kSegVecFlat : 0);
        p.segs.push_back(g);
        p.seg_bucket.push_back(b);
      }
    }
  }
  p.seg_first[B] = static_cast<int32_t>(p.segs.size());

  // Bucket-view work table: the bucket's flat range in kSegElems chunks. Bases
  // are 64-element aligned, so every chunk starts on a 16-byte boundary.
  p.view_seg_first.assign(B + 1, 0);
  for (int32_t b = 0; b < B; ++b) {
    p.view_seg_first[b] = static_cast<int32_t>(p.view_segs.size());
    for (int64_t k = 0; k < p.bucket_elems[b]; k += kSegElems) {
      Segment g;
      g.var = 0;
      g.start = p.flat_base[b] + k;
      g.len = std::min(kSegElems, p.bucket_elems[b] - k);
      g.boff = k;
      g.flags = kSegVecBoth;
      p.view_segs.push_back(g);
    }
  }
  p.view_seg_first[B] = static_cast<int32_t>(p.view_segs.size());
  return p;
}

int64_t workspace_bytes(const Plan& plan, int32_t mode) {
  if (mode == 1) return (static_cast<int64_t>(plan.R) + 1) * plan.flat_elems * plan.elem_size;
  return 0;
}

}  // namespace ddpb
