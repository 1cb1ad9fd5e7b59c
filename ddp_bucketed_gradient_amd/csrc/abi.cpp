// abi.cpp -- the extern "C" surface declared in include/ddpb.h. Argument
// checking and marshalling only; the work happens in plan.cpp, core.cpp and the
// launcher.
#include <algorithm>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/ddpb.h"
#include "core.hpp"

struct ddpb_reducer {
  explicit ddpb_reducer(ddpb::Plan p) : red(std::move(p)) {}
  ddpb::Reducer red;
};

namespace {
thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int pass(int code, const std::string& msg) {
  if (code != 0) g_err = msg;
  return code;
}
}  // namespace

extern "C" {

const char* ddpb_last_error(void) { return g_err.c_str(); }

int ddpb_reducer_create(const int64_t* shapes, const int32_t* ndims, int32_t P, int32_t dtype,
                        int64_t bucket_cap_bytes, int32_t R, ddpb_t* out) {
  if (out == nullptr) return fail(DDPB_E_ARG, "create: out is NULL");
  *out = nullptr;
  if (P < 0 || (P > 0 && ndims == nullptr)) return fail(DDPB_E_ARG, "create: bad P or ndims");
  if (dtype != DDPB_F32) return fail(DDPB_E_ARG, "create: only fp32 gradients are supported");
  if (bucket_cap_bytes < 0) return fail(DDPB_E_ARG, "create: negative bucket cap");
  if (R < 1 || R > ddpb::kMaxReplicas) return fail(DDPB_E_ARG, "create: R must be in 1..64");
  std::vector<int64_t> numel(P);
  int64_t k = 0;
  for (int32_t v = 0; v < P; ++v) {
    if (ndims[v] < 0 || ndims[v] > 16) return fail(DDPB_E_ARG, "create: bad ndims");
    if (ndims[v] > 0 && shapes == nullptr) return fail(DDPB_E_ARG, "create: shapes is NULL");
    int64_t n = 1;
    for (int32_t d = 0; d < ndims[v]; ++d) {
      const int64_t s = shapes[k++];
      if (s < 0) return fail(DDPB_E_ARG, "create: negative dimension");
      if (s != 0 && n > (int64_t(1) << 50) / s) return fail(DDPB_E_ARG, "create: tensor too large");
      n *= s;
    }
    numel[v] = n;
  }
  try {
    *out = new ddpb_reducer(ddpb::make_plan(numel, 4, bucket_cap_bytes, R));
  } catch (const std::bad_alloc&) {
    return fail(DDPB_E_NOMEM, "create: out of host memory");
  }
  return DDPB_OK;
}

void ddpb_destroy(ddpb_t h) { delete h; }

int ddpb_num_buckets(ddpb_t h, int32_t* B) {
  if (!h || !B) return fail(DDPB_E_ARG, "num_buckets: NULL argument");
  *B = h->red.plan().B();
  return DDPB_OK;
}

int ddpb_get_locator(ddpb_t h, int32_t v, int32_t* bucket, int32_t* intra, int64_t* offset,
                     int64_t* length) {
  if (!h) return fail(DDPB_E_ARG, "get_locator: NULL handle");
  const ddpb::Plan& p = h->red.plan();
  if (v < 0 || v >= p.P) return fail(DDPB_E_INDEX, "get_locator: variable index out of range");
  const ddpb::Locator& L = p.loc[v];
  if (bucket) *bucket = L.bucket;
  if (intra) *intra = L.intra;
  if (offset) *offset = L.offset;
  if (length) *length = L.length;
  return DDPB_OK;
}

int ddpb_get_bucket(ddpb_t h, int32_t b, int32_t* nvars, int64_t* bytes, int32_t* vars) {
  if (!h) return fail(DDPB_E_ARG, "get_bucket: NULL handle");
  const ddpb::Plan& p = h->red.plan();
  if (b < 0 || b >= p.B()) return fail(DDPB_E_INDEX, "get_bucket: bucket index out of range");
  if (nvars) *nvars = static_cast<int32_t>(p.members[b].size());
  if (bytes) *bytes = p.bucket_elems[b] * p.elem_size;
  if (vars) std::memcpy(vars, p.members[b].data(), p.members[b].size() * sizeof(int32_t));
  return DDPB_OK;
}

int ddpb_num_segments(ddpb_t h, int32_t* n, int64_t* seg_elems) {
  if (!h) return fail(DDPB_E_ARG, "num_segments: NULL handle");
  if (n) *n = static_cast<int32_t>(h->red.plan().segs.size());
  if (seg_elems) *seg_elems = ddpb::kSegElems;
  return DDPB_OK;
}

int ddpb_get_bucket_segments(ddpb_t h, int32_t b, int32_t* first, int32_t* count) {
  if (!h) return fail(DDPB_E_ARG, "get_bucket_segments: NULL handle");
  const ddpb::Plan& p = h->red.plan();
  if (b < 0 || b >= p.B()) return fail(DDPB_E_INDEX, "get_bucket_segments: bucket index out of range");
  if (first) *first = p.seg_first[b];
  if (count) *count = p.seg_first[b + 1] - p.seg_first[b];
  return DDPB_OK;
}

int ddpb_get_segment(ddpb_t h, int32_t s, int32_t* var, int32_t* bucket, int64_t* start,
                     int64_t* length, int64_t* bucket_offset) {
  if (!h) return fail(DDPB_E_ARG, "get_segment: NULL handle");
  const ddpb::Plan& p = h->red.plan();
  if (s < 0 || s >= static_cast<int32_t>(p.segs.size()))
    return fail(DDPB_E_INDEX, "get_segment: segment index out of range");
  const ddpb::Segment& g = p.segs[s];
  if (var) *var = g.var;
  if (bucket) *bucket = p.seg_bucket[s];
  if (start) *start = g.start;
  if (length) *length = g.len;
  if (bucket_offset) *bucket_offset = g.boff;
  return DDPB_OK;
}

int ddpb_workspace_bytes(ddpb_t h, int32_t mode, int64_t* bytes) {
  if (!h || !bytes) return fail(DDPB_E_ARG, "workspace_bytes: NULL argument");
  if (mode != DDPB_MODE_FUSED && mode != DDPB_MODE_STAGED) return fail(DDPB_E_ARG, "workspace_bytes: bad mode");
  *bytes = ddpb::workspace_bytes(h->red.plan(), mode);
  return DDPB_OK;
}

int ddpb_bind(ddpb_t h, void* const* grad_ptrs, void* workspace, int64_t ws_bytes, void* compute_stream,
              void* const* side_streams, int32_t n_side, int32_t mode, int32_t flags) {
  if (!h) return fail(DDPB_E_ARG, "bind: NULL handle");
  const ddpb::Plan& p = h->red.plan();
  if (mode != DDPB_MODE_FUSED && mode != DDPB_MODE_STAGED) return fail(DDPB_E_ARG, "bind: bad mode");
  if (flags & ~(DDPB_BIND_DEVICE_TIMESTAMPS | DDPB_BIND_TIME_LAUNCHES | DDPB_BIND_ROCTX | DDPB_BIND_OVERLAP)) return fail(DDPB_E_ARG, "bind: bad flags");
  if (n_side < 1 || n_side > 16 || side_streams == nullptr) return fail(DDPB_E_ARG, "bind: need 1..16 side streams");
  const int64_t need = ddpb::workspace_bytes(p, mode);
  if (ws_bytes < need || (need > 0 && workspace == nullptr))
    return fail(DDPB_E_ARG, "bind: workspace smaller than ddpb_workspace_bytes");
  const size_t n = static_cast<size_t>(p.R) * p.P;
  if (n > 0 && grad_ptrs == nullptr) return fail(DDPB_E_ARG, "bind: grad_ptrs is NULL");
  ddpb::BindArgs a;
  a.grad_ptrs.assign(grad_ptrs, grad_ptrs + n);
  for (size_t i = 0; i < n; ++i)
    if (a.grad_ptrs[i] == nullptr && p.numel[i % p.P] > 0) return fail(DDPB_E_ARG, "bind: NULL gradient pointer");
  a.workspace = workspace;
  a.ws_bytes = ws_bytes;
  a.compute_stream = compute_stream;
  a.side_streams.assign(side_streams, side_streams + n_side);
  a.mode = mode;
  a.flags = flags;
  std::string err;
  return pass(h->red.bind(a, &err), err);
}

int ddpb_bind_static(ddpb_t h, void* const* grad_ptrs, void* compute_stream, int32_t mode) {
  if (!h) return fail(DDPB_E_ARG, "bind_static: NULL handle");
  const ddpb::Plan& p = h->red.plan();
  if (mode != DDPB_MODE_FUSED && mode != DDPB_MODE_STAGED) return fail(DDPB_E_ARG, "bind_static: bad mode");
  const size_t n = static_cast<size_t>(p.R) * p.P;
  if (n > 0 && grad_ptrs == nullptr) return fail(DDPB_E_ARG, "bind_static: grad_ptrs is NULL");
  ddpb::BindArgs a;
  a.grad_ptrs.assign(grad_ptrs, grad_ptrs + n);
  for (size_t i = 0; i < n; ++i)
    if (a.grad_ptrs[i] == nullptr && p.numel[i % p.P] > 0) return fail(DDPB_E_ARG, "bind_static: NULL gradient pointer");
  a.compute_stream = compute_stream;
  a.side_streams.assign(1, compute_stream);
  a.mode = mode;
  a.no_alloc = true;
  std::string err;
  return pass(h->red.bind(a, &err), err);
}

int ddpb_rebuild_buckets(ddpb_t h, int64_t bucket_cap_bytes) {
  if (!h) return fail(DDPB_E_ARG, "rebuild_buckets: NULL handle");
  std::string err;
  return pass(h->red.rebuild_buckets(bucket_cap_bytes, &err), err);
}

int ddpb_get_ready_order(ddpb_t h, int32_t* order, int32_t cap, int32_t* n) {
  if (!h || !n || cap < 0 || (cap > 0 && !order)) return fail(DDPB_E_ARG, "get_ready_order: bad argument");
  const auto& o = h->red.last_ready_order();
  *n = static_cast<int32_t>(o.size());
  for (int32_t i = 0; i < std::min<int32_t>(cap, *n); ++i) order[i] = o[i];
  return DDPB_OK;
}

int ddpb_view_storage_elems(ddpb_t h, int64_t* elems) {
  if (!h || !elems) return fail(DDPB_E_ARG, "view_storage_elems: NULL argument");
  *elems = h->red.plan().flat_elems;
  return DDPB_OK;
}

int ddpb_get_view_offset(ddpb_t h, int32_t v, int64_t* offset) {
  if (!h || !offset) return fail(DDPB_E_ARG, "get_view_offset: NULL argument");
  const ddpb::Plan& p = h->red.plan();
  if (v < 0 || v >= p.P) return fail(DDPB_E_INDEX, "get_view_offset: variable index out of range");
  *offset = p.view_offset(v);
  return DDPB_OK;
}

int ddpb_bind_bucket_views(ddpb_t h, void* const* replica_storage, int64_t storage_elems, void* compute_stream,
                           void* const* side_streams, int32_t n_side, int32_t flags) {
  if (!h) return fail(DDPB_E_ARG, "bind_bucket_views: NULL handle");
  const ddpb::Plan& p = h->red.plan();
  if (flags & ~(DDPB_BIND_DEVICE_TIMESTAMPS | DDPB_BIND_TIME_LAUNCHES | DDPB_BIND_ROCTX | DDPB_BIND_OVERLAP))
    return fail(DDPB_E_ARG, "bind_bucket_views: bad flags");
  if (n_side < 1 || n_side > 16 || side_streams == nullptr)
    return fail(DDPB_E_ARG, "bind_bucket_views: need 1..16 side streams");
  if (storage_elems < p.flat_elems) return fail(DDPB_E_ARG, "bind_bucket_views: storage smaller than needed");
  if (replica_storage == nullptr) return fail(DDPB_E_ARG, "bind_bucket_views: replica_storage is NULL");
  ddpb::BindArgs a;
  a.view_bases.assign(replica_storage, replica_storage + p.R);
  for (void* s : a.view_bases)
    if (s == nullptr && p.flat_elems > 0) return fail(DDPB_E_ARG, "bind_bucket_views: NULL storage");
  a.compute_stream = compute_stream;
  a.side_streams.assign(side_streams, side_streams + n_side);
  a.mode = ddpb::kModeBucketView;
  a.flags = flags;
  std::string err;
  return pass(h->red.bind(a, &err), err);
}

int ddpb_ensure_prior_reduction_finished(ddpb_t h) {
  if (!h) return fail(DDPB_E_ARG, "NULL handle");
  std::string err;
  return pass(h->red.ensure_prior_reduction_finished(&err), err);
}

int ddpb_mark_ready(ddpb_t h, int32_t v) {
  if (!h) return fail(DDPB_E_ARG, "NULL handle");
  std::string err;
  const int rc = h->red.mark_ready(v, &err);
  if (rc != DDPB_OK) g_err = err;
  return rc;
}

int ddpb_mark_ready_many(ddpb_t h, const int32_t* vs, int32_t n) {
  if (!h || (n > 0 && vs == nullptr) || n < 0) return fail(DDPB_E_ARG, "mark_ready_many: bad argument");
  std::string err;
  for (int32_t i = 0; i < n; ++i) {
    const int rc = h->red.mark_ready(vs[i], &err);
    if (rc != DDPB_OK) return fail(rc, err);
  }
  return DDPB_OK;
}

int ddpb_finalize(ddpb_t h) {
  if (!h) return fail(DDPB_E_ARG, "NULL handle");
  std::string err;
  return pass(h->red.finalize(&err), err);
}

int ddpb_set_sync(ddpb_t h, int32_t enabled) {
  if (!h) return fail(DDPB_E_ARG, "NULL handle");
  std::string err;
  return pass(h->red.set_sync(enabled != 0, &err), err);
}

int ddpb_no_sync_accumulate(ddpb_t h, void* const* step_ptrs, int32_t step_dtype, int32_t first_step) {
  if (!h) return fail(DDPB_E_ARG, "NULL handle");
  std::string err;
  return pass(h->red.accumulate(step_ptrs, step_dtype, first_step != 0, &err), err);
}

int ddpb_reset(ddpb_t h) {
  if (!h) return fail(DDPB_E_ARG, "NULL handle");
  std::string err;
  return pass(h->red.reset(&err), err);
}

int ddpb_get_launch_log(ddpb_t h, int32_t* buckets, int32_t* trigger_call, int64_t* dev_t0,
                        int64_t* dev_t1, int32_t cap, int32_t* n) {
  if (!h || !n || cap < 0) return fail(DDPB_E_ARG, "get_launch_log: bad argument");
  const auto& log = h->red.log();
  *n = static_cast<int32_t>(log.size());
  const int32_t m = std::min<int32_t>(cap, *n);
  for (int32_t i = 0; i < m; ++i) {
    if (buckets) buckets[i] = log[i].bucket;
    if (trigger_call) trigger_call[i] = log[i].trigger_call;
  }
  if ((dev_t0 || dev_t1) && m > 0) {
    std::vector<ddpb::LaunchRecord> part(log.begin(), log.begin() + m);
    std::vector<int64_t> t0, t1;
    std::string err;
    const int rc = h->red.launcher()->read_stamps(part, &t0, &t1, &err);
    if (rc != DDPB_OK) return fail(rc, err);
    for (int32_t i = 0; i < m; ++i) {
      if (dev_t0) dev_t0[i] = t0[i];
      if (dev_t1) dev_t1[i] = t1[i];
    }
  }
  return DDPB_OK;
}

int ddpb_get_launch_times(ddpb_t h, int32_t iterations_ago, float* start_ms, float* ms, int32_t cap,
                          int32_t* n) {
  if (!h || !n || cap < 0 || (cap > 0 && !ms)) return fail(DDPB_E_ARG, "get_launch_times: bad argument");
  const int64_t fin = h->red.finalized();
  if (iterations_ago < 0 || iterations_ago >= ddpb::kTimeRing || iterations_ago >= fin)
    return fail(DDPB_E_INDEX, "get_launch_times: no such finalized iteration");
  const int64_t it = fin - 1 - iterations_ago;
  if (it < h->red.timed_from())
    return fail(DDPB_E_INDEX, "get_launch_times: that iteration ran before the current binding");
  const auto& log = h->red.log_of(it);
  *n = static_cast<int32_t>(log.size());
  const int32_t m = std::min<int32_t>(cap, *n);
  if (m == 0) return DDPB_OK;
  std::vector<ddpb::LaunchRecord> part(log.begin(), log.begin() + m);
  std::vector<float> st, t;
  std::string err;
  const int rc = h->red.launcher()->read_times(it, part, &st, &t, &err);
  if (rc != DDPB_OK) return fail(rc, err);
  for (int32_t i = 0; i < m; ++i) {
    ms[i] = t[i];
    if (start_ms) start_ms[i] = st[i];
  }
  return DDPB_OK;
}

int ddpb_set_local_used(ddpb_t h, const uint8_t* used) {
  if (!h) return fail(DDPB_E_ARG, "NULL handle");
  std::string err;
  return pass(h->red.set_local_used(used, &err), err);
}

int ddpb_set_launch_blocks(ddpb_t h, int32_t max_blocks) {
  if (!h || max_blocks < 0) return fail(DDPB_E_ARG, "set_launch_blocks: bad argument");
  h->red.launcher()->set_max_blocks(max_blocks);
  return DDPB_OK;
}

int ddpb_set_sync_step(ddpb_t h, void* const* step_ptrs, int32_t step_dtype, int32_t first_step) {
  if (!h) return fail(DDPB_E_ARG, "set_sync_step: NULL handle");
  std::string err;
  return pass(h->red.set_sync_step(step_ptrs, step_dtype, first_step != 0, &err), err);
}

int ddpb_set_workgroups_per_cu(ddpb_t h, int32_t n) {
  if (!h || n < 0 || n > 2) return fail(DDPB_E_ARG, "set_workgroups_per_cu: n must be 0, 1 or 2");
  std::string err;
  return pass(h->red.launcher()->set_workgroups_per_cu(n, &err), err);
}

int ddpb_device_clock_hz(ddpb_t h, int64_t* hz) {
  if (!h || !hz) return fail(DDPB_E_ARG, "device_clock_hz: NULL argument");
  std::string err;
  return pass(h->red.launcher()->clock_hz(hz, &err), err);
}

}  // extern "C"
