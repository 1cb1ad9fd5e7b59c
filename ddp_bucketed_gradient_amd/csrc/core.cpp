// core.cpp -- readiness state machine of the bucketed gradient reducer (the
// plan itself is built in plan.cpp). Page citations use the short names
// defined in core.hpp.
#include "core.hpp"

#include <utility>

namespace ddpb {

Reducer::Reducer(Plan plan) : plan_(std::move(plan)), launcher_(make_launcher()) {
  begin_iteration();
}

void Reducer::begin_iteration() {
  const int32_t B = plan_.B();
  pending_.resize(B);
  for (int32_t b = 0; b < B; ++b) pending_[b] = static_cast<int32_t>(plan_.members[b].size());
  ready_.assign(plan_.P, 0);
  next_bucket_ = 0;
  calls_ = 0;
  started_ = false;
  order_now_.clear();
}

int Reducer::bind(const BindArgs& args, std::string* err) {
  if (iteration_open()) {
    *err = "bind: an iteration is in progress";
    return kErrState;
  }
  int rc;
  if (args.mode == kModeBucketView) {
    // The gradient of variable v on replica r is the view at view_offset(v)
    // of replica r's storage; accumulation addresses it through that pointer.
    BindArgs a = args;
    a.grad_ptrs.resize(static_cast<size_t>(plan_.R) * plan_.P);
    for (int32_t r = 0; r < plan_.R; ++r)
      for (int32_t v = 0; v < plan_.P; ++v)
        a.grad_ptrs[static_cast<size_t>(r) * plan_.P + v] =
            static_cast<char*>(args.view_bases[r]) + plan_.view_offset(v) * plan_.elem_size;
    rc = launcher_->bind(plan_, a, err);
  } else {
    rc = launcher_->bind(plan_, args, err);
  }
  bound_ = (rc == kOk);
  static_bind_ = bound_ && args.no_alloc;
  sync_step_set_ = false;          // the launcher's tables were released
  // The launch log and the timing history refer to the previous binding's
  // buckets and events: start both afresh.
  log_.clear();
  timed_from_ = finalized_;
  return rc;
}

// [TP] "When a parameter never receives a gradient": the failure of an
// iteration that never finished reducing shows up at the next forward.
int Reducer::ensure_prior_reduction_finished(std::string* err) {
  if (failed_ || iteration_open()) {
    failed_ = true;
    *err = "the previous iteration left buckets unreduced; a new iteration cannot start before ddpb_reset";
    return kErrIncomplete;
  }
  return kOk;
}

int Reducer::mark_ready(int32_t v, std::string* err) {
  if (!bound_) {
    *err = "mark_ready: reducer is not bound";
    return kErrState;
  }
  if (v < 0 || v >= plan_.P) {
    *err = "mark_ready: variable index out of range";
    return kErrIndex;
  }
  if (!sync_) return kOk;     // no_sync: the hook runs but does nothing
  if (failed_) {
    *err = "the previous iteration left buckets unreduced; a new iteration cannot start before ddpb_reset";
    return kErrIncomplete;
  }
  if (!started_) {
    // [C30] "Unused Parameter": once per iteration, at its first hook (even if
    // that hook then fails), the unused variables are marked ready.
    started_ = true;
    log_.clear();
    const int rc = mark_unused_ready(calls_, err);
    if (rc != kOk) {
      failed_ = true;
      return rc;
    }
  }
  if (ready_[v]) {
    *err = "mark_ready: variable marked ready twice in one iteration";
    return kErrDoubleReady;
  }
  ready_[v] = 1;
  order_now_.push_back(v);
  const int32_t call = calls_++;
  const int32_t b = plan_.loc[v].bucket;
  // [Li] per-hook logic: decrement the bucket's pending count; at zero the
  // bucket is ready. [C30] "Bucket 必须按序发起": only the bucket at
  // next_bucket_ may launch, followed by every already complete successor; a
  // later bucket that completes first stays parked.
  if (--pending_[b] == 0 && b == next_bucket_) return launch_ready(call, err);
  return kOk;
}

int Reducer::launch_ready(int32_t call, std::string* err) {
  const int32_t first = next_bucket_;
  while (next_bucket_ < plan_.B() && pending_[next_bucket_] == 0) {
    log_.push_back(LaunchRecord{next_bucket_, call});
    ++next_bucket_;
  }
  if (next_bucket_ == first) return kOk;
  const int rc = launcher_->launch(first, next_bucket_ - 1, finalized_, err);
  if (rc != kOk) failed_ = true;
  return rc;
}

// [Li] "Handling Unused Parameters": variables no replica used are treated as
// ready (their buckets can complete) and their gradients are left alone; a
// replica that did not use a variable contributes zeros. [C30] "Unused
// Parameter": this happens when the iteration's first hook fires.
int Reducer::mark_unused_ready(int32_t call, std::string* err) {
  if (!used_set_) return kOk;
  const int32_t P = plan_.P, R = plan_.R;
  std::vector<uint8_t> global(P, 0);
  for (int32_t r = 0; r < R; ++r)
    for (int32_t v = 0; v < P; ++v) global[v] |= used_acc_[static_cast<size_t>(r) * P + v];
  int rc = launcher_->set_used(used_acc_.data(), global.data(), err);
  if (rc != kOk) return rc;
  for (int32_t v = 0; v < P; ++v) {
    if (global[v]) continue;
    ready_[v] = 1;
    --pending_[plan_.loc[v].bucket];
  }
  return launch_ready(call, err);
}

int Reducer::set_local_used(const uint8_t* used, std::string* err) {
  if (static_bind_) {
    *err = "set_local_used: a binding made by ddpb_bind_static has no staging for used flags";
    return kErrState;
  }
  if (iteration_open()) {
    *err = "set_local_used: must come before the iteration's hooks";
    return kErrState;
  }
  const size_t n = static_cast<size_t>(plan_.R) * plan_.P;
  if (!used_set_) used_acc_.assign(n, 0);
  // [Li] "Gradient Accumulation (no_sync)": under no_sync the flags of the
  // local steps accumulate (OR) until the next synchronisation.
  for (size_t i = 0; i < n; ++i) used_acc_[i] |= used ? (used[i] ? 1 : 0) : 1;
  used_set_ = true;
  return kOk;
}

int Reducer::set_sync_step(void* const* step_ptrs, int32_t step_dtype, bool first, std::string* err) {
  if (!bound_) {
    *err = "set_sync_step: reducer is not bound";
    return kErrState;
  }
  if (step_ptrs == nullptr || (step_dtype != 0 && step_dtype != 1)) {
    *err = "set_sync_step: bad step pointers or dtype";
    return kErrArg;
  }
  if (static_bind_) {
    *err = "set_sync_step: a binding made by ddpb_bind_static has no staging for step tables";
    return kErrState;
  }
  if (failed_) {
    *err = "the previous iteration left buckets unreduced; a new iteration cannot start before ddpb_reset";
    return kErrIncomplete;
  }
  if (iteration_open()) {
    *err = "set_sync_step: must come before the iteration's hooks";
    return kErrState;
  }
  if (!sync_) {
    *err = "set_sync_step: synchronisation is off; accumulate no_sync steps with ddpb_no_sync_accumulate";
    return kErrState;
  }
  const int rc = launcher_->set_sync_step(step_ptrs, step_dtype, first, err);
  if (rc == kOk) sync_step_set_ = true;
  return rc;
}

void Reducer::drop_sync_step() {
  if (!sync_step_set_) return;
  sync_step_set_ = false;
  std::string e2;
  launcher_->set_sync_step(nullptr, 0, false, &e2);
}

int Reducer::finalize(std::string* err) {
  if (!bound_) {
    *err = "finalize: reducer is not bound";
    return kErrState;
  }
  if (!sync_ && !started_) return kOk;
  if (!failed_ && !started_) {            // no hook fired: only unused variables, if any
    started_ = true;
    log_.clear();
    const int rc = mark_unused_ready(0, err);
    if (rc != kOk) {
      failed_ = true;
      return rc;
    }
  }
  if (failed_ || next_bucket_ != plan_.B()) {
    failed_ = true;
    // The buckets already launched keep running on the side streams: order
    // later compute-stream work (the caller's recovery, the next backward's
    // gradient writes) after them, so nothing races with their copy-back.
    std::string e2;
    launcher_->join(&e2);
    *err = "finalize: not every bucket was reduced in this iteration (" +
           std::to_string(next_bucket_) + " of " + std::to_string(plan_.B()) + " launched)";
    return kErrIncomplete;
  }
  // [C30] "Finalize Backward 与梯度可见性": the compute stream is ordered after
  // every bucket's reduction, without a host synchronization.
  const int rc = launcher_->join(err);
  log_ring_[finalized_ % kTimeRing] = log_;
  // a rebuild needs every variable's place in the ready order ([C30]: no
  // ready-order rebuild when the set of used parameters changes)
  has_order_ = (static_cast<int32_t>(order_now_.size()) == plan_.P);
  if (has_order_) last_order_ = order_now_;
  if (used_set_) {                        // the flags served this synchronisation
    used_set_ = false;
    std::string e2;
    launcher_->set_used(nullptr, nullptr, &e2);
  }
  drop_sync_step();                       // ... and so did the step
  ++finalized_;
  begin_iteration();
  return rc;
}

int Reducer::set_sync(bool enabled, std::string* err) {
  if (iteration_open()) {
    *err = "set_sync: an iteration is in progress";
    return kErrState;
  }
  if (!enabled && sync_step_set_) {
    *err = "set_sync: a step is set for the coming synchronisation (ddpb_set_sync_step)";
    return kErrState;
  }
  sync_ = enabled;
  return kOk;
}

int Reducer::accumulate(void* const* step_ptrs, int32_t step_dtype, bool first, std::string* err) {
  if (!bound_) {
    *err = "no_sync_accumulate: reducer is not bound";
    return kErrState;
  }
  if (step_ptrs == nullptr || (step_dtype != 0 && step_dtype != 1)) {
    *err = "no_sync_accumulate: bad step pointers or dtype";
    return kErrArg;
  }
  if (static_bind_) {
    *err = "no_sync_accumulate: a binding made by ddpb_bind_static has no staging for step tables";
    return kErrState;
  }
  if (failed_) {
    *err = "the previous iteration left buckets unreduced; a new iteration cannot start before ddpb_reset";
    return kErrIncomplete;
  }
  if (iteration_open()) {
    // Buckets of the open iteration may still be reducing on the side streams;
    // an accumulation on the compute stream would race with their copy-back.
    *err = "no_sync_accumulate: an iteration is in progress (finalize it first)";
    return kErrState;
  }
  return launcher_->accumulate(step_ptrs, step_dtype, first, err);
}

int Reducer::rebuild_buckets(int64_t cap_bytes, std::string* err) {
  if (failed_ || iteration_open()) {
    *err = "rebuild_buckets: the prior iteration has not finished reducing";
    return kErrIncomplete;
  }
  if (!has_order_) {
    *err = "rebuild_buckets: no finished iteration has recorded a ready order yet";
    return kErrState;
  }
  if (cap_bytes < 0) {
    *err = "rebuild_buckets: negative bucket cap";
    return kErrArg;
  }
  const std::vector<int32_t> order = last_order_;
  plan_ = make_plan(plan_.numel, plan_.elem_size, cap_bytes, plan_.R, &order);
  bound_ = false;                  // device tables and events follow the new plan at the next bind
  static_bind_ = false;
  drop_sync_step();
  log_.clear();
  begin_iteration();
  return kOk;
}

// Recovery after a failed or abandoned iteration. Buckets already launched keep
// running; the compute stream is made to wait for them, so that work the
// caller enqueues next cannot race with their copy-back. Everything the failed
// synchronisation held is dropped with it: its used flags (which serve one
// synchronising iteration, [Li] "Gradient Accumulation (no_sync)") and its
// synchronising step.
int Reducer::reset(std::string* err) {
  failed_ = false;
  drop_sync_step();
  int rc = kOk;
  if (bound_) rc = launcher_->join(err);
  if (used_set_) {
    std::string e2;
    launcher_->set_used(nullptr, nullptr, &e2);
  }
  used_set_ = false;
  used_acc_.clear();
  begin_iteration();
  return rc;
}

}  // namespace ddpb
