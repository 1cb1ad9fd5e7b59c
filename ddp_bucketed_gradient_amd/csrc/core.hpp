// core.hpp -- host side of the bucketed gradient reducer: bucket plan,
// variable locator, device work (segment) table and the readiness state
// machine. No HIP types appear here; device work goes through Launcher.
//
// Pages cited (titles shortened):
//   [Li]  "PyTorch Distributed: Experiences on Accelerating Data Parallel
//         Training" summary, §3.4 "Gradient Bucketing", "Overlapping
//         Computation with Communication", "Gradient Accumulation (no_sync)".
//   [TP]  tensorplay "Distributed Data Parallel" notes, "Internal Design",
//         "When a parameter never receives a gradient".
//   [C30] "NCCL 专家课程 30" blog, "Variable 到 Bucket", "Bucket 必须按序发起",
//         "bucket_cap_mb 不是张量切分器", "Finalize Backward 与梯度可见性".
#pragma once

#include <cstdint>
#include <memory>
#include <string>
#include <vector>

namespace ddpb {

// Elements per device segment: one wavefront processes one segment (32 KiB per
// replica). Measured on BERT-large shapes, R = 8, two side streams:
// 2048 / 4096 / 8192 / 16384 elements -> 4.95 / 5.40 / 5.49 / 5.38 TB/s.
constexpr int64_t kSegElems = 8192;
// Flat-bucket bases in the staged workspace are padded to this many elements.
constexpr int64_t kFlatAlignElems = 64;
constexpr int kMaxReplicas = 64;
// Launch-timing events are kept for this many most recent iterations.
constexpr int kTimeRing = 64;

enum Status : int {
  kOk = 0, kErrArg = -1, kErrIndex = -2, kErrDoubleReady = -3,
  kErrIncomplete = -4, kErrState = -5, kErrHip = -6, kErrNoMem = -7
};

// Device-side work descriptor, 32 bytes, read by the kernels.
struct Segment {
  int32_t var;        // variable index
  int32_t flags;      // kSegVec* bits: which float4 accesses are legal
  int64_t start;      // first element inside the variable
  int64_t len;        // number of elements
  int64_t boff;       // element offset inside the flat bucket
};
static_assert(sizeof(Segment) == 32, "segment layout is shared with the kernels");
constexpr int32_t kSegVecStart = 1;   // start is a multiple of 4 elements
constexpr int32_t kSegVecFlat = 2;    // boff is a multiple of 4 elements
constexpr int32_t kSegVecBoth = kSegVecStart | kSegVecFlat;

struct Locator {
  int32_t bucket;
  int32_t intra;
  int64_t offset;
  int64_t length;
};

struct Plan {
  int32_t P = 0;
  int32_t R = 0;
  int64_t cap_bytes = 0;
  int64_t elem_size = 4;
  std::vector<int64_t> numel;                  // per variable
  std::vector<std::vector<int32_t>> members;   // per bucket, in bucket order
  std::vector<int64_t> bucket_elems;           // per bucket
  std::vector<int64_t> flat_base;              // per bucket, padded element base in a flat buffer
  int64_t flat_elems = 0;                      // padded total (one replica)
  std::vector<Locator> loc;                    // per variable
  std::vector<Segment> segs;                   // bucket by bucket
  std::vector<int32_t> seg_first;              // per bucket, size B + 1
  std::vector<int32_t> seg_bucket;             // per segment
  // gradient_as_bucket_view: each replica's gradients live in one flat storage
  // of flat_elems floats in bucket layout; variable v is the view at
  // flat_base[bucket] + offset. The reduction then walks each bucket's flat
  // range in kSegElems chunks (var 0 = the replica's storage).
  std::vector<Segment> view_segs;
  std::vector<int32_t> view_seg_first;         // per bucket, size B + 1

  int64_t view_offset(int32_t v) const { return flat_base[loc[v].bucket] + loc[v].offset; }

  int32_t B() const { return static_cast<int32_t>(members.size()); }
};

// Reverse-order greedy assignment under the cap ([Li] "Gradient Bucketing";
// [C30] "bucket_cap_mb 不是张量切分器"), then locators, flat bases and segments.
// `order` (optional) is the visiting order; default is the reverse of the
// definition order, a rebuild passes the learned ready order.
Plan make_plan(const std::vector<int64_t>& numel, int64_t elem_size, int64_t cap_bytes, int32_t R,
               const std::vector<int32_t>* order = nullptr);

enum Mode : int32_t { kModeFused = 0, kModeStaged = 1, kModeBucketView = 2 };

struct BindArgs {
  std::vector<void*> grad_ptrs;     // R * P, replica-major
  std::vector<void*> view_bases;    // R flat storages (kModeBucketView only)
  void* workspace = nullptr;
  int64_t ws_bytes = 0;
  void* compute_stream = nullptr;
  std::vector<void*> side_streams;
  int32_t mode = 0;
  int32_t flags = 0;
  // Allocation-free binding (ddpb_bind_static): the device tables and the
  // staged workspace live in the library's static device array, the
  // reductions run on the compute stream, and nothing is allocated.
  bool no_alloc = false;
};

// Bytes of the static device array behind allocation-free bindings (one per
// device, shared by every such binding on it).
constexpr int64_t kStaticScratchBytes = int64_t(32) << 20;

int64_t workspace_bytes(const Plan& plan, int32_t mode);

struct LaunchRecord {
  int32_t bucket;
  int32_t trigger_call;
};

// Device work. The HIP implementation enqueues kernels; the test build only
// records what would be enqueued.
class Launcher {
 public:
  virtual ~Launcher() = default;
  virtual int bind(const Plan& plan, const BindArgs& args, std::string* err) = 0;
  // Buckets [first, last] are complete and every earlier bucket has been
  // launched: order them after the compute stream's current work and enqueue
  // their reduction on the side stream(s), in index order.
  // `iteration` counts finalized iterations before this one.
  virtual int launch(int32_t first, int32_t last, int64_t iteration, std::string* err) = 0;
  // End of iteration: the compute stream waits for every side stream.
  virtual int join(std::string* err) = 0;
  virtual int accumulate(void* const* step_ptrs, int32_t step_dtype, bool first, std::string* err) = 0;
  // Device clock stamps of the given launched buckets (zeros when disabled).
  virtual int read_stamps(const std::vector<LaunchRecord>& log, std::vector<int64_t>* t0,
                          std::vector<int64_t>* t1, std::string* err) = 0;
  // Waits for, then returns, the start (relative to the iteration's first
  // launch) and the duration of each launch of `iteration`, in milliseconds.
  virtual int read_times(int64_t iteration, const std::vector<LaunchRecord>& log, std::vector<float>* start_ms,
                         std::vector<float>* ms, std::string* err) = 0;
  virtual int clock_hz(int64_t* hz, std::string* err) = 0;
  // Caps the workgroups of each reduction launch (0 = one per four segments).
  virtual void set_max_blocks(int32_t n) = 0;
  // At most n fused-kernel workgroups per compute unit (0 = registers decide).
  virtual int set_workgroups_per_cu(int32_t n, std::string* err) = 0;
  // Used flags for the launches that follow (R * P replica-major, and the OR
  // over replicas per variable), or NULL for "all used". Ordered on the
  // compute stream before the next launch's ready event.
  virtual int set_used(const uint8_t* used, const uint8_t* global, std::string* err) = 0;
  // Step gradients (R * P, replica-major) that the coming synchronisation adds
  // to every replica's gradient as it reduces each bucket, or NULL for none.
  virtual int set_sync_step(void* const* step_ptrs, int32_t step_dtype, bool first, std::string* err) = 0;
};

std::unique_ptr<Launcher> make_launcher();

// The readiness state machine ([Li] per-hook logic and "Launching AllReduce in
// order"; [C30] "Variable 到 Bucket", "Bucket 必须按序发起").
class Reducer {
 public:
  explicit Reducer(Plan plan);
  const Plan& plan() const { return plan_; }

  int bind(const BindArgs& args, std::string* err);
  int ensure_prior_reduction_finished(std::string* err);
  int mark_ready(int32_t v, std::string* err);
  int finalize(std::string* err);
  int set_sync(bool enabled, std::string* err);
  int accumulate(void* const* step_ptrs, int32_t step_dtype, bool first, std::string* err);
  int reset(std::string* err);
  // [C30] "第一次迭代为何不同": re-plan from the hook order of the last finished
  // iteration (same cap rule); the handle must be bound again afterwards.
  int rebuild_buckets(int64_t cap_bytes, std::string* err);
  // Per-replica used flags (R * P, replica-major; NULL = all used) for the
  // coming synchronisation; OR-ed with earlier calls since the last sync.
  int set_local_used(const uint8_t* used, std::string* err);
  // [Li] "Gradient Accumulation (no_sync)": the last local step of a no_sync
  // run, accumulated by the coming synchronisation itself, bucket by bucket.
  int set_sync_step(void* const* step_ptrs, int32_t step_dtype, bool first, std::string* err);
  const std::vector<int32_t>& last_ready_order() const { return last_order_; }
  const std::vector<LaunchRecord>& log() const { return log_; }
  int64_t finalized() const { return finalized_; }
  // Launches of finalized iteration `it` (only the last kTimeRing are kept).
  const std::vector<LaunchRecord>& log_of(int64_t it) const { return log_ring_[it % kTimeRing]; }
  // First iteration launched with the current binding; launch times of
  // earlier iterations belong to device resources that no longer exist.
  int64_t timed_from() const { return timed_from_; }
  Launcher* launcher() { return launcher_.get(); }

 private:
  void begin_iteration();
  bool iteration_open() const { return started_; }

  Plan plan_;
  std::unique_ptr<Launcher> launcher_;
  bool bound_ = false;
  bool static_bind_ = false;       // bound by ddpb_bind_static: no staging for tables
  bool sync_ = true;
  bool failed_ = false;            // latched "prior reduction did not finish"
  std::vector<int32_t> pending_;   // per bucket
  std::vector<uint8_t> ready_;     // per variable
  int32_t next_bucket_ = 0;
  int32_t calls_ = 0;              // mark_ready calls that counted, this iteration
  bool started_ = false;           // the iteration's first hook has run (unused variables marked)
  std::vector<LaunchRecord> log_;
  std::vector<int32_t> order_now_;   // hook order of the current iteration
  std::vector<int32_t> last_order_;  // ... of the last finished iteration
  bool has_order_ = false;
  std::vector<uint8_t> used_acc_;    // R * P used flags, OR-ed until the next sync
  bool used_set_ = false;
  bool sync_step_set_ = false;       // a step for the coming synchronisation is set

  void drop_sync_step();

  int launch_ready(int32_t call, std::string* err);
  int mark_unused_ready(int32_t call, std::string* err);
  int64_t finalized_ = 0;          // iterations finalized so far
  int64_t timed_from_ = 0;         // finalized_ at the last successful bind
  std::vector<LaunchRecord> log_ring_[kTimeRing];
};

}  // namespace ddpb
