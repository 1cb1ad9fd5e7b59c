/*
 * ddpb.h -- C ABI of the bucketed gradient reducer for MI355X (gfx950).
 *
 * The library implements the gradient-reduction hot path of a data-parallel
 * wrapper as these pages describe it:
 *   [Li]   "PyTorch Distributed: Experiences on Accelerating Data Parallel
 *          Training" (paper-graph-ui summary of arXiv 2006.15704), §3.4,
 *          subsections "Gradient Bucketing", "Overlapping Computation with
 *          Communication", "Gradient Accumulation (no_sync)";
 *   [TP]   "Distributed Data Parallel" (tensorplay.cn notes), "Internal Design",
 *          "When a parameter never receives a gradient", "Gradient sync you can
 *          turn off";
 *   [C30]  "NCCL 专家课程 30：DDP Reducer、Bucket 与计算通信重叠" (blog.cptz.space),
 *          sections "Variable 到 Bucket", "Bucket 必须按序发起",
 *          "bucket_cap_mb 不是张量切分器", "Finalize Backward 与梯度可见性";
 *   [PDTI] "PyTorch Distributed Training Internals", §2 and §3.
 *
 * R data-parallel replicas live in one GPU's HBM. The all-reduce of a bucket
 * is emulated by an in-HBM elementwise mean over the R replicas' gradients,
 * summed in replica order 0..R-1 in fp32 and divided once by R (IEEE,
 * round to nearest even), after which the mean is written back into every
 * replica's gradient. There is no communication between GPUs.
 *
 * Conventions
 *  - Every call returns a status code (DDPB_OK or a negative DDPB_E_*); no
 *    C++ exception crosses the ABI. ddpb_last_error() describes the last
 *    failure on the calling thread.
 *  - Device pointers are HIP device addresses of memory the caller owns
 *    (allocated by PyTorch); they must stay valid until ddpb_destroy or the
 *    next ddpb_bind. Host pointers are read during the call only.
 *  - Streams are hipStream_t values passed as void*. The library owns its
 *    hipEvents and a small device copy of its pointer and segment tables.
 *  - A handle is driven by one host thread; the API is not thread-safe.
 *  - "Replica-major" arrays of R*P pointers hold replica r's variable v at
 *    index r*P + v.
 */
#ifndef DDPB_H
#define DDPB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ddpb_reducer* ddpb_t;

/* element types */
enum { DDPB_F32 = 0, DDPB_BF16 = 1 };

/* kernel modes for ddpb_bind */
enum {
  DDPB_MODE_FUSED = 0,  /* one kernel per bucket: gather, mean, write back; no flat copy */
  DDPB_MODE_STAGED = 1  /* three kernels per bucket: pack into flat buckets, mean, copy back */
};

/* flags for ddpb_bind */
enum {
  DDPB_BIND_DEVICE_TIMESTAMPS = 1, /* kernels stamp start/end device clock into the launch log; a
                                      diagnostic: each workgroup's closing fence and counter update
                                      cost about 10 % of the throughput of a BERT-large sync */
  DDPB_BIND_TIME_LAUNCHES = 2,     /* hipEvents around each bucket's kernels (ddpb_get_launch_times);
                                      about 0.8 % of that throughput */
  DDPB_BIND_ROCTX = 4,             /* host-side roctx ranges around each launch of complete buckets
                                      ("ddpb launch b0-b1"), the finalize join, no_sync_accumulate and
                                      set_sync_step, for rocprofv3 --marker-trace; no device work */
  DDPB_BIND_OVERLAP = 8            /* the reductions will run beside a backward on the compute stream:
                                      start with no per-CU limit on reduction workgroups (the
                                      same setting as ddpb_set_workgroups_per_cu(h, 0), which
                                      stays until changed) instead of one per CU, which
                                      hid more of the reduction behind a bf16 MLP backward of many
                                      buckets ([PDTI] §3.1, [Li] "Overlapping Computation with
                                      Communication"); a standalone sync runs faster without it */
};

/* status codes */
enum {
  DDPB_OK = 0,
  DDPB_E_ARG = -1,          /* bad argument (null pointer, size, dtype, misaligned buffer) */
  DDPB_E_INDEX = -2,        /* variable or bucket index out of range */
  DDPB_E_DOUBLE_READY = -3, /* a variable was marked ready twice in one iteration */
  DDPB_E_INCOMPLETE = -4,   /* the iteration did not reduce every bucket */
  DDPB_E_STATE = -5,        /* call not valid in the current state (e.g. not bound) */
  DDPB_E_HIP = -6,          /* a HIP runtime call failed */
  DDPB_E_NOMEM = -7         /* host or device allocation failed */
};

/* ---------------------------------------------------------------------------
 * Construction and plan ([Li] "Gradient Bucketing"; [C30] "Variable 到 Bucket",
 * "bucket_cap_mb 不是张量切分器").
 */

/* Plan the buckets for P parameters given in Model.parameters() order.
 *   shapes     concatenated dims of all parameters (sum(ndims) entries, >= 0)
 *   ndims      ndims[v] = number of dims of parameter v (0 = scalar, numel 1)
 *   dtype      gradient/bucket element type; DDPB_F32 only
 *   bucket_cap_bytes  the cap (>= 0). Parameters are visited in reverse
 *              order; each whole tensor joins the open bucket and the bucket
 *              closes once its byte size is >= the cap (so 0 = one bucket per
 *              tensor, and a tensor larger than the cap forms one larger
 *              bucket). Bucket 0 holds the last-defined parameters.
 *   R          number of emulated replicas, 1..64
 * Host-only: no device is touched. *out receives the handle. */
int ddpb_reducer_create(const int64_t* shapes, const int32_t* ndims, int32_t P,
                        int32_t dtype, int64_t bucket_cap_bytes, int32_t R, ddpb_t* out);

void ddpb_destroy(ddpb_t h);

int ddpb_num_buckets(ddpb_t h, int32_t* B);

/* The locator of variable v: bucket index, position inside the bucket, and
 * element offset/length of its narrowed view of the flat bucket. */
int ddpb_get_locator(ddpb_t h, int32_t v, int32_t* bucket, int32_t* intra,
                     int64_t* offset, int64_t* length);

/* Bucket b: number of member variables, byte size, and (if vars != NULL) its
 * member variable indices in bucket order (vars must hold nvars entries). */
int ddpb_get_bucket(ddpb_t h, int32_t b, int32_t* nvars, int64_t* bytes, int32_t* vars);

/* The device work table. Each bucket's members are cut into segments of at
 * most seg_elems elements; one wavefront processes one segment. Segments are
 * stored bucket by bucket; bucket b owns [first, first + count). */
int ddpb_num_segments(ddpb_t h, int32_t* n, int64_t* seg_elems);
int ddpb_get_bucket_segments(ddpb_t h, int32_t b, int32_t* first, int32_t* count);
int ddpb_get_segment(ddpb_t h, int32_t s, int32_t* var, int32_t* bucket,
                     int64_t* start, int64_t* length, int64_t* bucket_offset);

/* ---------------------------------------------------------------------------
 * Binding memory and streams.
 */

/* Device bytes of caller-provided workspace needed by a mode: 0 for FUSED;
 * for STAGED, R per-replica flat copies of every bucket plus one averaged
 * copy (each bucket starts on a 256-byte boundary). */
int ddpb_workspace_bytes(ddpb_t h, int32_t mode, int64_t* bytes);

/* Attach device memory and streams.
 *   grad_ptrs      R*P device pointers (replica-major) to each replica's fp32
 *                  gradient of each variable, numel[v] contiguous elements.
 *                  The reducer reads them and writes the averaged values back
 *                  in place.
 *   workspace      device buffer of >= ddpb_workspace_bytes(mode) bytes (may
 *                  be NULL when that is 0), 256-byte aligned.
 *   compute_stream stream on which gradients are produced (hipStream_t).
 *   side_streams   n_side (1..16) streams for the reduction kernels; bucket b
 *                  runs on side_streams[b % n_side]. Keep them on hardware
 *                  queues of their own (with 4 queues per process, the
 *                  compute stream and two side streams created one after the
 *                  other are placed apart). An entry may be the compute stream
 *                  itself: its buckets then run in order with the compute
 *                  work, with no cross-stream events (nothing overlaps them;
 *                  the lowest latency when there is no backward to hide
 *                  behind). A plan of a single bucket always reduces on the
 *                  compute stream: that bucket launches only once the last
 *                  gradient is ready, so there is nothing to overlap.
 *   mode, flags    DDPB_MODE_*, DDPB_BIND_*.
 * Synchronizes the compute stream once to upload the tables. Not allowed
 * while an iteration is in progress. */
int ddpb_bind(ddpb_t h, void* const* grad_ptrs, void* workspace, int64_t ws_bytes,
              void* compute_stream, void* const* side_streams, int32_t n_side,
              int32_t mode, int32_t flags);

/* Binding for callers that cannot allocate device memory: tight serving
 * loops, harnesses that forbid hipMalloc, programs that capture their steps
 * into HIP graphs and keep allocation out of them. Same as ddpb_bind (grad_ptrs, compute_stream and mode mean the
 * same) except that the library allocates nothing: its pointer and segment
 * tables and, in DDPB_MODE_STAGED, its flat buckets (no workspace argument)
 * are placed in a static device array of DDPB_STATIC_SCRATCH_BYTES bytes
 * that every device the library runs on holds until the process ends. No
 * hipMalloc, hipHostMalloc or hipEventCreate is called; the bucket reductions
 * run on the compute stream itself (no side streams, no events, no flags).
 * The bind uploads the tables and synchronises the compute stream once, so it
 * is not made during a capture; syncs on the binding may be captured and
 * replayed as with ddpb_bind.
 * Needs round256(R*P*8) + round256(segments*32) bytes (ddpb_num_segments),
 * plus ddpb_workspace_bytes(STAGED) in staged mode; a larger model gets
 * DDPB_E_ARG and is left unbound.
 * The array is shared by every static binding on a device and keeps the last
 * binding's tables: a later ddpb_bind_static on the same device (by this
 * handle or another) waits for the device to drain and takes the array over, after which the earlier handle's
 * launches fail with DDPB_E_STATE until it is bound again. Static bindings of
 * one device used from several threads at once race. Nothing in the array
 * needs to start at zero (every byte the kernels read is written first).
 * ddpb_no_sync_accumulate, ddpb_set_sync_step and ddpb_set_local_used need
 * pinned staging that only ddpb_bind allocates and return DDPB_E_STATE on a
 * static binding. Errors: DDPB_E_ARG, DDPB_E_STATE (iteration in progress),
 * DDPB_E_HIP. */
enum { DDPB_STATIC_SCRATCH_BYTES = 32 << 20 };
int ddpb_bind_static(ddpb_t h, void* const* grad_ptrs, void* compute_stream, int32_t mode);

/* Ready-order bucket rebuild ([C30] "第一次迭代为何不同"): re-plans the buckets
 * from the order in which the hooks fired in the last finished iteration,
 * first-ready variable first, with the same rule (whole tensors, the bucket
 * closes once its size is >= bucket_cap_bytes), so buckets follow the real
 * backward order and no bucket waits on a later gradient. A first iteration
 * planned with a huge cap (one bucket) learns the order without reducing
 * early. Needs a finished iteration and none in progress (DDPB_E_STATE /
 * DDPB_E_INCOMPLETE otherwise). Afterwards the plan queries describe the new
 * buckets and the handle must be bound again (ddpb_bind or
 * ddpb_bind_bucket_views; view offsets change). */
int ddpb_rebuild_buckets(ddpb_t h, int64_t bucket_cap_bytes);

/* Hook order of the last finished iteration (variable indices, first hook
 * first). Writes min(cap, count) entries and sets *n = count. */
int ddpb_get_ready_order(ddpb_t h, int32_t* order, int32_t cap, int32_t* n);

/* gradient_as_bucket_view ([TP] "Internal Design", backward pass; [C30]
 * section "gradient_as_bucket_view"; [PDTI] §4): each replica keeps all its
 * gradients in one flat fp32 storage laid out bucket by bucket, and the
 * gradient of variable v is the view of numel[v] elements at element offset
 * ddpb_get_view_offset(v) (bucket base, 64-element aligned, plus the
 * locator's offset). The hook then copies nothing and the bucket's reduction
 * walks its flat range contiguously.
 *   ddpb_view_storage_elems   elements each replica's storage must hold
 *   ddpb_get_view_offset      element offset of variable v in that storage
 *   ddpb_bind_bucket_views    R device pointers to the storages (replica r's
 *                             first; 256-byte aligned, >= storage_elems fp32
 *                             each, caller-owned), streams and flags as in
 *                             ddpb_bind. ddpb_no_sync_accumulate and every
 *                             other call work unchanged on the views. */
int ddpb_view_storage_elems(ddpb_t h, int64_t* elems);
int ddpb_get_view_offset(ddpb_t h, int32_t v, int64_t* offset);
int ddpb_bind_bucket_views(ddpb_t h, void* const* replica_storage, int64_t storage_elems,
                           void* compute_stream, void* const* side_streams, int32_t n_side,
                           int32_t flags);

/* Caps the number of workgroups (256 threads each) of every reduction launch;
 * 0 (the default) launches one workgroup per four segments, so a bucket uses
 * the whole GPU. A small cap keeps the reduction on a few compute units while
 * backward GEMMs keep the rest, the way a collective library restricts itself
 * to a few channels ([PDTI] §3.1 on collectives occupying compute units).
 * Each wavefront then strides over the bucket's segments; results do not
 * depend on the cap. May be called at any time; applies to later launches. */
int ddpb_set_launch_blocks(ddpb_t h, int32_t max_blocks);

/* At most n workgroups of the reduction kernels (fused, bucket-view and staged
 * modes; not the kernel that also accumulates a ddpb_set_sync_step step,
 * which runs without a limit) share one compute unit, counting every launch in flight: n = 1 (the
 * default) or 2, or 0 for no limit beyond the kernels' register budget (three
 * per CU for the fused kernel used without used flags). One per CU gives the
 * highest throughput for a synchronisation running alone: a CU holding two
 * workgroups of one launch finishes after the others. No limit lets the
 * reduction share CUs more densely with concurrent backward kernels, which hid
 * more of it behind a 48-bucket MLP backward ([PDTI] §3.1: collectives occupy
 * the compute units of the compute they overlap). Enforced by reserving, per
 * workgroup, more than 1/(n+1) of a CU's LDS (the kernels use none). The
 * no_sync accumulation always runs one workgroup per CU. Results do not
 * depend on it. May be called at any time; applies to later launches.
 * Returns DDPB_E_ARG for n outside 0..2. */
int ddpb_set_workgroups_per_cu(ddpb_t h, int32_t n);

/* ---------------------------------------------------------------------------
 * One iteration ([Li] "Overlapping Computation with Communication";
 * [C30] "Bucket 必须按序发起", "Finalize Backward 与梯度可见性").
 */

/* The check a wrapper's forward makes before a new iteration: returns
 * DDPB_E_INCOMPLETE (and latches that state until ddpb_reset) when the
 * previous iteration was left open -- its first hook ran but ddpb_finalize
 * did not complete it ([TP] "When a parameter never receives a gradient").
 * While latched, ddpb_mark_ready and ddpb_finalize fail the same way. */
int ddpb_ensure_prior_reduction_finished(ddpb_t h);

/* Hook for variable v: its gradient is final on every replica, ordered on the
 * compute stream. Decrements the pending count of v's bucket. When the count
 * reaches zero and every earlier bucket has been launched, launches that
 * bucket and then every following bucket that is already complete, in index
 * order: it records an event on the compute stream, makes the side stream
 * wait for it and enqueues the bucket's kernels. A bucket that completes
 * before an earlier one waits (parked) until the earlier one is launched.
 * With sync disabled it returns DDPB_OK and does nothing.
 * Errors: DDPB_E_INDEX, DDPB_E_DOUBLE_READY, DDPB_E_STATE (not bound),
 * DDPB_E_INCOMPLETE (latched failure), DDPB_E_HIP. */
int ddpb_mark_ready(ddpb_t h, int32_t v);

/* Same as calling ddpb_mark_ready for vs[0..n-1] in order; stops at the first
 * error and returns it. */
int ddpb_mark_ready_many(ddpb_t h, const int32_t* vs, int32_t n);

/* End of backward: every bucket must have been launched (else
 * DDPB_E_INCOMPLETE, latched; the compute stream is then still made to wait
 * for the buckets that did launch). Records a completion event on every side
 * stream and makes the compute stream wait for them, so later work on the
 * compute stream sees the averaged gradients without a host synchronization;
 * then resets the per-iteration state. A no-op while sync is disabled and no
 * variable was marked. */
int ddpb_finalize(ddpb_t h);

/* Graph capture. A whole synchronisation (the ddpb_mark_ready calls and
 * ddpb_finalize) may be recorded into a HIP graph by capturing the bound
 * compute stream: the library's event record on the compute stream forks the
 * side streams into the capture and finalize's join brings them back, so the
 * graph holds every bucket kernel with its ordering. Replaying the graph
 * repeats the device work only; the host state machine advanced once, at
 * capture. Refused during capture (DDPB_E_STATE, nothing recorded):
 * ddpb_no_sync_accumulate, ddpb_set_sync_step and an iteration with
 * ddpb_set_local_used flags (all upload tables from host staging that later
 * calls reuse), and any
 * launch of a binding made with DDPB_BIND_TIME_LAUNCHES. A refusal inside
 * ddpb_mark_ready latches DDPB_E_INCOMPLETE like any failed launch. */

/* The no_sync() switch ([Li] "Gradient Accumulation (no_sync)"; [TP] "Gradient
 * sync you can turn off"): enabled = 0 makes ddpb_mark_ready a no-op.
 * DDPB_E_STATE if an iteration is in progress. */
int ddpb_set_sync(ddpb_t h, int32_t enabled);

/* Local gradient accumulation of one backward pass into the bound fp32
 * gradients, on the compute stream: grad = float(step) when first_step != 0,
 * grad += float(step) otherwise, elementwise for every replica and variable.
 *   step_ptrs   R*P device pointers (replica-major), numel[v] elements each;
 *               NULL = that replica produced no gradient for the variable in
 *               this backward (zeros on the first step, unchanged otherwise)
 *   step_dtype  DDPB_F32 or DDPB_BF16 (widened exactly to fp32)
 * Belongs between iterations: DDPB_E_STATE while an iteration is in progress
 * (its buckets may still be reducing on the side streams), DDPB_E_INCOMPLETE
 * while a failed iteration is latched. */
int ddpb_no_sync_accumulate(ddpb_t h, void* const* step_ptrs, int32_t step_dtype,
                            int32_t first_step);

/* The last local step of a no_sync run, accumulated by the synchronisation
 * itself ([Li] "Gradient Accumulation (no_sync)": the backward that leaves
 * no_sync adds its gradients to the accumulated ones, then the buckets are
 * averaged). Instead of calling ddpb_no_sync_accumulate and then firing the
 * hooks, the caller sets the step here and fires the hooks as its gradients
 * become final: each bucket's reduction then forms, per replica and element,
 * exactly what ddpb_no_sync_accumulate(step_ptrs, step_dtype, first_step)
 * would leave in the gradient and averages that -- the same bits in one pass
 * over HBM instead of two. The step table is uploaded now (on the compute
 * stream); the step memory is read when each bucket is reduced, so it must
 * stay valid until ddpb_finalize.
 *   step_ptrs, step_dtype, first_step   as for ddpb_no_sync_accumulate
 * Must come before the iteration's first ddpb_mark_ready, with sync enabled
 * (else DDPB_E_STATE; DDPB_E_INCOMPLETE while a failed iteration is latched); consumed by that iteration's ddpb_finalize, dropped by
 * ddpb_reset, a rebind or a rebuild. While it is set, ddpb_set_sync(h, 0) is
 * refused. Fused and bucket-view modes reduce each bucket in one kernel; in
 * staged mode, or with used flags, each bucket's variables are accumulated
 * on its side stream just before its reduction. Refused during graph capture
 * (the table comes from host staging). */
int ddpb_set_sync_step(ddpb_t h, void* const* step_ptrs, int32_t step_dtype,
                       int32_t first_step);

/* Unused parameters ([Li] "Handling Unused Parameters and Sub-Graph
 * Execution"; [TP] "When a parameter never receives a gradient"; [C30]
 * "Unused Parameter"): which replicas will produce a gradient for which
 * variables in the coming backward pass, as the forward's graph walk finds
 * them.
 *   used   R*P host bytes, replica-major (used[r*P + v] != 0: replica r uses
 *          variable v), read before the call returns; NULL = all used
 * Calls before one synchronisation OR together (no_sync micro-steps each add
 * their flags); the flags serve the next synchronising iteration and are then
 * dropped. At that iteration's first ddpb_mark_ready (or at ddpb_finalize when
 * no hook fires), variables no replica used count as ready, so their buckets
 * can complete; they must not be marked again (DDPB_E_DOUBLE_READY). In the
 * reduction a replica that did not use a variable contributes zeros, and a
 * variable that no replica used keeps every replica's gradient untouched
 * (copy modes). With bucket views an unused view counts as zeros in its
 * bucket's average (it is not read) and, like every view of the bucket,
 * receives the mean, so a view no replica used ends as zeros. An iteration
 * with unused variables
 * records no ready order for ddpb_rebuild_buckets. DDPB_E_STATE if an
 * iteration is in progress. */
int ddpb_set_local_used(ddpb_t h, const uint8_t* used);

/* Recovery after a failed or abandoned iteration ([TP] "When a parameter never
 * receives a gradient": the failure surfaces at the next forward; clearing it
 * is this library's call). Clears a latched DDPB_E_INCOMPLETE, the
 * per-iteration state, the used flags set for the failed synchronisation
 * (ddpb_set_local_used) and a pending ddpb_set_sync_step. Buckets already
 * enqueued keep running; the compute stream is made to wait for every side
 * stream that ran one, so work enqueued on it afterwards cannot race with
 * their copy-back. Errors: DDPB_E_HIP. */
int ddpb_reset(ddpb_t h);

/* ---------------------------------------------------------------------------
 * Diagnostics.
 */

/* Launches of the current or last finished iteration, in launch order:
 * bucket index, index (0-based, within the iteration) of the ddpb_mark_ready
 * call that launched it, and, with DDPB_BIND_DEVICE_TIMESTAMPS, the device
 * clock (wall_clock64 ticks) at kernel start and end (else 0). Device values
 * are read with a blocking copy; synchronize the side streams first.
 * A bind or a bucket rebuild empties the log.
 * Writes min(cap, count) entries and sets *n = count. */
int ddpb_get_launch_log(ddpb_t h, int32_t* buckets, int32_t* trigger_call,
                        int64_t* dev_t0, int64_t* dev_t1, int32_t cap, int32_t* n);

/* With DDPB_BIND_TIME_LAUNCHES: per launched bucket, in launch order, for the
 * finalized iteration `iterations_ago` back (0 = the last one; the last 64
 * iterations are kept, and only those run with the current binding, else
 * DDPB_E_INDEX):
 *   ms[i]        duration from the start of the bucket's first kernel to the
 *                end of its last kernel (hipEvents attached to the dispatches)
 *   start_ms[i]  (may be NULL) start relative to the iteration's first launch,
 *                so overlapping launches on several side streams can be merged
 * Blocks the host until those events have completed; later iterations may
 * keep running on the device meanwhile. */
int ddpb_get_launch_times(ddpb_t h, int32_t iterations_ago, float* start_ms, float* ms, int32_t cap,
                          int32_t* n);

/* Device clock rate of wall_clock64 in Hz (for converting launch-log ticks). */
int ddpb_device_clock_hz(ddpb_t h, int64_t* hz);

const char* ddpb_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DDPB_H */
