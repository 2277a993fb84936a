/*
 * moe_mk.h -- C ABI of the MoE-layer megakernel for AMD Instinct MI355X (gfx950).
 *
 * One call of moe_mk_forward runs a whole top-k Mixture-of-Experts layer as ONE
 * persistent kernel launch:
 *   router GEMM (fp32) -> top-k + softmax over the selected logits -> per-expert
 *   histogram and exp_indptr prefix sum -> token grouping (permutation + row gather)
 *   -> expert GroupGEMM 1 (gate/up, SwiGLU) -> expert GroupGEMM 2 (down)
 *   -> weighted combine.
 *
 * Pages cited below ("Source:" on every declaration):
 *   [ET]   "Event Tensor: A Unified Abstraction for Compiling Dynamic Megakernel (MLSys
 *          2026)", sections Problem, Core method, Key results.
 *   [L112] "Lecture 112: Production Megakernels for Real-World Inference", Key takeaways
 *          and Technical details.
 *   [RaMP] "RaMP: Runtime-Aware Megakernel Polymorphism for Mixture-of-Experts", abstract.
 *
 * Conventions for every entry point:
 *   - Device pointers point to device memory of the plan's device; host pointers are
 *     marked "host".  The caller owns every buffer; the library never allocates or frees
 *     device memory.  A plan owns host memory only.
 *   - Tensors are row-major and contiguous.  bf16 is stored as uint16_t (IEEE binary32
 *     upper half).  Device buffers must be 16-byte aligned.
 *   - Functions return a moe_mk_status_t; nothing throws or aborts across the ABI.
 *     Arguments are checked before anything is enqueued.
 *   - The batch size B is symbolic: it is an argument of every forward, never of the
 *     plan, and one compiled kernel serves every B with no recompilation and no graph.
 *     Counts that follow from B (routing tiles, router and combine task shapes, f splits of
 *     the down projection) are kernel arguments; the GroupGEMM tile shape of each expert
 *     (64-row or 256-row tiles) is chosen on the device from that expert's row count.
 *   - Host-side calls on one plan may come from several threads at once, except
 *     moe_mk_plan_set_debug and moe_mk_plan_destroy.
 */
#ifndef MOE_MK_H
#define MOE_MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Opaque host-side plan: the layer shape (E, k, d, f), the schedule and the device.  It is
 * never written after creation.
 * Source: [ET] Core method (shape dynamism: one runtime instantiated for the actual values
 * of symbolic dimensions such as the batch, without recompiling).
 */
typedef struct moe_mk_plan_s *moe_mk_plan_t;

/*
 * Task scheduling.
 * Source: [ET] Core method (static scheduling: tasks assigned to per-SM queues ahead of
 * time, synchronised by counter semaphores and spin-waits; dynamic scheduling: the event
 * that fires pushes its consumer tasks onto a shared queue with an atomic, idle SMs pop).
 */
typedef enum {
    MOE_MK_SCHED_STATIC = 0,  /* persistent workgroups take tasks from fixed per-XCD lists (then what the other XCDs'
                                 lists have left: any GroupGEMM position, or with wide row tiles down-projection
                                 positions only) and spin-wait on events; relies on the whole grid
                                 (one workgroup per CU) being resident at once, as on a GPU not shared with other
                                 kernels: a workgroup held back by another stream's kernel delays the forward until
                                 it is scheduled, and a wait longer than the watchdog (2 s) ends the forward with
                                 MOE_MK_ERR_WATCHDOG instead of hanging */
    MOE_MK_SCHED_DYNAMIC = 1, /* the task that fires an event pushes its consumers onto a shared queue; idle workgroups
                                 pop.  Every task handed out is ready, so any number of resident workgroups progresses */
    MOE_MK_SCHED_STATIC_COOPERATIVE = 2 /* the static schedule launched as a cooperative kernel: the runtime guarantees
                                 the grid is co-resident, or refuses the launch (MOE_MK_EHIP).  Measured on MI355X it
                                 adds about 15-45 us per forward; for GPUs shared with other kernels */
} moe_mk_sched_t;

/*
 * Status of every call.
 * Source: none on the pages (this library's error reporting).
 */
typedef enum {
    MOE_MK_OK = 0,
    MOE_MK_EINVAL = -1,        /* bad argument: null pointer, misalignment, negative size, ... */
    MOE_MK_EUNSUPPORTED = -2,  /* shape or device outside the supported range */
    MOE_MK_EWORKSPACE = -3,    /* workspace too small, or not initialised */
    MOE_MK_EHIP = -4,          /* a HIP runtime call failed (including a refused cooperative launch) */
    MOE_MK_EDEVICE = -5        /* the kernel reported an error in the workspace (watchdog, bad routing) */
} moe_mk_status_t;

/*
 * Create a plan for a layer with E experts, top-k routing, model width d and expert
 * hidden width f, on the current HIP device, with schedule sched.
 *   Supported: gfx950; d and f multiples of 128; 1 <= E <= 256; 1 <= k <= min(E, 16).
 *   The plan fixes no batch size and no tile configuration (see moe_mk_forward_info).
 *   *plan (host) receives a new plan, owned by the caller (release with
 *   moe_mk_plan_destroy); on an error it receives NULL.
 * Errors: EINVAL (plan == NULL, bad sched), EUNSUPPORTED (shape, device, or no cooperative
 * launch for MOE_MK_SCHED_STATIC_COOPERATIVE), EHIP.
 * Source: [ET] Core method (symbolic shapes: the batch is a symbolic dimension, bound at
 * run time); [L112] Key takeaways, "Symbolic Representation of Work".
 */
moe_mk_status_t moe_mk_plan(moe_mk_plan_t *plan, int E, int k, int d, int f, moe_mk_sched_t sched);

/*
 * Release a plan (NULL is ignored).  No forward of it may be pending on the host side.
 * Source: none on the pages (plan bookkeeping).
 */
void moe_mk_plan_destroy(moe_mk_plan_t plan);

/*
 * Bytes of device workspace that a forward with batch size B needs (grows with B).
 * Returns 0 for an invalid plan or B < 0 or B*k >= 2^31.
 * A workspace of N bytes serves every B whose requirement is <= N; its internal layout
 * depends only on N, so one workspace can serve a sequence of different batch sizes.  It
 * holds the event counters (sized from the symbolic batch), the task queue and the
 * intermediates.
 * Source: [ET] Core method (event tensors with symbolic dimensions, lowered to plain
 * integer tensors).
 */
size_t moe_mk_workspace_bytes(moe_mk_plan_t plan, int64_t B);

/*
 * Prepare a workspace (device pointer ws, ws_bytes bytes): clears it and sets the
 * control block and every event counter to its rest state, enqueued on stream
 * (hipStream_t, may be NULL) as fill kernels (no memset).  Needed once per allocation, and
 * again after a forward reported MOE_MK_EDEVICE.  Afterwards every forward leaves the
 * control block in its rest state by itself.
 * Errors: EINVAL, EWORKSPACE (ws_bytes smaller than the B = 1 requirement), EHIP.
 * Source: [ET] Core method (an event is an integer counter with a wait count).
 */
moe_mk_status_t moe_mk_workspace_init(moe_mk_plan_t plan, void *ws, size_t ws_bytes, void *stream);

/*
 * Run the layer on B tokens.  Enqueues exactly one kernel on stream (hipStream_t, may be
 * NULL) and returns without synchronising.  B = 0 enqueues nothing.
 *   x            bf16 [B, d]           token activations
 *   Wr           fp32 [d, E]           router weights
 *   router_bias  fp32 [E] or NULL      added to the logits before top-k and softmax
 *   W1           bf16 [E, d, f]        gate projection of every expert
 *   W3           bf16 [E, d, f]        up projection of every expert
 *   W2           bf16 [E, f, d]        down projection of every expert
 *   out          bf16 [B, d]           layer output (written, never read)
 *   ws, ws_bytes device workspace prepared by moe_mk_workspace_init; it must not be used
 *                by two forwards at the same time.  Every buffer stays owned by the caller.
 * Routing is exact: logits use 64 interleaved fp32 fma chains over d (chain j mod 64,
 * ascending j) folded in halves, plus the bias; top-k orders by logit, ties to the
 * lower expert index; within an expert the grouped rows keep ascending token order.
 * Errors: EINVAL (null or misaligned pointer, B < 0, B*k >= 2^31), EWORKSPACE, EHIP.
 * Faults detected on the device (a wait that exceeds the watchdog, a non-finite
 * logit) are recorded in the workspace; see moe_mk_workspace_error.
 * Source: [ET] Problem (MoE routing, token grouping and the GroupGEMM depend on the
 * runtime top-k; batch sizes change between calls) and Core method (data-dependent event
 * update: a grouping tile updates the event of the expert each token chose; data-dependent
 * task triggering: the exp_indptr prefix sum sets how many GroupGEMM tiles each expert
 * triggers; notify is an atomic decrement, wait a spin on zero); [L112] Technical
 * details, "Execution Model" (one persistent kernel whose cores take tasks from a queue).
 */
moe_mk_status_t moe_mk_forward(moe_mk_plan_t plan, const void *x, const float *Wr, const float *router_bias,
                               const void *W1, const void *W3, const void *W2, void *out, int64_t B,
                               void *ws, size_t ws_bytes, void *stream);

/*
 * The same layer as moe_mk_forward, run as seven kernels launched one after another on
 * stream (router, top-k, scan, grouping, gate/up GroupGEMM, down GroupGEMM, combine), one
 * task per workgroup, synchronised by the kernel boundaries alone: the launch-per-phase
 * baseline the megakernel is measured against, plainly or captured in a HIP graph (the
 * launches record no memset).  Same arguments, ownership and errors as moe_mk_forward;
 * the output is bitwise that of moe_mk_forward (same tile code and summation order).  A
 * graph of it holds B and the pointers: another B needs another capture.
 * Source: [ET] Problem (launch overhead of 5-10 us per kernel and coarse synchronisation at
 * kernel boundaries; a CUDA graph removes the launch overhead but keeps the boundaries) and
 * Key results (warm-up without re-capture); [L112] Technical details, "Kernel Launch
 * Overhead Mitigation".
 */
moe_mk_status_t moe_mk_forward_unfused(moe_mk_plan_t plan, const void *x, const float *Wr, const float *router_bias,
                                       const void *W1, const void *W3, const void *W2, void *out, int64_t B,
                                       void *ws, size_t ws_bytes, void *stream);

/*
 * moe_mk_forward without a caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  It allocates nothing: no hipMalloc, no hipFree, no allocating library call.
 * The workspace is a static scratch array of MOE_MK_SCRATCH_BYTES in the library's device
 * code, one per GPU, held by each GPU that loads the library until the process ends.
 *   x .. out, B, stream  as for moe_mk_forward.
 *   err   device int32 (4-byte aligned) or NULL: receives this forward's device error bits
 *         (MOE_MK_ERR_*, 0 when none) when the kernel ends.  After a device error the
 *         kernel puts the scratch back to its rest state itself, so the next call runs clean.
 * The largest B is the capacity of the scratch for this plan's shape (the B for which
 * moe_mk_workspace_bytes(plan, B) <= MOE_MK_SCRATCH_BYTES); a larger B returns EWORKSPACE
 * and enqueues nothing.  The first call on a device looks up the scratch's device address;
 * the first call of a plan on a device (after another plan used it, or ever) also enqueues
 * the scratch's preparation (two small fill kernels) on stream before the forward.
 * Every call on one GPU shares that GPU's scratch: calls that overlap in time on one GPU
 * (other streams, other threads) race and give undefined results.
 * Errors: EINVAL, EWORKSPACE, EUNSUPPORTED (device index >= 64), EHIP.
 * Source: none on the pages; for callers that cannot allocate (above).
 */
#define MOE_MK_SCRATCH_BYTES ((size_t)64 << 20)
moe_mk_status_t moe_mk_forward_noalloc(moe_mk_plan_t plan, const void *x, const float *Wr, const float *router_bias,
                                       const void *W1, const void *W3, const void *W2, void *out, int64_t B,
                                       int32_t *err, void *stream);

/*
 * Device pointers into the workspace of the most recent forward with batch size B (no
 * copies; they stay owned by the workspace and are valid until its next forward).
 *   topk_idx  int32 [B, k]   expert of each (token, slot), slot 0 = largest logit
 *   topk_w    fp32  [B, k]   softmax weight of each slot
 *   hist      int32 [E]      rows routed to each expert
 *   exp_indptr int32 [E+1]   exclusive prefix sum of hist
 *   perm      int32 [B*k]    perm[p] = b*k + i: the assignment held by grouped row p
 *   inv       int32 [B*k]    inverse of perm
 *   logits    fp32  [B, E]   router logits
 *   ctl       int32 [512]    control block (ctl[2] is the error word, see below; ctl[9] the
 *                            number of (expert, row tile) pairs, ctl[10] how many of them are
 *                            wide; ctl[192..198] per-kind task counters accumulated over
 *                            forwards)
 *   mt_*      int32 [mt_cap] the forward's row tiles (see the struct)
 * Errors: EINVAL, EWORKSPACE.
 * Source: [ET] Core method (data-dependent event update by the grouping tiles; the
 * exp_indptr prefix sum triggers each expert's GroupGEMM tiles); [RaMP] abstract (the
 * runtime expert histogram sets each expert's tile configuration).
 */
typedef struct {
    const int32_t *topk_idx;
    const float *topk_w;
    const int32_t *hist;
    const int32_t *exp_indptr;
    const int32_t *perm;
    const int32_t *inv;
    const float *logits;
    const int32_t *ctl;
    const int32_t *mt_expert;  /* row tile i (i < ctl[9], in expert order): expert, first    */
    const int32_t *mt_row0;    /* grouped row, rows; a row tile of more than BM rows is wide */
    const int32_t *mt_rows;    /* (up to wide_BM rows), ctl[10] of them                       */
    int64_t mt_cap;            /* length of the three row-tile arrays (host value)            */
} moe_mk_routing_view_t;

/*
 * Fill *view (host) with the pointers above for the last forward of B tokens on the
 * workspace ws (ws_bytes bytes).  Errors: EINVAL, EWORKSPACE.
 * Source: [ET] Core method (data-dependent event update and task triggering).
 */
moe_mk_status_t moe_mk_routing_view(moe_mk_plan_t plan, int64_t B, const void *ws, size_t ws_bytes,
                                    moe_mk_routing_view_t *view /* host */);

/*
 * Read the workspace's error word (synchronises stream).  *err (host) receives 0 when no
 * device fault was recorded, otherwise a bit set of MOE_MK_ERR_*.
 * Returns OK, EINVAL or EHIP.
 * Source: [ET] Core method (wait is a spin on zero; here every spin is bounded by a
 * watchdog, whose expiry is recorded instead of hanging).
 */
#define MOE_MK_ERR_WATCHDOG 1   /* a wait or queue pop exceeded the watchdog */
#define MOE_MK_ERR_NONFINITE 2  /* a router logit was NaN or infinite */
#define MOE_MK_ERR_QUEUE 4      /* the dynamic queue overflowed its capacity */
#define MOE_MK_ERR_UNINIT 8     /* the workspace was not prepared by moe_mk_workspace_init */
moe_mk_status_t moe_mk_workspace_error(moe_mk_plan_t plan, const void *ws, size_t ws_bytes, void *stream,
                                       int32_t *err /* host */);

/*
 * Plan facts (host).  Keys: "E" "k" "d" "f" "sched" "grid" "cus" "wg_per_cu" "BM" "BN1"
 * "BN2" "BK" "wide_BM" "wide_BN1" "wide_BN2" "wide_BK" "wide_min_rows" "route_experts"
 * "threads".  Narrow GroupGEMM tiles are BM rows x BN1 gate/up (BN2 down) columns (half as
 * many in the forwards where forward_info("BN") says so) with K steps of BK; wide ones
 * wide_BM rows x wide_BN1 gate/up (wide_BN2 down) columns with K
 * steps of wide_BK, taken by experts with at least wide_min_rows rows.  Returns -1 for an
 * unknown key or invalid plan.
 * Source: none on the pages (plan bookkeeping).
 */
int64_t moe_mk_plan_info(moe_mk_plan_t plan, const char *key);

/*
 * Per-forward facts of a batch of B tokens on this plan (host, no device access): the
 * counts and tile shapes the library picks from B for one forward.  Keys:
 *   "T"                       64-token routing tiles (top-k and grouping tasks)
 *   "route_tasks"             router tasks; "route_tokens_per_wave", "route_experts_per_task"
 *   "combine_tasks"           combine tasks; "combine_tokens" tokens per combine task
 *   "BN"                      columns of a narrow tile in this forward: plan_info("BN1"), or
 *                             half of it for the smallest batches (every expert narrow and
 *                             twice the gate/up tiles of all its row tiles still at most one
 *                             per workgroup), so that more compute units stream the weights
 *   "NB1"                     gate/up tiles per row tile (f / BN, or f / wide_BN1 = f / BN1
 *                             for a wide row tile)
 *   "NB2" "NB2_wide"          down-projection tiles per row tile and f range in a forward
 *                             without wide row tiles (d / down_cols), and per row tile in one
 *                             with them (d / wide_BN2)
 *   "down_cols"               columns of a down-projection tile in a forward without wide row
 *                             tiles: wide_BN2 (two narrow column blocks in one tile) when BN is
 *                             BN1, d a multiple of wide_BN2 and min(B*k, E) * (d / wide_BN2) * S
 *                             such tasks would fill one round of the grid (256), else BN
 *   "S"                       f ranges of the down projection (1: not split)
 *   "wide_ok"                 1 when experts may take wide row tiles in this forward (the
 *                             kernel then gives them to experts with at least
 *                             plan_info("wide_min_rows") rows; see moe_mk_routing_view)
 *   "all_token_gate_up"       1 when gate/up tiles that start before the routing is known run
 *                             over all B tokens and keep their expert's rows at the end (a
 *                             batch of one routing tile in which an expert gets no token with
 *                             probability (1 - k/E)^B <= 1/4, full-width tiles); the routing
 *                             view then lists one row tile per expert (rows 0 for an expert
 *                             without tokens).  The probability assumes roughly uniform routing;
 *                             under strong skew the early tiles of idle experts stream their
 *                             weights for nothing (at most one round of the grid's tiles).  0 with
 *                             MOE_MK_DEBUG_GROUPED_GATE_UP set.
 * Returns -1 for an unknown key, an invalid plan, B < 1 or B*k >= 2^31.
 * Source: [RaMP] abstract (what follows from the batch size alone, as opposed to the
 * routing distribution, which only the device sees).
 */
int64_t moe_mk_forward_info(moe_mk_plan_t plan, int64_t B, const char *key);

/*
 * Debug controls for tests (host): watchdog limit in GPU real-time ticks (100 MHz;
 * 0 restores the default of 2 s) and a flag word (MOE_MK_DEBUG_*).  They apply to later
 * forwards of this plan; no forward may be issued on the plan from another thread meanwhile.
 * MOE_MK_DEBUG_DROP_NOTIFY makes the first grouping task skip one of its event
 * notifications, so the waiting GroupGEMM tasks must leave through the watchdog and record
 * MOE_MK_ERR_WATCHDOG instead of hanging.
 * Source: none on the pages (test and measurement controls).
 */
#define MOE_MK_DEBUG_DROP_NOTIFY 1
#define MOE_MK_DEBUG_TRACE 2  /* record per-task timestamps, see moe_mk_trace_view */
#define MOE_MK_DEBUG_NO_PREFETCH 4  /* static schedule: no weight prefetch while a small batch is routed (A/B timing) */
#define MOE_MK_DEBUG_NARROW_ONLY 8  /* every expert takes narrow row tiles (A/B timing of the tile choice) */
#define MOE_MK_DEBUG_BATCH_RULE 16  /* tile shape from the batch size alone: every expert with more than BM
                                       rows wide when B*k >= 128*E, else all narrow (A/B timing) */
#define MOE_MK_DEBUG_GROUPED_GATE_UP 32  /* never the all-token gate/up: gate/up tiles over grouped rows only,
                                            after the routing (A/B timing; see forward_info) */
moe_mk_status_t moe_mk_plan_set_debug(moe_mk_plan_t plan, int64_t watchdog_ticks, int32_t flags);

/*
 * Debug view of the task trace of the last forward run with MOE_MK_DEBUG_TRACE: *trace
 * (host) receives a device pointer (into the workspace) to *n (host) records of eight
 * int64 each:
 *   [0] task index g | kind << 32 | workgroup << 40   (kind: 0 router, 1 top-k, 2 scan,
 *       3 grouping, 4 gate/up GEMM, 5 down GEMM, 6 combine)
 *   [1] time the workgroup obtained the task, [2] time its dependencies were satisfied,
 *   [3] time it finished, [4] time its compute ended (before its notifications),
 *   all in GPU real-time clock ticks (100 MHz); [5] the XCD (accelerator die, 0..7) that
 *   ran it; [6], [7] ends of the scan and of the grouping when the top-k task of a
 *   one-tile batch runs both itself (else 0).
 * Records of tasks that did not run in that forward are stale.  Errors: EINVAL, EWORKSPACE.
 * Source: [L112] Key takeaways, "Dependency Tracking (Barriers)" (consumers start before
 * all producers have finished: the trace shows when each task's dependencies were met).
 */
moe_mk_status_t moe_mk_trace_view(moe_mk_plan_t plan, int64_t B, const void *ws, size_t ws_bytes,
                                  const int64_t **trace /* host */, int64_t *n /* host */);

/*
 * Short static description of a status code (never NULL; owned by the library).
 * Source: none on the pages (error reporting).
 */
const char *moe_mk_status_str(moe_mk_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MK_H */
