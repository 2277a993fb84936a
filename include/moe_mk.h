/*
 * moe_mk.h -- C ABI of the MoE-layer megakernel for AMD Instinct MI355X (gfx950).
 *
 * One call of moe_mk_forward runs a whole top-k Mixture-of-Experts layer as ONE
 * persistent kernel launch:
 *   router GEMM (fp32) -> top-k + softmax over the selected logits -> per-expert
 *   histogram and exp_indptr prefix sum -> token grouping (permutation + row gather)
 *   -> expert GroupGEMM 1 (gate/up, SwiGLU) -> expert GroupGEMM 2 (down)
 *   -> weighted combine.
 * The steps follow "Event Tensor: A Unified Abstraction for Compiling Dynamic
 * Megakernel" (MLSys 2026): section "Problem" (MoE routing, token grouping and
 * GroupGEMM depend on the runtime top-k; dynamic batch sizes must not force a
 * recompile) and section "Core method" (grouping tiles update the event of the expert
 * chosen at run time; the exp_indptr prefix sum decides how many GroupGEMM tiles each
 * expert triggers; events are integer counters where notify is an atomic decrement
 * and wait is a spin until zero; static per-CU queues or a dynamic atomic queue).
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
 *     plan, and the kernel (compiled once per GroupGEMM tile shape, narrow or wide) serves
 *     every B with no recompilation and no graph.
 */
#ifndef MOE_MK_H
#define MOE_MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_mk_plan_s *moe_mk_plan_t;  /* opaque, host-side, immutable after creation */

/* Task scheduling ("Event Tensor", Core method, static and dynamic scheduling). */
typedef enum {
    MOE_MK_SCHED_STATIC = 0,  /* persistent workgroups take tasks from fixed per-XCD lists (then, with narrow tiles, what
                                 the other XCDs' lists have left) and spin-wait on events */
    MOE_MK_SCHED_DYNAMIC = 1  /* the task that fires an event pushes its consumers onto a shared queue; idle workgroups pop */
} moe_mk_sched_t;

typedef enum {
    MOE_MK_OK = 0,
    MOE_MK_EINVAL = -1,        /* bad argument: null pointer, misalignment, negative size, ... */
    MOE_MK_EUNSUPPORTED = -2,  /* shape or device outside the supported range */
    MOE_MK_EWORKSPACE = -3,    /* workspace too small, or not initialised */
    MOE_MK_EHIP = -4,          /* a HIP runtime call failed */
    MOE_MK_EDEVICE = -5        /* the kernel reported an error in the workspace (watchdog, bad routing) */
} moe_mk_status_t;

/*
 * Create a plan for a layer with E experts, top-k routing, model width d and expert
 * hidden width f, on the current HIP device.
 *   Supported: gfx950; d and f multiples of 128; 1 <= E <= 256; 1 <= k <= min(E, 16).
 *   The tile configuration depends on (E, k, d, f) only.
 *   *plan receives a new plan (release with moe_mk_plan_destroy).
 * Errors: EINVAL (plan == NULL, bad sched), EUNSUPPORTED (shape, device), EHIP.
 */
moe_mk_status_t moe_mk_plan(moe_mk_plan_t *plan, int E, int k, int d, int f, moe_mk_sched_t sched);

/* Release a plan (NULL is ignored). */
void moe_mk_plan_destroy(moe_mk_plan_t plan);

/*
 * Bytes of device workspace that a forward with batch size B needs (monotone in B).
 * Returns 0 for an invalid plan or B < 0 or B*k >= 2^31.
 * A workspace of N bytes serves every B whose requirement is <= N; its internal layout
 * depends only on N, so one workspace can serve a sequence of different batch sizes.
 */
size_t moe_mk_workspace_bytes(moe_mk_plan_t plan, int64_t B);

/*
 * Prepare a workspace (device pointer ws, ws_bytes bytes): clears it and sets the
 * control block to its rest state, enqueued on stream (hipStream_t, may be NULL).
 * Needed once per allocation, and again after a forward reported MOE_MK_EDEVICE.
 * Afterwards every forward leaves the control block in its rest state by itself.
 * Errors: EINVAL, EWORKSPACE (ws_bytes smaller than the B = 1 requirement), EHIP.
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
 *                by two forwards at the same time.
 * Routing is exact: logits use 64 interleaved fp32 fma chains over d (chain j mod 64,
 * ascending j) folded in halves, plus the bias; top-k orders by logit, ties to the
 * lower expert index; within an expert the grouped rows keep ascending token order.
 * Errors: EINVAL (null or misaligned pointer, B < 0, B*k >= 2^31), EWORKSPACE, EHIP.
 * Faults detected on the device (a wait that exceeds the watchdog, a non-finite
 * logit) are recorded in the workspace; see moe_mk_workspace_error.
 */
moe_mk_status_t moe_mk_forward(moe_mk_plan_t plan, const void *x, const float *Wr, const float *router_bias,
                               const void *W1, const void *W3, const void *W2, void *out, int64_t B,
                               void *ws, size_t ws_bytes, void *stream);

/*
 * Device pointers into the workspace of the most recent forward with batch size B.
 * Valid until the next forward on that workspace.
 *   topk_idx  int32 [B, k]   expert of each (token, slot), slot 0 = largest logit
 *   topk_w    fp32  [B, k]   softmax weight of each slot
 *   hist      int32 [E]      rows routed to each expert
 *   exp_indptr int32 [E+1]   exclusive prefix sum of hist
 *   perm      int32 [B*k]    perm[p] = b*k + i: the assignment held by grouped row p
 *   inv       int32 [B*k]    inverse of perm
 *   logits    fp32  [B, E]   router logits
 *   ctl       int32 [512]    control block (ctl[2] is the error word, see below; ctl[9] the
 *                            number of (expert, row tile) pairs; ctl[192..198] per-kind task
 *                            counters accumulated over forwards)
 * Errors: EINVAL, EWORKSPACE.
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
} moe_mk_routing_view_t;

moe_mk_status_t moe_mk_routing_view(moe_mk_plan_t plan, int64_t B, const void *ws, size_t ws_bytes,
                                    moe_mk_routing_view_t *view /* host */);

/*
 * Read the workspace's error word (synchronises stream).  *err (host) receives 0 when no
 * device fault was recorded, otherwise a bit set of MOE_MK_ERR_*.
 * Returns OK, EINVAL or EHIP.
 */
#define MOE_MK_ERR_WATCHDOG 1   /* a wait or queue pop exceeded the watchdog */
#define MOE_MK_ERR_NONFINITE 2  /* a router logit was NaN or infinite */
#define MOE_MK_ERR_QUEUE 4      /* the dynamic queue overflowed its capacity */
#define MOE_MK_ERR_UNINIT 8     /* the workspace was not prepared by moe_mk_workspace_init */
moe_mk_status_t moe_mk_workspace_error(moe_mk_plan_t plan, const void *ws, size_t ws_bytes, void *stream,
                                       int32_t *err /* host */);

/* Plan facts (host).  Keys: "E" "k" "d" "f" "sched" "grid" "cus" "wg_per_cu" "BM" "BN1" "BN2" "BK"
 * "wide_BM" "wide_BN1" "wide_BN2" "wide_BK" "wide_min_rows" "route_experts" "threads".
 * GroupGEMM tiles are BM x BN1 (gate/up) and BM x BN2 (down) with K steps of BK, except in
 * forwards where B*k >= wide_min_rows*E (an expert averages that many rows): there tiles
 * have wide_BM rows, wide_BN1 gate/up columns, wide_BN2 down columns and K steps of wide_BK.  Returns -1 for an
 * unknown key or invalid plan. */
int64_t moe_mk_plan_info(moe_mk_plan_t plan, const char *key);

/*
 * Debug controls for tests (host): watchdog limit in GPU real-time ticks (100 MHz;
 * 0 restores the default of 2 s) and a flag word (MOE_MK_DEBUG_*).  They apply to later
 * forwards of this plan.  MOE_MK_DEBUG_DROP_NOTIFY makes the first grouping task skip
 * one of its event notifications, so the waiting GroupGEMM tasks must leave through the
 * watchdog and record MOE_MK_ERR_WATCHDOG instead of hanging.
 */
#define MOE_MK_DEBUG_DROP_NOTIFY 1
#define MOE_MK_DEBUG_TRACE 2  /* record per-task timestamps, see moe_mk_trace_view */
#define MOE_MK_DEBUG_NO_PREFETCH 4  /* static schedule: no weight prefetch while a small batch is routed (A/B timing) */
moe_mk_status_t moe_mk_plan_set_debug(moe_mk_plan_t plan, int64_t watchdog_ticks, int32_t flags);

/*
 * Debug view of the task trace of the last forward run with MOE_MK_DEBUG_TRACE: *trace
 * (host) receives a device pointer to *n (host) records of eight int64 each:
 *   [0] task index g | kind << 32 | workgroup << 40   (kind: 0 router, 1 top-k, 2 scan,
 *       3 grouping, 4 gate/up GEMM, 5 down GEMM, 6 combine)
 *   [1] time the workgroup obtained the task, [2] time its dependencies were satisfied,
 *   [3] time it finished, [4] time its compute ended (before its notifications),
 *   all in GPU real-time clock ticks (100 MHz); [5] the XCD (accelerator die, 0..7) that
 *   ran it; [6], [7] ends of the scan and of the grouping when the top-k task of a
 *   one-tile batch runs both itself (else 0).
 * Records of tasks that did not run in that forward are stale.  Errors: EINVAL, EWORKSPACE.
 */
moe_mk_status_t moe_mk_trace_view(moe_mk_plan_t plan, int64_t B, const void *ws, size_t ws_bytes,
                                  const int64_t **trace /* host */, int64_t *n /* host */);

/* Short static description of a status code. */
const char *moe_mk_status_str(moe_mk_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MK_H */
