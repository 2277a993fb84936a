// host.cpp -- the C ABI of include/moe_mk.h: plans, workspace layout, argument checks and
// the single kernel launch per forward.  Host code only (the device pass sees nothing).
#include <hip/hip_runtime.h>
#if !defined(__HIP_DEVICE_COMPILE__)

#include <atomic>
#include <cstdint>
#include <mutex>
#include <cstdlib>
#include <cstring>
#include <new>

#include "../../include/moe_mk.h"
#include "mk_capacity.h"
#include "mk_common.h"

hipError_t mk_launch(const mk::Params &p, int grid, hipStream_t stream, bool cooperative);
hipError_t mk_ws_init(void *ws, size_t bytes, hipStream_t stream);
hipError_t mk_occupancy(int *blocks_per_cu);
hipError_t mk_scratch(void **ptr, size_t *bytes);
hipError_t mk_launch_unfused(const mk::Params &p, hipStream_t stream);

struct moe_mk_plan_s {
    mk::Shape s;
    int sched;
    int device;
    int cus;
    int wg_per_cu;
    int grid;
    long long watchdog;
    int debug;
    uint64_t id;  // unique over the process lifetime (keys the per-thread capacity cache)
};

namespace {

constexpr long long kDefaultWatchdog = 200000000LL;  // 2 s at the 100 MHz real-time clock

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool plan_ok(moe_mk_plan_t p) { return p != nullptr && p->s.E > 0; }

size_t bytes_for(const mk::Shape &s, int64_t B) { return mk::workspace_bytes_for(s, B); }

std::atomic<uint64_t> g_next_plan_id{1};

int64_t capacity(moe_mk_plan_t p, size_t ws_bytes) { return mk::workspace_capacity(p->s, p->id, ws_bytes); }

}  // namespace

extern "C" {

const char *moe_mk_status_str(moe_mk_status_t s) {
    switch (s) {
        case MOE_MK_OK: return "ok";
        case MOE_MK_EINVAL: return "invalid argument";
        case MOE_MK_EUNSUPPORTED: return "unsupported shape or device";
        case MOE_MK_EWORKSPACE: return "workspace too small or not initialised";
        case MOE_MK_EHIP: return "HIP runtime error";
        case MOE_MK_EDEVICE: return "device-side error recorded in the workspace";
    }
    return "unknown status";
}

moe_mk_status_t moe_mk_plan(moe_mk_plan_t *plan, int E, int k, int d, int f, moe_mk_sched_t sched) {
    if (!plan) return MOE_MK_EINVAL;
    *plan = nullptr;
    if (sched != MOE_MK_SCHED_STATIC && sched != MOE_MK_SCHED_DYNAMIC && sched != MOE_MK_SCHED_STATIC_COOPERATIVE)
        return MOE_MK_EINVAL;
    if (sched == MOE_MK_SCHED_STATIC_COOPERATIVE) {
        int coop = 0;
        int d = 0;
        if (hipGetDevice(&d) != hipSuccess) return MOE_MK_EHIP;
        if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, d) != hipSuccess) return MOE_MK_EHIP;
        if (!coop) return MOE_MK_EUNSUPPORTED;
    }
    if (E < 1 || E > mk::kMaxE || k < 1 || k > mk::kMaxK || k > E) return MOE_MK_EUNSUPPORTED;
    if (d < 128 || f < 128 || d % 128 != 0 || f % 128 != 0) return MOE_MK_EUNSUPPORTED;
    if ((int64_t)d * f * E >= ((int64_t)1 << 40)) return MOE_MK_EUNSUPPORTED;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_MK_EHIP;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_MK_EHIP;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MOE_MK_EUNSUPPORTED;
    int occ = 0;
    if (mk_occupancy(&occ) != hipSuccess || occ < 1) return MOE_MK_EHIP;
    if (occ > 2) occ = 2;
    moe_mk_plan_s *p = new (std::nothrow) moe_mk_plan_s;
    if (!p) return MOE_MK_EINVAL;
    p->s = mk::Shape{E, k, d, f};
    p->sched = (int)sched;
    p->device = dev;
    p->cus = prop.multiProcessorCount;
    p->wg_per_cu = occ;
    p->grid = p->cus * occ;
    const char *env = std::getenv("MOE_MK_GRID");  // debugging aid: cap the persistent grid
    if (env) {
        // whole groups of 8 workgroups: the static schedule gives each of the 8 XCDs its own
        // list, taken by the workgroups w with w % 8 == x, so every list needs a workgroup
        const int g = std::atoi(env) / 8 * 8;
        if (g >= 8 && g < p->grid) p->grid = g;
    }
    p->watchdog = kDefaultWatchdog;
    p->debug = 0;
    p->id = g_next_plan_id.fetch_add(1);
    *plan = p;
    return MOE_MK_OK;
}

void moe_mk_plan_destroy(moe_mk_plan_t plan) { delete plan; }

size_t moe_mk_workspace_bytes(moe_mk_plan_t plan, int64_t B) {
    if (!plan_ok(plan) || B < 0 || B * plan->s.k >= ((int64_t)1 << 31)) return 0;
    return bytes_for(plan->s, B);
}

moe_mk_status_t moe_mk_workspace_init(moe_mk_plan_t plan, void *ws, size_t ws_bytes, void *stream) {
    if (!plan_ok(plan) || !ws || !aligned16(ws)) return MOE_MK_EINVAL;
    if (ws_bytes < bytes_for(plan->s, 1)) return MOE_MK_EWORKSPACE;
    if (hipSetDevice(plan->device) != hipSuccess) return MOE_MK_EHIP;
    if (mk_ws_init(ws, ws_bytes, (hipStream_t)stream) != hipSuccess) return MOE_MK_EHIP;
    return MOE_MK_OK;
}

}  // extern "C"

namespace {

// Checks shared by both forward entry points (everything but the workspace).
moe_mk_status_t check_forward(moe_mk_plan_t plan, const void *x, const float *Wr, const float *router_bias,
                              const void *W1, const void *W3, const void *W2, void *out, int64_t B) {
    if (!plan_ok(plan)) return MOE_MK_EINVAL;
    if (B < 0 || B * plan->s.k >= ((int64_t)1 << 31)) return MOE_MK_EINVAL;
    if (B == 0) return MOE_MK_OK;
    if (!x || !Wr || !W1 || !W3 || !W2 || !out) return MOE_MK_EINVAL;
    if (!aligned16(x) || !aligned16(Wr) || !aligned16(W1) || !aligned16(W3) || !aligned16(W2) || !aligned16(out))
        return MOE_MK_EINVAL;
    if (router_bias && ((uintptr_t)router_bias & 3u)) return MOE_MK_EINVAL;
    return MOE_MK_OK;
}

// Kernel arguments of a forward of B tokens whose workspace (a layout for cap tokens)
// starts at base.
bool dense_forward(moe_mk_plan_t plan, int64_t B) {
    return !(plan->debug & MOE_MK_DEBUG_GROUPED_GATE_UP) && mk::all_token_gate_up(plan->s, B);
}

mk::Params make_params(moe_mk_plan_t plan, const void *x, const float *Wr, const float *router_bias, const void *W1,
                       const void *W3, const void *W2, void *out, int64_t B, char *base, int64_t cap) {
    const mk::Shape &s = plan->s;
    const mk::Layout L = mk::make_layout(s, cap);
    const mk::Counts c = mk::make_counts(s, B);
    const mk::Counts cc = mk::make_counts(s, cap);
    mk::Params P;
    P.x = (const uint16_t *)x;
    P.Wr = Wr;
    P.bias = router_bias;
    P.W1 = (const uint16_t *)W1;
    P.W3 = (const uint16_t *)W3;
    P.W2 = (const uint16_t *)W2;
    P.out = (uint16_t *)out;
    P.B = (int)B;
    P.E = s.E;
    P.k = s.k;
    P.d = s.d;
    P.f = s.f;
    P.sched = plan->sched == MOE_MK_SCHED_DYNAMIC ? 1 : 0;  // the kernel knows static (0) or dynamic (1)
    P.debug = plan->debug;
    P.nR = (int)c.nR;
    P.nTG = (int)c.nTG;
    P.tpw = (int)c.tpw;
    P.nEB = (int)c.nEB;
    P.reb = (int)c.reb;
    P.T = (int)c.T;
    P.nC = (int)c.nC;
    P.CT = mk::combine_tokens(B, s.k);
    const mk::Tiles tl = mk::tile_config(s, B);
    P.BN = tl.BN;
    P.NB1 = tl.NB1;
    P.NB2 = tl.NB2;
    P.NB2w = tl.NB2w;
    P.DC = tl.DC;
    P.S = tl.S;
    P.wide_ok = tl.wide_ok;
    // experts with at least wide_min rows take wide row tiles (always more than one routing
    // tile's worth of rows, so a batch of one routing tile has narrow row tiles only)
    if (plan->debug & MOE_MK_DEBUG_NARROW_ONLY)
        P.wide_min = 1 << 30;
    else if (plan->debug & MOE_MK_DEBUG_BATCH_RULE)
        P.wide_min = B * s.k >= (int64_t)mk::kBatchRuleRows * s.E ? mk::kWideMinRows : 1 << 30;
    else
        P.wide_min = mk::kWideMinRows;
    P.dense = dense_forward(plan, B) ? 1 : 0;
    // dynamic schedule: tickets without a queue slot (the routers; with the all-token gate/up also
    // the top-k task and the gate/up tiles of every expert, in f-range order)
    P.nImp = P.nR + (P.dense ? 1 + s.E * P.NB1 : 0);
    {  // after the tile configuration: the prefetch follows the gate/up tiles (none is needed when
       // they run from the start)
        const mk::Prefetch pf = (plan->debug & MOE_MK_DEBUG_NO_PREFETCH) || P.dense
                                    ? mk::Prefetch{0, 0}
                                    : mk::prefetch_plan(s, B, P.NB1, false);
        P.pf_nt = pf.nt;
        P.pf_lines = pf.lines;
    }
    P.q_cap = (int)cc.q_cap;
    P.mt_cap = (int)cc.mt_cap;
    P.watchdog = plan->watchdog;
    P.ctl = (int *)(base + L.ctl);
    P.ev_logit = (int *)(base + L.ev_logit);
    P.ev_exp = (int *)(base + L.ev_exp);
    P.ev_h = (int *)(base + L.ev_h);
    P.ev_d = (int *)(base + L.ev_d);
    P.nch = (int)mk::ceil_div(s.d, mk::kCombineCols);
    P.logits = (float *)(base + L.logits);
    P.topk_idx = (int *)(base + L.topk_idx);
    P.topk_w = (float *)(base + L.topk_w);
    P.tile_hist = (int *)(base + L.tile_hist);
    P.hist = (int *)(base + L.hist);
    P.indptr = (int *)(base + L.indptr);
    P.mt_base = (int *)(base + L.mt_base);
    P.mt_expert = (int *)(base + L.mt_expert);
    P.mt_row0 = (int *)(base + L.mt_row0);
    P.mt_rows = (int *)(base + L.mt_rows);
    P.perm = (int *)(base + L.perm);
    P.inv = (int *)(base + L.inv);
    P.amt = (int *)(base + L.amt);
    P.h = (uint16_t *)(base + L.h);
    P.y = (uint16_t *)(base + L.y);
    P.yp = (float *)(base + L.yp);
    P.qslots = (unsigned long long *)(base + L.qslots);
    P.red_ctr = (int *)(base + L.red_ctr);
    P.trace = (long long *)(base + L.trace);
    P.err_out = nullptr;
    P.heal = 0;
    P.unfused = 0;
    return P;
}

static_assert(MOE_MK_SCRATCH_BYTES == mk::kScratchBytes, "the header states the scratch size");

// Per device: the plan whose layout the static scratch currently holds (0: none yet).
std::mutex g_scratch_mu;
uint64_t g_scratch_plan[64] = {};

}  // namespace

extern "C" {

moe_mk_status_t moe_mk_forward(moe_mk_plan_t plan, const void *x, const float *Wr, const float *router_bias,
                               const void *W1, const void *W3, const void *W2, void *out, int64_t B, void *ws,
                               size_t ws_bytes, void *stream) {
    const moe_mk_status_t st = check_forward(plan, x, Wr, router_bias, W1, W3, W2, out, B);
    if (st != MOE_MK_OK || B == 0) return st;
    if (!ws || !aligned16(ws)) return MOE_MK_EINVAL;
    const int64_t cap = capacity(plan, ws_bytes);
    if (cap < B) return MOE_MK_EWORKSPACE;
    const mk::Params P = make_params(plan, x, Wr, router_bias, W1, W3, W2, out, B, (char *)ws, cap);
    if (hipSetDevice(plan->device) != hipSuccess) return MOE_MK_EHIP;
    if (mk_launch(P, plan->grid, (hipStream_t)stream, plan->sched == MOE_MK_SCHED_STATIC_COOPERATIVE) != hipSuccess)
        return MOE_MK_EHIP;
    return MOE_MK_OK;
}

moe_mk_status_t moe_mk_forward_unfused(moe_mk_plan_t plan, const void *x, const float *Wr, const float *router_bias,
                                       const void *W1, const void *W3, const void *W2, void *out, int64_t B, void *ws,
                                       size_t ws_bytes, void *stream) {
    const moe_mk_status_t st = check_forward(plan, x, Wr, router_bias, W1, W3, W2, out, B);
    if (st != MOE_MK_OK || B == 0) return st;
    if (!ws || !aligned16(ws)) return MOE_MK_EINVAL;
    const int64_t cap = capacity(plan, ws_bytes);
    if (cap < B) return MOE_MK_EWORKSPACE;
    mk::Params P = make_params(plan, x, Wr, router_bias, W1, W3, W2, out, B, (char *)ws, cap);
    P.unfused = 1;
    P.dense = 0;  // one kernel per phase: the gate/up kernel runs after the grouping
    P.nImp = P.nR;
    if (hipSetDevice(plan->device) != hipSuccess) return MOE_MK_EHIP;
    if (mk_launch_unfused(P, (hipStream_t)stream) != hipSuccess) return MOE_MK_EHIP;
    return MOE_MK_OK;
}

moe_mk_status_t moe_mk_forward_noalloc(moe_mk_plan_t plan, const void *x, const float *Wr, const float *router_bias,
                                       const void *W1, const void *W3, const void *W2, void *out, int64_t B,
                                       int32_t *err, void *stream) {
    const moe_mk_status_t st = check_forward(plan, x, Wr, router_bias, W1, W3, W2, out, B);
    if (st != MOE_MK_OK || B == 0) return st;
    if (err && ((uintptr_t)err & 3u)) return MOE_MK_EINVAL;
    if (hipSetDevice(plan->device) != hipSuccess) return MOE_MK_EHIP;
    if (plan->device < 0 || plan->device >= 64) return MOE_MK_EUNSUPPORTED;
    void *base = nullptr;
    size_t bytes = 0;
    if (mk_scratch(&base, &bytes) != hipSuccess) return MOE_MK_EHIP;
    const int64_t cap = capacity(plan, bytes);
    if (cap < B) return MOE_MK_EWORKSPACE;
    {
        // The scratch is shared by every plan on this device.  Its rest state is valid for
        // one layout (one plan shape), so it is prepared again whenever another plan uses it:
        // the zero fill and the control block's rest values, enqueued before the forward.
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (g_scratch_plan[plan->device] != plan->id) {
            if (mk_ws_init(base, mk::make_layout(plan->s, cap).total, (hipStream_t)stream) != hipSuccess)
                return MOE_MK_EHIP;
            g_scratch_plan[plan->device] = plan->id;
        }
    }
    mk::Params P = make_params(plan, x, Wr, router_bias, W1, W3, W2, out, B, (char *)base, cap);
    P.err_out = err;
    P.heal = 1;
    if (mk_launch(P, plan->grid, (hipStream_t)stream, plan->sched == MOE_MK_SCHED_STATIC_COOPERATIVE) != hipSuccess)
        return MOE_MK_EHIP;
    return MOE_MK_OK;
}

moe_mk_status_t moe_mk_routing_view(moe_mk_plan_t plan, int64_t B, const void *ws, size_t ws_bytes,
                                    moe_mk_routing_view_t *view) {
    if (!plan_ok(plan) || !ws || !view || B < 0) return MOE_MK_EINVAL;
    const int64_t cap = capacity(plan, ws_bytes);
    if (cap < B || cap < 1) return MOE_MK_EWORKSPACE;
    const mk::Layout L = mk::make_layout(plan->s, cap);
    const char *base = (const char *)ws;
    view->topk_idx = (const int32_t *)(base + L.topk_idx);
    view->topk_w = (const float *)(base + L.topk_w);
    view->hist = (const int32_t *)(base + L.hist);
    view->exp_indptr = (const int32_t *)(base + L.indptr);
    view->perm = (const int32_t *)(base + L.perm);
    view->inv = (const int32_t *)(base + L.inv);
    view->logits = (const float *)(base + L.logits);
    view->ctl = (const int32_t *)(base + L.ctl);
    view->mt_expert = (const int32_t *)(base + L.mt_expert);
    view->mt_row0 = (const int32_t *)(base + L.mt_row0);
    view->mt_rows = (const int32_t *)(base + L.mt_rows);
    view->mt_cap = mk::make_counts(plan->s, cap).mt_cap;
    return MOE_MK_OK;
}

moe_mk_status_t moe_mk_trace_view(moe_mk_plan_t plan, int64_t B, const void *ws, size_t ws_bytes,
                                  const int64_t **trace, int64_t *n) {
    if (!plan_ok(plan) || !ws || !trace || !n || B < 1) return MOE_MK_EINVAL;
    const int64_t cap = capacity(plan, ws_bytes);
    if (cap < B) return MOE_MK_EWORKSPACE;
    const mk::Layout L = mk::make_layout(plan->s, cap);
    const mk::Counts c = mk::make_counts(plan->s, cap);
    *trace = (const int64_t *)((const char *)ws + L.trace);
    *n = c.q_cap + c.nR_max;
    return MOE_MK_OK;
}

moe_mk_status_t moe_mk_workspace_error(moe_mk_plan_t plan, const void *ws, size_t ws_bytes, void *stream,
                                       int32_t *err) {
    if (!plan_ok(plan) || !ws || !err) return MOE_MK_EINVAL;
    if (ws_bytes < bytes_for(plan->s, 1)) return MOE_MK_EWORKSPACE;
    if (hipSetDevice(plan->device) != hipSuccess) return MOE_MK_EHIP;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return MOE_MK_EHIP;
    int32_t words[mk::CTL_WORDS];
    if (hipMemcpy(words, ws, sizeof words, hipMemcpyDeviceToHost) != hipSuccess) return MOE_MK_EHIP;
    *err = words[mk::CTL_ERR];
    if (words[mk::CTL_MAGIC] != mk::kMagic) *err |= 8;
    return MOE_MK_OK;
}

int64_t moe_mk_plan_info(moe_mk_plan_t plan, const char *key) {
    if (!plan_ok(plan) || !key) return -1;
    struct {
        const char *k;
        int64_t v;
    } t[] = {{"E", plan->s.E},
             {"k", plan->s.k},
             {"d", plan->s.d},
             {"f", plan->s.f},
             {"sched", plan->sched},
             {"grid", plan->grid},
             {"cus", plan->cus},
             {"wg_per_cu", plan->wg_per_cu},
             {"BM", mk::kBM},
             {"BN1", mk::kBN},
             {"BN2", mk::kBN},
             {"BK", mk::kBK},
             {"wide_BM", mk::kWideBM},
             {"wide_BN1", mk::kWideBN1},
             {"wide_BN2", mk::kWideBN},
             {"wide_BK", mk::kWideBK},
             {"wide_min_rows", mk::kWideMinRows},
             {"route_experts", mk::kRouteExperts},
             {"threads", mk::kThreads}};
    for (auto &e : t)
        if (std::strcmp(e.k, key) == 0) return e.v;
    return -1;
}

int64_t moe_mk_forward_info(moe_mk_plan_t plan, int64_t B, const char *key) {
    if (!plan_ok(plan) || !key || B < 1 || B * plan->s.k >= ((int64_t)1 << 31)) return -1;
    const mk::Shape &s = plan->s;
    const mk::Counts c = mk::make_counts(s, B);
    const mk::Tiles t = mk::tile_config(s, B);
    struct {
        const char *k;
        int64_t v;
    } tab[] = {{"T", c.T},
               {"route_tasks", c.nR},
               {"route_tokens_per_wave", c.tpw},
               {"route_experts_per_task", c.reb},
               {"combine_tasks", c.nC},
               {"combine_tokens", mk::combine_tokens(B, s.k)},
               {"BN", t.BN},
               {"NB1", t.NB1},
               {"NB2", t.NB2},
               {"NB2_wide", t.NB2w},
               {"down_cols", t.DC},
               {"S", t.S},
               {"wide_ok", t.wide_ok},
               {"all_token_gate_up", dense_forward(plan, B) ? 1 : 0}};
    for (auto &e : tab)
        if (std::strcmp(e.k, key) == 0) return e.v;
    return -1;
}

moe_mk_status_t moe_mk_plan_set_debug(moe_mk_plan_t plan, int64_t watchdog_ticks, int32_t flags) {
    if (!plan_ok(plan) || watchdog_ticks < 0) return MOE_MK_EINVAL;
    plan->watchdog = watchdog_ticks ? watchdog_ticks : kDefaultWatchdog;
    plan->debug = flags;
    return MOE_MK_OK;
}

}  // extern "C"

#endif  // !__HIP_DEVICE_COMPILE__
