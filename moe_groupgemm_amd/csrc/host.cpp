// host.cpp -- the C ABI of include/moe_mk.h: plans, workspace layout, argument checks and
// the single kernel launch per forward.  Host code only (the device pass sees nothing).
#include <hip/hip_runtime.h>
#if !defined(__HIP_DEVICE_COMPILE__)

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <new>

#include "../../include/moe_mk.h"
#include "mk_common.h"

hipError_t mk_launch(const mk::Params &p, int grid, hipStream_t stream);
hipError_t mk_ws_init(void *ws, size_t bytes, hipStream_t stream);
hipError_t mk_occupancy(int *blocks_per_cu);

struct moe_mk_plan_s {
    mk::Shape s;
    int sched;
    int device;
    int cus;
    int wg_per_cu;
    int grid;
    long long watchdog;
    int debug;
    // cache of the last workspace size -> capacity lookup
    size_t cached_bytes;
    int64_t cached_cap;
};

namespace {

constexpr long long kDefaultWatchdog = 200000000LL;  // 2 s at the 100 MHz real-time clock

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool plan_ok(moe_mk_plan_t p) { return p != nullptr && p->s.E > 0; }

size_t bytes_for(const mk::Shape &s, int64_t B) {
    if (B < 1) B = 1;
    return mk::make_layout(s, B).total;
}

// Largest B whose requirement fits in ws_bytes (0 when even B = 1 does not fit).
int64_t capacity(moe_mk_plan_t p, size_t ws_bytes) {
    if (p->cached_bytes == ws_bytes) return p->cached_cap;
    int64_t lo = 0, hi = ((int64_t)1 << 31) / p->s.k;  // B*k < 2^31
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo + 1) / 2;
        if (bytes_for(p->s, mid) <= ws_bytes)
            lo = mid;
        else
            hi = mid - 1;
    }
    p->cached_bytes = ws_bytes;
    p->cached_cap = lo;
    return lo;
}

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
    if (sched != MOE_MK_SCHED_STATIC && sched != MOE_MK_SCHED_DYNAMIC) return MOE_MK_EINVAL;
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
        const int g = std::atoi(env);
        if (g > 0 && g < p->grid) p->grid = g;
    }
    p->watchdog = kDefaultWatchdog;
    p->debug = 0;
    p->cached_bytes = (size_t)-1;
    p->cached_cap = 0;
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

moe_mk_status_t moe_mk_forward(moe_mk_plan_t plan, const void *x, const float *Wr, const float *router_bias,
                               const void *W1, const void *W3, const void *W2, void *out, int64_t B, void *ws,
                               size_t ws_bytes, void *stream) {
    if (!plan_ok(plan)) return MOE_MK_EINVAL;
    const mk::Shape &s = plan->s;
    if (B < 0 || B * s.k >= ((int64_t)1 << 31)) return MOE_MK_EINVAL;
    if (B == 0) return MOE_MK_OK;
    if (!x || !Wr || !W1 || !W3 || !W2 || !out || !ws) return MOE_MK_EINVAL;
    if (!aligned16(x) || !aligned16(Wr) || !aligned16(W1) || !aligned16(W3) || !aligned16(W2) ||
        !aligned16(out) || !aligned16(ws))
        return MOE_MK_EINVAL;
    if (router_bias && ((uintptr_t)router_bias & 3u)) return MOE_MK_EINVAL;
    const int64_t cap = capacity(plan, ws_bytes);
    if (cap < B) return MOE_MK_EWORKSPACE;
    const mk::Layout L = mk::make_layout(s, cap);
    const mk::Counts c = mk::make_counts(s, B);
    const mk::Counts cc = mk::make_counts(s, cap);
    char *base = (char *)ws;

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
    P.sched = plan->sched;
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
    P.NB1 = tl.NB1;
    P.NB2 = tl.NB2;
    P.S = tl.S;
    P.BM = tl.BM;
    {  // after the tile configuration: the prefetch follows the gate/up tiles
        const mk::Prefetch pf = (plan->debug & MOE_MK_DEBUG_NO_PREFETCH) ? mk::Prefetch{0, 0}
                                                                           : mk::prefetch_plan(s, B, P.NB1, P.BM == mk::kWideBM);
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
    P.logits = (float *)(base + L.logits);
    P.topk_idx = (int *)(base + L.topk_idx);
    P.topk_w = (float *)(base + L.topk_w);
    P.tile_hist = (int *)(base + L.tile_hist);
    P.tile_off = (int *)(base + L.tile_off);
    P.hist = (int *)(base + L.hist);
    P.indptr = (int *)(base + L.indptr);
    P.mt_base = (int *)(base + L.mt_base);
    P.mt_expert = (int *)(base + L.mt_expert);
    P.mt_row0 = (int *)(base + L.mt_row0);
    P.mt_rows = (int *)(base + L.mt_rows);
    P.perm = (int *)(base + L.perm);
    P.inv = (int *)(base + L.inv);
    P.h = (uint16_t *)(base + L.h);
    P.y = (uint16_t *)(base + L.y);
    P.yp = (float *)(base + L.yp);
    P.qslots = (unsigned long long *)(base + L.qslots);
    P.red_ctr = (int *)(base + L.red_ctr);
    P.trace = (long long *)(base + L.trace);
    if (hipSetDevice(plan->device) != hipSuccess) return MOE_MK_EHIP;
    if (mk_launch(P, plan->grid, (hipStream_t)stream) != hipSuccess) return MOE_MK_EHIP;
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

moe_mk_status_t moe_mk_plan_set_debug(moe_mk_plan_t plan, int64_t watchdog_ticks, int32_t flags) {
    if (!plan_ok(plan) || watchdog_ticks < 0) return MOE_MK_EINVAL;
    plan->watchdog = watchdog_ticks ? watchdog_ticks : kDefaultWatchdog;
    plan->debug = flags;
    return MOE_MK_OK;
}

}  // extern "C"

#endif  // !__HIP_DEVICE_COMPILE__
