// mk_common.h -- constants, workspace layout and kernel parameters shared by the host
// library and the megakernel (both are compiled into the same shared library).
#pragma once

#include <stddef.h>
#include <stdint.h>

// Global (device) memory pointers: in device code they carry address space 1 so every
// access compiles to global_* instructions (flat accesses would also count against the
// LDS wait counter and stall the software pipeline).  Host code sees plain pointers.
#if defined(__HIP_DEVICE_COMPILE__)
#define MK_G __attribute__((address_space(1)))
#define MK_C __attribute__((address_space(4)))  // constant (kernel-argument) memory
#else
#define MK_G
#define MK_C
#endif

namespace mk {

constexpr int kWaves = 8;            // waves per persistent workgroup (one workgroup per CU)
constexpr int kThreads = 64 * kWaves;
constexpr int kTileTokens = 64;      // tokens per top-k / grouping tile (one lane per token)
constexpr int kRouteExperts = 16;    // experts per router task (4 at small batches: route_reb)
constexpr int kCombineTokens = 8;    // most tokens per combine task (see combine_tokens)
constexpr int kCombineCols = 4 * kThreads;  // model columns per combine task (4 per thread)
constexpr int kBM = 64;              // GroupGEMM rows per narrow tile (one expert's rows)
constexpr int kBN = 16 * kWaves;     // GroupGEMM columns per narrow tile (16 per wave)
constexpr int kHalfBN = kBN / 2;     // columns of a half-width narrow tile (smallest batches)
constexpr int kGridDefault = 256;    // persistent workgroups per forward (one per CU)
constexpr int kBK = 64;              // narrow GroupGEMM K step staged through LDS
constexpr int kMaxE = 256;
constexpr int kMaxK = 16;

// Control block: int32 words at the start of the workspace.  Words that many workgroups
// update or poll at once sit on cache lines of their own (32 words = 128 bytes apart).
enum CtlWord {
    CTL_EPOCH = 0,      // forward counter; tags queue slots and the published task totals
    CTL_EXIT = 1,       // workgroups that left the current forward
    CTL_ERR = 2,        // sticky error bits (MOE_MK_ERR_*)
    CTL_EV_TOPK = 5,    // event: all top-k tiles done (one consumer: the scan task)
    CTL_EV_SCAN = 6,    // event: scan done; rest value 1
    CTL_MAGIC = 8,      // set by workspace init
    CTL_MT_TOTAL = 9,   // number of (expert, row-tile) pairs, written by the scan task
    CTL_MW = 10,        // how many of them are wide row tiles, written by the scan task
    CTL_TOTAL64 = 12,   // int64 at words 12..13: (epoch << 32) | task count (dynamic mode)
    CTL_SCAN64 = 14,    // int64 at words 14..15: (epoch << 32) | (1 << 31 if any row tile is wide) | row
                        // tiles, stored by the scan after its tables (static mode: the GroupGEMM
                        // workgroups wait on this word, which gives the event and the layout at once)
    CTL_QHEAD = 32,     // dynamic queue: next ticket
    CTL_QTAIL = 64,     // dynamic queue: slots reserved by pushers
    CTL_PF = 96,        // weight prefetch: lines claimed (rest 0)
    CTL_CQ = 128,       // static schedule: combine tasks claimed (rest 0)
    CTL_EV_G1 = 160,    // event: (row tile, f range) gate/up groups still open (dynamic schedule; fires the combine pushes)
    CTL_DBG = 192,      // 8 per-kind task counters (accumulate across forwards)
    CTL_XQ = 256,       // static schedule: claim counter of XCD x's GroupGEMM list at 256 + 32x
    CTL_WORDS = 512
};

constexpr int32_t kMagic = 0x4d4f4531;  // "MOE1"

enum TaskKind { K_ROUTE = 0, K_TOPK = 1, K_SCAN = 2, K_GROUP = 3, K_GEMM1 = 4, K_GEMM2 = 5, K_COMBINE = 6 };

struct Shape {
    int E, k, d, f;
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tokens per combine task: eight at large batches with k <= 8 (twice the rows in flight per
// task, and half the tasks each paying a round trip for its indices), one for a batch of
// one routing tile (the combine is then two round trips of latency, run on as many
// workgroups as there are tokens), else four.
inline int combine_tokens(int64_t B, int k) { return B >= 1024 && k <= 8 ? 8 : B <= kTileTokens ? 1 : 4; }
static_assert(kTileTokens % kCombineTokens == 0, "a combine task's tokens lie in one routing tile");

// Router tokens per wave: one at small batches (more, shorter tasks), four at large ones
// (each expert-weight row read from LDS serves four tokens), eight once that still leaves
// two tasks per workgroup (each row read serves eight tokens: the reads, not the FMAs, had
// set a task's pace; needs E % 4 == 0 and d % 128 == 0).  A task covers kWaves waves;
// 512 tasks are two per workgroup on 256 CUs.
inline int route_tpw(int64_t B, int64_t E, int64_t d) {
    if (B <= 512) return 1;
    if (E % 4 == 0 && d % 128 == 0 && ceil_div(B, 8 * kWaves) * ceil_div(E, kRouteExperts) >= 512) return 8;
    return 4;
}

// Experts per router task: 16, or 4 when one token per wave and 16-expert blocks would
// give fewer than 64 tasks.  Every task streams its block's whole Wr slice (4*d bytes per
// expert), so at small batches a few CUs each read a large slice; blocks of 4 spread the
// same bytes over four times the tasks (needs E % 4 == 0 and d % 512 == 0).
inline int route_reb(int64_t B, int64_t E, int64_t d, int64_t tpw) {
    if (tpw == 1 && E % 4 == 0 && d % 512 == 0 && ceil_div(B, kWaves) * ceil_div(E, kRouteExperts) < 64) return 4;
    return kRouteExperts;
}

// K splits S of the down projection: at small batches with a long f, each down-projection
// tile covers f/S of the reduction (partial results summed in a fixed order by the last
// split to finish), so tiles are smaller and each split can start as soon as the gate/up
// tiles of its f range are done.  S > 1 only when B*k <= 1024 (bounds the partial
// buffers).  (Eight splits at f = 14336 were measured slower: twice the tiles, each with
// its own ring fill and partial write.)
inline int down_splits(const Shape &s, int64_t B) {
    const int64_t a = B * s.k;
    const int64_t nb1 = s.f / kBN;
    if (a <= 1024 && s.f >= 8192 && nb1 % 4 == 0) return 4;
    if (a <= 1024 && s.f >= 4096 && nb1 % 2 == 0) return 2;
    return 1;
}
constexpr int kMaxSplits = 4;
// The most splits any batch size takes for this shape (sizes the partial buffers).
inline int max_down_splits(const Shape &s) {
    const int64_t nb1 = s.f / kBN;
    if (s.f >= 8192 && nb1 % 4 == 0) return 4;
    if (s.f >= 4096 && nb1 % 2 == 0) return 2;
    return 1;
}

// GroupGEMM tiles.  Every expert's rows are cut into row tiles of one of two shapes, chosen
// per expert on the device from its row count once the histogram is known (the scan task):
//   narrow  kBM = 64 rows; gate/up tiles of kBN = 128 columns of each weight, down-projection
//           tiles of kBN columns, the down projection optionally split over f (S ranges);
//           when d allows, a down-projection tile takes two such column blocks (kWideBN
//           columns, two weight blocks against one staged h tile);
//   wide    kWideBM = 256 rows; gate/up tiles of kWideBN1 = 128 columns of each weight,
//           down-projection tiles of kWideBN = 256 columns, so that each staged byte serves
//           more multiply-adds.  An expert with wide row tiles puts a remainder of at most
//           kBM rows in one narrow row tile.
// Wide row tiles need S = 1 and d, f multiples of their widths.  By default they go to every
// expert with more than kBM rows: such an expert needs two or more narrow row tiles, each of
// which streams all of its weight tiles again, where wide row tiles stream them once per
// kWideBM rows (debug flags force narrow tiles, or a choice from the batch size alone).
constexpr int kWideMinRows = kBM + 1;
// The batch-size-only choice the debug flag reproduces: every expert wide when the batch
// averages at least this many rows per expert.
constexpr int kBatchRuleRows = 128;
constexpr int kWideBM = 256;
constexpr int kWideBN = 256;   // down-projection columns per wide tile
constexpr int kWideBN1 = 128;  // gate/up columns of each weight per wide tile
constexpr int kWideBK = 32;
static_assert(kWideBN1 == kBN, "gate/up tiles of both shapes span the same columns");
// Half-width narrow tiles.  When even half-width gate/up tiles of every row tile the batch can
// have fit in one round of the grid, and the batch's experts all take narrow row tiles (B*k <=
// kBM rows in all, so no expert reaches kWideMinRows), the narrow tiles span kHalfBN columns:
// twice as many tiles, each streaming half the weight bytes, so that twice as many compute
// units stream the few experts of a tiny batch.  Inside a half-width tile the eight waves take
// four 16-column blocks and two halves of every K step, and add the halves through LDS.
inline bool half_width(const Shape &s, int64_t B) {
    const int64_t a = B * s.k, rt = a < s.E ? a : s.E;  // most row tiles such a batch can have
    // (a half-width gate/up tile of a short reduction, under 256 KB of weights, is all fixed
    // cost: ring fill, epilogue, notify; halving it gains nothing)
    return a <= kBM && 2 * rt * (s.f / kBN) <= kGridDefault && (int64_t)s.d * kHalfBN * 4 >= (256 << 10);
}
// All-token gate/up (a batch of one routing tile in which most experts get tokens): gate/up
// tiles that start before the routing is known run over all B tokens instead of waiting for
// their expert's grouped rows, and keep the rows of the tokens that chose the expert once the
// routing is out; tiles that start later run over the grouped rows (or only notify, for an
// expert without tokens).  The extra multiply-adds cost nothing at these batch sizes (the tiles
// are bound by their weight bytes); the cost is the weight bytes of the early tiles whose expert
// ends up without tokens, so the mode is taken when an expert is idle with probability at most
// 1/4 under uniform routing ((1 - k/E)^B <= 1/4) and the tiles are full width.
inline bool all_token_gate_up(const Shape &s, int64_t B) {
    if (B < 1 || B > kTileTokens || half_width(s, B)) return false;
    double p = 1.0;
    for (int64_t i = 0; i < B; ++i) p *= 1.0 - (double)s.k / (double)s.E;
    return p <= 0.25;
}
struct Tiles {
    int BN;      // columns of a narrow tile: kBN, or kHalfBN (half_width)
    int NB1;     // gate/up tiles per row tile (f / BN; f / 128 for wide row tiles)
    int NB2;     // down-projection tiles per narrow row tile and f range (d / DC)
    int NB2w;    // down-projection tiles per wide row tile (d / 256)
    int DC;      // columns of a down-projection task in a forward without wide row tiles: 256
                 // (both 128-column halves in one two-weight tile) with full-width tiles, d a
                 // multiple of 256 and enough such tasks to fill a round of the grid, BN otherwise
    int S;       // f ranges of the down projection
    int wide_ok; // wide row tiles allowed in this forward
};
inline Tiles tile_config(const Shape &s, int64_t B) {
    Tiles t;
    t.BN = half_width(s, B) ? kHalfBN : kBN;
    t.NB1 = s.f / t.BN;
    t.S = down_splits(s, B);
    t.DC = t.BN == kBN && s.d % kWideBN == 0 ? kWideBN : t.BN;
    {
        // ... unless the forward's down-projection tasks of that width would not fill one round of
        // the grid (at most min(B*k, E) row tiles): then the more, narrower tasks finish sooner
        const int64_t rt = B * s.k < s.E ? B * s.k : s.E;
        if (t.DC == kWideBN && rt * (s.d / kWideBN) * t.S < kGridDefault) t.DC = t.BN;
    }
    t.NB2 = s.d / t.DC;
    t.NB2w = s.d / kWideBN;
    t.wide_ok = t.S == 1 && t.BN == kBN && s.d % kWideBN == 0 && s.f % kWideBN1 == 0;
    return t;
}

// Weight prefetch while a small batch is routed (static schedule).  Until the scan event
// fires (the whole routing phase), a workgroup with nothing to do reads the leading rows of
// the gate/up weight tiles that the first round of tasks will stream, so that those rows
// come from the Infinity Cache (256 MB) rather than HBM once the tiles run.  (The dynamic
// schedule does not prefetch: a workgroup waiting on its queue slot between prefetch chunks
// started its task later, which cost more than the prefetch saved.)  Only for a batch
// of one routing tile with narrow tiles, where each expert has at most one row tile and
// the first round of tasks is known from the shapes (the gate/up tiles in task order, if
// every expert has rows), and only when B*k >= E, so that most experts do.
constexpr int64_t kPrefetchBytes = 96ll << 20;
struct Prefetch {
    int nt, lines;
};
inline Prefetch prefetch_plan(const Shape &s, int64_t B, int nb1, bool wide) {
    Prefetch p{0, 0};
    if (B < 1 || B > kTileTokens || wide || nb1 < 1 || B * s.k < s.E || half_width(s, B)) return p;
    const int64_t nt = (int64_t)s.E * nb1 < 256 ? (int64_t)s.E * nb1 : 256;
    int64_t depth = kPrefetchBytes / (nt * 4 * 128);  // rows of K: 4 lines per tile row (two of each weight)
    depth = depth < s.d ? depth : s.d;
    depth -= depth % 64;
    if (depth <= 0) return p;
    p.nt = (int)nt;
    p.lines = (int)(depth * nt * 4);
    return p;
}

// Task counts that depend on B only.
struct Counts {
    int64_t T;      // top-k / grouping tiles
    int64_t tpw;    // router tokens per wave
    int64_t nTG;    // router token groups
    int64_t reb;    // experts per router task
    int64_t nEB;    // router expert blocks
    int64_t nR;     // router tasks
    int64_t nC;     // combine tasks
    int64_t mt_cap; // upper bound of sum_e ceil(hist[e] / kBM)
    int64_t NB1, NB2;
    int64_t S;      // down-projection K splits
    int64_t q_cap;  // upper bound of the tasks pushed to the dynamic queue in one forward
    int64_t nR_max; // upper bound of the router tasks of any batch up to B
};

inline Counts make_counts(const Shape &s, int64_t B) {
    Counts c;
    c.T = ceil_div(B, kTileTokens);
    c.tpw = route_tpw(B, s.E, s.d);
    c.nTG = ceil_div(B, kWaves * c.tpw);
    c.reb = route_reb(B, s.E, s.d, c.tpw);
    c.nEB = ceil_div(s.E, c.reb);
    c.nR = c.nTG * c.nEB;
    c.nC = ceil_div(B, combine_tokens(B, s.k)) * ceil_div(s.d, kCombineCols);
    int64_t a = B * s.k;
    c.mt_cap = a / kBM + (a < s.E ? a : s.E) + 1;
    c.NB1 = s.f / kHalfBN;  // upper bounds over both narrow tile widths (sizes the queue
    c.NB2 = s.d / kHalfBN;  // and the split counters)
    c.S = down_splits(s, B);
    // combine tasks of any batch up to B (a task has at least one token), so that the queue,
    // and with it the workspace, grows with B
    const int64_t nC_max = B * ceil_div(s.d, kCombineCols);
    c.q_cap = 2 * c.T + 1 + c.mt_cap * c.NB1 + c.mt_cap * kMaxSplits * c.NB2 + nC_max + 128;  // + block padding
    c.nR_max = ceil_div(B, kWaves) * ceil_div(s.E, 4);
    return c;
}

// Byte offsets of every workspace array, for a workspace sized for B = cap tokens.
struct Layout {
    size_t ctl, ev_logit, ev_exp, ev_h, ev_d, logits, topk_idx, topk_w, tile_hist, hist, indptr,
        mt_base, mt_expert, mt_row0, mt_rows, perm, inv, amt, h, y, yp, red_ctr, qslots, trace, total;
    int64_t cap;
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline Layout make_layout(const Shape &s, int64_t cap) {
    Counts c = make_counts(s, cap);
    Layout L;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t r = o;
        o = align_up(o + bytes, 256);
        return r;
    };
    const int64_t A = cap * s.k;
    L.cap = cap;
    L.ctl = take(CTL_WORDS * 4);
    L.ev_logit = take((size_t)c.T * 4);
    L.ev_exp = take((size_t)s.E * 4);
    L.ev_h = take((size_t)c.mt_cap * kMaxSplits * 4);
    L.ev_d = take((size_t)c.mt_cap * ceil_div(s.d, kCombineCols) * 4);
    L.logits = take((size_t)cap * s.E * 4);
    L.topk_idx = take((size_t)A * 4);
    L.topk_w = take((size_t)A * 4);
    L.tile_hist = take((size_t)c.T * s.E * 4);
    L.hist = take((size_t)s.E * 4);
    L.indptr = take((size_t)(s.E + 1) * 4);
    L.mt_base = take((size_t)(s.E + 1) * 4);
    L.mt_expert = take((size_t)c.mt_cap * 4);
    L.mt_row0 = take((size_t)c.mt_cap * 4);
    L.mt_rows = take((size_t)c.mt_cap * 4);
    L.perm = take((size_t)A * 4);
    L.inv = take((size_t)A * 4);
    L.amt = take((size_t)A * 4);
    L.h = take((size_t)A * s.f * 2);
    L.y = take((size_t)A * s.d * 2);
    // yp holds S fp32 partial results of B*k rows each; S > 1 only when B*k <= 1024, and
    // never for a shape whose f is too short to split
    const int smax = max_down_splits(s);
    L.yp = take(smax > 1 ? (size_t)smax * (A < 1024 ? A : 1024) * s.d * 4 : 0);
    L.red_ctr = take((size_t)c.mt_cap * c.NB2 * 4);
    L.qslots = take((size_t)c.q_cap * 8);
    L.trace = take((size_t)(c.q_cap + c.nR_max) * 8 * 8);
    L.total = o;
    return L;
}

// Kernel arguments (passed by value).
struct Params {
    const MK_G uint16_t *x;
    const MK_G float *Wr;
    const MK_G float *bias;
    const MK_G uint16_t *W1, *W3, *W2;
    MK_G uint16_t *out;
    int B, E, k, d, f;
    int sched;       // 0 static, 1 dynamic
    int debug;       // MOE_MK_DEBUG_* bits
    int nR, nTG, nEB, T, nC, tpw;
    int BN, NB1, NB2, NB2w, S, wide_ok, DC;  // see Tiles
    int wide_min;    // an expert takes wide row tiles when it has at least this many rows (> kTileTokens)
    int reb;         // experts per router task (4 or 16)
    int CT;          // tokens per combine task
    int pf_nt, pf_lines;  // weight prefetch during routing: first gate/up tiles covered, 128-byte lines
    int q_cap, mt_cap;
    long long watchdog;  // real-time ticks (100 MHz)
    MK_G int *ctl, *ev_logit, *ev_exp, *ev_h;
    // ev_d[mt * nch + c]: down-projection tiles of row tile mt in column chunk c (kCombineCols
    // columns, the span of one combine task) not yet written; the combine tasks wait on the
    // events of the row tiles their tokens' rows sit in (rest 0)
    MK_G int *ev_d;
    int nch;
    MK_G float *logits;
    MK_G int *topk_idx;
    MK_G float *topk_w;
    MK_G int *tile_hist, *hist, *indptr, *mt_base, *mt_expert, *mt_row0, *mt_rows, *perm, *inv;
    MK_G int *amt;  // row tile of each assignment b*k+i (written by the grouping)
    MK_G uint16_t *h;
    MK_G uint16_t *y;   // down-projection output, bf16 [B*k, d] in grouped row order
    MK_G float *yp;     // fp32 partials of the split down projection
    MK_G unsigned long long *qslots;
    MK_G int *red_ctr;      // per down-projection tile: splits finished (rest 0)
    MK_G long long *trace;  // 8 int64 per task when tracing is on
    // Used by the allocation-free entry point: the error bits of the forward are stored at
    // *err_out (0 when none; NULL: not reported), and with heal set the last workgroup out
    // puts the control block and the event counters back to their rest state even after a
    // device error (clearing the error word), so the next forward starts clean.
    MK_G int *err_out;
    int heal;
    // Set for the phase-per-kernel pipeline (the unfused baseline): kernel boundaries order
    // the phases, so the scan arms no events and the workspace stays at its rest state.
    int unfused;
    // All-token gate/up (all_token_gate_up): row tile e is expert e's rows (possibly none); a
    // gate/up tile that starts before the routing is known runs over every token and keeps its
    // expert's grouped rows at the end; in the dynamic schedule the top-k task and the gate/up
    // tiles are handed out without a push.
    int dense;
    int nImp;  // dynamic schedule: tickets handed out without a queue slot (routers, and with dense the top-k
               // task and the gate/up tiles)
};

// The static scratch of the allocation-free entry point (one per GPU).
constexpr size_t kScratchBytes = (size_t)64 << 20;

}  // namespace mk
