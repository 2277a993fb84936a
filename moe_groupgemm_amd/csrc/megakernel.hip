// megakernel.hip -- one persistent HIP kernel that runs a whole top-k MoE layer.
//
// Design ("Event Tensor: A Unified Abstraction for Compiling Dynamic Megakernel",
// MLSys 2026, section "Core method"): the layer is a graph of tasks whose dependencies
// are event counters in device memory.  notify = atomic decrement; wait = spin until the
// counter is zero.  Two schedulers run the same graph:
//   static  -- workgroup w runs the tasks whose global index g satisfies g = w (mod G), in
//              increasing g, spin-waiting on events (phases are numbered in topological
//              order, so the smallest unfinished task can always run: no deadlock with a
//              co-resident grid);
//   dynamic -- the router tasks are implicitly queued; every other task is pushed onto a
//              shared queue by the task whose notification brings its event to zero
//              ("data-dependent task triggering"), and idle workgroups pop from it.
// The batch size B is a kernel argument: every count after the routing stage (histogram,
// exp_indptr, tiles per expert) is derived on the device, so one compiled kernel serves
// every B (section "Core method", symbolic shapes).
//
// Task kinds and their events:
//   ROUTE(tg,eb)  fp32 router logits for 16 tokens x 16 experts  -> ev_logit[tile]
//   TOPK(t)       top-k + softmax + tile histogram, 64 tokens    -> ev_topk
//   SCAN          hist, exp_indptr, per-tile offsets, row tiles; arms ev_exp/ev_h/ev_y -> ev_scan
//   GROUP(t)      stable ranks, perm/inv, gather of token rows    -> ev_exp[e] -= rows of e
//   GEMM1(mt,n)   gate/up GroupGEMM tile + SwiGLU -> h            -> ev_h[mt]
//   GEMM2(mt,n)   down GroupGEMM tile -> y                        -> ev_y
//   COMBINE(c)    out[b] = sum_i w[b,i] y[inv[b,i]] for 16 tokens
#include <hip/hip_runtime.h>

#include "mk_common.h"
#include "mk_device.h"

namespace mk {

// ------------------------------------------------------------------------------ LDS
struct GemmSmem {
    uint16_t A[2][kBM * kBK];
    uint16_t B0[2][kBN * kBK];
    uint16_t B1[2][kBN * kBK];
};
struct TopkSmem {
    int hist[kMaxE];
};
struct ScanSmem {
    int part[8];
};
struct GroupSmem {
    unsigned long long mask[kMaxE];
    int rowmap[kTileTokens * kMaxK];
    int fired[kMaxE];
    int nfired;
};
struct Smem {
    union {
        GemmSmem g;
        TopkSmem t;
        ScanSmem s;
        GroupSmem gr;
    } u;
    int bcast[4];
    int epoch;
};

// The workgroup's LDS, shared by every task kind (file scope, so out-of-line task bodies
// still address it as LDS).
__shared__ Smem g_sm;

// Phase bases of the global task index g.
struct Bases {
    int K, S, G, M1, M2, C, total;
    bool known;  // M2/C/total are known once the scan has run
};

__device__ __forceinline__ Bases initial_bases(const MK_C Params &P) {
    Bases b;
    b.K = P.nR;
    b.S = b.K + P.T;
    b.G = b.S + 1;
    b.M1 = b.G + P.T;
    b.M2 = b.C = b.total = 0x7fffffff;
    b.known = false;
    return b;
}

__device__ __forceinline__ void complete_bases(const MK_C Params &P, Bases &b, int mt_total) {
    b.M2 = b.M1 + mt_total * P.NB1;
    b.C = b.M2 + mt_total * P.NB2;
    b.total = b.C + P.nC;
    b.known = true;
}

// ------------------------------------------------------------------------------ event helpers (workgroup level)

// Thread 0 waits for *ctr == 0 and acquires (the acquire also invalidates this CU's
// vector L1, which every wave of the group reads through); the barrier then releases the
// group.  Returns false on error/watchdog.
__device__ __forceinline__ bool wg_wait_zero(const MK_C Params &P, const MK_G int *ctr) {
    if (threadIdx.x == 0) {
        const bool ok = spin_until(ctr, 0, P.ctl, P.watchdog);
        fence_acquire();
        g_sm.bcast[0] = ok ? 1 : 0;
    }
    __syncthreads();
    const bool ok = g_sm.bcast[0] != 0;
    __syncthreads();
    return ok;
}

// Every wave waits for its own global stores to complete, then the group synchronises;
// after this, one agent-scope release by a single thread publishes all of them.
__device__ __forceinline__ void wg_stores_done() {
    wave_drain_vm();
    __syncthreads();
}

// Push the contiguous task range [g0, g0 + cnt) onto the dynamic queue (all threads call,
// after wg_stores_done() or another point where the data the tasks read is complete).
__device__ __forceinline__ void wg_push_range(const MK_C Params &P, int g0, int cnt) {
    if (cnt <= 0) return;
    if (threadIdx.x == 0) {
        fence_release();
        g_sm.bcast[1] = add_relaxed(P.ctl + CTL_QTAIL, cnt);
    }
    __syncthreads();
    const int s0 = g_sm.bcast[1];
    __syncthreads();
    if (s0 + cnt > P.q_cap) {
        if (threadIdx.x == 0) set_error(P.ctl, 4 /* MOE_MK_ERR_QUEUE */);
        return;
    }
    const unsigned long long tag = (unsigned long long)(uint32_t)g_sm.epoch << 32;
    for (int i = threadIdx.x; i < cnt; i += kThreads)
        st_relaxed64(P.qslots + s0 + i, tag | (uint32_t)(g0 + i));
}

// Notify one counter: the group's stores complete, thread 0 adds delta (negative =
// decrement) with acquire-release ordering.  Returns (to every thread) whether this
// notification brought the counter to zero, i.e. fired the event.
__device__ __forceinline__ bool wg_notify(const MK_C Params &P, MK_G int *ctr, int delta) {
    wg_stores_done();
    if (threadIdx.x == 0) {
        const int old = add_acq_rel(ctr, delta);
        g_sm.bcast[2] = (old + delta == 0) ? 1 : 0;
    }
    __syncthreads();
    const bool fired = g_sm.bcast[2] != 0;
    __syncthreads();
    return fired;
}

// ------------------------------------------------------------------------------ ROUTE
// logit[b,e] = sum_j x[b,j] Wr[j,e] (+ bias[e]) in the fixed fp32 order: lane l of the
// wave accumulates j = l, l+64, ... with fma (one chain per lane), then the 64 chains are
// combined by a butterfly that pairs lanes l and l^32, then l^16, ... (the halves fold),
// which every lane evaluates in the same association; the bias is added last.

template <int N>
__device__ __forceinline__ void reduce_scatter(float (&v)[64], int lane) {
    if constexpr (N >= 2) {
        constexpr int H = N / 2;
        const bool up = (lane & H) != 0;
#pragma unroll
        for (int i = 0; i < H; ++i) {
            const float send = up ? v[i] : v[i + H];
            const float keep = up ? v[i + H] : v[i];
            v[i] = keep + shfl_xor_f(send, H);
        }
        reduce_scatter<H>(v, lane);
    }
}

__device__ __attribute__((noinline)) void task_route(const MK_C Params &P, int tg, int eb) {
    const int lane = lane_id(), w = wave_id();
    const int b0 = tg * kRouteTokens + w * 4;
    const int e0 = eb * kRouteExperts;
    float acc[4][16];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;

    bool tv[4];
    const MK_G uint16_t *xp[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        tv[t] = (b0 + t) < P.B;
        xp[t] = P.x + (size_t)(tv[t] ? b0 + t : 0) * P.d + lane;
    }
    const bool vec = (P.E & 3) == 0;
    bool ev[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) ev[q] = (e0 + 4 * q) < P.E;
    const MK_G float *wp = P.Wr + (size_t)lane * P.E + e0;
    const size_t wstep = (size_t)64 * P.E;
    const int nst = P.d / 64;
#pragma unroll 4
    for (int s = 0; s < nst; ++s) {
        float xv[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) xv[t] = tv[t] ? bf16_to_f32(xp[t][(size_t)s * 64]) : 0.0f;
        float wr[16];
        if (vec) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f32x4 v = {0.f, 0.f, 0.f, 0.f};
                if (ev[q]) v = *(const MK_G f32x4 *)(wp + 4 * q);
                wr[4 * q + 0] = v[0];
                wr[4 * q + 1] = v[1];
                wr[4 * q + 2] = v[2];
                wr[4 * q + 3] = v[3];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) wr[e] = (e0 + e) < P.E ? wp[e] : 0.0f;
        }
        wp += wstep;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[t][e] = fmaf(xv[t], wr[e], acc[t][e]);
    }
    float v[64];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) v[t * 16 + e] = acc[t][e];
    reduce_scatter<64>(v, lane);
    // lane L now holds the full sum of value L = (token L/16, expert L%16)
    const int b = b0 + (lane >> 4), e = e0 + (lane & 15);
    if (b < P.B && e < P.E) {
        const float bias = P.bias ? P.bias[e] : 0.0f;
        const float lg = v[0] + bias;
        if (!__builtin_isfinite(lg)) set_error(P.ctl, 2 /* MOE_MK_ERR_NONFINITE */);
        P.logits[(size_t)b * P.E + e] = lg;
    }
}

// ------------------------------------------------------------------------------ TOPK
// For each token: the k largest logits (ties to the lower expert index; -0 equals +0),
// then softmax over them in fp32.  Keys are (order-preserving logit bits, ~expert) so a
// wave-wide max picks the largest logit and, among equals, the smallest expert.
__device__ __attribute__((noinline)) void task_topk(const MK_C Params &P, int t) {
    int *sh = g_sm.u.t.hist;
    for (int i = threadIdx.x; i < P.E; i += kThreads) sh[i] = 0;
    __syncthreads();
    const int lane = lane_id(), w = wave_id();
    for (int q = w; q < kTileTokens; q += 4) {
        const int b = t * kTileTokens + q;
        if (b >= P.B) break;
        const MK_G float *lg = P.logits + (size_t)b * P.E;
        unsigned long long key[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int e = lane + 64 * c;
            key[c] = 0ull;
            if (e < P.E) {
                const float l = lg[e] + 0.0f;  // folds -0 onto +0
                key[c] = ((unsigned long long)float_key(l) << 32) | (0xffffffffu - (uint32_t)e);
            }
        }
        int sel_e[kMaxK];
        float sel_l[kMaxK];
#pragma unroll
        for (int s = 0; s < kMaxK; ++s) {
            sel_e[s] = 0;
            sel_l[s] = 0.0f;
            if (s < P.k) {
                unsigned long long best = key[0];
#pragma unroll
                for (int c = 1; c < 4; ++c) best = key[c] > best ? key[c] : best;
                best = wave_max_u64(best);
                const int eb = (int)(0xffffffffu - (uint32_t)best);
                if ((eb & 63) == lane) {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if ((eb >> 6) == c) key[c] = 0ull;
                }
                sel_e[s] = eb;
                sel_l[s] = key_float((uint32_t)(best >> 32));
            }
        }
        const float m = sel_l[0];
        float ex[kMaxK];
        float sum = 0.0f;
#pragma unroll
        for (int s = 0; s < kMaxK; ++s) {
            ex[s] = 0.0f;
            if (s < P.k) {
                ex[s] = expf(sel_l[s] - m);
                sum += ex[s];
            }
        }
        int my_e = 0;
        float my_x = 0.0f;
#pragma unroll
        for (int s = 0; s < kMaxK; ++s)
            if (s == lane) {
                my_e = sel_e[s];
                my_x = ex[s];
            }
        if (lane < P.k) {
            P.topk_idx[(size_t)b * P.k + lane] = my_e;
            P.topk_w[(size_t)b * P.k + lane] = my_x / sum;
            atomicAdd(&sh[my_e], 1);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < P.E; i += kThreads) P.tile_hist[(size_t)t * P.E + i] = sh[i];
}

// ------------------------------------------------------------------------------ SCAN
__device__ __forceinline__ int block_excl_scan(int v, int *part, int *total) {
    const int lane = lane_id(), w = wave_id();
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) part[w] = x;
    __syncthreads();
    int pre = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) {
        pre += (i < w) ? part[i] : 0;
        tot += part[i];
    }
    __syncthreads();
    *total = tot;
    return pre + x - v;
}

// hist[e] = sum_t tile_hist[t,e]; exp_indptr = exclusive prefix sum; tile_off[t,e] =
// exp_indptr[e] + rows of e in tiles before t; row tiles of kBM rows per expert; arms
// ev_exp[e] with hist[e], ev_h[mt] with the gate/up tiles of each row tile, and ev_y with
// the number of down-projection tiles ("Core method": the prefix sum decides how many
// GroupGEMM tiles each expert triggers).  Returns the number of row tiles.
__device__ __attribute__((noinline)) int task_scan(const MK_C Params &P) {
    const int e = threadIdx.x;
    const int E = P.E;
    int h = 0;
    if (e < E)
        for (int t = 0; t < P.T; ++t) h += P.tile_hist[(size_t)t * E + e];
    const int mt = (h + kBM - 1) / kBM;
    int total_h, total_mt;
    const int off = block_excl_scan(h, g_sm.u.s.part, &total_h);
    const int mbase = block_excl_scan(mt, g_sm.u.s.part, &total_mt);
    if (e < E) {
        P.hist[e] = h;
        P.indptr[e] = off;
        P.mt_base[e] = mbase;
        int run = off;
        for (int t = 0; t < P.T; ++t) {
            P.tile_off[(size_t)t * E + e] = run;
            run += P.tile_hist[(size_t)t * E + e];
        }
        for (int m = 0; m < mt; ++m) {
            const int i = mbase + m;
            P.mt_expert[i] = e;
            P.mt_row0[i] = off + m * kBM;
            P.mt_rows[i] = min(kBM, h - m * kBM);
            add_relaxed(P.ev_h + i, P.NB1);
        }
        if (h) add_relaxed(P.ev_exp + e, h);
    }
    if (e == 0) {
        P.indptr[E] = total_h;
        P.mt_base[E] = total_mt;
        st_relaxed(P.ctl + CTL_MT_TOTAL, total_mt);
        add_relaxed(P.ctl + CTL_EV_Y, total_mt * P.NB2);
    }
    return total_mt;
}

// ------------------------------------------------------------------------------ GROUP
// Stable grouping of one 64-token tile: rank of (b, i) among the tile's rows of expert e
// is the number of earlier tokens of the tile routed to e (a token uses an expert at most
// once), read off a 64-bit token mask per expert.  Row p = tile_off[t,e] + rank;
// perm[p] = b*k+i, inv[b*k+i] = p, and the token's row of x is copied to xg[p].
__device__ __attribute__((noinline)) void task_group(const MK_C Params &P, int t) {
    GroupSmem &g = g_sm.u.gr;
    const int E = P.E, k = P.k;
    for (int i = threadIdx.x; i < E; i += kThreads) g.mask[i] = 0ull;
    __syncthreads();
    const int lane = lane_id(), w = wave_id();
    const int ntok = min(kTileTokens, P.B - t * kTileTokens);
    const int b = t * kTileTokens + lane;
    for (int i = w; i < k; i += 4)
        if (lane < ntok) atomicOr(&g.mask[P.topk_idx[(size_t)b * k + i]], 1ull << lane);
    __syncthreads();
    for (int i = w; i < k; i += 4) {
        if (lane < ntok) {
            const int a = b * k + i;
            const int e = P.topk_idx[a];
            const int rank = __popcll(g.mask[e] & ((1ull << lane) - 1ull));
            const int p = P.tile_off[(size_t)t * E + e] + rank;
            P.perm[p] = a;
            P.inv[a] = p;
            g.rowmap[lane * k + i] = p;
        }
    }
    __syncthreads();
    const int cpr = P.d / 8;  // 16-byte chunks per row
    const int total = ntok * k * cpr;
    for (int idx = threadIdx.x; idx < total; idx += kThreads) {
        const int q = idx / cpr, c = idx - q * cpr;
        const int tok = t * kTileTokens + q / k;
        const u32x4 v = *((const MK_G u32x4 *)(P.x + (size_t)tok * P.d) + c);
        *((MK_G u32x4 *)(P.xg + (size_t)g.rowmap[q] * P.d) + c) = v;
    }
}

// ------------------------------------------------------------------------------ GroupGEMM tiles
// C[rows, 64 cols] = A[rows, K] * B[K, 64 cols] on v_mfma_f32_16x16x32_bf16 with fp32
// accumulation.  A is K-contiguous (grouped token rows); B is a weight slice with N
// contiguous ([K][ldb] row-major).  Tiles of kBK = 64 along K are staged through LDS in
// two buffers while the next two stages are in flight in registers.  In LDS both tiles
// are stored K-contiguous per row (A: per token row, B: per output column; B is
// transposed in registers while being written), in 16-byte chunks XOR-swizzled by row
// so fragment reads and transposing writes are free of bank conflicts.  Wave w owns
// output columns [16w, 16w+16); 16-row blocks beyond the tile's rows are skipped.

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

template <bool DUAL>
struct GemmRegs {
    u32x4 a[2];
    u32x4 b0[2];
    u32x4 b1[DUAL ? 2 : 1];
};

struct GemmArgs {
    const MK_G uint16_t *A;
    int lda, nrows;
    const MK_G uint16_t *B0, *B1;
    int ldb, K;
};

template <bool DUAL>
__device__ __forceinline__ void gemm_load(GemmRegs<DUAL> &R, const GemmArgs &g, int k0) {
    const int tid = threadIdx.x;
    const int ar = tid >> 3, ac = tid & 7;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int r = ar + 32 * hh;
        u32x4 z = {0u, 0u, 0u, 0u};
        if (r < g.nrows) z = *(const MK_G u32x4 *)(g.A + (size_t)r * g.lda + k0 + ac * 8);
        R.a[hh] = z;
    }
    const int kp = tid >> 3, c = tid & 7;
    const MK_G uint16_t *p0 = g.B0 + (size_t)(k0 + 2 * kp) * g.ldb + c * 8;
    R.b0[0] = *(const MK_G u32x4 *)p0;
    R.b0[1] = *(const MK_G u32x4 *)(p0 + g.ldb);
    if constexpr (DUAL) {
        const MK_G uint16_t *p1 = g.B1 + (size_t)(k0 + 2 * kp) * g.ldb + c * 8;
        R.b1[0] = *(const MK_G u32x4 *)p1;
        R.b1[1] = *(const MK_G u32x4 *)(p1 + g.ldb);
    }
}

__device__ __forceinline__ void store_b_transposed(const u32x4 &r0, const u32x4 &r1, uint16_t *sB) {
    const int tid = threadIdx.x;
    const int kp = tid >> 3, c = tid & 7;
    const int kc = kp >> 2, kw = (kp & 3) * 2;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const uint32_t lo = r0[q >> 1], hi = r1[q >> 1];
        const uint32_t v = (q & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        const int n = 8 * c + q;
        *(uint32_t *)(sB + n * kBK + ((kc ^ swz(n)) * 8) + kw) = v;
    }
}

template <bool DUAL>
__device__ __forceinline__ void gemm_store_lds(const GemmRegs<DUAL> &R, uint16_t *sA, uint16_t *sB0, uint16_t *sB1) {
    const int tid = threadIdx.x;
    const int ar = tid >> 3, ac = tid & 7;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int r = ar + 32 * hh;
        *(u32x4 *)(sA + r * kBK + ((ac ^ swz(r)) * 8)) = R.a[hh];
    }
    store_b_transposed(R.b0[0], R.b0[1], sB0);
    if constexpr (DUAL) store_b_transposed(R.b1[0], R.b1[1], sB1);
}

template <bool DUAL>
__device__ __forceinline__ void gemm_compute(const uint16_t *sA, const uint16_t *sB0, const uint16_t *sB1, int nrb,
                                             f32x4 (&acc0)[4], f32x4 (&acc1)[4]) {
    const int lane = lane_id(), w = wave_id();
    const int g = lane >> 4, j = lane & 15;
    const int n = 16 * w + j;
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
        const int ch = ks * 4 + g;
        const u32x4 b0 = *(const u32x4 *)(sB0 + n * kBK + ((ch ^ swz(n)) * 8));
        u32x4 b1 = b0;
        if constexpr (DUAL) b1 = *(const u32x4 *)(sB1 + n * kBK + ((ch ^ swz(n)) * 8));
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            if (rb < nrb) {
                const int r = 16 * rb + j;
                const u32x4 a = *(const u32x4 *)(sA + r * kBK + ((ch ^ swz(r)) * 8));
                acc0[rb] = mfma_bf16_16x16x32(a, b0, acc0[rb]);
                if constexpr (DUAL) acc1[rb] = mfma_bf16_16x16x32(a, b1, acc1[rb]);
            }
        }
    }
}

// PF register stages are in flight while LDS buffer (s & 1) holds stage s; stage s sits
// in register set s % PF until it is written to LDS one step before its use.
template <bool DUAL, int PF>
__device__ __forceinline__ void gemm_tile(const GemmArgs &ga, f32x4 (&acc0)[4], f32x4 (&acc1)[4], GemmSmem &s) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        acc0[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc1[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int nrb = (ga.nrows + 15) / 16;
    const int nk = ga.K / kBK;
    GemmRegs<DUAL> R[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (p < nk) gemm_load<DUAL>(R[p], ga, p * kBK);
    gemm_store_lds<DUAL>(R[0], s.A[0], s.B0[0], s.B1[0]);
    if (PF < nk) gemm_load<DUAL>(R[0], ga, PF * kBK);
    __syncthreads();
    for (int kk = 0; kk < nk; kk += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int st = kk + u;
            if (st < nk) {
                const int buf = st & 1;
                gemm_compute<DUAL>(s.A[buf], s.B0[buf], s.B1[buf], nrb, acc0, acc1);
                if (st + 1 < nk) {
                    gemm_store_lds<DUAL>(R[(u + 1) % PF], s.A[buf ^ 1], s.B0[buf ^ 1], s.B1[buf ^ 1]);
                    if (st + 1 + PF < nk) gemm_load<DUAL>(R[(u + 1) % PF], ga, (st + 1 + PF) * kBK);
                }
                __syncthreads();
            }
        }
    }
}

constexpr int kPF = 4;  // register prefetch depth of the GroupGEMM tiles

// GEMM1 tile: h[rows, n0:n0+64] = bf16( silu(xg W1[e]) * (xg W3[e]) ) for one row tile.
__device__ __attribute__((noinline)) void task_gemm1(const MK_C Params &P, int e, int row0, int nrows, int n) {
    GemmArgs ga;
    ga.A = P.xg + (size_t)row0 * P.d;
    ga.lda = P.d;
    ga.nrows = nrows;
    ga.B0 = P.W1 + (size_t)e * P.d * P.f + (size_t)n * kBN;
    ga.B1 = P.W3 + (size_t)e * P.d * P.f + (size_t)n * kBN;
    ga.ldb = P.f;
    ga.K = P.d;
    f32x4 acc0[4], acc1[4];
    gemm_tile<true, kPF>(ga, acc0, acc1, g_sm.u.g);
    const int lane = lane_id(), w = wave_id();
    const int g = lane >> 4, j = lane & 15;
    const int col = n * kBN + 16 * w + j;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * rb + 4 * g + r;
            if (row < nrows) {
                const float gv = acc0[rb][r], uv = acc1[rb][r];
                const float hv = gv / (1.0f + __expf(-gv)) * uv;
                P.h[(size_t)(row0 + row) * P.f + col] = f32_to_bf16(hv);
            }
        }
    }
}

// GEMM2 tile: y[rows, n0:n0+64] = h[rows, :] W2[e][:, n0:n0+64] in fp32.
__device__ __attribute__((noinline)) void task_gemm2(const MK_C Params &P, int e, int row0, int nrows, int n) {
    GemmArgs ga;
    ga.A = P.h + (size_t)row0 * P.f;
    ga.lda = P.f;
    ga.nrows = nrows;
    ga.B0 = P.W2 + (size_t)e * P.f * P.d + (size_t)n * kBN;
    ga.B1 = ga.B0;
    ga.ldb = P.d;
    ga.K = P.f;
    f32x4 acc0[4], acc1[4];
    gemm_tile<false, kPF>(ga, acc0, acc1, g_sm.u.g);
    const int lane = lane_id(), w = wave_id();
    const int g = lane >> 4, j = lane & 15;
    const int col = n * kBN + 16 * w + j;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * rb + 4 * g + r;
            if (row < nrows) P.y[(size_t)(row0 + row) * P.d + col] = acc0[rb][r];
        }
    }
}

// ------------------------------------------------------------------------------ COMBINE
// out[b, :] = bf16( sum_{i<k} w[b,i] * y[inv[b*k+i], :] ), slot order, fp32.
__device__ __attribute__((noinline)) void task_combine(const MK_C Params &P, int c) {
    const int b_lo = c * kCombineTokens;
    const int b_hi = min(P.B, b_lo + kCombineTokens);
    const int nq = P.d / 4;
    for (int b = b_lo; b < b_hi; ++b) {
        for (int q = threadIdx.x; q < nq; q += kThreads) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int i = 0; i < P.k; ++i) {
                const int p = P.inv[(size_t)b * P.k + i];
                const float wgt = P.topk_w[(size_t)b * P.k + i];
                const f32x4 yv = *(const MK_G f32x4 *)(P.y + (size_t)p * P.d + 4 * q);
#pragma unroll
                for (int z = 0; z < 4; ++z) acc[z] = fmaf(wgt, yv[z], acc[z]);
            }
            const uint32_t lo = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
            MK_G uint32_t *o = (MK_G uint32_t *)(P.out + (size_t)b * P.d + 4 * q);
            o[0] = lo;
            o[1] = hi;
        }
    }
}

// ------------------------------------------------------------------------------ task dispatch
__device__ __forceinline__ int route_tasks_of_tile(const MK_C Params &P, int t) {
    const int g0 = t * (kTileTokens / kRouteTokens);
    const int g1 = min(g0 + kTileTokens / kRouteTokens, P.nTG);
    return (g1 - g0) * P.nEB;
}

__device__ __forceinline__ void count_task(const MK_C Params &P, int kind) {
    if (threadIdx.x == 0) add_relaxed(P.ctl + CTL_DBG + kind, 1);
}

// Debug trace (MOE_MK_DEBUG_TRACE): per task {g | kind << 32 | workgroup << 40, obtained,
// dependencies satisfied, finished} in real-time ticks.
__device__ __forceinline__ void trace_task(const MK_C Params &P, int g, int kind, unsigned long long t0,
                                           unsigned long long t1) {
    if ((P.debug & 2) && threadIdx.x == 0) {
        MK_G long long *e = P.trace + (size_t)g * 4;
        e[0] = (long long)g | ((long long)kind << 32) | ((long long)blockIdx.x << 40);
        e[1] = (long long)t0;
        e[2] = (long long)t1;
        e[3] = (long long)now_ticks();
    }
}

// Runs task g (obtained at time t0).  Returns false when the forward must be abandoned.
__device__ __forceinline__ bool run_task(const MK_C Params &P, int g, Bases &bs, unsigned long long t0) {
    const bool dyn = P.sched != 0;
    if (g < bs.K) {  // ---------------------------------------------------------- ROUTE
        const int tg = g / P.nEB, eb = g - tg * P.nEB;
        task_route(P, tg, eb);
        count_task(P, K_ROUTE);
        const int t = tg / (kTileTokens / kRouteTokens);
        int delta = -1;
        if (dyn && (tg % (kTileTokens / kRouteTokens)) == 0 && eb == 0) delta += route_tasks_of_tile(P, t);
        if (wg_notify(P, P.ev_logit + t, delta) && dyn) wg_push_range(P, bs.K + t, 1);
        trace_task(P, g, K_ROUTE, t0, t0);
        return true;
    }
    if (g < bs.S) {  // ---------------------------------------------------------- TOPK
        const int t = g - bs.K;
        if (!dyn) {
            if (threadIdx.x == 0) add_relaxed(P.ev_logit + t, route_tasks_of_tile(P, t));  // arm
            if (!wg_wait_zero(P, P.ev_logit + t)) return false;
        }
        const unsigned long long t1 = now_ticks();
        task_topk(P, t);
        count_task(P, K_TOPK);
        int delta = -1;
        if (dyn && t == 0) delta += P.T;
        if (wg_notify(P, P.ctl + CTL_EV_TOPK, delta) && dyn) wg_push_range(P, bs.S, 1);
        trace_task(P, g, K_TOPK, t0, t1);
        return true;
    }
    if (g == bs.S) {  // --------------------------------------------------------- SCAN
        if (!dyn) {
            if (threadIdx.x == 0) add_relaxed(P.ctl + CTL_EV_TOPK, P.T);  // arm
            if (!wg_wait_zero(P, P.ctl + CTL_EV_TOPK)) return false;
        }
        const unsigned long long t1 = now_ticks();
        const int mt_total = task_scan(P);
        count_task(P, K_SCAN);
        complete_bases(P, bs, mt_total);
        wg_notify(P, P.ctl + CTL_EV_SCAN, -1);
        if (dyn) {
            wg_push_range(P, bs.G, P.T);
            if (threadIdx.x == 0)
                st_relaxed64((MK_G unsigned long long *)(P.ctl + CTL_TOTAL64),
                             ((unsigned long long)(uint32_t)g_sm.epoch << 32) | (uint32_t)bs.total);
        }
        trace_task(P, g, K_SCAN, t0, t1);
        return true;
    }
    if (g < bs.M1) {  // --------------------------------------------------------- GROUP
        const int t = g - bs.G;
        if (!dyn && !wg_wait_zero(P, P.ctl + CTL_EV_SCAN)) return false;
        const unsigned long long t1 = now_ticks();
        task_group(P, t);
        count_task(P, K_GROUP);
        GroupSmem &gr = g_sm.u.gr;
        if (threadIdx.x == 0) gr.nfired = 0;
        wg_stores_done();
        int skip = -1;
        if ((P.debug & 1) && t == 0) {  // debug: drop the notification of the tile's first expert
            for (int e = 0; e < P.E; ++e)
                if (gr.mask[e]) {
                    skip = e;
                    break;
                }
        }
        for (int e = threadIdx.x; e < P.E; e += kThreads) {
            const int cnt = __popcll(gr.mask[e]);
            if (cnt && e != skip) {
                const int old = add_acq_rel(P.ev_exp + e, -cnt);
                if (dyn && old == cnt) gr.fired[atomicAdd(&gr.nfired, 1)] = e;
            }
        }
        __syncthreads();
        if (dyn) {
            const int nf = gr.nfired;
            for (int i = 0; i < nf; ++i) {
                const int e = gr.fired[i];
                const int m0 = P.mt_base[e], m1 = P.mt_base[e + 1];
                wg_push_range(P, bs.M1 + m0 * P.NB1, (m1 - m0) * P.NB1);
            }
        }
        trace_task(P, g, K_GROUP, t0, t1);
        return true;
    }
    if (!bs.known) complete_bases(P, bs, ld_relaxed(P.ctl + CTL_MT_TOTAL));
    if (g < bs.M2) {  // --------------------------------------------------------- GEMM1
        const int i = g - bs.M1;
        const int mt = i / P.NB1, n = i - mt * P.NB1;
        const int e = P.mt_expert[mt];
        if (!dyn && !wg_wait_zero(P, P.ev_exp + e)) return false;
        const unsigned long long t1 = now_ticks();
        task_gemm1(P, e, P.mt_row0[mt], P.mt_rows[mt], n);
        count_task(P, K_GEMM1);
        if (wg_notify(P, P.ev_h + mt, -1) && dyn) wg_push_range(P, bs.M2 + mt * P.NB2, P.NB2);
        trace_task(P, g, K_GEMM1, t0, t1);
        return true;
    }
    if (g < bs.C) {  // ---------------------------------------------------------- GEMM2
        const int i = g - bs.M2;
        const int mt = i / P.NB2, n = i - mt * P.NB2;
        if (!dyn && !wg_wait_zero(P, P.ev_h + mt)) return false;
        const unsigned long long t1 = now_ticks();
        task_gemm2(P, P.mt_expert[mt], P.mt_row0[mt], P.mt_rows[mt], n);
        count_task(P, K_GEMM2);
        if (wg_notify(P, P.ctl + CTL_EV_Y, -1) && dyn) wg_push_range(P, bs.C, P.nC);
        trace_task(P, g, K_GEMM2, t0, t1);
        return true;
    }
    {  // ------------------------------------------------------------------------ COMBINE
        const int c = g - bs.C;
        if (!dyn && !wg_wait_zero(P, P.ctl + CTL_EV_Y)) return false;
        const unsigned long long t1 = now_ticks();
        task_combine(P, c);
        count_task(P, K_COMBINE);
        __syncthreads();
        trace_task(P, g, K_COMBINE, t0, t1);
        return true;
    }
}

// Dynamic queue pop.  Returns a task index, -1 when the forward is complete, -2 on error.
__device__ __forceinline__ int wg_pop(const MK_C Params &P) {
    if (threadIdx.x == 0) {
        int g = -1;
        const int claim = add_relaxed(P.ctl + CTL_QHEAD, 1);
        if (claim < P.nR) {
            g = claim;
        } else {
            const int slot = claim - P.nR;
            const uint32_t ep = (uint32_t)g_sm.epoch;
            const unsigned long long t0 = now_ticks();
            for (unsigned it = 0;; ++it) {
                if (slot < P.q_cap) {
                    const unsigned long long v = ld_relaxed64(P.qslots + slot);
                    if ((uint32_t)(v >> 32) == ep) {
                        g = (int)(uint32_t)v;
                        break;
                    }
                }
                const unsigned long long tot = ld_relaxed64((const MK_G unsigned long long *)(P.ctl + CTL_TOTAL64));
                if ((uint32_t)(tot >> 32) == ep && claim >= (int)(uint32_t)tot) {
                    g = -1;
                    break;
                }
                if ((it & 31u) == 31u) {
                    if (ld_relaxed(P.ctl + CTL_ERR) != 0) {
                        g = -2;
                        break;
                    }
                    if ((long long)(now_ticks() - t0) > P.watchdog) {
                        set_error(P.ctl, 1);
                        g = -2;
                        break;
                    }
                }
                __builtin_amdgcn_s_sleep(1);
            }
            fence_acquire();
        }
        g_sm.bcast[3] = g;
    }
    __syncthreads();
    const int g = g_sm.bcast[3];
    __syncthreads();
    return g;
}

__global__ void __launch_bounds__(kThreads, 2) moe_megakernel(Params Parg) {
    // Parg is the first kernel argument, at offset 0 of the kernel-argument segment: read it
    // there in place rather than from a private copy.
    (void)Parg;
    const MK_C Params &P = *(const MK_C Params *)__builtin_amdgcn_kernarg_segment_ptr();
    if (threadIdx.x == 0) {
        g_sm.epoch = ld_relaxed(P.ctl + CTL_EPOCH);
        g_sm.bcast[0] = ld_relaxed(P.ctl + CTL_MAGIC) == kMagic;
    }
    __syncthreads();
    if (!g_sm.bcast[0]) {  // workspace never prepared: record it and touch nothing else
        if (threadIdx.x == 0) set_error(P.ctl, 8 /* MOE_MK_ERR_UNINIT */);
        return;
    }
    Bases bs = initial_bases(P);
    if (P.sched == 0) {
        for (int g = blockIdx.x;; g += gridDim.x) {
            if (g >= bs.M1 && !bs.known) {
                if (!wg_wait_zero(P, P.ctl + CTL_EV_SCAN)) break;
                complete_bases(P, bs, ld_relaxed(P.ctl + CTL_MT_TOTAL));
            }
            if (bs.known && g >= bs.total) break;
            if (!run_task(P, g, bs, now_ticks())) break;
        }
    } else {
        for (;;) {
            const unsigned long long t0 = now_ticks();
            const int g = wg_pop(P);
            if (g < 0) break;
            if (!run_task(P, g, bs, t0)) break;
        }
    }
    // Leave: the last workgroup out puts the control block back to its rest state.
    __syncthreads();
    if (threadIdx.x == 0) {
        fence_release();
        const int old = add_acq_rel(P.ctl + CTL_EXIT, 1);
        if (old == (int)gridDim.x - 1) {
            if (ld_relaxed(P.ctl + CTL_ERR) == 0) {
                st_relaxed(P.ctl + CTL_QHEAD, 0);
                st_relaxed(P.ctl + CTL_QTAIL, 0);
                st_relaxed(P.ctl + CTL_EV_SCAN, 1);
            }
            st_relaxed(P.ctl + CTL_EXIT, 0);
            st_release(P.ctl + CTL_EPOCH, g_sm.epoch + 1);
        }
    }
}

// Workspace preparation: zero everything, then set the rest values.
// (Kernel signatures use plain pointers: the host pass must mangle them identically.)
__global__ void moe_ws_init(uint32_t *ws_generic, size_t words) {
    MK_G uint32_t *ws = (MK_G uint32_t *)ws_generic;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += stride) ws[i] = 0u;
}
__global__ void moe_ws_init_ctl(int *ctl_generic) {
    MK_G int *ctl = (MK_G int *)ctl_generic;
    if (threadIdx.x == 0) {
        ctl[CTL_EPOCH] = 1;
        ctl[CTL_EV_SCAN] = 1;
        ctl[CTL_MAGIC] = kMagic;
    }
}

}  // namespace mk

// ------------------------------------------------------------------------------ launch glue
hipError_t mk_launch(const mk::Params &p, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(mk::moe_megakernel, dim3(grid), dim3(mk::kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t mk_ws_init(void *ws, size_t bytes, hipStream_t stream) {
    const size_t words = bytes / 4;
    int blocks = (int)((words + 255) / 256);
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(mk::moe_ws_init, dim3(blocks), dim3(256), 0, stream, (uint32_t *)ws, words);
    hipLaunchKernelGGL(mk::moe_ws_init_ctl, dim3(1), dim3(64), 0, stream, (int *)ws);
    return hipGetLastError();
}

hipError_t mk_occupancy(int *blocks_per_cu) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, mk::moe_megakernel, mk::kThreads, 0);
}
