// megakernel.hip -- one persistent HIP kernel that runs a whole top-k MoE layer.
//
// Design ("Event Tensor: A Unified Abstraction for Compiling Dynamic Megakernel",
// MLSys 2026, section "Core method"): the layer is a graph of tasks whose dependencies
// are event counters in device memory.  notify = atomic decrement; wait = spin until the
// counter is zero.  Two schedulers run the same graph:
//   static  -- the routing tasks go to workgroups round-robin (workgroup w runs g = w,
//              w + G, ...); the GroupGEMM tasks are partitioned over the 8 XCDs and each
//              XCD's workgroups take its list in order, then what the other XCDs have left;
//              the combine tasks come last from one shared counter; tasks spin-wait on their
//              events (every list is in topological order, so the smallest unfinished task
//              can always run: no deadlock with a co-resident grid);
//   dynamic -- the router tasks are implicitly queued; every other task is pushed onto a
//              shared queue by the task whose notification brings its event to zero
//              ("data-dependent task triggering"), and idle workgroups pop from it.
// The batch size B is a kernel argument: every count after the routing stage (histogram,
// exp_indptr, tiles per expert) is derived on the device, so one compiled kernel serves
// every B and every routing (section "Core method", symbolic shapes).  The scan chooses
// each expert's GroupGEMM tile shape from its row count (64-row narrow tiles, or 256-row
// wide tiles above 64 rows).  The task loop exists twice in the kernel: the wide tiles use
// nearly every register and are inlined into the copy that runs forwards with wide row
// tiles (called out of line, each tile saved and restored about 60 registers per wave
// through memory), and the other copy, which runs every task until a forward is known to
// have them, carries none of their code or register pressure (the narrow tiles are
// out-of-line functions that both copies call).
//
// Task kinds and their events:
//   ROUTE(tg,eb)  fp32 router logits, 8*tpw tokens x reb experts   -> ev_logit[tile]
//   TOPK(t)       top-k + softmax + tile histogram, 64 tokens    -> ev_topk
//   SCAN          hist, exp_indptr, row tiles and their shapes; arms ev_exp/ev_h/ev_d and
//                 re-arms ev_logit as the tiles' grouping events -> ev_scan, scan result word
//   GROUP(t)      stable ranks -> perm/inv/amt (GEMM1 gathers the rows) -> ev_exp[e] -= rows
//                 of e, ev_logit[t]
//   GEMM1(mt,n)   gate/up GroupGEMM tile + SwiGLU -> h            -> ev_h[mt,s] (s: n's f range)
//   GEMM2(mt,s,n) down GroupGEMM tile over f range s -> y         -> ev_d[mt, column chunk]
//   COMBINE(c)    out[b] = sum_i w[b,i] y[inv[b,i]] for 1, 4 or 8 tokens and 2048 columns,
//                 after its tokens' grouping and the row tiles its rows use
// In a batch of one routing tile where nearly every expert gets tokens (Params::dense), the
// row tiles are one per expert and known from the start; a GEMM1 tile that starts before the
// scan's result word is out runs over every token and keeps its expert's rows at the end, so
// the gate/up weights stream while the batch is routed, and the scan arms ev_h with atomic adds.
// Weight loads of experts that have a single row tile carry the non-temporal hint.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mk_common.h"
#include "mk_device.h"

#define MK_L __attribute__((address_space(3)))  // LDS pointers

namespace mk {

// ------------------------------------------------------------------------------ LDS
constexpr int kRingBytes = 144 * 1024;  // LDS ring of the GroupGEMM and router tiles
struct GemmSmem {
    uint16_t ring[kRingBytes / 2];
};
// Scratch of the single-tile routing tail, over the top-k staging area once top-k is done.
struct FusedWork {
    unsigned long long mask[kMaxE];  // tokens of the tile per expert
    int off[kMaxE];                  // exp_indptr[e]
    int mtb[kMaxE + 1];              // first row tile of each expert
    int poff[kMaxE], pnm[kMaxE];     // queue offset and row tiles of each fired expert
    int perm[kTileTokens * kMaxK];   // the batch's perm, inv and row tiles, written out contiguously
    int inv[kTileTokens * kMaxK];
    int amt[kTileTokens * kMaxK];
    int part[kWaves];
    int base;
};
struct TopkSmem {
    union {
        float lg[kTileTokens * kMaxE];  // a tile's logits, then the candidate lists
        FusedWork fw;
    };
    int hist[kMaxE];
    int tk[kTileTokens * kMaxK];        // the tile's selected experts, [token][slot]
    float tw[kTileTokens * kMaxK];      // and their weights
};
constexpr int kScanStage = 16384;  // ints of tile_hist staged per round
struct ScanSmem {
    int part[8];
    int ps[kThreads];      // partial sums, [thread group r][expert]
    int tiles[kScanStage];
};
struct GroupSmem {
    unsigned long long mask[kMaxE];
    int toff[kMaxE];  // the tile's row offsets: exp_indptr[e] + rows of e in earlier tiles
    int ps[kThreads];  // partial sums of the earlier tiles' rows, [thread group r][expert]
    int eoff[kMaxE], emt[kMaxE], erows[kMaxE];  // per expert: exp_indptr, first row tile, rows per row tile
    int poff[kMaxE], pm0[kMaxE], pnm[kMaxE];  // per expert: queue offset, first row tile, row tiles
    int part[kWaves];
    int base;
};
struct CombineSmem {
    int row[kCombineTokens * kMaxK];
    float w[kCombineTokens * kMaxK];
};
struct Smem {
    union {
        GemmSmem g;
        TopkSmem t;
        ScanSmem s;
        GroupSmem gr;
        CombineSmem c;
    } u;
    int bcast[4];
    int epoch;
    int total;  // the forward's task count once read (dynamic mode), else -1
};

// The workgroup's LDS, shared by every task kind (file scope, so out-of-line task bodies
// still address it as LDS).
__shared__ Smem g_sm;

// Layout of the global task index g (the static schedule walks it in order; dynamic
// pushes use the same indices):
//   [ROUTE][TOPK][SCAN][GROUP] then the GroupGEMM tiles by f range s (S ranges):
//   [G1(0)] [G1(1)] [G2(0)] [G1(2)] [G2(1)] ... [G1(S-1)] [G2(S-2)] [G2(S-1)] [COMBINE]
// where G1(s) holds the gate/up tiles whose columns fall in f range s (for every row
// tile, Q = NB1/S per row tile) and G2(s) the down-projection tiles reducing over f range
// s (N2 per row tile: NB2w tasks of kWideBN columns when the forward has a wide row tile,
// where a narrow row tile's task runs kWideBN / kBN narrow tiles; else NB2 of kBN).  Row
// tiles are numbered in expert order, so that an expert's tiles (a wide one and its thin
// remainder) sit side by side in every list and share the expert's weights in L2.  Each G2
// block comes one G1 block after the G1 block it consumes, so the two GEMMs overlap
// instead of running as two phases.
//
// GroupGEMM blocks start at multiples of 8 and are padded to multiples of 8 (padding
// positions are empty tasks).  Workgroups are dealt to the 8 XCDs round-robin, so in the
// static schedule position p of a block runs on XCD p % 8 (unless another XCD takes it once
// its own positions are done).  Static mode therefore maps
// the positions of XCD x, in order, to the tiles of row tiles [mt x / 8, mt (x+1) / 8) (row
// tile major; see xcd_blocks) when the forward has wide row tiles, so that the tiles sharing a
// row tile's activations or an expert's weight columns run together on the same L2, and both
// GEMMs of a row tile on one XCD.  Otherwise, and in dynamic mode (whose pushes follow the
// linear order), position p is linear tile p.
struct Bases {
    int K, S, G, M1, M1p, C, total;
    int mt;        // row tiles
    int q1, q2;    // tiles per G1(s) block and per G2(s) block
    int q1p, q2p;  // block sizes: q1, q2 rounded up to multiples of 8 (see complete_bases)
    int N2;        // down-projection tasks per row tile and f range
    bool wide;     // the forward has wide row tiles
    bool known;    // GroupGEMM layout known once the scan has run (all-token gate/up: from the start)
    bool routed;   // static schedule: this workgroup has seen the scan's result word
};

__device__ __forceinline__ int round8(int v) { return (v + 7) & ~7; }

__device__ __forceinline__ Bases initial_bases(const MK_C Params &P) {
    Bases b;
    b.K = P.nR;
    b.S = b.K + P.T;
    b.G = b.S + 1;
    b.M1 = b.G + P.T;
    b.M1p = round8(b.M1);
    b.C = b.total = 0x7fffffff;
    b.mt = b.q1 = b.q2 = b.q1p = b.q2p = b.N2 = 0;
    b.wide = false;
    b.known = false;
    b.routed = false;
    return b;
}

// mt_total row tiles, mw of them wide.  The counts are made visibly wave-uniform so that
// the layout lives in scalar registers: held in vector registers across the task body, it
// pushed the wide tiles' K loops into spills.
// In the static schedule with wide row tiles the blocks are dealt to the XCDs by whole row
// tiles (xcd_blocks): XCD x takes row tiles [mt x / 8, mt (x+1) / 8) in both blocks, each list
// padded to ceil(mt / 8) row tiles' worth, so that no row tile's gate/up tiles are split
// between two XCDs (a down-projection list that began with a row tile shared with the previous
// XCD's list waited for that list's last gate/up tiles).
__device__ __forceinline__ bool xcd_blocks(const MK_C Params &P, const Bases &b) { return P.sched == 0 && b.wide; }
__device__ __forceinline__ void complete_bases(const MK_C Params &P, Bases &b, int mt_total, int mw) {
    mt_total = uni(mt_total);
    b.mt = mt_total;
    b.wide = uni(mw) > 0;
    b.N2 = b.wide ? P.NB2w : P.NB2;
    b.q1 = mt_total * (P.NB1 / P.S);
    b.q2 = mt_total * b.N2;
    if (xcd_blocks(P, b)) {
        const int per = (mt_total + 7) >> 3;  // row tiles of the longest XCD list
        b.q1p = 8 * per * (P.NB1 / P.S);
        b.q2p = 8 * per * b.N2;
    } else {
        b.q1p = round8(b.q1);
        b.q2p = round8(b.q2);
    }
    b.C = b.M1p + P.S * (b.q1p + b.q2p);
    b.total = b.C + P.nC;
    b.known = true;
}

__device__ __forceinline__ int base_g1(const Bases &b, int s) {
    return s == 0 ? b.M1p : b.M1p + b.q1p + (s - 1) * (b.q1p + b.q2p);
}
__device__ __forceinline__ int base_g2(const Bases &b, int s, int S) {
    return s < S - 1 ? base_g1(b, s + 1) + b.q1p : b.M1p + S * b.q1p + (S - 1) * b.q2p;
}
// The layout as the scan task published it (row tiles and wide row tiles, one line).
__device__ __forceinline__ void complete_bases_from_ctl(const MK_C Params &P, Bases &b) {
    complete_bases(P, b, ld_relaxed(P.ctl + CTL_MT_TOTAL), ld_relaxed(P.ctl + CTL_MW));
}

// Decode a GroupGEMM task index: returns 1 for gate/up, 2 for down, 0 for a padding
// position; sets the f range s and the linear tile j inside its block.  xcd_map: the blocks
// are dealt to the XCDs by whole row tiles (xcd_blocks); Q: gate/up tiles per row tile and f
// range (a down-projection row tile has b.N2).
__device__ __forceinline__ int decode_gemm(const Bases &b, int S, bool xcd_map, int g, int &s, int &j, int Q) {
    int o = g - b.M1p, kind = 0, cnt = 0, size = 0;
    if (o < b.q1p) {
        s = 0;
        kind = 1;
    } else {
        o -= b.q1p;
        for (int r = 1; r < S && kind == 0; ++r) {
            if (o < b.q1p) {
                s = r;
                kind = 1;
            } else {
                o -= b.q1p;
                if (o < b.q2p) {
                    s = r - 1;
                    kind = 2;
                } else {
                    o -= b.q2p;
                }
            }
        }
        if (kind == 0) {
            s = S - 1;
            kind = 2;
        }
    }
    cnt = kind == 1 ? b.q1 : b.q2;
    size = kind == 1 ? b.q1p : b.q2p;
    (void)size;
    if (xcd_map) {  // position o runs on XCD o % 8: the (o / 8)-th tile of that XCD's row tiles
        const int per = kind == 1 ? Q : b.N2, x = o & 7;
        const int r0 = (b.mt * x) >> 3, r1 = (b.mt * (x + 1)) >> 3;
        const int i = o >> 3;
        j = r0 * per + i;
        return i < (r1 - r0) * per ? kind : 0;
    }
    j = o;
    return j < cnt ? kind : 0;
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

// Every wave waits for its own (agent-scope) stores to complete, then the group
// synchronises: after this, all of them are visible to every XCD.
__device__ __forceinline__ void wg_stores_done() {
    wave_drain_vm();
    __syncthreads();
}

// Make data other workgroups (or this one) published visible to this workgroup's loads:
// thread 0 acquires at agent scope (invalidating the CU's vector L1), then the group syncs.
__device__ __forceinline__ void wg_acquire() {
    if (threadIdx.x == 0) fence_acquire();
    __syncthreads();
}

// Push the contiguous task range [g0, g0 + cnt) onto the dynamic queue (all threads call;
// the data the pushed tasks read was published before the event that fired them).
__device__ __forceinline__ void wg_push_range(const MK_C Params &P, int g0, int cnt) {
    if (cnt <= 0) return;
    if (threadIdx.x == 0) g_sm.bcast[1] = add_relaxed(P.ctl + CTL_QTAIL, cnt);
    __syncthreads();
    const int s0 = g_sm.bcast[1];
    __syncthreads();
    if (s0 + cnt > P.q_cap) {
        if (threadIdx.x == 0) set_error(P.ctl, 4 /* MOE_MK_ERR_QUEUE */);
        return;
    }
    const unsigned long long tag = (unsigned long long)(uint32_t)g_sm.epoch << 32;
    for (int i = threadIdx.x; i < cnt; i += kThreads) st_relaxed64(P.qslots + s0 + i, tag | (uint32_t)(g0 + i));
}

// The same from one thread (the slots' data was published before the event that fired them).
__device__ __forceinline__ void thread_push_range(const MK_C Params &P, int g0, int cnt) {
    if (cnt <= 0) return;
    const int s0 = add_relaxed(P.ctl + CTL_QTAIL, cnt);
    if (s0 + cnt > P.q_cap) {
        set_error(P.ctl, 4 /* MOE_MK_ERR_QUEUE */);
        return;
    }
    const unsigned long long tag = (unsigned long long)(uint32_t)g_sm.epoch << 32;
    for (int i = 0; i < cnt; ++i) st_relaxed64(P.qslots + s0 + i, tag | (uint32_t)(g0 + i));
}

// Notify one counter: the group's published stores complete, then thread 0 adds delta
// (negative = decrement).  Returns (to every thread) whether this notification brought
// the counter to zero, i.e. fired the event.  In the static schedule nobody acts on the
// firing (the consumers poll), so the add goes out without waiting for its reply, and the
// result is false.
__device__ __forceinline__ bool wg_notify(const MK_C Params &P, MK_G int *ctr, int delta) {
    wg_stores_done();
    if (P.sched == 0) {
        if (threadIdx.x == 0) add_relaxed_noret(ctr, delta);
        return false;
    }
    if (threadIdx.x == 0) {
        const int old = add_relaxed(ctr, delta);
        g_sm.bcast[2] = (old + delta == 0) ? 1 : 0;
    }
    __syncthreads();
    const bool fired = g_sm.bcast[2] != 0;
    __syncthreads();
    return fired;
}

// ------------------------------------------------------------------------------ LDS DMA helpers
// 16 bytes per lane from global memory straight into LDS: lane L's bytes land at
// dst_wave_base + 16 L.
__device__ __forceinline__ void lds_dma16(const MK_G void *src, MK_L void *dst_wave_base) {
    __builtin_amdgcn_global_load_lds(src, dst_wave_base, 16, 0, 0);
}
// The same with the non-temporal hint (cache policy bit nt), for the weight tiles of an expert
// that has a single row tile: its weight bytes are read once.  On MI355X such loads measured
// much faster (a decode forward streaming 2.8 GB of weights: 491 -> 446 us); for experts whose
// row tiles share weight columns through L2 the hint measured slower, so they keep plain loads.
// (Narrow tiles take the choice as a template argument; the wide tiles, whose K loop is
// inlined, branch on a wave-uniform flag at each weight load.)
__device__ __forceinline__ void lds_dma16_nt(const MK_G void *src, MK_L void *dst_wave_base) {
    __builtin_amdgcn_global_load_lds(src, dst_wave_base, 16, 0, 2);
}

__device__ __forceinline__ uint32_t lds_addr(const uint16_t *p) {
    return (uint32_t)(uintptr_t)(const MK_L uint16_t *)p;
}

// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

// Wait until at most n stages of L loads each are outstanding (n clamped to 0 .. MAXN; the
// count of s_waitcnt is an immediate, so this picks one of MAXN + 1 waits).
template <int L, int MAXN>
__device__ __forceinline__ void wait_vm_stages(int n) {
    if constexpr (MAXN > 0) {
        if (n >= MAXN) {
            wait_vm<MAXN * L>();
            return;
        }
        wait_vm_stages<L, MAXN - 1>(n);
    } else {
        wait_vm<0>();
    }
}

// Workgroup barrier without the memory-model fences of __syncthreads (which would wait
// for every LDS-DMA load in flight); the empty asm statements keep the compiler from
// moving memory operations across it.
__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Round v to bf16 and store it at row[col], two adjacent columns per 4-byte store: the
// value of column col+1 sits in the next lane, and the even lane stores both.  Every lane
// of the wave must call (the pair is exchanged across lanes); ok masks the store.
__device__ __forceinline__ void store_bf16_pair(MK_G uint16_t *row, int col, float v, bool ok) {
    const uint32_t hv = f32_to_bf16(v);
    const uint32_t nb = (uint32_t)__shfl_xor((int)hv, 1, 64);
    if (ok && (col & 1) == 0) pub((MK_G uint32_t *)(row + col), hv | (nb << 16));
}

// The kernel parameters through a wave-uniform reference.  A callee receives its reference
// in vector registers, so field reads through it would be vector loads from the kernel-
// argument segment, each followed by a wait for all of the wave's loads; through a uniform
// address they are scalar loads that the scalar cache keeps.
__device__ __forceinline__ const MK_C Params &uni_params(const MK_C Params &P) {
    const uint64_t a = (uint64_t)(uintptr_t)&P;
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    return *(const MK_C Params *)(uintptr_t)(lo | (hi << 32));
}

// ------------------------------------------------------------------------------ ROUTE
// logit[b,e] = sum_j x[b,j] Wr[j,e] (+ bias[e]) in the fixed fp32 order: lane l of the
// wave accumulates j = l, l+64, ... with fma (one chain per lane), then the 64 chains are
// combined by a butterfly that pairs lanes l and l^32, then l^16, ... (the halves fold),
// which every lane evaluates in the same association; the bias is added last.

// Lane l ^ M's value (M = 1, 2, 4, 8: within rows of 16 lanes) by DPP, without LDS.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
    int x = __float_as_int(v);
    if constexpr (M == 1) {
        x = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
    } else if constexpr (M == 2) {
        x = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
    } else if constexpr (M == 4) {
        x = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true);  // row_half_mirror: j -> 7 - j
        x = __builtin_amdgcn_mov_dpp(x, 0x1B, 0xF, 0xF, true);   // quad_perm [3,2,1,0]
    } else {
        static_assert(M == 8, "xor within a row");
        x = __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true);  // row_ror:8
    }
    return __int_as_float(x);
}

// Sum each of NV per-lane values over the 64 lanes, leaving value v (v = 0..NV-1) in the
// lanes whose bits 5, 4, ... (most significant first) spell v.  Level by level, lane l
// adds the partial sum of lane l ^ M (M = 32, 16, ..., 1); the values a lane stops
// carrying are sent to its partner instead of both lanes adding everything.  Every
// value is therefore the sum of the 64 chains in the association of the halves fold.
// The exchanges are cross-lane VALU operations (no LDS round trips): for M = 32 and 16,
// v_permlane32_swap / v_permlane16_swap of the pair (v[i], v[i+H]) leave each lane its own
// kept value and its partner's copy of it (lanes with bit M clear keep v[i], the others
// v[i+H]), whose sum is the level's result; for M <= 8, DPP moves within rows.
template <int NV, int M>
__device__ __forceinline__ void reduce_scatter(float *v, int lane) {
    if constexpr (M >= 1) {
        if constexpr (NV >= 2) {
            constexpr int H = NV / 2;
            if constexpr (M >= 16) {
#pragma unroll
                for (int i = 0; i < H; ++i) {
                    const unsigned a = __float_as_uint(v[i]), b = __float_as_uint(v[i + H]);
                    unsigned p0, p1;
                    if constexpr (M == 32) {
                        const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
                        p0 = r[0];
                        p1 = r[1];
                    } else {
                        const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
                        p0 = r[0];
                        p1 = r[1];
                    }
                    v[i] = __uint_as_float(p0) + __uint_as_float(p1);
                }
            } else {
                const bool up = (lane & M) != 0;
#pragma unroll
                for (int i = 0; i < H; ++i) {
                    const float send = up ? v[i] : v[i + H];
                    const float keep = up ? v[i + H] : v[i];
                    v[i] = keep + lane_xor<M>(send);
                }
            }
            reduce_scatter<H, M / 2>(v, lane);
        } else {
            if constexpr (M >= 16)
                v[0] = v[0] + shfl_xor_f(v[0], M);
            else
                v[0] = v[0] + lane_xor<M>(v[0]);
            reduce_scatter<1, M / 2>(v, lane);
        }
    }
}

// Sums of one wave (lane l holds chain l of every (token, expert) pair it owns) reduced
// over the lanes in the halves-fold order and written as logits (bias added last).
template <int TPW, int EPT = 16>
__device__ __forceinline__ void route_write(const MK_C Params &P, float (&acc)[TPW * EPT], int b0, int e0) {
    constexpr int NV = TPW * EPT;
    const int lane = lane_id();
    reduce_scatter<NV, 32>(acc, lane);
    if constexpr (NV == 128) {
        // lane L holds values 2L (acc[0]) and 2L+1 (acc[1]): token L / 8, experts
        // e0 + 2 * (L % 8) and the next
        const int b = b0 + (lane >> 3), e = e0 + 2 * (lane & 7);
        if (b < P.B) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                if (e + i < P.E) {
                    const float lg = acc[i] + (P.bias ? P.bias[e + i] : 0.0f);
                    if (!__builtin_isfinite(lg)) set_error(P.ctl, 2 /* MOE_MK_ERR_NONFINITE */);
                    pub(P.logits + (size_t)b * P.E + e + i, lg);
                }
        }
        return;
    }
    // lane L holds value L >> SH: token t = value / EPT, expert e0 + value % EPT
    constexpr int SH = NV == 64 ? 0 : NV == 16 ? 2 : 4;
    static_assert(NV == 128 || NV == 64 || NV == 16 || NV == 4, "values per lane");
    if ((lane & ((1 << SH) - 1)) == 0) {
        const int v = lane >> SH;
        const int b = b0 + v / EPT, e = e0 + v % EPT;
        if (b < P.B && e < P.E) {
            const float bias = P.bias ? P.bias[e] : 0.0f;
            const float lg = acc[0] + bias;
            if (!__builtin_isfinite(lg)) set_error(P.ctl, 2 /* MOE_MK_ERR_NONFINITE */);
            pub(P.logits + (size_t)b * P.E + e, lg);
        }
    }
}

// Router tile through LDS (E a multiple of 4).  The workgroup's kWaves*TPW tokens (wave w
// owns TPW of them) and EPT experts (16, or 4 when a small batch spreads its router over
// more workgroups) share every staged slice: per RPS values of j, the RPS x EPT block of Wr
// (each wave moving 1/8 of it, 1 KB per load) and the tokens' RPS x values (each wave
// moving its own), in a ring of as many stages as LDS holds (up to 16), filled by
// global_load_lds.  Deeper stages (RPS = 512 with one token per wave) move
// more bytes per ring iteration, which sets a workgroup's streaming rate; with four tokens
// per wave the stages hold 256 values when d allows.  Lane l
// accumulates chain l (j = l, l+64, ... in order) of every (token, expert) pair of its
// wave; a stage holds RPS/64 consecutive steps of every chain.
//   Wr stage in LDS: [RPS rows][EPT/4 chunks of 4 experts]; with EPT = 16 chunk c of row r
//     sits at c ^ rswz(r), so the 16 rows a quarter-wave reads fall on distinct 16-byte
//     bank groups (one chunk per row needs no swizzle).
//   x stage: per wave, TPW blocks of 2*RPS bytes, each one token's RPS bf16 values.
// Tokens past B and experts past E load clamped (valid) addresses; their sums are never
// written.
__device__ __forceinline__ int rswz(int r) { return (r >> 2) & 3; }

template <int TPW, int RPS, int EPT = 16>
struct RouteCfg {
    static constexpr int WR_BYTES = RPS * EPT * 4;
    static constexpr int WR_LOADS = WR_BYTES / 1024 / kWaves;  // 1 KB Wr loads per wave and stage
    static constexpr int XB = 2 * RPS * TPW;                   // x bytes per wave and stage
    static constexpr int X_LOADS = XB >= 1024 ? XB / 1024 : XB / 256;  // 16-byte lanes, else 4-byte lanes
    static constexpr int STAGE_BYTES = WR_BYTES + kWaves * XB;
    static constexpr int LOADS = WR_LOADS + X_LOADS;
    static constexpr int NS = kRingBytes / STAGE_BYTES < 16 ? kRingBytes / STAGE_BYTES : 16;
    static_assert(WR_LOADS >= 1 && WR_LOADS * 1024 * kWaves == WR_BYTES, "whole Wr loads per wave");
    static_assert(XB % 1024 == 0 || (XB < 1024 && XB % 256 == 0), "whole x loads per wave");
    static_assert(NS >= 3 && NS * STAGE_BYTES <= kRingBytes, "router ring");
    static_assert((NS - 2) * LOADS < 64, "vmcnt range");
};

// One step of a router stage: this lane's Wr row (16 experts, four 16-byte chunks at wa and
// its swizzled neighbours) and its value of each of the wave's TPW tokens (token t at
// xa + t * XS bytes).  The reads do not wait: route_wait names the same registers as inputs
// and outputs, so no use of them can be placed before it.
template <int TPW, int XS, int EPT = 16>
__device__ __forceinline__ void route_reads(uint32_t wa, uint32_t xa, f32x4 (&wv)[4], uint32_t (&xr)[TPW]) {
    const uint32_t w1 = wa ^ 16u, w2 = wa ^ 32u, w3 = wa ^ 48u;
    if constexpr (EPT == 4) {
        static_assert(TPW == 1, "four-expert blocks with one token per wave");
        asm volatile("ds_read_b128 %0, %2\n\tds_read_u16 %1, %3" : "=&v"(wv[0]), "=&v"(xr[0]) : "v"(wa), "v"(xa));
    } else if constexpr (TPW == 1) {
        asm volatile(
            "ds_read_b128 %0, %5\n\tds_read_b128 %1, %6\n\tds_read_b128 %2, %7\n\tds_read_b128 %3, %8\n\t"
            "ds_read_u16 %4, %9"
            : "=&v"(wv[0]), "=&v"(wv[1]), "=&v"(wv[2]), "=&v"(wv[3]), "=&v"(xr[0])
            : "v"(wa), "v"(w1), "v"(w2), "v"(w3), "v"(xa));
    } else if constexpr (TPW == 4) {
        asm volatile(
            "ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\tds_read_b128 %3, %11\n\t"
            "ds_read_u16 %4, %12\n\tds_read_u16 %5, %12 offset:%13\n\t"
            "ds_read_u16 %6, %12 offset:%14\n\tds_read_u16 %7, %12 offset:%15"
            : "=&v"(wv[0]), "=&v"(wv[1]), "=&v"(wv[2]), "=&v"(wv[3]), "=&v"(xr[0]), "=&v"(xr[1]), "=&v"(xr[2]),
              "=&v"(xr[3])
            : "v"(wa), "v"(w1), "v"(w2), "v"(w3), "v"(xa), "i"(XS), "i"(2 * XS), "i"(3 * XS));
    } else {
        static_assert(TPW == 8, "router tokens per wave");
        asm volatile(
            "ds_read_b128 %0, %12\n\tds_read_b128 %1, %13\n\tds_read_b128 %2, %14\n\tds_read_b128 %3, %15\n\t"
            "ds_read_u16 %4, %16\n\tds_read_u16 %5, %16 offset:%17\n\t"
            "ds_read_u16 %6, %16 offset:%18\n\tds_read_u16 %7, %16 offset:%19\n\t"
            "ds_read_u16 %8, %16 offset:%20\n\tds_read_u16 %9, %16 offset:%21\n\t"
            "ds_read_u16 %10, %16 offset:%22\n\tds_read_u16 %11, %16 offset:%23"
            : "=&v"(wv[0]), "=&v"(wv[1]), "=&v"(wv[2]), "=&v"(wv[3]), "=&v"(xr[0]), "=&v"(xr[1]), "=&v"(xr[2]),
              "=&v"(xr[3]), "=&v"(xr[4]), "=&v"(xr[5]), "=&v"(xr[6]), "=&v"(xr[7])
            : "v"(wa), "v"(w1), "v"(w2), "v"(w3), "v"(xa), "i"(XS), "i"(2 * XS), "i"(3 * XS), "i"(4 * XS),
              "i"(5 * XS), "i"(6 * XS), "i"(7 * XS));
    }
}

// Holds the accumulators at this point of the program: the FMAs that produce them cannot
// be moved past it (the compiler otherwise sinks a pipelined step's FMAs behind the next
// steps' reads and waits).
template <int N>
__device__ __forceinline__ void pin_acc(float (&acc)[N]) {
    if constexpr (N == 4) {
        asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
    } else {
        static_assert(N % 16 == 0, "blocks of 16");
#pragma unroll
        for (int i = 0; i < N; i += 16)
            asm volatile(""
                         : "+v"(acc[i]), "+v"(acc[i + 1]), "+v"(acc[i + 2]), "+v"(acc[i + 3]), "+v"(acc[i + 4]),
                           "+v"(acc[i + 5]), "+v"(acc[i + 6]), "+v"(acc[i + 7]), "+v"(acc[i + 8]), "+v"(acc[i + 9]),
                           "+v"(acc[i + 10]), "+v"(acc[i + 11]), "+v"(acc[i + 12]), "+v"(acc[i + 13]),
                           "+v"(acc[i + 14]), "+v"(acc[i + 15]));
    }
}

template <int TPW, int EPT = 16>
__device__ __forceinline__ void route_wait(f32x4 (&wv)[4], uint32_t (&xr)[TPW]) {
    if constexpr (EPT == 4)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(wv[0]), "+v"(xr[0]));
    else if constexpr (TPW == 1)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(wv[0]), "+v"(wv[1]), "+v"(wv[2]), "+v"(wv[3]), "+v"(xr[0]));
    else if constexpr (TPW == 4)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(wv[0]), "+v"(wv[1]), "+v"(wv[2]), "+v"(wv[3]), "+v"(xr[0]), "+v"(xr[1]), "+v"(xr[2]),
                       "+v"(xr[3]));
    else
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(wv[0]), "+v"(wv[1]), "+v"(wv[2]), "+v"(wv[3]), "+v"(xr[0]), "+v"(xr[1]), "+v"(xr[2]),
                       "+v"(xr[3]), "+v"(xr[4]), "+v"(xr[5]), "+v"(xr[6]), "+v"(xr[7]));
}

template <int TPW, int RPS, int EPT = 16>
__device__ __forceinline__ void route_tile_body(const MK_C Params &Pa, int b0, int e0) {
    const MK_C Params &P = uni_params(Pa);
    using C = RouteCfg<TPW, RPS, EPT>;
    static_assert(EPT == 16 || (EPT == 4 && TPW == 1 && RPS == 512), "router block shapes");
    constexpr int NS = C::NS;
    b0 = uni(b0);
    e0 = uni(e0);
    uint8_t *ring = (uint8_t *)g_sm.u.g.ring;
    const int lane = lane_id(), w = wave_id();
    const int nst = uni(P.d / RPS);
    const int E = P.E;
    // this lane's Wr DMA source.  16 experts (64-byte rows): load i of wave w covers rows
    // RPS/8*w + 16*i + lane/4 (chunk position lane%4; the swizzle of those rows does not
    // depend on i).  4 experts (16-byte rows, not swizzled): rows RPS/8*w + 64*i + lane.
    constexpr int RB = 4 * EPT;     // bytes of one staged Wr row
    constexpr int RPL = 1024 / RB;  // rows per 1 KB load
    const int wrow = (RPS / kWaves) * w + (EPT == 16 ? (lane >> 2) : lane);
    const int wcol = EPT == 16 ? min(e0 + 4 * ((lane & 3) ^ rswz(wrow)), E - 4) : e0;
    const MK_G float *wsrc = P.Wr + (size_t)wrow * E + wcol;
    // x DMA sources: byte q of the wave's x block (q = 1024*i + 16*lane, or 256*i + 4*lane)
    // is value (q % (2*RPS))/2 of the wave's token q / (2*RPS)
    const MK_G uint16_t *xsrc[C::X_LOADS];
#pragma unroll
    for (int i = 0; i < C::X_LOADS; ++i) {
        const int q = C::XB >= 1024 ? 1024 * i + 16 * lane : 256 * i + 4 * lane;
        const int tok = min(b0 + w * TPW + q / (2 * RPS), P.B - 1);
        xsrc[i] = P.x + (size_t)tok * P.d + (q % (2 * RPS)) / 2;
    }
    const size_t wstep = (size_t)RPS * E;
    auto load = [&](int st, int s) {
        uint8_t *sp = ring + s * C::STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < C::WR_LOADS; ++i)
            lds_dma16(wsrc + (size_t)st * wstep + (size_t)RPL * i * E,
                      (MK_L void *)(sp + ((RPS / kWaves) * w + RPL * i) * RB));
        uint8_t *xd = sp + C::WR_BYTES + w * C::XB;
#pragma unroll
        for (int i = 0; i < C::X_LOADS; ++i) {
            if constexpr (C::XB >= 1024)
                lds_dma16(xsrc[i] + (size_t)st * RPS, (MK_L void *)(xd + 1024 * i));
            else
                __builtin_amdgcn_global_load_lds(xsrc[i] + (size_t)st * RPS, (MK_L void *)(xd + 256 * i), 4, 0, 0);
        }
    };
    float acc[TPW * EPT];
#pragma unroll
    for (int i = 0; i < TPW * EPT; ++i) acc[i] = 0.0f;
    // Software-pipelined: the LDS reads of the next step (group of steps) are issued before
    // the FMAs of the current one and waited for after them, so the two waves of a SIMD (which leave every stage
    // barrier together) do not both sit out the LDS latency.  The reads of a stage's first
    // step are issued in the previous stage's last step, after that stage's barrier (stage
    // st+1 has landed; every wave has read all of stage st, whose slot then takes the
    // loads of stage st+NS).  Register sets alternate per step (RPS/64 steps per stage, an
    // even count), and every read is issued unconditionally (past the last stage, from a
    // slot of the ring, unused) so that no set is merged with another while in flight.
    constexpr int NSUB = RPS / 64;
    static_assert(NSUB % 2 == 0, "even steps per stage");
    const uint32_t rbase = lds_addr((const uint16_t *)ring);
    auto reads = [&](int slot, int sub, f32x4 (&wv)[4], uint32_t (&xr)[TPW]) {
        const uint32_t sb = rbase + (uint32_t)(slot * C::STAGE_BYTES);
        const int row = 64 * sub + lane;  // j = RPS*st + row: chain `lane`, step NSUB*st + sub
        route_reads<TPW, 2 * RPS, EPT>(sb + (uint32_t)(EPT == 16 ? row * 64 + 16 * rswz(row) : row * RB),
                                       sb + (uint32_t)(C::WR_BYTES + w * C::XB + 2 * row), wv, xr);
    };
    auto fmas = [&](const f32x4 (&wv)[4], const uint32_t (&xr)[TPW]) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const float xf = __uint_as_float(xr[t] << 16);
#pragma unroll
            for (int q = 0; q < EPT / 4; ++q)
#pragma unroll
                for (int z = 0; z < 4; ++z) acc[t * EPT + 4 * q + z] = fmaf(xf, wv[q][z], acc[t * EPT + 4 * q + z]);
        }
    };
#pragma unroll
    for (int p = 0; p < NS - 1; ++p)
        if (p < nst) load(p, p);
    if (NS - 2 < nst)
        wait_vm<(NS - 2) * C::LOADS>();
    else
        wait_vm<0>();
    bare_barrier();
    if (NS - 1 < nst) load(NS - 1, NS - 1);
    // With one token per wave a step has only 4 or 16 FMAs per lane, too few to cover an LDS
    // round trip: U consecutive steps (the same chains, in ascending order) share one.
    constexpr int UW = TPW == 1 ? (EPT == 4 ? 4 : 2) : 1;
    constexpr int U = UW <= NSUB / 2 ? UW : NSUB / 2;
    constexpr int NG = NSUB / U;  // read groups per stage (even: the register sets alternate)
    static_assert(NSUB % U == 0 && NG % 2 == 0, "whole, even groups per stage");
    f32x4 wvA[U][4], wvB[U][4];
    uint32_t xrA[U][TPW], xrB[U][TPW];
    auto reads_g = [&](int slot, int grp, f32x4 (&wv)[U][4], uint32_t (&xr)[U][TPW]) {
#pragma unroll
        for (int u = 0; u < U; ++u) reads(slot, grp * U + u, wv[u], xr[u]);
    };
    auto wait_g = [&](f32x4 (&wv)[U][4], uint32_t (&xr)[U][TPW]) {
#pragma unroll
        for (int u = 0; u < U; ++u) route_wait<TPW, EPT>(wv[u], xr[u]);
    };
    reads_g(0, 0, wvA, xrA);
    wait_g(wvA, xrA);
    int slot = 0;
    for (int st = 0; st < nst; ++st) {
        const int nslot = slot == NS - 1 ? 0 : slot + 1;
#pragma unroll
        for (int grp = 0; grp < NG; ++grp) {
            f32x4 (&wc)[U][4] = (grp & 1) ? wvB : wvA;
            uint32_t (&xc)[U][TPW] = (grp & 1) ? xrB : xrA;
            f32x4 (&wn)[U][4] = (grp & 1) ? wvA : wvB;
            uint32_t (&xn)[U][TPW] = (grp & 1) ? xrA : xrB;
            if (grp + 1 < NG) {
                reads_g(slot, grp + 1, wn, xn);
            } else {
                if (st + 1 < nst) {
                    if (st + NS - 1 < nst)
                        wait_vm<(NS - 2) * C::LOADS>();  // after stage st+1: stages st+2 .. st+NS-1
                    else
                        wait_vm<0>();
                    bare_barrier();
                    if (st + NS < nst) load(st + NS, slot);
                }
                reads_g(nslot, 0, wn, xn);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < U; ++u) fmas(wc[u], xc[u]);
            pin_acc(acc);
            __builtin_amdgcn_sched_barrier(0);
            wait_g(wn, xn);
        }
        slot = nslot;
    }
    wait_vm<0>();
    __syncthreads();  // the ring may be reused by the next task
    route_write<TPW, EPT>(P, acc, b0 + w * TPW, e0);
}
template <int TPW, int RPS, int EPT = 16>
__device__ __attribute__((noinline)) void route_tile(const MK_C Params &Pa, int b0, int e0) {
    route_tile_body<TPW, RPS, EPT>(Pa, b0, e0);
}

// Router wave for E not a multiple of 4: plain scalar loads, same summation order.
__device__ __attribute__((noinline)) void route_wave_scalar(const MK_C Params &Pa, int b0, int e0) {
    const MK_C Params &P = uni_params(Pa);
    const int lane = lane_id();
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    const MK_G uint16_t *xp = P.x + (size_t)min(b0, P.B - 1) * P.d + lane;
    const int nst = P.d / 64;
    for (int st = 0; st < nst; ++st) {
        const int j = st * 64 + lane;
        const float xv = bf16_to_f32(xp[(size_t)st * 64]);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float wv = P.Wr[(size_t)j * P.E + min(e0 + e, P.E - 1)];
            acc[e] = fmaf(xv, wv, acc[e]);
        }
    }
    route_write<1>(P, acc, b0, e0);
}

// Router task (tg, eb): tokens [kWaves*tpw*tg, +kWaves*tpw), wave w taking tpw of them,
// experts [reb*eb, +reb) (reb = 16, or 4 at small batches).  The eight-tokens-per-wave
// tile (nearly every register) is inlined instead of called, so it saves no registers
// through memory; the other tiles fit in the caller-saved registers and stay calls.
__device__ __forceinline__ void task_route_body(const MK_C Params &P, int tg, int eb) {
    const int e0 = eb * P.reb;
    if (P.reb == 4) {  // one token per wave, d % 512 == 0, E % 4 == 0
        route_tile<1, 512, 4>(P, tg * kWaves, e0);
    } else if ((P.E & 3) != 0) {
        const int tpw = uni(P.tpw);
        for (int t = 0; t < tpw; ++t) route_wave_scalar(P, (tg * kWaves + wave_id()) * tpw + t, e0);
    } else if (P.tpw == 1) {
        // 512-value stages for long rows; at d <= 2048 stages of 256 let the whole slice be
        // in flight at once (7 stages of the ring), which matters more than the stage size
        if (P.d % 512 == 0 && P.d > 2048)
            route_tile<1, 512>(P, tg * kWaves, e0);
        else if (P.d % 256 == 0)
            route_tile<1, 256>(P, tg * kWaves, e0);
        else
            route_tile<1, 128>(P, tg * kWaves, e0);
    } else if (P.tpw == 8) {  // d % 128 == 0
        route_tile_body<8, 128>(P, tg * kWaves * 8, e0);
    } else {
        if (P.d % 256 == 0)
            route_tile<4, 256>(P, tg * kWaves * 4, e0);
        else
            route_tile<4, 128>(P, tg * kWaves * 4, e0);
    }
}

// ------------------------------------------------------------------------------ TOPK
// For each token: the k largest logits (ties to the lower expert index; -0 equals +0),
// then softmax over them in fp32.  Keys are (order-preserving logit bits, ~expert) so the
// larger key is the larger logit and, among equal logits, the smaller expert; keys are
// unique, so the selected set and its order do not depend on the order of insertion.
// The tile's logits are staged in LDS.  Eight lanes share a token (8 tokens per wave):
// lane part q keeps a sorted list of the best keys among experts [q*per, (q+1)*per),
// visited from a per-token starting offset so the lanes of a wave read distinct LDS
// banks, eight at a time (sorted, then merged into the list); three butterfly rounds over
// lane pairs (xor 1, 2, then 4) merge the eight lists.

// Sorted lists are combined with bitonic networks (compare-exchanges of one level are
// independent, so a lane's work is a few short dependency chains rather than one long one).
// A list of KB keys is held in P = max(8, next power of two >= KB) slots, padded with key 0.
__device__ __forceinline__ void key_cx(unsigned long long &a, unsigned long long &b) {  // a = max, b = min
    const bool c = a < b;
    const unsigned long long hi = c ? b : a;
    b = c ? a : b;
    a = hi;
}
// Sort N keys into descending order.
template <int N>
__device__ __forceinline__ void keys_sort(unsigned long long (&v)[N]) {
#pragma unroll
    for (int k = 2; k <= N; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int l = i ^ j;
                if (l > i) {
                    if ((i & k) == 0)
                        key_cx(v[i], v[l]);
                    else
                        key_cx(v[l], v[i]);
                }
            }
}
// keys (KB, descending) := the KB largest of keys and other (P slots, descending): the
// elementwise max of one list and the other reversed is bitonic and holds the P largest;
// a bitonic merge sorts it.
template <int KB, int P>
__device__ __forceinline__ void keys_merge(unsigned long long (&keys)[KB], const unsigned long long (&other)[P]) {
    static_assert(P >= KB && (P & (P - 1)) == 0, "power-of-two slots");
    unsigned long long c[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const unsigned long long a = i < KB ? keys[i] : 0ull, b = other[P - 1 - i];
        c[i] = a > b ? a : b;
    }
#pragma unroll
    for (int j = P >> 1; j > 0; j >>= 1)
#pragma unroll
        for (int i = 0; i < P; ++i)
            if ((i ^ j) > i) key_cx(c[i], c[i ^ j]);
#pragma unroll
    for (int i = 0; i < KB; ++i) keys[i] = c[i];
}
template <int KB>
constexpr int key_slots() { return KB <= 8 ? 8 : 16; }

// Exchange with lane ^ M: M = 1, 2 by DPP quad permutes, M = 4 by a swizzle in bit mode
// (and-mask 31, xor-mask 4); neither makes an LDS memory round trip.
template <int M>
__device__ __forceinline__ unsigned long long lane_xor_u64(unsigned long long v) {
    int lo, hi;
    if constexpr (M == 4) {
        lo = __builtin_amdgcn_ds_swizzle((int)(uint32_t)v, 0x101F);
        hi = __builtin_amdgcn_ds_swizzle((int)(uint32_t)(v >> 32), 0x101F);
    } else {
        constexpr int ctrl = M == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] or [2,3,0,1]
        lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, ctrl, 0xF, 0xF, false);
        hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), ctrl, 0xF, 0xF, false);
    }
    return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

template <int KB>
__device__ __attribute__((noinline)) void topk_tile(const MK_C Params &Pa, int t) {
    const MK_C Params &P = uni_params(Pa);
    TopkSmem &ts = g_sm.u.t;
    const int lane = lane_id(), w = wave_id();
    const int E = P.E, k = P.k;
    const int ntok = min(kTileTokens, P.B - t * kTileTokens);
    // stage the tile's logits: 1 KB blocks straight into LDS, all in flight at once (the
    // tail of the last block may read past the tile, still inside the workspace)
    const MK_G float *src = P.logits + (size_t)t * kTileTokens * E;
    if ((E & 3) == 0) {
        const int nblk = (ntok * E * 4 + 1023) / 1024;
        for (int bk = wave_id(); bk < nblk; bk += kWaves)
            __builtin_amdgcn_global_load_lds((const MK_G void *)(src + bk * 256 + lane_id() * 4),
                                             (MK_L void *)(ts.lg + bk * 256), 16, 0, 0);
        wave_drain_vm();
    } else {
        for (int i = threadIdx.x; i < ntok * E; i += kThreads) ts.lg[i] = src[i];
    }
    for (int i = threadIdx.x; i < E; i += kThreads) ts.hist[i] = 0;
    __syncthreads();
    const int tok = 8 * w + (lane >> 3), q = lane & 7;
    const int per = (E + 7) / 8;
    const int e_lo = q * per, n_e = max(0, min(per, E - e_lo));
    const int s0 = tok % per;
    unsigned long long keys[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) keys[i] = 0ull;
    const float *row = ts.lg + tok * E + e_lo;
    // eight logits read ahead of their insertions; visits past the quarter read a valid
    // address and insert nothing (key 0 ranks below every real key)
    for (int i0 = 0; i0 < per; i0 += 8) {
        float lv[8];
        int ev[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            int idx = i0 + u + s0;
            idx -= idx >= per ? per : 0;
            idx -= idx >= per ? per : 0;
            ev[u] = i0 + u < per && idx < n_e ? idx : -1;
            lv[u] = row[ev[u] >= 0 ? idx : 0];
        }
        constexpr int PS = key_slots<KB>();
        unsigned long long nk[PS];
#pragma unroll
        for (int u = 0; u < PS; ++u) {
            nk[u] = 0ull;
            if (u < 8) {
                const float l = lv[u] + 0.0f;  // folds -0 onto +0
                const unsigned long long key =
                    ((unsigned long long)float_key(l) << 32) | (0xffffffffu - (uint32_t)(e_lo + ev[u]));
                nk[u] = ev[u] >= 0 ? key : 0ull;
            }
        }
        keys_sort<PS>(nk);
        keys_merge<KB, PS>(keys, nk);
    }
    // merge with lane ^ 1, lane ^ 2, then lane ^ 4 (every lane takes part in the exchanges)
    {
        constexpr int PS = key_slots<KB>();
        unsigned long long other[PS];
#pragma unroll
        for (int i = 0; i < PS; ++i) other[i] = 0ull;
#pragma unroll
        for (int i = 0; i < KB; ++i) other[i] = lane_xor_u64<1>(keys[i]);
        keys_merge<KB, PS>(keys, other);
#pragma unroll
        for (int i = 0; i < KB; ++i) other[i] = lane_xor_u64<2>(keys[i]);
        keys_merge<KB, PS>(keys, other);
#pragma unroll
        for (int i = 0; i < KB; ++i) other[i] = lane_xor_u64<4>(keys[i]);
        keys_merge<KB, PS>(keys, other);
    }
    if (q == 0 && tok < ntok) {
        const float mx = key_float((uint32_t)(keys[0] >> 32));
        float ex[KB];
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < KB; ++i) {
            ex[i] = 0.0f;
            if (i < k) {
                ex[i] = expf(key_float((uint32_t)(keys[i] >> 32)) - mx);
                sum += ex[i];
            }
        }
#pragma unroll
        for (int i = 0; i < KB; ++i) {
            if (i < k) {
                const int e = (int)(0xffffffffu - (uint32_t)keys[i]);
                atomicAdd(&ts.hist[e], 1);
                ts.tk[tok * k + i] = e;
                ts.tw[tok * k + i] = ex[i] / sum;
            }
        }
    }
    __syncthreads();
    // the tile's selections and weights leave as contiguous rows (whole lines, not 4-byte
    // pieces 4k bytes apart), then its histogram
    const size_t a0 = (size_t)t * kTileTokens * k;
    for (int i = threadIdx.x; i < ntok * k; i += kThreads) {
        pub(P.topk_idx + a0 + i, ts.tk[i]);
        pub(P.topk_w + a0 + i, ts.tw[i]);
    }
    for (int i = threadIdx.x; i < E; i += kThreads) pub(P.tile_hist + (size_t)t * E + i, ts.hist[i]);
}

__device__ __attribute__((noinline)) void task_topk(const MK_C Params &Pa, int t) {
    const MK_C Params &P = uni_params(Pa);
    if (P.k <= 2)
        topk_tile<2>(P, t);
    else if (P.k <= 4)
        topk_tile<4>(P, t);
    else if (P.k <= 6)
        topk_tile<6>(P, t);
    else if (P.k <= 8)
        topk_tile<8>(P, t);
    else
        topk_tile<16>(P, t);
}

// ------------------------------------------------------------------------------ SCAN
// Exclusive prefix sum of v over the workgroup's threads (and the total).  The wave's
// inclusive scan is done with DPP moves, no LDS round trips: within each row of 16 lanes the
// sums of the previous 1, 2, 4, 8 lanes (row_shr; lanes without a source add 0), then lane 15
// of rows 0 and 2 into rows 1 and 3 (row_bcast:15) and lane 31 into rows 2 and 3
// (row_bcast:31).
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15, rows 1 and 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31, rows 2 and 3
    return x;
}
__device__ __forceinline__ int block_excl_scan(int v, int *part, int *total) {
    const int lane = lane_id(), w = wave_id();
    const int x = wave_incl_scan(v);
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

// Row tiles of an expert with h rows: nw wide ones (kWideBM rows each, the last possibly
// fewer but more than kBM) and nn narrow ones (kBM rows each, the last possibly fewer).
// The shape is chosen per expert from its own row count ("RaMP": the best kernel
// configuration follows the routing histogram, not the batch size): wide row tiles read
// an expert's weight tiles once for up to kWideBM rows, narrow ones keep more weight bytes
// in flight per workgroup and split the down projection at small batches.  A wide expert's
// remainder of at most kBM rows goes to one narrow row tile.
struct ExpertTiles {
    int nw, nn, full, rem;
};
__device__ __forceinline__ ExpertTiles expert_tiles(const MK_C Params &P, int h) {
    ExpertTiles t;
    if (P.wide_ok && h >= P.wide_min) {
        t.full = h / kWideBM;
        t.rem = h - t.full * kWideBM;
        t.nw = t.full + (t.rem > kBM ? 1 : 0);
        t.nn = t.rem > 0 && t.rem <= kBM ? 1 : 0;
    } else {
        t.full = t.rem = t.nw = 0;
        t.nn = (h + kBM - 1) / kBM;
    }
    return t;
}

// Events of row tile i: its gate/up tiles per f range (NB1/S each, ev_h) and its
// down-projection tiles of bn2 columns per combine chunk (ev_d).
// (gate_up = false: only ev_d; the all-token gate/up arms ev_h with atomic adds, since its
// gate/up tiles may have counted them down before the scan)
__device__ __forceinline__ void arm_row_tile(const MK_C Params &P, int i, int bn2, bool gate_up = true) {
    if (P.unfused) return;  // kernel boundaries order the phases there
    if (gate_up)
        for (int sp = 0; sp < P.S; ++sp) pub(P.ev_h + i * P.S + sp, P.NB1 / P.S);
    for (int c = 0; c < P.nch; ++c) pub(P.ev_d + i * P.nch + c, min(kCombineCols, P.d - c * kCombineCols) / bn2);
}

// Publish expert e's row tiles (h rows from grouped row off) as row tiles mbase.. (its wide
// ones first), each with its events armed (arm_row_tile; bn2 columns per down-projection
// tile).  A row tile's shape follows from its rows: wide ones hold more than kBM rows, narrow
// ones at most kBM.
__device__ __forceinline__ void publish_row_tiles(const MK_C Params &P, int e, int h, int off, const ExpertTiles &t,
                                                  int mbase, int bn2) {
    for (int m = 0; m < t.nw; ++m) {
        const int i = mbase + m;
        pub(P.mt_expert + i, e);
        pub(P.mt_row0 + i, off + m * kWideBM);
        pub(P.mt_rows + i, min(kWideBM, h - m * kWideBM));
        arm_row_tile(P, i, bn2);
    }
    const int r0 = t.nw ? t.full * kWideBM : 0;  // a wide expert's remainder, or all rows
    for (int m = 0; m < t.nn; ++m) {
        const int i = mbase + t.nw + m;
        pub(P.mt_expert + i, e);
        pub(P.mt_row0 + i, off + r0 + m * kBM);
        pub(P.mt_rows + i, min(kBM, h - r0 - m * kBM));
        arm_row_tile(P, i, bn2);
    }
}

// hist[e] = sum_t tile_hist[t,e]; exp_indptr = exclusive prefix sum; each expert's row tiles
// (expert_tiles); arms ev_h[mt,s] with the gate/up tiles of each (row tile, f range), ev_d
// with the down-projection tiles of each (row tile, column chunk) and ev_exp[e] with
// hist[e] ("Core method": the prefix sum decides how many GroupGEMM tiles each expert
// triggers).  Events are at rest (zero) and nothing decrements them before the scan is
// published, so arming is a plain store.  (Each grouping task sums the earlier tiles' rows
// of every expert itself, so no per-tile offsets are published here.)  Returns the number of
// row tiles and (mw) of wide ones; ph (optional) receives the times the histogram scans and
// the publication ended (trace records).
__device__ __attribute__((noinline)) int task_scan(const MK_C Params &Pa, int &mw_out,
                                                   unsigned long long *ph = nullptr) {
    const MK_C Params &P = uni_params(Pa);
    ScanSmem &ss = g_sm.u.s;
    const int e = threadIdx.x;
    const int E = P.E;
    int *tb = ss.tiles;
    const int rows = kScanStage / E;  // tile_hist rows staged per round (coalesced loads)
    // R threads per expert: thread (ex, r) = (tid % E, tid / E) sums the r-th contiguous
    // chunk of each round's tiles
    const int R = kThreads / E;
    const int ex = threadIdx.x % E, r = threadIdx.x / E;
    const bool act = r < R;
    int hp = 0;
    for (int t0 = 0; t0 < P.T; t0 += rows) {
        const int nr = min(rows, P.T - t0);
        // stage rows [t0, t0 + nr) of tile_hist, sixteen loads of each thread in flight at once
        const MK_G int *src = P.tile_hist + (size_t)t0 * E;
        const int n = nr * E;
        __syncthreads();
        for (int i0 = threadIdx.x; i0 < n; i0 += 16 * kThreads) {
            int v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = i0 + u * kThreads < n ? src[i0 + u * kThreads] : 0;
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (i0 + u * kThreads < n) tb[i0 + u * kThreads] = v[u];
        }
        __syncthreads();
        const int c = (nr + R - 1) / R;
        if (act)
            for (int t = r * c; t < min(nr, (r + 1) * c); ++t) hp += tb[t * E + ex];
    }
    ss.ps[threadIdx.x] = hp;
    __syncthreads();
    int h = 0;
    if (e < E)
        for (int q = 0; q < R; ++q) h += ss.ps[q * E + e];
    const ExpertTiles et = expert_tiles(P, e < E ? h : 0);
    int total_h, total_mt, total_w;
    const int off = block_excl_scan(h, ss.part, &total_h);
    const int mbase = block_excl_scan(et.nw + et.nn, ss.part, &total_mt);
    block_excl_scan(et.nw, ss.part, &total_w);
    if (ph) ph[0] = now_ticks();
    if (e < E) {
        pub(P.hist + e, h);
        pub(P.indptr + e, off);
        pub(P.mt_base + e, mbase);
        publish_row_tiles(P, e, h, off, et, mbase, total_w > 0 ? kWideBN : P.DC);
        if (h && !P.unfused) pub(P.ev_exp + e, h);
    }
    if (e == 0) {
        pub(P.indptr + E, total_h);
        pub(P.mt_base + E, total_mt);
        st_relaxed(P.ctl + CTL_MT_TOTAL, total_mt);
        st_relaxed(P.ctl + CTL_MW, total_w);
        if (!P.unfused && P.sched) pub(P.ctl + CTL_EV_G1, P.S * total_mt);
    }
    // The routing tiles' events (at rest once their top-k ran) now count each tile's
    // grouping task: the combine tasks of a tile's tokens read its perm/inv and row tiles.
    if (!P.unfused)
        for (int t = threadIdx.x; t < P.T; t += kThreads) pub(P.ev_logit + t, 1);
    mw_out = total_w;
    if (ph) ph[1] = now_ticks();
    return total_mt;
}

// ------------------------------------------------------------------------------ GROUP
// Stable grouping of one 64-token tile: the rank of (b, i) among the tile's rows of expert
// e is the number of earlier tokens of the tile routed to e (a token uses an expert at
// most once), read off a 64-bit token mask per expert.  Row p = toff[e] + rank, where toff[e] =
// exp_indptr[e] + the rows of e in earlier tiles (summed here from tile_hist);
// perm[p] = b*k+i and inv[b*k+i] = p.  The rows themselves are not copied: the gate/up
// GroupGEMM reads each grouped row of x through perm.
__device__ __attribute__((noinline)) void task_group(const MK_C Params &Pa, int t) {
    const MK_C Params &P = uni_params(Pa);
    GroupSmem &g = g_sm.u.gr;
    const int E = P.E, k = P.k;
    const int lane = lane_id(), w = wave_id();
    const int ntok = min(kTileTokens, P.B - t * kTileTokens);
    const int b = t * kTileTokens + lane;
    // every load of the task at once: the lane's assignments (slots w and w + kWaves;
    // k <= 2 * kWaves) and the tile's row offsets
    static_assert(kMaxK <= 2 * kWaves, "two slots per lane");
    int ev[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int i = w + j * kWaves;
        ev[j] = i < k && lane < ntok ? P.topk_idx[(size_t)b * k + i] : -1;
    }
    // rows of each expert in the tiles before this one: thread (ex, r) sums the r-th chunk of
    // tiles [0, t) of tile_hist (R threads per expert), eight loads in flight at a time
    {
        const int R = kThreads / E, ex = threadIdx.x % E, r = threadIdx.x / E;
        const int c = (t + R - 1) / R, ta = min(t, r * c), tz = r < R ? min(t, (r + 1) * c) : ta;
        int sum = 0;
        for (int t0 = ta; t0 < tz; t0 += 8) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = t0 + u < tz ? P.tile_hist[(size_t)(t0 + u) * E + ex] : 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) sum += v[u];
        }
        g.ps[threadIdx.x] = sum;
    }
    for (int i = threadIdx.x; i < E; i += kThreads) {
        g.eoff[i] = P.indptr[i];
        g.emt[i] = P.mt_base[i];
        const int h = P.hist[i];
        g.erows[i] = expert_tiles(P, h).nw ? kWideBM : kBM;
        g.mask[i] = 0ull;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < E; i += kThreads) {
        int o = g.eoff[i];
        for (int q = 0; q < kThreads / E; ++q) o += g.ps[q * E + i];
        g.toff[i] = o;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
        if (ev[j] >= 0) atomicOr(&g.mask[ev[j]], 1ull << lane);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (ev[j] >= 0) {
            const int e = ev[j];
            const int a = b * k + w + j * kWaves;
            const int rank = __popcll(g.mask[e] & ((1ull << lane) - 1ull));
            const int p = g.toff[e] + rank;
            pub(P.perm + p, a);
            pub(P.inv + a, p);
            // the row tile of grouped row p: the expert's tiles hold erows rows each from its
            // first row (a wide expert's last tile holds the remainder)
            pub(P.amt + a, g.emt[e] + (p - g.eoff[e]) / g.erows[e]);
        }
    }
}

// ------------------------------------------------------------------------------ GroupGEMM tiles
// C[rows, kBN cols] = A[rows, K] * B[K, kBN cols] on v_mfma_f32_16x16x32_bf16 with fp32
// accumulation.  A is K-contiguous (grouped token rows); B is a weight slice with N
// contiguous ([K][ldb] row-major), exactly as stored.  Tiles of kBK = 64 along K go
// straight from global memory into a ring of LDS stages (global_load_lds, no staging
// registers), all but one of them in flight while one is consumed.
//   A tile in LDS: [row][k], 128-byte rows; 16-byte chunk c of row r sits at c ^ swa(r).
//     MFMA A fragment (lane i of group g: 8 consecutive k of row i) = one ds_read_b128.
//   B tile in LDS: [k][n], 256-byte rows as in memory; chunk c of row k sits at c ^ wswb(k).
//     MFMA B fragment (8 consecutive k of column j) = two ds_read_b64_tr_b16: within each
//     16-lane group, lane l addresses row (k0 + l/4), columns (n0 + 4*(l%4) .. +3) and
//     receives the 4 rows' values of column n0 + l.
// The swizzles make both fragment reads conflict-free (checked with the LDS bank-conflict
// counter on probes of these address patterns).  Wave w owns output columns
// [16w, 16w+16); 16-row blocks beyond the tile's rows are skipped, and rows of a partial
// block past the tile's rows are never loaded (their outputs are discarded).
// Half-width tiles (BN = kHalfBN = 64 columns, the smallest batches): the B tile rows are 128
// bytes, chunk c of row k at c ^ hswb(k); wave w owns columns [16 (w%4), +16) and the K step of
// 32 in each 64-deep stage that its half (w/4) takes; waves 4-7 hand their sums to waves 0-3
// through LDS at the end, which add them (first half + second half) and write the outputs.
//   hswb keeps the two chunks of a fragment read adjacent and gives the four even (and the four
//   odd) rows that one half-wave's ds_read_b64_tr_b16 touches four different chunk pairs, so
//   each half-wave reads 256 bytes from 64 distinct banks.

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Chosen by timing every chunk swizzle that is a linear (XOR) function of row bits 0..4 and
// checking the winner with the LDS bank-conflict counter: zero conflict cycles, where
// (r ^ (r >> 3)) & 7 spent half the read cycles in conflicts on MI355X.
__device__ __forceinline__ int swa(int r) {
    return ((r >> 1) & 1) | ((((r >> 1) ^ (r >> 2) ^ (r >> 4)) & 1) << 1) | (((r >> 2) & 1) << 2);
}
__device__ __forceinline__ int wswb(int k) { return ((k & 3) | (((k >> 3) & 1) << 2)) << 1; }
__device__ __forceinline__ int hswb(int k) { return (((k >> 1) & 1) | (((k >> 3) & 1) << 1)) << 1; }

// Tile variants: DUAL (gate and up weights share the A tile) and AR, the A rows staged
// (16 when the tile has at most 16 rows, as at decode batch sizes, else 64).  The ring of
// stages fills the same LDS either way, so smaller A tiles buy deeper rings: more weight
// bytes in flight per workgroup.
template <bool DUAL, int AR, int BN = kBN>
struct GemmCfg {
    static constexpr int A_ELEMS = AR * kBK;
    static constexpr int B_ELEMS = kBK * BN;
    static constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS * (DUAL ? 2 : 1);
    static constexpr int NS = (kRingBytes / 2) / STAGE_ELEMS < 8 ? (kRingBytes / 2) / STAGE_ELEMS : 8;
    static constexpr int B_BLOCKS = B_ELEMS / 512;                  // 1 KB blocks per weight and stage
    static constexpr int LOADS = 1 + (B_BLOCKS / kWaves) * (DUAL ? 2 : 1);  // global_load_lds per wave per stage
    static_assert(AR / 8 <= kWaves && B_BLOCKS % kWaves == 0, "one A block, whole B blocks per wave");
    static_assert(NS >= 3, "ring too shallow");
    static_assert((NS - 2) * LOADS < 64, "vmcnt range");
};

struct GemmArgs {
    const MK_G uint16_t *arow[1];  // this lane's A row (in the 1 KB block it loads)
    int nrows;
    const MK_G uint16_t *B0, *B1;
    int ldb, K;
};


// The 1 KB block of the A tile (8 rows of 128 bytes) this wave loads: block w, or with
// 16 rows block w % 2 (waves past the first two repeat their loads, writing identical
// bytes, so every wave issues the same number of loads per stage).
template <int AR>
__device__ __forceinline__ int a_block() {
    return wave_id() % (AR / 8);
}

// Issue the loads of one K stage.  A: one 1 KB block per wave; B: each wave moves
// B_BLOCKS / kWaves 1 KB blocks (4 k-rows of 256 bytes, or 8 of 128 bytes at half width) of
// every weight tile.
template <bool DUAL, int AR, int BN = kBN, bool NT = false>
__device__ __forceinline__ void stage_load(const GemmArgs &g, int k0, uint16_t *stage) {
    using C = GemmCfg<DUAL, AR, BN>;
    uint16_t *sA = stage, *sB0 = stage + C::A_ELEMS, *sB1 = sB0 + C::B_ELEMS;
    const int lane = lane_id(), w = wave_id();
    {
        const int blk = a_block<AR>();
        const int row = 8 * blk + (lane >> 3);
        lds_dma16(g.arow[0] + k0 + 8 * ((lane & 7) ^ swa(row)), (MK_L void *)(sA + blk * 512));
    }
#pragma unroll
    for (int i = 0; i < C::B_BLOCKS / kWaves; ++i) {
        const int blk = (C::B_BLOCKS / kWaves) * w + i;
        constexpr int CPR = BN / 8;  // 16-byte chunks per k-row
        const int kr = (64 / CPR) * blk + lane / CPR;
        const int lc = (lane % CPR) ^ (BN == kBN ? wswb(kr) : hswb(kr));
        const MK_G uint16_t *b0 = g.B0 + (size_t)(k0 + kr) * g.ldb + 8 * lc;
        const MK_G uint16_t *b1 = g.B1 + (size_t)(k0 + kr) * g.ldb + 8 * lc;
        if constexpr (NT) {
            lds_dma16_nt(b0, (MK_L void *)(sB0 + blk * 512));
            if constexpr (DUAL) lds_dma16_nt(b1, (MK_L void *)(sB1 + blk * 512));
        } else {
            lds_dma16(b0, (MK_L void *)(sB0 + blk * 512));
            if constexpr (DUAL) lds_dma16(b1, (MK_L void *)(sB1 + blk * 512));
        }
    }
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));


// LDS byte address of this lane's half of a B fragment (rows kbase + l/4, columns
// ncol0 + 4*(l%4)) in a B tile of BN columns.
template <int BN = kBN>
__device__ __forceinline__ uint32_t b_frag_addr(const uint16_t *sB, int kbase, int ncol0) {
    const int l = lane_id() & 15;
    const int k = kbase + (l >> 2);
    const int col = ncol0 + 4 * (l & 3);
    const int sw = BN == kBN ? wswb(k) : hswb(k);
    return lds_addr(sB + k * BN + ((((col >> 3) ^ sw) << 3) | (col & 7)));
}

__device__ __forceinline__ u32x4 join(u32x2 lo, u32x2 hi) { return u32x4{lo[0], lo[1], hi[0], hi[1]}; }

// Fragment reads of one K step of 32 (B halves: b[0..1] for W1 / W2, b[2..3] for W3;
// A: one fragment per 16-row block).  They are issued together in one asm block that
// also waits for them: the compiler cannot tell these reads from the DMA writes into
// other ring buffers and would otherwise wait for every load in flight.
template <bool DUAL, int AR>
__device__ __forceinline__ void frag_reads(const uint32_t (&ba)[4], const uint32_t (&aa)[4], u32x2 (&b)[4],
                                           u32x4 (&a)[4]) {
    if constexpr (DUAL && AR == 64) {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %8\n\tds_read_b64_tr_b16 %1, %9\n\t"
            "ds_read_b64_tr_b16 %2, %10\n\tds_read_b64_tr_b16 %3, %11\n\t"
            "ds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\tds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3]), "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
            : "v"(ba[0]), "v"(ba[1]), "v"(ba[2]), "v"(ba[3]), "v"(aa[0]), "v"(aa[1]), "v"(aa[2]), "v"(aa[3]));
    } else if constexpr (DUAL && AR == 32) {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %6\n\tds_read_b64_tr_b16 %1, %7\n\t"
            "ds_read_b64_tr_b16 %2, %8\n\tds_read_b64_tr_b16 %3, %9\n\t"
            "ds_read_b128 %4, %10\n\tds_read_b128 %5, %11\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3]), "=&v"(a[0]), "=&v"(a[1])
            : "v"(ba[0]), "v"(ba[1]), "v"(ba[2]), "v"(ba[3]), "v"(aa[0]), "v"(aa[1]));
    } else if constexpr (DUAL) {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %5\n\tds_read_b64_tr_b16 %1, %6\n\t"
            "ds_read_b64_tr_b16 %2, %7\n\tds_read_b64_tr_b16 %3, %8\n\t"
            "ds_read_b128 %4, %9\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3]), "=&v"(a[0])
            : "v"(ba[0]), "v"(ba[1]), "v"(ba[2]), "v"(ba[3]), "v"(aa[0]));
        static_assert(AR == 16, "two-weight tiles stage 16, 32 or 64 A rows");
    } else if constexpr (AR == 64) {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %6\n\tds_read_b64_tr_b16 %1, %7\n\t"
            "ds_read_b128 %2, %8\n\tds_read_b128 %3, %9\n\tds_read_b128 %4, %10\n\tds_read_b128 %5, %11\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(b[0]), "=&v"(b[1]), "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
            : "v"(ba[0]), "v"(ba[1]), "v"(aa[0]), "v"(aa[1]), "v"(aa[2]), "v"(aa[3]));
    } else {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %3\n\tds_read_b64_tr_b16 %1, %4\n\t"
            "ds_read_b128 %2, %5\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(b[0]), "=&v"(b[1]), "=&v"(a[0])
            : "v"(ba[0]), "v"(ba[1]), "v"(aa[0]));
        static_assert(AR == 16, "one-weight tiles stage 16 or 64 A rows");
    }
}

template <bool DUAL, int AR, int BN = kBN>
__device__ __forceinline__ void stage_compute(const uint16_t *stage, int nrb, f32x4 (&acc0)[4], f32x4 (&acc1)[4]) {
    using C = GemmCfg<DUAL, AR, BN>;
    constexpr bool HALF = BN == kHalfBN;
    const uint16_t *sA = stage, *sB0 = stage + C::A_ELEMS, *sB1 = sB0 + C::B_ELEMS;
    const int lane = lane_id(), w = wave_id();
    const int g = lane >> 4, i = lane & 15;
    const int n0 = 16 * (HALF ? (w & 3) : w);  // this wave's 16 columns
#pragma unroll
    for (int kq = 0; kq < (HALF ? 1 : kBK / 32); ++kq) {
        const int ks = HALF ? (w >> 2) : kq;  // at half width each half of the waves takes one K step
        const int kb = 32 * ks + 8 * g;  // this lane group's 8 k values: kb .. kb+7
        uint32_t aa[4], ba[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const int r = 16 * rb + i;
            aa[rb] = lds_addr(sA + (r % AR) * kBK + (((kb >> 3) ^ swa(r % AR)) << 3));
        }
        ba[0] = b_frag_addr<BN>(sB0, kb, n0);
        ba[1] = b_frag_addr<BN>(sB0, kb + 4, n0);
        ba[2] = DUAL ? b_frag_addr<BN>(sB1, kb, n0) : 0u;
        ba[3] = DUAL ? b_frag_addr<BN>(sB1, kb + 4, n0) : 0u;
        u32x2 b[4];
        u32x4 a[4];
        frag_reads<DUAL, AR>(ba, aa, b, a);
        const u32x4 b0 = join(b[0], b[1]);
        const u32x4 b1 = DUAL ? join(b[2], b[3]) : b0;
#pragma unroll
        for (int rb = 0; rb < AR / 16; ++rb) {
            if (rb < nrb) {
                acc0[rb] = mfma_bf16_16x16x32(a[rb], b0, acc0[rb]);
                if constexpr (DUAL) acc1[rb] = mfma_bf16_16x16x32(a[rb], b1, acc1[rb]);
            }
        }
    }
}



template <bool DUAL, int AR, int BN = kBN, bool NT = false>
__device__ __forceinline__ void gemm_tile(const GemmArgs &ga, f32x4 (&acc0)[4], f32x4 (&acc1)[4], GemmSmem &s) {
    using C = GemmCfg<DUAL, AR, BN>;
    constexpr int NS = C::NS;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        acc0[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc1[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int nrb = uni((ga.nrows + 15) / 16);
    const int nk = uni(ga.K / kBK);
#pragma unroll
    for (int p = 0; p < NS - 1; ++p)
        if (p < nk) stage_load<DUAL, AR, BN, NT>(ga, p * kBK, s.ring + p * C::STAGE_ELEMS);
    int slot = 0;  // ring slot of stage st
    if constexpr (AR == 16) {
        // Small tiles (decode batch sizes): the stages that issue the loads of stage st + NS - 1,
        // then the last NS - 1 stages, which issue none, as two loops, so no stage branches on
        // whether it loads.  (For 64-row tiles the two copies of the stage body cost more
        // registers than the called function keeps free, so they keep one loop.)
        int st = 0;
        for (; st < nk - (NS - 1); ++st) {
            wait_vm<(NS - 2) * C::LOADS>();  // stage st has landed: at most NS - 2 newer stages outstanding
            bare_barrier();  // every wave's part of stage st is in LDS; the slot of st-1 is free
            const int ns = slot == 0 ? NS - 1 : slot - 1;  // (st - 1) mod NS
            stage_load<DUAL, AR, BN, NT>(ga, (st + NS - 1) * kBK, s.ring + ns * C::STAGE_ELEMS);
            stage_compute<DUAL, AR, BN>(s.ring + slot * C::STAGE_ELEMS, nrb, acc0, acc1);
            slot = slot == NS - 1 ? 0 : slot + 1;
        }
        for (; st < nk; ++st) {
            wait_vm_stages<C::LOADS, NS - 2>(nk - 1 - st);  // stage st has landed (nk-1-st newer ones may not have)
            bare_barrier();
            stage_compute<DUAL, AR, BN>(s.ring + slot * C::STAGE_ELEMS, nrb, acc0, acc1);
            slot = slot == NS - 1 ? 0 : slot + 1;
        }
    } else {
        for (int st = 0; st < nk; ++st) {
            // stage st has landed once at most NS - 2 newer stages are outstanding
            if (st + NS - 2 < nk)
                wait_vm<(NS - 2) * C::LOADS>();
            else
                wait_vm<0>();
            bare_barrier();  // every wave's part of stage st is in LDS; the slot of st-1 is free
            const int nxt = st + NS - 1;
            if (nxt < nk) {
                const int ns = slot == 0 ? NS - 1 : slot - 1;  // (st - 1) mod NS
                stage_load<DUAL, AR, BN, NT>(ga, nxt * kBK, s.ring + ns * C::STAGE_ELEMS);
            }
            stage_compute<DUAL, AR, BN>(s.ring + slot * C::STAGE_ELEMS, nrb, acc0, acc1);
            slot = slot == NS - 1 ? 0 : slot + 1;
        }
    }
    wait_vm<0>();
    __syncthreads();  // the ring may be reused by the next task
    if constexpr (BN == kHalfBN) {
        // waves 4-7 (second K half) hand their sums to waves 0-3 (same columns), which add
        // them after their own: [wave % 4][row block][gate, up][4 values][64 lanes] floats
        constexpr int NRB = AR / 16;
        float *red = (float *)s.ring;
        const int w = wave_id(), lane = lane_id();
        auto at = [&](int rb, int q, int r) { return (((((w & 3) * NRB + rb) * 2 + q) * 4 + r) << 6) + lane; };
        if (w >= 4) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    red[at(rb, 0, r)] = acc0[rb][r];
                    if constexpr (DUAL) red[at(rb, 1, r)] = acc1[rb][r];
                }
        }
        __syncthreads();
        if (w < 4) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    acc0[rb][r] = acc0[rb][r] + red[at(rb, 0, r)];
                    if constexpr (DUAL) acc1[rb][r] = acc1[rb][r] + red[at(rb, 1, r)];
                }
        }
        __syncthreads();  // the ring may be reused by the next task
    }
}

// Row of the A block this lane loads (8 rows of 128 bytes per block).  Rows past the
// tile's end re-read its last row (every wave must issue the same number of loads per
// stage for the vmcnt-based waits); their outputs are discarded.
template <int AR>
__device__ __forceinline__ int a_row(int nrows) {
    return min(8 * a_block<AR>() + (lane_id() >> 3), nrows - 1);
}

// All-token gate/up: wait until this forward's routing tables are out (the scan's result word
// carries the forward's epoch), then acquire.  Returns false on an error or the watchdog.
__device__ __forceinline__ bool wg_wait_routed(const MK_C Params &P) {
    if (threadIdx.x == 0) {
        const uint32_t ep = (uint32_t)g_sm.epoch;
        const MK_G unsigned long long *word = (const MK_G unsigned long long *)(P.ctl + CTL_SCAN64);
        bool ok = true;
        const unsigned long long t0 = now_ticks();
        for (unsigned it = 1; (uint32_t)(ld_relaxed64(word) >> 32) != ep; ++it) {
            if (it < 64)
                __builtin_amdgcn_s_sleep(1);
            else
                __builtin_amdgcn_s_sleep(8);
            if ((it & 31u) == 0) {
                if (ld_relaxed(P.ctl + CTL_ERR) != 0) {
                    ok = false;
                    break;
                }
                if ((long long)(now_ticks() - t0) > P.watchdog) {
                    set_error(P.ctl, 1 /* MOE_MK_ERR_WATCHDOG */);
                    ok = false;
                    break;
                }
            }
        }
        fence_acquire();
        g_sm.bcast[0] = ok ? 1 : 0;
    }
    __syncthreads();
    const bool ok = g_sm.bcast[0] != 0;
    __syncthreads();
    return ok;
}

// Gate/up tile of row tile (e, row0, nrows), columns n*BN.. of f, written to h rows row0...
// DENSE (all-token gate/up, a tile that started before the routing was known): the A rows are
// x rows 0..nrows-1, every token of the batch, in order; once the K loop is done the tile waits
// for the routing and writes the row of each token that chose expert e to that token's grouped
// h row (inv), dropping the others.  Otherwise the A rows are grouped rows, gathered from x
// through perm.  Returns false when the wait for the routing failed.
// NT: the weight loads carry the non-temporal hint (the expert has this row tile only).
template <int AR, int BN = kBN, bool DENSE = false, bool NT = false>
__device__ __forceinline__ bool gemm1_tile(const MK_C Params &P, int e, int row0, int nrows, int n) {
    GemmArgs ga;
    const int ar = a_row<AR>(nrows);
    ga.arow[0] = P.x + (size_t)(DENSE ? ar : P.perm[row0 + ar] / P.k) * P.d;
    ga.nrows = nrows;
    ga.B0 = P.W1 + (size_t)e * P.d * P.f + (size_t)n * BN;
    ga.B1 = P.W3 + (size_t)e * P.d * P.f + (size_t)n * BN;
    ga.ldb = P.f;
    ga.K = P.d;
    f32x4 acc0[4], acc1[4];
    gemm_tile<true, AR, BN, NT>(ga, acc0, acc1, g_sm.u.g);
    int *dmap = (int *)g_sm.u.g.ring;  // DENSE: grouped h row of each token, or -1 (the ring is free now)
    if constexpr (DENSE) {
        static_assert(BN == kBN, "all-token tiles are full width");
        if (!wg_wait_routed(P)) return false;
        for (int t = threadIdx.x; t < nrows; t += kThreads) {
            int dst = -1;
            for (int i = 0; i < P.k; ++i)
                if (P.topk_idx[(size_t)t * P.k + i] == e) dst = P.inv[(size_t)t * P.k + i];
            dmap[t] = dst;
        }
        __syncthreads();  // (the notify that follows the tile syncs again before the ring is reused)
    }
    const int lane = lane_id(), w = wave_id();
    const int g = lane >> 4, j = lane & 15;
    if (BN == kHalfBN && w >= 4) return true;  // (their sums went to waves 0-3)
    const int col = n * BN + 16 * (BN == kHalfBN ? (w & 3) : w) + j;
#pragma unroll
    for (int rb = 0; rb < AR / 16; ++rb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * rb + 4 * g + r;
            const float gv = acc0[rb][r], uv = acc1[rb][r];
            const uint32_t hv = f32_to_bf16(gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv);
            // columns col and col+1 sit in lanes j and j+1: even lanes store both
            const uint32_t nb = (uint32_t)__shfl_xor((int)hv, 1, 64);
            if (row < nrows && (j & 1) == 0) {
                const int dr = DENSE ? dmap[row] : row0 + row;
                if (dr >= 0) pub((MK_G uint32_t *)(P.h + (size_t)dr * P.f + col), hv | (nb << 16));
            }
        }
    }
    return true;
}

// Down-projection tile over f range sp.  With S = 1 the tile writes y (bf16) directly.
// With S > 1 splits, every split stores its fp32 partial in yp[sp]; the split that
// finishes a tile last (a per-tile counter) adds the S partials in split order and writes
// the rounded sum to y, so the result does not depend on which split finished last.
// PAIR: the task spans kWideBN = 2 kBN columns from kWideBN*n, run as one two-weight tile
// whose weight slots (those of gate and up in a gate/up tile) hold the two column halves, so
// it streams 512-byte W2 row segments through one K loop instead of two 256-byte ones.
// Returns whether this call completed the y tile (always with S = 1; with S > 1 only for the
// split that added the partials).  SPLITS = false: code for S = 1 only.
template <int AR, int BN = kBN, bool PAIR = false, bool SPLITS = true, bool NT = false>
__device__ __forceinline__ bool gemm2_tile(const MK_C Params &P, int e, int row0, int nrows, int n, int sp,
                                           int mt) {
    static_assert(!PAIR || (BN == kBN && kWideBN == 2 * kBN), "a pair of narrow column blocks spans a wide task");
    const int kl = P.f / P.S;  // reduction range of this split: [sp*kl, (sp+1)*kl)
    GemmArgs ga;
    ga.arow[0] = P.h + (size_t)(row0 + a_row<AR>(nrows)) * P.f + (size_t)sp * kl;
    ga.nrows = nrows;
    ga.B0 = P.W2 + (size_t)e * P.f * P.d + (size_t)sp * kl * P.d + (size_t)n * (PAIR ? kWideBN : BN);
    ga.B1 = PAIR ? ga.B0 + kBN : ga.B0;
    ga.ldb = P.d;
    ga.K = kl;
    f32x4 acc0[4], acc1[4];
    gemm_tile<PAIR, AR, BN, NT>(ga, acc0, acc1, g_sm.u.g);
    const int lane = lane_id(), w = wave_id();
    const int g = lane >> 4, j = lane & 15;
    // at half width waves 4-7 handed their sums to waves 0-3 and write nothing
    const bool own = BN == kBN || w < 4;
    const int col = n * (PAIR ? kWideBN : BN) + 16 * (BN == kHalfBN ? (w & 3) : w) + j;
    if (!SPLITS || P.S == 1) {
#pragma unroll
        for (int rb = 0; rb < AR / 16; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rb + 4 * g + r;
                MK_G uint16_t *yr = P.y + (size_t)(row0 + row) * P.d;
                store_bf16_pair(yr, col, acc0[rb][r], own && row < nrows);
                if constexpr (PAIR) store_bf16_pair(yr, col + kBN, acc1[rb][r], row < nrows);
            }
        return true;
    }
    const size_t split_stride = (size_t)P.B * P.k * P.d;  // floats between partial buffers
    MK_G float *ys = P.yp + (size_t)sp * split_stride;
#pragma unroll
    for (int rb = 0; rb < AR / 16; ++rb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * rb + 4 * g + r;
            if (own && row < nrows) {
                pub(ys + (size_t)(row0 + row) * P.d + col, acc0[rb][r]);
                if constexpr (PAIR) pub(ys + (size_t)(row0 + row) * P.d + col + kBN, acc1[rb][r]);
            }
        }
    }
    // count finished splits of this tile; the last one reduces
    wg_stores_done();
    if (threadIdx.x == 0) {
        MK_G int *ctr = P.red_ctr + (size_t)mt * P.NB2 + n;
        const int old = add_relaxed(ctr, 1);
        const bool last = old == P.S - 1;
        if (last) st_relaxed(ctr, 0);  // rest state for the next forward
        g_sm.bcast[2] = last ? 1 : 0;
    }
    __syncthreads();
    const bool last = g_sm.bcast[2] != 0;
    __syncthreads();
    if (!last) return false;
    fence_acquire();
    if (!own) return true;
#pragma unroll
    for (int half = 0; half < (PAIR ? 2 : 1); ++half) {
        const int c = col + half * kBN;
#pragma unroll
        for (int rb = 0; rb < AR / 16; ++rb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rb + 4 * g + r;
                const size_t o = (size_t)(row0 + min(row, nrows - 1)) * P.d + c;
                const float mine = half ? acc1[rb][r] : acc0[rb][r];
                float v[kMaxSplits];  // every partial loaded at once, then added in split order
#pragma unroll
                for (int q = 0; q < kMaxSplits; ++q)
                    v[q] = q < P.S && q != sp ? P.yp[(size_t)q * split_stride + o] : mine;
                float sum = v[0];
#pragma unroll
                for (int q = 1; q < kMaxSplits; ++q)
                    if (q < P.S) sum += v[q];
                store_bf16_pair(P.y + (size_t)(row0 + row) * P.d, c, sum, row < nrows);
            }
        }
    }
    return true;
}

// ------------------------------------------------------------------------------ wide tiles
// At large batches (an expert averages kWideMinRows rows or more) a tile has kWideBM = 256
// rows, K steps are 32 deep, and the eight waves split the tile 2 x 4: wave w owns rows
// 128*(w/4) .. +128 and the (w%4)-th quarter of the columns.  Gate/up tiles are kWideBN1 =
// 128 columns of each weight (a wave: 128 x 32 of gate and of up) and down-projection tiles
// kWideBN = 256 columns (a wave: 128 x 64); 128 accumulator registers either way.  Per K
// step a wave reads 8 A fragments and 8 B fragment halves and issues 32 MFMAs in two groups
// of 16 (rows 0-63, rows 64-127 of its block); the workgroup stages 32 KB per 4.2 MFLOP.
//   A tile in LDS: [row][k], 64-byte rows; 16-byte chunk c of row r sits at c ^ wswa(r).
//     Measured with the LDS bank-conflict counter on MI355X: rows r and r+4 of a fragment
//     read have to differ in the 32-byte half of their chunk; a swizzle of bits 2 and 3 of
//     the row that flips both chunk bits between them reads conflict-free, where XORing
//     (r >> 2) & 3 alone spent half the read cycles in conflicts.
//   B tile in LDS: [k][n], 256- or 512-byte rows as in memory; chunk c of row k sits at
//     c ^ wswb(k), so the rows one ds_read_b64_tr_b16 touches spread over distinct bank
//     groups (the bank pattern repeats every 256 bytes).
// The fragments are register-pipelined: a group's MFMAs run while the fragments of the
// next group (or of the next stage) are read, so a wave never waits on LDS before its MFMAs.
constexpr int kWBK = kWideBK;
constexpr int kWR = kWideBM / 2;  // rows per wave row
constexpr int kWRB = kWR / 16;    // 16-row blocks per wave row (two groups of four)
__device__ __forceinline__ int wswa(int r) { return ((r >> 2) & 1) | ((((r >> 2) ^ (r >> 3)) & 1) << 1); }

template <bool DUAL, int BN>
struct WideCfg {
    static constexpr int CB = BN / 64;                // 16-column blocks per wave and weight
    static constexpr int NACC = kWRB * CB;            // accumulators per weight
    static constexpr int A_ELEMS = kWideBM * kWBK;
    static constexpr int B_ELEMS = kWBK * BN;
    static constexpr int B_BLOCKS = B_ELEMS / 512;    // 1 KB blocks per weight and stage
    static constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS * (DUAL ? 2 : 1);
    static constexpr int STAGE_BYTES = 2 * STAGE_ELEMS;
    static constexpr int NS = (kRingBytes / 2) / STAGE_ELEMS;
    static constexpr int A_LOADS = 2;                 // global_load_lds per wave and stage: A, then B
    static constexpr int LOADS = A_LOADS + (B_BLOCKS / kWaves) * (DUAL ? 2 : 1);
    static_assert(NS >= 4, "ring too shallow");
    static_assert(kWRB == 8, "two groups of four row blocks per wave");
    static_assert(CB * (DUAL ? 2 : 1) == 4, "eight B fragment halves per K step");
    static_assert(A_ELEMS / 512 == A_LOADS * kWaves && B_BLOCKS % kWaves == 0, "whole blocks per wave");
    static_assert((NS - 2) * LOADS < 64, "vmcnt range");
};

// Operands of a wide tile: wave-uniform bases plus 32-bit per-lane element offsets that
// stay fixed over the K loop (each K stage only moves the uniform bases).
struct WideArgs {
    const MK_G uint16_t *A;   // activation base (x or h)
    uint32_t a_off[2];        // this lane's row start + 16-byte chunk, per A block it loads
    const MK_G uint16_t *B0, *B1;  // weight tile bases (k 0, column n0)
    uint32_t b_off[2];        // this lane's k-row * ldb + 16-byte chunk, per B block it loads
    int ldb, K, nrows;
    int nt;  // weight loads with the non-temporal hint (the expert has this row tile only)
};

// Issue all four loads of one K stage (PART 0) or only load PART (1 .. 4: the two A blocks
// of the wave, then its two B blocks).  A: sixteen 1 KB blocks of 16 rows x 64 bytes, two
// per wave (lane -> row 16*blk + lane/4, position lane%4).  B: 1 KB blocks of 1024/(2*BN)
// k-rows of 2*BN bytes (lane -> k-row lane/(BN/8), position lane%(BN/8)); a wave moves one
// block of each weight (gate/up) or two blocks of the down projection.
template <bool DUAL, int BN, int PART>
__device__ __forceinline__ void wstage_load(const WideArgs &g, int k0, uint16_t *stage) {
    using C = WideCfg<DUAL, BN>;
    static_assert(C::LOADS == 4 && C::B_BLOCKS / kWaves == (DUAL ? 1 : 2), "four loads per wave and stage");
    uint16_t *sA = stage, *sB0 = stage + C::A_ELEMS, *sB1 = sB0 + C::B_ELEMS;
    const int w = wave_id();
    const MK_G uint16_t *ab = g.A + k0;
    const size_t kk = (size_t)k0 * g.ldb;
    if constexpr (PART == 0 || PART == 1) lds_dma16(ab + g.a_off[0], (MK_L void *)(sA + (2 * w) * 512));
    if constexpr (PART == 0 || PART == 2) lds_dma16(ab + g.a_off[1], (MK_L void *)(sA + (2 * w + 1) * 512));
    auto wl = [&](const MK_G uint16_t *src, uint16_t *dst) {
        if (g.nt)
            lds_dma16_nt(src, (MK_L void *)dst);
        else
            lds_dma16(src, (MK_L void *)dst);
    };
    if constexpr (DUAL) {
        if constexpr (PART == 0 || PART == 3) wl(g.B0 + kk + g.b_off[0], sB0 + w * 512);
        if constexpr (PART == 0 || PART == 4) wl(g.B1 + kk + g.b_off[0], sB1 + w * 512);
    } else {
        if constexpr (PART == 0 || PART == 3) wl(g.B0 + kk + g.b_off[0], sB0 + (2 * w) * 512);
        if constexpr (PART == 0 || PART == 4) wl(g.B0 + kk + g.b_off[1], sB0 + (2 * w + 1) * 512);
    }
}

// Per-lane offsets of a wide tile's loads; arow(i) gives the element offset of the start
// of the A row this lane loads for A block i.
template <bool DUAL, int BN, typename RowOf>
__device__ __forceinline__ void wide_offsets(WideArgs &g, RowOf arow) {
    using C = WideCfg<DUAL, BN>;
    const int lane = lane_id(), w = wave_id();
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) {
        const int row = 16 * (2 * w + i) + (lane >> 2);
        g.a_off[i] = arow(i) + 8u * (uint32_t)((lane & 3) ^ wswa(row));
    }
    constexpr int CPR = BN / 8;    // 16-byte chunks per k-row
    constexpr int RPB = 64 / CPR;  // k-rows per 1 KB block
#pragma unroll
    for (int i = 0; i < C::B_BLOCKS / kWaves; ++i) {
        const int blk = (C::B_BLOCKS / kWaves) * w + i;
        const int kr = RPB * blk + lane / CPR;
        g.b_off[i] = (uint32_t)kr * (uint32_t)g.ldb + 8u * (uint32_t)((lane % CPR) ^ wswb(kr));
    }
}

// Byte offsets (within a stage) of this lane's fragment reads: `a` for the wave's first A
// fragment (row block rb adds 1024 * rb: rows 16 apart keep the lane's swizzle), b[cb] for
// the B fragment half of column block cb of the wave's quarter (rows kb + l/4, columns
// 16*cb + 4*(l%4)) in the first weight.  The other halves are fixed distances away: rows
// kb + 4 + l/4 (same swizzle) at +8*BN bytes, the up weight at +2*B_ELEMS bytes.
template <bool DUAL, int BN>
struct WideFragOff {
    static constexpr int CB = WideCfg<DUAL, BN>::CB;
    uint32_t a, b[CB];
    __device__ __forceinline__ WideFragOff() {
        using C = WideCfg<DUAL, BN>;
        const int lane = lane_id(), w = wave_id();
        const int g = lane >> 4, l = lane & 15;
        const int r = kWR * (w >> 2) + l;
        a = 2u * (uint32_t)(r * kWBK + ((g ^ wswa(r)) << 3));
        const int c0 = (BN / 4) * (w & 3);
        const int k = 8 * g + (l >> 2);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const int col = c0 + 16 * cb + 4 * (l & 3);
            b[cb] = 2u * (uint32_t)(C::A_ELEMS + k * BN + ((((col >> 3) ^ wswb(k)) << 3) | (col & 7)));
        }
    }
};

// Fragment reads that do not wait: the wait is wfrag_wait, which names the same registers
// as inputs and outputs, so no use of them can be placed before it.  OFF: byte offset of
// the first of four A fragments (row blocks 16 rows = 1024 bytes apart).
template <int OFF>
__device__ __forceinline__ void wfrag_read_a(uint32_t addr, u32x4 (&a)[4]) {
    asm volatile(
        "ds_read_b128 %0, %4 offset:%5\n\tds_read_b128 %1, %4 offset:%6\n\t"
        "ds_read_b128 %2, %4 offset:%7\n\tds_read_b128 %3, %4 offset:%8"
        : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
        : "v"(addr), "i"(OFF), "i"(OFF + 1024), "i"(OFF + 2048), "i"(OFF + 3072));
}
// The eight B fragment halves of a stage at byte address `stage`: b[2*jj + h] for block
// jj (CB blocks of gate then CB of up, or four of the down projection) and row half h.
// The reads wait for themselves in the same asm block (the halves are joined into MFMA
// operands, which must not be assembled before the data is there), and that wait also
// covers the A fragments a0 read earlier without one.
template <bool DUAL, int BN>
__device__ __forceinline__ void wfrag_read_b_wait(uint32_t stage, const WideFragOff<DUAL, BN> &fo, u32x2 (&b)[8],
                                                  u32x4 (&a0)[4]) {
    constexpr int HO = 8 * BN;                                 // rows kb + 4 + l/4
    constexpr int QO = 2 * WideCfg<DUAL, BN>::B_ELEMS;          // the up weight
    if constexpr (DUAL) {
        static_assert(WideFragOff<DUAL, BN>::CB == 2, "two blocks per weight");
        const uint32_t v0 = stage + fo.b[0], v1 = stage + fo.b[1];
        asm volatile(
            "ds_read_b64_tr_b16 %0, %12\n\tds_read_b64_tr_b16 %1, %12 offset:%14\n\t"
            "ds_read_b64_tr_b16 %2, %13\n\tds_read_b64_tr_b16 %3, %13 offset:%14\n\t"
            "ds_read_b64_tr_b16 %4, %12 offset:%15\n\tds_read_b64_tr_b16 %5, %12 offset:%16\n\t"
            "ds_read_b64_tr_b16 %6, %13 offset:%15\n\tds_read_b64_tr_b16 %7, %13 offset:%16\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3]), "=&v"(b[4]), "=&v"(b[5]), "=&v"(b[6]), "=&v"(b[7]),
              "+v"(a0[0]), "+v"(a0[1]), "+v"(a0[2]), "+v"(a0[3])
            : "v"(v0), "v"(v1), "i"(HO), "i"(QO), "i"(QO + HO));
    } else {
        static_assert(WideFragOff<DUAL, BN>::CB == 4, "four blocks");
        const uint32_t v0 = stage + fo.b[0], v1 = stage + fo.b[1], v2 = stage + fo.b[2], v3 = stage + fo.b[3];
        asm volatile(
            "ds_read_b64_tr_b16 %0, %12\n\tds_read_b64_tr_b16 %1, %12 offset:%16\n\t"
            "ds_read_b64_tr_b16 %2, %13\n\tds_read_b64_tr_b16 %3, %13 offset:%16\n\t"
            "ds_read_b64_tr_b16 %4, %14\n\tds_read_b64_tr_b16 %5, %14 offset:%16\n\t"
            "ds_read_b64_tr_b16 %6, %15\n\tds_read_b64_tr_b16 %7, %15 offset:%16\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3]), "=&v"(b[4]), "=&v"(b[5]), "=&v"(b[6]), "=&v"(b[7]),
              "+v"(a0[0]), "+v"(a0[1]), "+v"(a0[2]), "+v"(a0[3])
            : "v"(v0), "v"(v1), "v"(v2), "v"(v3), "i"(HO));
    }
}
__device__ __forceinline__ void wfrag_wait(u32x4 (&a)[4]) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
}

// The 16 MFMAs of row blocks [4*G + lo, 4*G + hi) (those below NRB) with fragments a, b.
template <bool DUAL, int BN, int NRB, int G>
__device__ __forceinline__ void wide_mfma(int lo, int hi, const u32x4 (&a)[4], const u32x2 (&b)[8],
                                          f32x4 (&acc0)[WideCfg<DUAL, BN>::NACC],
                                          f32x4 (&acc1)[WideCfg<DUAL, BN>::NACC]) {
    constexpr int CB = WideCfg<DUAL, BN>::CB;
#pragma unroll
    for (int rb = lo; rb < hi; ++rb) {
        const int rr = 4 * G + rb;
        if (rr < NRB)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int q = jj / CB, cb = jj % CB;
                const u32x4 bf = join(b[2 * jj], b[2 * jj + 1]);
                if (q == 0)
                    acc0[CB * rr + cb] = mfma_bf16_16x16x32(a[rb], bf, acc0[CB * rr + cb]);
                else
                    acc1[CB * rr + cb] = mfma_bf16_16x16x32(a[rb], bf, acc1[CB * rr + cb]);
            }
    }
}

// One K stage st (in ring slot st % NS), entered with its group-0 A fragments (a0) and its
// B fragments (b) in registers:
//   read group 1's A fragments; group-0 MFMAs with two loads of stage st+NS-1 (into the
//   slot of stage st-1, which every wave finished reading before the last barrier); wait
//   for group 1's fragments; this wave's loads of stage st+1 complete, then the barrier
//   (every wave's loads of stage st+1 have landed and every wave is done with slot st);
//   read stage st+1's group-0 A fragments into a0 (their MFMAs are issued); group-1 MFMAs
//   with the other two loads; read stage st+1's B fragments into b once those MFMAs are
//   issued, and wait for all of them.
// A wave that issues a load can stall until the memory pipeline takes it, and issues no
// MFMA meanwhile.  So the two waves that share a SIMD (w and w + 4: LATE is w >= 4) place
// their loads at opposite points: one after each run of 8 MFMAs, the other before it, and
// one wave's stall overlaps the other's MFMAs.
// NRB = 16-row blocks of the wave that hold rows, rounded up to even (a compile-time count,
// so no branches surround the MFMAs); every variant issues the same loads and barriers.
// TAIL: 0 for the stages that issue loads (st + NS - 1 < nk), 1 for the later ones but the
// last, 2 for the last; the three variants are separate loops, so no stage branches on them.
template <bool DUAL, int BN, int NRB, bool LATE, int TAIL>
__device__ __forceinline__ void wide_stage(int st, int nk, const WideArgs &ga, const WideFragOff<DUAL, BN> &fo,
                                           uint32_t ring, uint16_t *ring_p, u32x4 (&a0)[4], u32x2 (&b)[8],
                                           u32x4 (&a1)[4],
                                           f32x4 (&acc0)[WideCfg<DUAL, BN>::NACC],
                                           f32x4 (&acc1)[WideCfg<DUAL, BN>::NACC]) {
    using C = WideCfg<DUAL, BN>;
    constexpr int NS = C::NS;
    const uint32_t sb = ring + (uint32_t)((st % NS) * C::STAGE_BYTES);
    const int ld = st + NS - 1;  // the stage whose loads this one issues
    uint16_t *ld_p = ring_p + ((st + NS - 1) % NS) * C::STAGE_ELEMS;
    constexpr bool lds = TAIL == 0;
    if constexpr (NRB > 4) wfrag_read_a<4096>(sb + fo.a, a1);
    if constexpr (LATE) {
        if (lds) wstage_load<DUAL, BN, 1>(ga, ld * kWBK, ld_p);
        __builtin_amdgcn_sched_barrier(0);
    }
    wide_mfma<DUAL, BN, NRB, 0>(0, 2, a0, b, acc0, acc1);
    __builtin_amdgcn_sched_barrier(0);
    if (lds) {
        if constexpr (LATE)
            wstage_load<DUAL, BN, 2>(ga, ld * kWBK, ld_p);
        else
            wstage_load<DUAL, BN, 1>(ga, ld * kWBK, ld_p);
    }
    __builtin_amdgcn_sched_barrier(0);
    wide_mfma<DUAL, BN, NRB, 0>(2, 4, a0, b, acc0, acc1);
    if constexpr (!LATE) {
        __builtin_amdgcn_sched_barrier(0);
        if (lds) wstage_load<DUAL, BN, 2>(ga, ld * kWBK, ld_p);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NRB > 4) wfrag_wait(a1);
    constexpr bool more = TAIL < 2;
    if (more) {
        if constexpr (lds)
            wait_vm<(NS - 3) * C::LOADS + 2>();  // after stage st+1: stages st+2 .. st+NS-2, two of st+NS-1
        else
            wait_vm<0>();
        bare_barrier();
        if constexpr (NRB > 0) wfrag_read_a<0>(ring + (uint32_t)(((st + 1) % NS) * C::STAGE_BYTES) + fo.a, a0);
    }
    if constexpr (LATE) {
        __builtin_amdgcn_sched_barrier(0);
        if (lds) wstage_load<DUAL, BN, 3>(ga, ld * kWBK, ld_p);
    }
    __builtin_amdgcn_sched_barrier(0);
    wide_mfma<DUAL, BN, NRB, 1>(0, 2, a1, b, acc0, acc1);
    __builtin_amdgcn_sched_barrier(0);
    if (lds) {
        if constexpr (LATE)
            wstage_load<DUAL, BN, 4>(ga, ld * kWBK, ld_p);
        else
            wstage_load<DUAL, BN, 3>(ga, ld * kWBK, ld_p);
    }
    __builtin_amdgcn_sched_barrier(0);
    wide_mfma<DUAL, BN, NRB, 1>(2, 4, a1, b, acc0, acc1);
    if constexpr (!LATE) {
        __builtin_amdgcn_sched_barrier(0);
        if (lds) wstage_load<DUAL, BN, 4>(ga, ld * kWBK, ld_p);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NRB > 0)
        if (more) wfrag_read_b_wait<DUAL, BN>(ring + (uint32_t)(((st + 1) % NS) * C::STAGE_BYTES), fo, b, a0);
}

template <bool DUAL, int BN, int NRB, bool LATE>
__device__ __forceinline__ void wide_loop(const WideArgs &ga, int nk, f32x4 (&acc0)[WideCfg<DUAL, BN>::NACC],
                                          f32x4 (&acc1)[WideCfg<DUAL, BN>::NACC], GemmSmem &s) {
    using C = WideCfg<DUAL, BN>;
    constexpr int NS = C::NS;
    const WideFragOff<DUAL, BN> fo;
    const uint32_t ring = lds_addr(s.ring);
#pragma unroll
    for (int p = 0; p < NS - 1; ++p)
        if (p < nk) wstage_load<DUAL, BN, 0>(ga, p * kWBK, s.ring + p * C::STAGE_ELEMS);
    // stage 0 complete (this wave's loads, then everyone's), then its fragments
    if (nk >= NS - 1)
        wait_vm<(NS - 2) * C::LOADS>();
    else
        wait_vm<0>();
    bare_barrier();
    u32x4 a0[4], a1[4];
    u32x2 b[8];
    if constexpr (NRB > 0) {
        wfrag_read_a<0>(ring + fo.a, a0);
        wfrag_read_b_wait<DUAL, BN>(ring, fo, b, a0);
    }
    int st = 0;
    for (; st < nk - (NS - 1); ++st)
        wide_stage<DUAL, BN, NRB, LATE, 0>(st, nk, ga, fo, ring, s.ring, a0, b, a1, acc0, acc1);
    for (; st < nk - 1; ++st)
        wide_stage<DUAL, BN, NRB, LATE, 1>(st, nk, ga, fo, ring, s.ring, a0, b, a1, acc0, acc1);
    if (st < nk) wide_stage<DUAL, BN, NRB, LATE, 2>(st, nk, ga, fo, ring, s.ring, a0, b, a1, acc0, acc1);
    wait_vm<0>();
    __syncthreads();
}

// The K loop of a wide tile.  Each wave runs the loop variant for the number of its
// 16-row blocks that hold rows (waves of one tile may differ; every variant issues the
// same loads and barriers).
template <bool DUAL, int BN>
__device__ __forceinline__ void wide_tile(const WideArgs &ga, f32x4 (&acc0)[WideCfg<DUAL, BN>::NACC],
                                          f32x4 (&acc1)[WideCfg<DUAL, BN>::NACC], GemmSmem &s) {
    using C = WideCfg<DUAL, BN>;
#pragma unroll
    for (int q = 0; q < C::NACC; ++q) {
        acc0[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc1[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int wrows = min(max(uni(ga.nrows) - kWR * (wave_id() >> 2), 0), kWR);
    const int nrb2 = uni((wrows + 31) / 32);  // pairs of 16-row blocks
    const int nk = uni(ga.K / kWBK);
    if (wave_id() < 4) {  // rows 0-127 of the tile
        switch (nrb2) {
            case 4: wide_loop<DUAL, BN, 8, false>(ga, nk, acc0, acc1, s); break;
            case 3: wide_loop<DUAL, BN, 6, false>(ga, nk, acc0, acc1, s); break;
            case 2: wide_loop<DUAL, BN, 4, false>(ga, nk, acc0, acc1, s); break;
            default: wide_loop<DUAL, BN, 2, false>(ga, nk, acc0, acc1, s); break;  // a tile has a row
        }
    } else {
        switch (nrb2) {
            case 4: wide_loop<DUAL, BN, 8, true>(ga, nk, acc0, acc1, s); break;
            case 3: wide_loop<DUAL, BN, 6, true>(ga, nk, acc0, acc1, s); break;
            case 2: wide_loop<DUAL, BN, 4, true>(ga, nk, acc0, acc1, s); break;
            case 1: wide_loop<DUAL, BN, 2, true>(ga, nk, acc0, acc1, s); break;
            default: wide_loop<DUAL, BN, 0, true>(ga, nk, acc0, acc1, s); break;
        }
    }
}

// Row of A block i (16 rows) loaded by this lane in a wide tile, clamped to the tile's rows.
__device__ __forceinline__ int wa_row(int i, int nrows) {
    return min(16 * (2 * wave_id() + i) + (lane_id() >> 2), nrows - 1);
}

// Output of a wide tile through LDS.  The MFMA layout gives a lane one column of four rows,
// so stored directly every store instruction writes 32-byte pieces of lines, and with the
// write-through stores that publish results across XCDs those partial lines dominated a
// tile's time.  Instead every wave puts its bf16 results into a [kWideBM][BN] tile in the
// (then idle) LDS ring, 16-byte chunks of a row XOR-swizzled by row % 8 so that the 16 rows
// one write instruction touches spread over the banks, and the workgroup then stores
// whole rows, 8 bytes per lane.
template <int BN>
__device__ __forceinline__ uint32_t wout_off(int row, int byte) {  // byte offset in the LDS tile
    return (uint32_t)(row * (2 * BN) + ((((byte >> 4) ^ (row & 7)) << 4) | (byte & 15)));
}
template <int BN>
__device__ __forceinline__ void wout_put(uint8_t *tile, int row, int col, uint32_t bf) {
    *(uint16_t *)(tile + wout_off<BN>(row, 2 * col)) = (uint16_t)bf;
}
// Rows [0, nrows) of the LDS tile to dst (row r at dst + r * ld elements); all threads
// call it after the tile is complete, and the ring is free again when it returns.
template <int BN>
__device__ __forceinline__ void wout_store(const uint8_t *tile, MK_G uint16_t *dst, size_t ld, int nrows) {
    constexpr int LPR = BN / 4;          // lanes per row, 8 bytes each
    constexpr int RPI = kThreads / LPR;  // rows per pass of the workgroup
    const int q = threadIdx.x % LPR, r = threadIdx.x / LPR;
    for (int row = r; row < nrows; row += RPI) {
        const unsigned long long v = *(const unsigned long long *)(tile + wout_off<BN>(row, 8 * q));
        st_relaxed64((MK_G unsigned long long *)(dst + (size_t)row * ld + 4 * q), v);
    }
    __syncthreads();
}

// Wide gate/up tile: kWideBM rows x kWideBN1 columns of h.
__device__ __forceinline__ void wide_gemm1(const MK_C Params &Pa, int e, int row0, int nrows, int n, bool single) {
    const MK_C Params &P = uni_params(Pa);
    e = uni(e);
    row0 = uni(row0);
    nrows = uni(nrows);
    n = uni(n);
    constexpr int BN = kWideBN1;
    using C = WideCfg<true, BN>;
    WideArgs ga;
    ga.A = P.x;
    ga.nrows = nrows;
    ga.B0 = P.W1 + (size_t)e * P.d * P.f + (size_t)n * BN;
    ga.B1 = P.W3 + (size_t)e * P.d * P.f + (size_t)n * BN;
    ga.ldb = P.f;
    ga.K = P.d;
    ga.nt = uni(single ? 1 : 0);
    wide_offsets<true, BN>(ga, [&](int i) {
        return (uint32_t)(P.perm[row0 + wa_row(i, nrows)] / P.k) * (uint32_t)P.d;
    });
    f32x4 acc0[C::NACC], acc1[C::NACC];
    wide_tile<true, BN>(ga, acc0, acc1, g_sm.u.g);
    const int lane = lane_id(), w = wave_id();
    const int g = lane >> 4, j = lane & 15;
    const int r0 = kWR * (w >> 2), c0 = (BN / 4) * (w & 3);  // tile-relative
    uint8_t *tile = (uint8_t *)g_sm.u.g.ring;
#pragma unroll
    for (int rb = 0; rb < kWRB; ++rb)
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float gv = acc0[C::CB * rb + cb][r], uv = acc1[C::CB * rb + cb][r];
                const uint32_t hv = f32_to_bf16(gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv);
                wout_put<BN>(tile, r0 + 16 * rb + 4 * g + r, c0 + 16 * cb + j, hv);
            }
    __syncthreads();
    wout_store<BN>(tile, P.h + (size_t)row0 * P.f + (size_t)n * BN, (size_t)P.f, nrows);
}

// Wide down-projection tile: kWideBM rows x kWideBN columns of y.
__device__ __forceinline__ void wide_gemm2(const MK_C Params &Pa, int e, int row0, int nrows, int n, bool single) {
    const MK_C Params &P = uni_params(Pa);
    e = uni(e);
    row0 = uni(row0);
    nrows = uni(nrows);
    n = uni(n);
    constexpr int BN = kWideBN;
    using C = WideCfg<false, BN>;
    WideArgs ga;
    ga.A = P.h + (size_t)row0 * P.f;
    ga.nrows = nrows;
    ga.B0 = P.W2 + (size_t)e * P.f * P.d + (size_t)n * BN;
    ga.B1 = ga.B0;
    ga.ldb = P.d;
    ga.K = P.f;
    ga.nt = uni(single ? 1 : 0);
    wide_offsets<false, BN>(ga, [&](int i) { return (uint32_t)wa_row(i, nrows) * (uint32_t)P.f; });
    f32x4 acc0[C::NACC], acc1[C::NACC];
    wide_tile<false, BN>(ga, acc0, acc1, g_sm.u.g);
    const int lane = lane_id(), w = wave_id();
    const int g = lane >> 4, j = lane & 15;
    const int r0 = kWR * (w >> 2), c0 = (BN / 4) * (w & 3);  // tile-relative
    uint8_t *tile = (uint8_t *)g_sm.u.g.ring;
#pragma unroll
    for (int rb = 0; rb < kWRB; ++rb)
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                wout_put<BN>(tile, r0 + 16 * rb + 4 * g + r, c0 + 16 * cb + j, f32_to_bf16(acc0[C::CB * rb + cb][r]));
    __syncthreads();
    wout_store<BN>(tile, P.y + (size_t)row0 * P.d + (size_t)n * BN, (size_t)P.d, nrows);
}

// Narrow GEMM tiles as functions of their own, each called straight from the task loop.
// They fit in the caller-saved registers, so a call saves and restores nothing (a function
// that uses callee-saved registers stores them to scratch memory and reloads them on every
// call; the wide tiles, which need nearly all registers, are inlined for that reason).
// GEMM1 tile: h[rows, n0:n0+128] = bf16( silu(x_g W1[e]) * (x_g W3[e]) ) for one row tile,
// where row p of the tile is token perm[p] / k of x; AR = staged A rows (16 or 64).
template <int AR, int BN = kBN, bool DENSE = false, bool NT = false>
__device__ __attribute__((noinline)) bool narrow_gemm1(const MK_C Params &Pa, int e, int row0, int nrows, int n) {
    const MK_C Params &P = uni_params(Pa);
    return gemm1_tile<AR, BN, DENSE, NT>(P, uni(e), uni(row0), uni(nrows), uni(n));
}
// All-token gate/up tile of expert e over every token of the batch (see gemm1_tile).
__device__ __forceinline__ bool dense_gemm1(const MK_C Params &P, int e, int n) {
    const int B = uni(P.B);
    // (an all-token forward's expert has one row tile)
    if (B <= 16) return narrow_gemm1<16, kBN, true, true>(P, e, 0, B, n);
    if (B <= 32) return narrow_gemm1<32, kBN, true, true>(P, e, 0, B, n);
    return narrow_gemm1<64, kBN, true, true>(P, e, 0, B, n);
}
// GEMM2 tile: y[rows, n0:n0+128] (or its split-sp partial) = h[rows, f range sp] W2[e][f range sp, n0:n0+128].
template <int AR, int BN = kBN, bool NT = false>
__device__ __attribute__((noinline)) bool narrow_gemm2(const MK_C Params &Pa, int e, int row0, int nrows, int n,
                                                       int sp, int mt) {
    const MK_C Params &P = uni_params(Pa);
    return gemm2_tile<AR, BN, false, true, NT>(P, uni(e), uni(row0), uni(nrows), uni(n), uni(sp), uni(mt));
}

// ... over kWideBN columns as one two-weight tile (gemm2_tile PAIR); SPLITS: S > 1 possible
// (the split code raises a 64-row tile's registers past the caller-saved set, so S = 1 has
// its own copy).
template <int AR, bool SPLITS, bool NT = false>
__device__ __attribute__((noinline)) bool narrow_gemm2_pair(const MK_C Params &Pa, int e, int row0, int nrows,
                                                            int n2, int sp, int mt) {
    const MK_C Params &P = uni_params(Pa);
    return gemm2_tile<AR, kBN, true, SPLITS, NT>(P, uni(e), uni(row0), uni(nrows), uni(n2), uni(sp), uni(mt));
}

// The tile code follows the row tile's rows: a row tile of more than kBM rows is a wide one
// (see expert_tiles), narrow row tiles of at most 16 rows stage only 16 A rows.  In a forward
// with wide row tiles, and in any forward with full-width narrow tiles and d a multiple of
// kWideBN (Params::DC), a down-projection task spans kWideBN columns, which a narrow row tile
// covers with one two-weight narrow tile over both column halves.
// WIDE: the code may meet wide row tiles (the task loop of forwards that have them).
template <bool WIDE, bool NT>
__device__ __forceinline__ void narrow_task_gemm1(const MK_C Params &P, int e, int row0, int nrows, int n) {
    if (!WIDE && uni(P.BN) == kHalfBN)  // (never in a forward with wide row tiles)
        nrows <= 16 ? narrow_gemm1<16, kHalfBN, false, NT>(P, e, row0, nrows, n)
                    : narrow_gemm1<64, kHalfBN, false, NT>(P, e, row0, nrows, n);
    else if (nrows <= 16)
        narrow_gemm1<16, kBN, false, NT>(P, e, row0, nrows, n);
    else
        narrow_gemm1<64, kBN, false, NT>(P, e, row0, nrows, n);
}
// single: the row tile holds all of its expert's rows (its narrow tiles' weight loads then
// carry the non-temporal hint; see lds_dma16_nt).
template <bool WIDE>
__device__ __forceinline__ void task_gemm1(const MK_C Params &P, int e, int row0, int nrows, int n, bool single) {
    if (WIDE && nrows > kBM)
        wide_gemm1(P, e, row0, nrows, n, single);
    else if (single)
        narrow_task_gemm1<WIDE, true>(P, e, row0, nrows, n);
    else
        narrow_task_gemm1<WIDE, false>(P, e, row0, nrows, n);
}
template <bool WIDE, bool NT>
__device__ __forceinline__ bool narrow_task_gemm2(const MK_C Params &P, int e, int row0, int nrows, int n, int sp,
                                                  int mt) {
    if (WIDE || uni(P.DC) == kWideBN) {  // both column halves in one tile
        if (!WIDE && uni(P.S) > 1)  // (never in a forward with wide row tiles)
            return nrows <= 16 ? narrow_gemm2_pair<16, true, NT>(P, e, row0, nrows, n, sp, mt)
                               : narrow_gemm2_pair<64, true, NT>(P, e, row0, nrows, n, sp, mt);
        return nrows <= 16 ? narrow_gemm2_pair<16, false, NT>(P, e, row0, nrows, n, sp, mt)
                           : narrow_gemm2_pair<64, false, NT>(P, e, row0, nrows, n, sp, mt);
    }
    if (uni(P.BN) == kHalfBN)
        return nrows <= 16 ? narrow_gemm2<16, kHalfBN, NT>(P, e, row0, nrows, n, sp, mt)
                           : narrow_gemm2<64, kHalfBN, NT>(P, e, row0, nrows, n, sp, mt);
    if (nrows <= 16) return narrow_gemm2<16, kBN, NT>(P, e, row0, nrows, n, sp, mt);
    return narrow_gemm2<64, kBN, NT>(P, e, row0, nrows, n, sp, mt);
}
// Returns whether the task completed its y tile (see gemm2_tile).
template <bool WIDE>
__device__ __forceinline__ bool task_gemm2(const MK_C Params &P, int e, int row0, int nrows, int n, int sp, int mt,
                                           bool single) {
    static_assert(kWideBN % kBN == 0, "a wide down tile spans whole narrow tiles");
    if (WIDE && nrows > kBM) {
        wide_gemm2(P, e, row0, nrows, n, single);
        return true;
    }
    return single ? narrow_task_gemm2<WIDE, true>(P, e, row0, nrows, n, sp, mt)
                  : narrow_task_gemm2<WIDE, false>(P, e, row0, nrows, n, sp, mt);
}

// Whether row tile mt (of expert e, mt_total row tiles in expert order) holds all of the
// expert's rows: neither neighbour belongs to e.  (The neighbours' entries are loaded with the
// tile's own, in one round trip.)
__device__ __forceinline__ bool single_row_tile(int e, int e_prev, int e_next) { return e_prev != e && e_next != e; }

// ------------------------------------------------------------------------------ COMBINE
// out[b, :] = bf16( sum_{i<k} w[b,i] * y[inv[b*k+i], :] ), slot order, fp32, for
// a combine task: CT tokens x kCombineCols columns (4 columns per thread).
// The task first waits for the down-projection tiles its rows need: each (token, slot) row
// lies in one row tile, whose event for this column chunk counts its y tiles not yet written
// (in the unfused pipeline the kernel boundary has already ordered them).  Returns false
// when a wait ended on the watchdog or the error word; t1 receives the time the waits ended.
template <int KB, int CT>
__device__ __forceinline__ bool combine_tile(const MK_C Params &P, int c, unsigned long long &t1) {
    CombineSmem &cs = g_sm.u.c;
    const int nchunks = P.nch;
    const int grp = c / nchunks, chunk = c - grp * nchunks;
    const int b_lo = grp * CT;
    const int nb = min(CT, P.B - b_lo);
    const int k = P.k;
    // the grouping of the tokens' routing tile is done (a batch of one routing tile is grouped
    // before the scan result that every combine task comes after)
    if (!P.unfused && P.T > 1 && !wg_wait_zero(P, P.ev_logit + b_lo / kTileTokens)) return false;
    bool ok = true;
    for (int i = threadIdx.x; i < nb * k; i += kThreads) {
        cs.row[i] = P.inv[(size_t)b_lo * k + i];
        cs.w[i] = P.topk_w[(size_t)b_lo * k + i];
        if (!P.unfused) ok = ok && spin_until(P.ev_d + P.amt[(size_t)b_lo * k + i] * nchunks + chunk, 0, P.ctl,
                                             P.watchdog);
    }
    if (__syncthreads_or(!ok)) return false;
    if (!P.unfused) wg_acquire();  // the rows written on other CUs, visible to this CU's loads
    t1 = now_ticks();
    const int q = (chunk * kCombineCols) / 4 + threadIdx.x;  // this thread's 4-column group
    if (4 * q < P.d) {
        // the rows of every token of the task in flight before any is used
        u32x2 yv[CT][KB];
#pragma unroll
        for (int bb = 0; bb < CT; ++bb)
#pragma unroll
            for (int i = 0; i < KB; ++i)
                if (bb < nb && i < k) yv[bb][i] = *(const MK_G u32x2 *)(P.y + (size_t)cs.row[bb * k + i] * P.d + 4 * q);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int bb = 0; bb < CT; ++bb) {
            if (bb >= nb) break;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < KB; ++i) {
                if (i < k) {
                    const float wgt = cs.w[bb * k + i];
                    const u32x2 v = yv[bb][i];
                    acc[0] = fmaf(wgt, __uint_as_float(v[0] << 16), acc[0]);
                    acc[1] = fmaf(wgt, __uint_as_float(v[0] & 0xffff0000u), acc[1]);
                    acc[2] = fmaf(wgt, __uint_as_float(v[1] << 16), acc[2]);
                    acc[3] = fmaf(wgt, __uint_as_float(v[1] & 0xffff0000u), acc[3]);
                }
            }
            const uint32_t lo = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
            *(MK_G u32x2 *)(P.out + (size_t)(b_lo + bb) * P.d + 4 * q) = u32x2{lo, hi};
        }
    }
    __syncthreads();
    return true;
}

__device__ __attribute__((noinline)) bool task_combine(const MK_C Params &Pa, int c, unsigned long long &t1) {
    const MK_C Params &P = uni_params(Pa);
    if (P.CT == 8) {  // k <= 8
        if (P.k <= 2)
            return combine_tile<2, 8>(P, c, t1);
        else if (P.k <= 4)
            return combine_tile<4, 8>(P, c, t1);
        else
            return combine_tile<8, 8>(P, c, t1);
    } else if (P.CT == 1) {
        if (P.k <= 2)
            return combine_tile<2, 1>(P, c, t1);
        else if (P.k <= 4)
            return combine_tile<4, 1>(P, c, t1);
        else if (P.k <= 8)
            return combine_tile<8, 1>(P, c, t1);
        else
            return combine_tile<16, 1>(P, c, t1);
    } else if (P.k <= 2) {
        return combine_tile<2, 4>(P, c, t1);
    } else if (P.k <= 4) {
        return combine_tile<4, 4>(P, c, t1);
    } else if (P.k <= 8) {
        return combine_tile<8, 4>(P, c, t1);
    } else {
        return combine_tile<16, 4>(P, c, t1);
    }
}

// ------------------------------------------------------------------------------ task dispatch
// Router token groups of one 64-token tile (a group is 4 * tpw tokens).
__device__ __forceinline__ int route_groups_per_tile(const MK_C Params &P) { return kTileTokens / (kWaves * P.tpw); }

__device__ __forceinline__ int route_tasks_of_tile(const MK_C Params &P, int t) {
    const int g0 = t * route_groups_per_tile(P);
    const int g1 = min(g0 + route_groups_per_tile(P), P.nTG);
    return (g1 - g0) * P.nEB;
}

__device__ __forceinline__ void count_task(const MK_C Params &P, int kind) {
    if (threadIdx.x == 0) add_relaxed(P.ctl + CTL_DBG + kind, 1);
}

// Debug trace (MOE_MK_DEBUG_TRACE): per task {g | kind << 32 | workgroup << 40, obtained,
// dependencies satisfied, finished, compute ended} in real-time ticks.
__device__ __forceinline__ void trace_task(const MK_C Params &P, int g, int kind, unsigned long long t0,
                                           unsigned long long t1, unsigned long long t2,
                                           unsigned long long t3 = 0, unsigned long long t4 = 0) {
    if ((P.debug & 2) && threadIdx.x == 0) {
        MK_G long long *e = P.trace + (size_t)g * 8;
        e[0] = (long long)g | ((long long)kind << 32) | ((long long)blockIdx.x << 40);
        e[1] = (long long)t0;
        e[2] = (long long)t1;
        e[3] = (long long)now_ticks();
        e[4] = (long long)t2;
        uint32_t xcc;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(xcc));
        e[5] = (long long)xcc;  // the XCD that ran the task
        e[6] = (long long)t3;   // optional phase ends inside the task (0 when unused)
        e[7] = (long long)t4;
    }
}

// Grouping of routing tile t and its notifications: perm/inv for the tile's assignments,
// then each expert's event is decremented by the tile's rows of that expert; in dynamic
// mode the gate/up tiles of every expert this brought to zero are pushed, with one
// reservation of queue slots for all of them (a prefix sum over the experts places each
// expert's tasks, in expert order).
// ph (optional): receives the times the grouping's stores were issued and had completed.
__device__ __forceinline__ void group_and_notify(const MK_C Params &P, Bases &bs, int t, bool dyn,
                                                 unsigned long long *ph = nullptr) {
    static_assert(kMaxE <= kThreads, "one thread per expert");
    task_group(P, t);
    count_task(P, K_GROUP);
    GroupSmem &gr = g_sm.u.gr;
    if (ph) ph[0] = now_ticks();
    wg_stores_done();
    if (ph) ph[1] = now_ticks();
    if (threadIdx.x == 0) add_relaxed(P.ev_logit + t, -1);  // the tile is grouped (see task_scan)
    int skip = -1;
    if ((P.debug & 1) && t == 0) {  // debug: drop the notification of the tile's first expert
        for (int e = 0; e < P.E; ++e)
            if (gr.mask[e]) {
                skip = e;
                break;
            }
    }
    const int e = threadIdx.x;
    const int cnt = e < P.E ? __popcll(gr.mask[e]) : 0;
    bool fire = false;
    if (cnt && e != skip) {
        if (dyn)
            fire = add_relaxed(P.ev_exp + e, -cnt) == cnt;
        else
            add_relaxed_noret(P.ev_exp + e, -cnt);
    }
    if (!dyn) return;
    // push the gate/up tiles of every expert this tile completed
    if (!bs.known) complete_bases_from_ctl(P, bs);  // block bases for the pushes
    int m0 = 0, nm = 0;
    if (fire) {
        m0 = ld_relaxed(P.mt_base + e);
        nm = ld_relaxed(P.mt_base + e + 1) - m0;
    }
    const int Q = P.NB1 / P.S;  // gate/up tasks per row tile and split
    int tot;
    const int off = block_excl_scan(nm * Q * P.S, gr.part, &tot);
    if (!tot) return;
    if (threadIdx.x == 0) gr.base = add_relaxed(P.ctl + CTL_QTAIL, tot);
    __syncthreads();
    const int base = gr.base;
    if (base + tot > P.q_cap) {
        if (threadIdx.x == 0) set_error(P.ctl, 4 /* MOE_MK_ERR_QUEUE */);
        return;
    }
    if (e < P.E) {
        gr.poff[e] = base + off;
        gr.pm0[e] = m0;
        gr.pnm[e] = nm;
    }
    __syncthreads();
    // wave w writes the slots of experts w, w + kWaves, ..., 64 slots per store
    const unsigned long long tag = (unsigned long long)(uint32_t)g_sm.epoch << 32;
    const int lane = lane_id();
    for (int x = wave_id(); x < P.E; x += kWaves) {
        const int n = gr.pnm[x] * Q;
        if (!n) continue;
        int slot = gr.poff[x];
        for (int sp = 0; sp < P.S; ++sp) {
            const int g0 = base_g1(bs, sp) + gr.pm0[x] * Q;
            for (int i = lane; i < n; i += 64) st_relaxed64(P.qslots + slot + i, tag | (uint32_t)(g0 + i));
            slot += n;
        }
    }
}

// Publish the scan's result word (static schedule, and dynamic all-token gate/up forwards; called
// after the scan's stores were drained): the row-tile count and whether any row tile is wide, tagged with the epoch.
__device__ __forceinline__ void publish_scan(const MK_C Params &P, int mt_total, int mw) {
    if (threadIdx.x == 0) {
        const unsigned long long v = ((unsigned long long)(uint32_t)g_sm.epoch << 32) | (mw > 0 ? 0x80000000ull : 0ull) |
                                     (uint32_t)mt_total;
        st_relaxed64((MK_G unsigned long long *)(P.ctl + CTL_SCAN64), v);
    }
}

// The scan and the grouping of a batch that is one routing tile, run by its top-k task
// right after top-k, from what top-k left in LDS (the tile histogram is the histogram, the
// tile's row offsets are exp_indptr): everything is published and nothing is read back.
// In dynamic mode the task count is published and the gate/up tiles of every expert with
// rows are pushed with one reservation of queue slots, made right after the scan so that
// the atomic's round trip overlaps the grouping.  t3 receives the end time of the scan.
__device__ __forceinline__ void fused_scan_group(const MK_C Params &P, Bases &bs, bool dyn, unsigned long long &t3) {
    static_assert(kMaxE <= kThreads, "one thread per expert");
    TopkSmem &ts = g_sm.u.t;
    FusedWork &W = ts.fw;
    const int e = threadIdx.x;
    // A batch of one routing tile gives an expert at most kTileTokens rows, fewer than
    // wide_min: every row tile is narrow (at most one per expert).
    const int E = P.E, k = P.k, BM = kBM;
    int skip = -1;
    if (P.debug & 1) {  // debug: drop the notification of the first expert with rows
        for (int x = 0; x < E; ++x)
            if (ts.hist[x]) {
                skip = x;
                break;
            }
    }
    // scan ("Core method": the prefix sum decides how many GroupGEMM tiles each expert triggers)
    const int h = e < E ? ts.hist[e] : 0;
    // (all-token gate/up: row tile e is expert e's rows, none for an expert without tokens)
    const int mt = P.dense ? (e < E ? 1 : 0) : (h + BM - 1) / BM;
    int total_h, total_mt;
    const int off = block_excl_scan(h, W.part, &total_h);
    const int mbase = block_excl_scan(mt, W.part, &total_mt);
    if (e < E) {
        W.off[e] = off;
        W.mtb[e] = mbase;
        W.mask[e] = 0ull;
        pub(P.hist + e, h);
        pub(P.indptr + e, off);
        pub(P.mt_base + e, mbase);
        for (int m = 0; m < mt; ++m) {
            const int i = mbase + m;
            pub(P.mt_expert + i, e);
            pub(P.mt_row0 + i, off + m * BM);
            pub(P.mt_rows + i, min(BM, h - m * BM));
            if (!P.dense || h > 0) arm_row_tile(P, i, P.DC, !P.dense);
        }
    }
    if (e == 0) {
        W.mtb[E] = total_mt;
        pub(P.indptr + E, total_h);
        pub(P.mt_base + E, total_mt);
        st_relaxed(P.ctl + CTL_MT_TOTAL, total_mt);
        st_relaxed(P.ctl + CTL_MW, 0);
        if (P.sched) pub(P.ctl + CTL_EV_G1, P.S * total_mt);
    }
    count_task(P, K_SCAN);
    complete_bases(P, bs, total_mt, 0);
    // all-token gate/up: the down-projection tasks of the experts with tokens are the only
    // GroupGEMM tasks pushed
    int active = 0;
    if (dyn && P.dense) (void)block_excl_scan(h > 0 ? 1 : 0, W.part, &active);
    if (dyn && threadIdx.x == 0) {
        // tickets: routers, this task, and the GroupGEMM and combine tasks
        const int real = bs.K + 1 + P.S * (P.dense ? bs.q1 + active * bs.N2 : bs.q1 + bs.q2) + P.nC;
        const unsigned long long tag = (unsigned long long)(uint32_t)g_sm.epoch << 32;
        st_relaxed64((MK_G unsigned long long *)(P.ctl + CTL_TOTAL64), tag | (uint32_t)real);
    }
    // reserve the queue slots of the pushes (the reply is first needed after the grouping)
    const int Q = P.NB1 / P.S;  // gate/up tasks per row tile and split
    int tot = 0, qbase = 0;
    if (dyn && !P.dense) {
        const int nm = e < E && h > 0 && e != skip ? mt : 0;
        const int poff = block_excl_scan(nm * Q * P.S, W.part, &tot);
        if (e < E) {
            W.poff[e] = poff;
            W.pnm[e] = nm;
        }
        if (threadIdx.x == 0 && tot) qbase = add_relaxed(P.ctl + CTL_QTAIL, tot);
    }
    t3 = now_ticks();
    __syncthreads();
    // grouping: rank of each (token, slot) among the expert's rows, tokens in order
    const int lane = lane_id(), w = wave_id();
    const int ntok = P.B;
    static_assert(kMaxK <= 2 * kWaves, "two slots per lane");
    int ev[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int i = w + j * kWaves;
        ev[j] = i < k && lane < ntok ? ts.tk[lane * k + i] : -1;
        if (ev[j] >= 0) atomicOr(&W.mask[ev[j]], 1ull << lane);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (ev[j] >= 0) {
            const int a = lane * k + w + j * kWaves;
            const int p = W.off[ev[j]] + __popcll(W.mask[ev[j]] & ((1ull << lane) - 1ull));
            W.perm[p] = a;
            W.inv[a] = p;
            W.amt[a] = W.mtb[ev[j]];  // an expert of a one-tile batch has at most one row tile
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < ntok * k; i += kThreads) {
        pub(P.perm + i, W.perm[i]);
        pub(P.inv + i, W.inv[i]);
        pub(P.amt + i, W.amt[i]);
    }
    count_task(P, K_GROUP);
    if (P.dense) {
        // Arm each (expert, f range) gate/up event with its tile count.  Its gate/up tiles have
        // been counting it down since the forward began, so the add that brings it to zero (this
        // one, or a tile's later) fires it; whoever fires it pushes the expert's down-projection
        // tasks of that f range (dynamic schedule; static ones wait for the scan's result word
        // and then for zero).  Everything the down projection reads goes out first.
        wg_stores_done();
        const int Q1 = P.NB1 / P.S;
        if (e < E) {
            // (debug: a skipped expert's events are armed with one count too many, so they never fire)
            const int arm = e == skip ? Q1 + 1 : Q1;
            for (int sp = 0; sp < P.S; ++sp) {
                MK_G int *ctr = P.ev_h + e * P.S + sp;
                if (!dyn) {
                    add_relaxed_noret(ctr, arm);  // (drained by the caller's notification)
                    continue;
                }
                if (add_relaxed(ctr, arm) + arm != 0) continue;  // a gate/up tile will fire it
                if (h > 0) thread_push_range(P, base_g2(bs, sp, P.S) + e * bs.N2, bs.N2);
                if (add_relaxed(P.ctl + CTL_EV_G1, -1) == 1) thread_push_range(P, bs.C, P.nC);
            }
        }
        // dynamic: the result word tells the gate/up tiles that the routing is known (the tables
        // went out above); static: the caller's notification drains the arming and publishes it
        if (dyn) publish_scan(P, E, 0);
        return;
    }
    if (!dyn) {
        if (skip >= 0 && threadIdx.x == 0) pub(P.ev_exp + skip, 1);  // a wait that never ends (debug)
        return;  // the caller's notification publishes everything
    }
    wg_stores_done();  // every table and perm/inv is out before any GroupGEMM task can start
    if (!tot) return;
    // push the gate/up tiles of every expert with rows (all but a debug-skipped one)
    if (threadIdx.x == 0) W.base = qbase;
    __syncthreads();
    const int base = W.base;
    if (base + tot > P.q_cap) {
        if (threadIdx.x == 0) set_error(P.ctl, 4 /* MOE_MK_ERR_QUEUE */);
        return;
    }
    // wave w writes the slots of experts w, w + kWaves, ..., 64 slots per store
    const unsigned long long tag = (unsigned long long)(uint32_t)g_sm.epoch << 32;
    for (int x = w; x < E; x += kWaves) {
        const int n = W.pnm[x] * Q;
        if (!n) continue;
        int slot = base + W.poff[x];
        for (int sp = 0; sp < P.S; ++sp) {
            const int g0 = base_g1(bs, sp) + W.mtb[x] * Q;
            for (int i = lane; i < n; i += 64) st_relaxed64(P.qslots + slot + i, tag | (uint32_t)(g0 + i));
            slot += n;
        }
    }
}

// Token group and expert block of router task g.  A task reads its group's activation rows
// and its block's router-weight columns, and workgroup w (hence task position g in the
// static schedule) runs on XCD w % 8.  Token-group major order (tg = g / nEB) gives XCD x
// the expert blocks = x (mod 8) of every group: each XCD keeps its weight columns in L2 but
// fetches all of x.  When x is the larger of the two (B > 2E: B*d bf16 values against E*d
// fp32 ones), positions g = 8l + x instead take group 8*(l / nEB) + x and block l % nEB,
// so the blocks of a group run together on one XCD and its rows are fetched into that L2
// once; groups past the last multiple of 8 keep the plain order.
__device__ __forceinline__ void route_task_coords(const MK_C Params &P, int g, int &tg, int &eb) {
    const int full = P.nTG & ~7;
    if (P.B > 2 * P.E && g < full * P.nEB) {
        const int x = g & 7, l = g >> 3, lg = l / P.nEB;
        tg = 8 * lg + x;
        eb = l - lg * P.nEB;
    } else {
        tg = g / P.nEB;
        eb = g - tg * P.nEB;
    }
}

// Runs task g (obtained at time t0).  Returns false when the forward must be abandoned.
// WIDE: the copy of the task code that can run wide row tiles.  The other copy (used until a
// forward is known to have them, and throughout forwards that have none) leaves them out, so
// its routing and narrow-tile paths are compiled without the wide tiles' register pressure;
// it returns kNeedWide, without running the task, for a GroupGEMM task of a forward that
// has wide row tiles.
constexpr int kTaskDone = 1, kNeedWide = 2;
__device__ __forceinline__ bool wg_wait_scan(const MK_C Params &P, Bases &bs);

// All-token gate/up forwards: whether this forward's routing tables are out (the scan's result
// word carries the forward's epoch), with an acquire when they are.  One load, until this
// workgroup has once seen them.
__device__ __forceinline__ bool routing_seen(const MK_C Params &P, Bases &bs) {
    if (bs.routed) return true;
    if (threadIdx.x == 0) {
        const unsigned long long v = ld_relaxed64((const MK_G unsigned long long *)(P.ctl + CTL_SCAN64));
        const bool r = (uint32_t)(v >> 32) == (uint32_t)g_sm.epoch;
        if (r) fence_acquire();
        g_sm.bcast[0] = r ? 1 : 0;
    }
    __syncthreads();
    const bool r = g_sm.bcast[0] != 0;
    __syncthreads();
    bs.routed = r;
    return r;
}
template <bool WIDE>
__device__ __forceinline__ int run_task(const MK_C Params &P, int g, Bases &bs, unsigned long long t0) {
    const bool dyn = P.sched != 0;
    if (g < bs.K) {  // ---------------------------------------------------------- ROUTE
        int tg, eb;
        route_task_coords(P, g, tg, eb);
        task_route_body(P, tg, eb);
        const unsigned long long t2 = now_ticks();
        count_task(P, K_ROUTE);
        const int t = tg / route_groups_per_tile(P);
        // (dynamic: the first task of the tile arms its event and the one that fires it pushes the
        // top-k task, except with the all-token gate/up, whose top-k task arms and waits as in
        // the static schedule)
        const bool push = dyn && !P.dense;
        int delta = -1;
        if (push && (tg % route_groups_per_tile(P)) == 0 && eb == 0) delta += route_tasks_of_tile(P, t);
        if (wg_notify(P, P.ev_logit + t, delta) && push) wg_push_range(P, bs.K + t, 1);
        trace_task(P, g, K_ROUTE, t0, t0, t2);
        return kTaskDone;
    }
    if (g < bs.S) {  // ---------------------------------------------------------- TOPK
        const int t = g - bs.K;
        if (!dyn || P.dense) {
            if (threadIdx.x == 0) add_relaxed(P.ev_logit + t, route_tasks_of_tile(P, t));  // arm
            if (!wg_wait_zero(P, P.ev_logit + t)) return 0;
        }
        const unsigned long long t1 = now_ticks();
        task_topk(P, t);
        const unsigned long long t2 = now_ticks();
        count_task(P, K_TOPK);
        if (P.T == 1) {
            // The only routing tile: its histogram is the whole histogram, so the scan and
            // the grouping run here, without the two joins between separate tasks.
            unsigned long long t3;
            fused_scan_group(P, bs, dyn, t3);
            const unsigned long long t4 = now_ticks();
            // static GroupGEMM tasks start once this is seen: the tables and perm/inv are out
            // (dynamic ones are pushed, and no task waits on the event)
            if (!dyn) {
                wg_notify(P, P.ctl + CTL_EV_SCAN, -1);
                publish_scan(P, bs.q1 / (P.NB1 / P.S), 0);  // (q1 = row tiles x gate/up tiles per f range)
            }
            trace_task(P, g, K_TOPK, t0, t1, t2, t3, t4);
            return kTaskDone;
        }
        int delta = -1;
        if (dyn && t == 0) delta += P.T;
        if (wg_notify(P, P.ctl + CTL_EV_TOPK, delta) && dyn) wg_push_range(P, bs.S, 1);
        trace_task(P, g, K_TOPK, t0, t1, t2);
        return kTaskDone;
    }
    if (g == bs.S) {  // --------------------------------------------------------- SCAN
        if (P.T == 1) return kTaskDone;  // a single routing tile is scanned by its top-k task
        if (!dyn) {
            if (threadIdx.x == 0) add_relaxed(P.ctl + CTL_EV_TOPK, P.T);  // arm
            if (!wg_wait_zero(P, P.ctl + CTL_EV_TOPK)) return 0;
        }
        const unsigned long long t1 = now_ticks();
        int mw = 0;
        unsigned long long ph[2];
        const int mt_total = task_scan(P, mw, ph);
        const unsigned long long t2 = now_ticks();
        count_task(P, K_SCAN);
        complete_bases(P, bs, mt_total, mw);
        wg_notify(P, P.ctl + CTL_EV_SCAN, -1);
        if (!dyn) publish_scan(P, mt_total, mw);
        if (dyn) {
            wg_push_range(P, bs.G, P.T);
            if (threadIdx.x == 0) {  // every task of this forward now has a ticket number
                // (padding positions of the static layout are never pushed)
                const int real = bs.M1 + P.S * (bs.q1 + bs.q2) + P.nC;
                const unsigned long long tag = (unsigned long long)(uint32_t)g_sm.epoch << 32;
                st_relaxed64((MK_G unsigned long long *)(P.ctl + CTL_TOTAL64), tag | (uint32_t)real);
            }
        }
        trace_task(P, g, K_SCAN, t0, t1, t2, ph[0], ph[1]);
        return kTaskDone;
    }
    if (g < bs.M1p) {  // -------------------------------------------------------- GROUP
        const int t = g - bs.G;
        if (t >= P.T) return kTaskDone;  // padding before the GroupGEMM blocks
        if (P.T == 1) return kTaskDone;  // a single routing tile is grouped by its top-k task
        if (!dyn && !wg_wait_zero(P, P.ctl + CTL_EV_SCAN)) return 0;
        const unsigned long long t1 = now_ticks();
        unsigned long long ph[2];
        group_and_notify(P, bs, t, dyn, ph);
        trace_task(P, g, K_GROUP, t0, t1, now_ticks(), ph[0], ph[1]);
        return kTaskDone;
    }
    if (!bs.known) complete_bases_from_ctl(P, bs);
    if constexpr (!WIDE) {
        if (bs.wide && g < bs.C) return kNeedWide;
    }
    if (g < bs.C) {
        int sp, j;
        // static schedule with wide row tiles: each XCD takes a contiguous eighth of a block
        const int kind = decode_gemm(bs, P.S, xcd_blocks(P, bs), g, sp, j, P.NB1 / P.S);
        if (kind == 0) return kTaskDone;  // padding position
        const int Q = P.NB1 / P.S;
        if (kind == 1) {  // ---------------------------------------------------- GEMM1
            const int mt = j / Q, n = sp * Q + (j - (j / Q) * Q);
            if constexpr (!WIDE) {  // (an all-token forward has no wide row tiles)
            if (P.dense) {
                // All-token gate/up forward: row tile mt is expert mt's rows.  A tile that starts
                // before the routing is known runs over every token and keeps the expert's rows
                // at its end; one that starts later runs over the expert's grouped rows, if any.
                const unsigned long long t1 = now_ticks();
                if (routing_seen(P, bs)) {
                    const int r0_ = P.mt_row0[mt], nr_ = P.mt_rows[mt];
                    if (uni(nr_) > 0) task_gemm1<false>(P, mt, uni(r0_), uni(nr_), n, true);
                } else {
                    if (!dense_gemm1(P, mt, n)) return 0;
                    bs.routed = true;  // (it waited for the scan's result word)
                }
                const unsigned long long t2 = now_ticks();
                count_task(P, K_GEMM1);
                // Firing the event means the scan has armed it, so the routing tables are out:
                // push the expert's down-projection tiles of this f range if it has rows.
                if (wg_notify(P, P.ev_h + mt * P.S + sp, -1) && dyn) {
                    if (threadIdx.x == 0) {
                        fence_acquire();
                        g_sm.bcast[0] = ld_relaxed(P.mt_rows + mt);
                    }
                    __syncthreads();
                    const int rows = g_sm.bcast[0];
                    __syncthreads();
                    if (rows > 0) wg_push_range(P, base_g2(bs, sp, P.S) + mt * bs.N2, bs.N2);
                    if (wg_notify(P, P.ctl + CTL_EV_G1, -1)) wg_push_range(P, bs.C, P.nC);
                }
                trace_task(P, g, K_GEMM1, t0, t1, t2);
                return kTaskDone;
            }
            }
            // the row tile's table entries (and its neighbours' experts) are read together (one
            // round trip)
            const int e_ = P.mt_expert[mt], r0_ = P.mt_row0[mt], nr_ = P.mt_rows[mt];
            const int ep_ = mt > 0 ? P.mt_expert[mt - 1] : -1, en_ = mt + 1 < bs.mt ? P.mt_expert[mt + 1] : -1;
            const int e = uni(e_);
            // (a batch of one routing tile was grouped before the layout was published, and its
            // experts' events stay at rest, unless the debug flag holds one back)
            if (!dyn && (P.T > 1 || (P.debug & 1)) && !wg_wait_zero(P, P.ev_exp + e)) return 0;
            const unsigned long long t1 = now_ticks();
            task_gemm1<WIDE>(P, e, uni(r0_), uni(nr_), n, single_row_tile(e, uni(ep_), uni(en_)));
            const unsigned long long t2 = now_ticks();
            count_task(P, K_GEMM1);
            // f range sp of this row tile complete: its down-projection tiles are ready; once
            // every row tile's have been pushed, the combine tasks follow them in the queue
            // (each waits for the down-projection tiles of its own rows)
            if (wg_notify(P, P.ev_h + mt * P.S + sp, -1) && dyn) {
                wg_push_range(P, base_g2(bs, sp, P.S) + mt * bs.N2, bs.N2);
                if (wg_notify(P, P.ctl + CTL_EV_G1, -1)) wg_push_range(P, bs.C, P.nC);
            }
            trace_task(P, g, K_GEMM1, t0, t1, t2);
            return kTaskDone;
        }
        // --------------------------------------------------------------------- GEMM2
        const int mt = j / bs.N2, n = j - mt * bs.N2;
        // (all-token gate/up, static: the layout was known from the start, the routing tables
        // are out once the scan's result word is)
        if (P.dense && !dyn && !bs.routed) {
            if (!wg_wait_scan(P, bs)) return 0;
            bs.routed = true;
        }
        // the row tile's table entries (published with the scan result this workgroup has
        // acquired) are read before the wait, so the two round trips overlap
        const int e_ = P.mt_expert[mt], r0_ = P.mt_row0[mt], nr_ = P.mt_rows[mt];
        const int ep_ = mt > 0 ? P.mt_expert[mt - 1] : -1, en_ = mt + 1 < bs.mt ? P.mt_expert[mt + 1] : -1;
        if (P.dense && uni(nr_) == 0) return kTaskDone;  // an expert without tokens (static positions)
        if (!dyn && !wg_wait_zero(P, P.ev_h + mt * P.S + sp)) return 0;
        const unsigned long long t1 = now_ticks();
        const bool done = task_gemm2<WIDE>(P, uni(e_), uni(r0_), uni(nr_), n, sp, mt,
                                           single_row_tile(uni(e_), uni(ep_), uni(en_)));
        const unsigned long long t2 = now_ticks();
        count_task(P, K_GEMM2);
        // y tile (mt, n) written: one fewer tile of its combine chunk
        if (done) wg_notify(P, P.ev_d + mt * P.nch + n * (bs.wide ? kWideBN : P.DC) / kCombineCols, -1);
        trace_task(P, g, K_GEMM2, t0, t1, t2);
        return kTaskDone;
    }
    {  // ------------------------------------------------------------------------ COMBINE
        const int c = g - bs.C;
        unsigned long long t1 = 0;
        if (P.dense && !dyn && !bs.routed) {  // (see GEMM2)
            if (!wg_wait_scan(P, bs)) return 0;
            bs.routed = true;
        }
        if (!task_combine(P, c, t1)) return 0;
        const unsigned long long t2 = now_ticks();
        count_task(P, K_COMBINE);
        __syncthreads();
        trace_task(P, g, K_COMBINE, t0, t1, t2);
        return kTaskDone;
    }
}

// One chunk of the weight prefetch (512 lines, one per thread; see prefetch_plan): line L
// is line L % 4 (W1 or W3, first or second 128 bytes) of row L / (4 pf_nt) of gate/up tile
// (L / 4) % pf_nt in task order.  Returns false when no line is left.
__device__ __forceinline__ bool prefetch_chunk(const MK_C Params &P) {
    if (P.pf_lines <= 0) return false;
    if (threadIdx.x == 0) g_sm.bcast[1] = add_relaxed(P.ctl + CTL_PF, kThreads);
    __syncthreads();
    const int l0 = g_sm.bcast[1];
    __syncthreads();
    if (l0 >= P.pf_lines) return false;
    const int L = l0 + (int)threadIdx.x;
    if (L < P.pf_lines) {
        const int per_row = 4 * P.pf_nt;
        const int r = L / per_row, rem = L - r * per_row;
        const int i = rem >> 2, c = rem & 3;
        const int Q = P.NB1 / P.S;
        const int sp = i / (P.E * Q), e = (i / Q) % P.E, n = i % Q;
        const int col = sp * (P.f / P.S) + n * kBN + (c & 1) * 64;
        const MK_G uint16_t *W = (c >> 1) ? P.W3 : P.W1;
        const uint32_t v = *(const MK_G uint32_t *)(W + (size_t)e * P.d * P.f + (size_t)r * P.f + col);
        asm volatile("" ::"v"(v));  // the value is not needed, only the line's trip through the caches
    }
    return true;
}

// Wait for a counter to reach zero (as wg_wait_zero), prefetching weight lines meanwhile.
__device__ __forceinline__ bool wg_wait_zero_prefetching(const MK_C Params &P, const MK_G int *ctr) {
    for (;;) {
        if (threadIdx.x == 0) g_sm.bcast[0] = ld_relaxed(ctr) == 0 ? 1 : 0;
        __syncthreads();
        const bool zero = g_sm.bcast[0] != 0;
        __syncthreads();
        if (zero || !prefetch_chunk(P)) break;
    }
    return wg_wait_zero(P, ctr);
}

// Static schedule: wait for this forward's scan result word (prefetching weight lines
// meanwhile), acquire, and complete the GroupGEMM layout from it.  One load gives both the
// event and the layout, where waiting on the scan event and then reading the row-tile counts
// took two round trips.  Returns false on error or watchdog.
__device__ __forceinline__ bool wg_wait_scan(const MK_C Params &P, Bases &bs) {
    const uint32_t ep = (uint32_t)g_sm.epoch;
    const MK_G unsigned long long *word = (const MK_G unsigned long long *)(P.ctl + CTL_SCAN64);
    if (P.pf_lines > 0) {
        for (;;) {
            if (threadIdx.x == 0) g_sm.bcast[0] = (uint32_t)(ld_relaxed64(word) >> 32) == ep ? 1 : 0;
            __syncthreads();
            const bool ready = g_sm.bcast[0] != 0;
            __syncthreads();
            if (ready || !prefetch_chunk(P)) break;
        }
    }
    if (threadIdx.x == 0) {
        unsigned long long v = ld_relaxed64(word);
        bool ok = true;
        const unsigned long long t0 = now_ticks();
        for (unsigned it = 1; (uint32_t)(v >> 32) != ep; ++it) {
            if (it < 64)
                __builtin_amdgcn_s_sleep(1);
            else
                __builtin_amdgcn_s_sleep(8);
            v = ld_relaxed64(word);
            if ((it & 31u) == 0) {
                if (ld_relaxed(P.ctl + CTL_ERR) != 0) {
                    ok = false;
                    break;
                }
                if ((long long)(now_ticks() - t0) > P.watchdog) {
                    set_error(P.ctl, 1 /* MOE_MK_ERR_WATCHDOG */);
                    ok = false;
                    break;
                }
            }
        }
        fence_acquire();
        g_sm.bcast[0] = ok ? 1 : 0;
        g_sm.bcast[1] = (int)(uint32_t)v;
    }
    __syncthreads();
    const bool ok = g_sm.bcast[0] != 0;
    const uint32_t v = (uint32_t)g_sm.bcast[1];
    __syncthreads();
    if (ok) complete_bases(P, bs, (int)(v & 0x7fffffffu), (int)(v >> 31));
    return ok;
}

// Dynamic pop.  A workgroup takes the next ticket with one atomic add; tickets below nImp are
// handed out without a queue slot (the router tasks, and with the all-token gate/up the top-k
// task and every gate/up tile), ticket nImp + i is queue slot i.  The holder of a ticket
// whose slot is not yet filled waits on that slot alone, so idle workgroups poll distinct
// words instead of contending for one.  Every pushed task is ready, so a filled slot runs
// at once.  Returns a task index, -1 when the ticket lies beyond the forward's task count,
// -2 on error.
__device__ __forceinline__ int wg_pop(const MK_C Params &P, const Bases &bs) {
    if (threadIdx.x == 0) {
        int g;
        const uint32_t ep = (uint32_t)g_sm.epoch;
        const int t = add_relaxed(P.ctl + CTL_QHEAD, 1);
        if (t < P.nR) {
            g = t;
        } else if (t < P.nImp) {
            // all-token gate/up: ticket nR is the top-k task (index nR), then come the gate/up
            // tiles of every expert, f range by f range
            const int u = t - P.nR - 1;
            const int sp = u < 0 ? 0 : u / bs.q1;
            g = u < 0 ? t : base_g1(bs, sp) + (u - sp * bs.q1);
        } else if (g_sm.total >= 0 && t >= g_sm.total) {
            g = -1;  // beyond the forward's tasks: nothing will fill this slot
        } else {
            const int i = t - P.nImp;
            const unsigned long long t0 = now_ticks();
            for (unsigned it = 0;; ++it) {
                if (i < P.q_cap) {
                    const unsigned long long v = ld_relaxed64(P.qslots + i);
                    if ((uint32_t)(v >> 32) == ep) {
                        g = (int)(uint32_t)v;
                        break;
                    }
                }
                if (g_sm.total < 0 && (it & 3u) == 0u) {  // the task count, until it is known
                    const unsigned long long tot =
                        ld_relaxed64((const MK_G unsigned long long *)(P.ctl + CTL_TOTAL64));
                    if ((uint32_t)(tot >> 32) == ep) {
                        g_sm.total = (int)(uint32_t)tot;
                        if (t >= g_sm.total) {
                            g = -1;
                            break;
                        }
                    }
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
                if (it < 64)
                    __builtin_amdgcn_s_sleep(1);
                else
                    __builtin_amdgcn_s_sleep(4);
            }
        }
        fence_acquire();
        g_sm.bcast[3] = g;
    }
    __syncthreads();
    const int g = g_sm.bcast[3];
    __syncthreads();
    return g;
}

// Static schedule: the next task of this workgroup.
//   Routing tasks (phase 0): workgroup w runs g = w, w + G, ... below the GroupGEMM blocks.
//   GroupGEMM positions (phase 1, once the scan's result word is out) are claimed per XCD.  Position p
// belongs to XCD p % 8 (the blocks start at multiples of 8); the workgroups of an XCD
// (w % 8 == x, as the hardware deals them) take that XCD's positions in increasing order from
// its claim counter, so tiles adjacent in the list start together and share operands in L2.
// Each XCD's list is in topological order, so the smallest unfinished task of the forward
// always has its inputs done or in progress.
//   With at least two GroupGEMM positions per workgroup, once its XCD's list has no GroupGEMM
// position left, a workgroup takes unclaimed GroupGEMM positions of the other XCDs from their
// counters (thread 0 looks at a counter first and claims only while it shows a position to
// take), so that the XCDs finish the GroupGEMM phase together even when skewed routing or
// heavy tiles give them unequal work.  In a forward with wide row tiles only down-projection
// positions are taken that way: a gate/up tile run away from its list's XCD loses the L2
// neighbours that share its weights and activations (taking those too made prefill slower),
// while a down-projection tile left at the end of a list would otherwise hold the combine up.
// Claims are monotonic, so a position seen there is at most claimed later.  Combine tasks,
// which wait for down-projection tiles and read rows written on every XCD, are then claimed
// from one counter shared by all workgroups; a workgroup reaches them only when no
// GroupGEMM position is left that it may take.  A claim is exclusive whoever makes it and a
// claimed position is always run, so every task runs exactly once.  (Other XCDs' gate/up
// positions of a wide forward are left to their own workgroups, which take their list in
// order and so reach them.)
//   A forward with no more GroupGEMM and combine positions than workgroups claims nothing:
// workgroup w runs position M1p + w (again on XCD w % 8), which spares each one a claim on a
// counter that its XCD's other workgroups hit at the same moment.
// Returns -1 when this workgroup has nothing left, -2 on an error.
struct StaticCursor {
    int g;       // next routing position (phase 0); the fixed position (phase 2)
    int phase;   // 0 routing, 1 GroupGEMM and combine claims, 2 one fixed position
    int y;       // list of XCD x + y being claimed from: 0 its own, 1..7 the others, 8 combine
    bool steal;  // take other XCDs' positions once the own list is done
};
__device__ __forceinline__ int static_next(const MK_C Params &P, Bases &bs, StaticCursor &c) {
    if (c.phase == 0) {
        if (c.g < bs.M1p) {
            const int g = c.g;
            c.g += gridDim.x;
            return g;
        }
        // (all-token gate/up: the layout is known from the start and the gate/up tiles wait for
        // nothing; the tasks that read routing results wait for the result word themselves)
        if (!P.dense && !wg_wait_scan(P, bs)) return -2;
        // (a forward of a few tiles per workgroup gains nothing from stealing, and its idle
        // workgroups would only load the counters that the busy ones claim from)
        c.steal = bs.C - bs.M1p >= 2 * (int)gridDim.x;
        c.phase = bs.total - bs.M1p <= (int)gridDim.x ? 2 : 1;
        c.g = bs.M1p + (int)blockIdx.x;
    }
    if (c.phase == 2) {
        const int g = c.g;
        c.g = 0x7fffffff;
        return g >= bs.total ? -1 : g;
    }
    const int x = blockIdx.x & 7;
    for (;;) {
        if (!c.steal || c.y < 8) {
            const int xs = (x + c.y) & 7;
            if (threadIdx.x == 0) {
                MK_G int *ctr = P.ctl + CTL_XQ + 32 * xs;
                int take = 1;
                if (c.y != 0) {  // another XCD's list: claim only while it shows a position to take
                    const int nx = bs.M1p + 8 * ld_relaxed(ctr) + xs;
                    take = nx < bs.C && (!bs.wide || nx >= bs.M1p + bs.q1p);
                }
                g_sm.bcast[3] = take ? add_relaxed(ctr, 1) : -1;
            }
            __syncthreads();
            const int cl = g_sm.bcast[3];
            __syncthreads();
            const int g = bs.M1p + 8 * cl + xs;
            if (!c.steal) return g >= bs.total ? -1 : g;
            if (cl < 0 || g >= bs.C) {  // no GroupGEMM position left in this list
                ++c.y;
                continue;
            }
            return g;
        }
        if (threadIdx.x == 0) g_sm.bcast[3] = add_relaxed(P.ctl + CTL_CQ, 1);
        __syncthreads();
        const int g = bs.C + g_sm.bcast[3];
        __syncthreads();
        return g >= bs.total ? -1 : g;
    }
}

__global__ void __launch_bounds__(kThreads, 1) moe_megakernel(Params Parg) {
    // Parg is the first kernel argument, at offset 0 of the kernel-argument segment: read it
    // there in place rather than from a private copy.
    (void)Parg;
    const MK_C Params &P = *(const MK_C Params *)__builtin_amdgcn_kernarg_segment_ptr();
    {
        // Touch every 64-byte line of the parameter block once, all at the start: the first
        // read of a line from a compute unit misses the scalar cache and waits on the
        // kernel-argument memory, which would otherwise happen inside the first task of each
        // kind that reads a new field.
        static_assert(sizeof(Params) % 4 == 0, "whole words");
        static_assert(kWideBM * 2 * kWideBN <= kRingBytes && kWideBM * 2 * kWideBN1 <= kRingBytes, "wide output tiles fit the ring");
        const MK_C uint32_t *pw = (const MK_C uint32_t *)&P;
        uint32_t acc = 0;
#pragma unroll
        for (int i = 0; i < (int)(sizeof(Params) / 4); i += 16) acc ^= pw[i];
        asm volatile("" ::"s"(acc));
    }
    if (threadIdx.x == 0) {
        g_sm.epoch = ld_relaxed(P.ctl + CTL_EPOCH);
        g_sm.total = -1;
        g_sm.bcast[0] = ld_relaxed(P.ctl + CTL_MAGIC) == kMagic;
    }
    __syncthreads();
    if (!g_sm.bcast[0]) {  // workspace never prepared: record it and touch nothing else
        if (threadIdx.x == 0) set_error(P.ctl, 8 /* MOE_MK_ERR_UNINIT */);
        if (P.err_out && blockIdx.x == 0 && threadIdx.x == 0) st_relaxed(P.err_out, 8);
        return;
    }
    Bases bs = initial_bases(P);
    if (P.dense) complete_bases(P, bs, P.E, 0);  // one row tile per expert, known before routing
    // Two task loops, each with one call site of its copy of the task code: the first runs
    // forwards without wide row tiles, and every task until a forward is known to have them;
    // the second takes over from there (with the task that found out, if any).
    StaticCursor cur;
    cur.g = blockIdx.x;
    cur.phase = 0;
    cur.y = 0;
    cur.steal = false;
    int g = -1;
    unsigned long long t0 = 0;
    bool wide_loop = false, pending = false;
    for (;;) {
        t0 = now_ticks();
        g = uni(P.sched != 0 ? wg_pop(P, bs) : static_next(P, bs, cur));
        if (g < 0) break;
        const int r = run_task<false>(P, g, bs, t0);
        if (r != kTaskDone) {
            wide_loop = pending = r == kNeedWide;
            break;
        }
        if (bs.known && bs.wide) {
            wide_loop = true;
            break;
        }
    }
    while (wide_loop) {
        if (!pending) {
            t0 = now_ticks();
            g = uni(P.sched != 0 ? wg_pop(P, bs) : static_next(P, bs, cur));
            if (g < 0) break;
        }
        pending = false;
        if (run_task<true>(P, g, bs, t0) != kTaskDone) break;
    }
    // Leave: the last workgroup out puts the control block back to its rest state.
    __syncthreads();
    wave_drain_vm();
    if (threadIdx.x == 0) {
        const int old = add_relaxed(P.ctl + CTL_EXIT, 1);
        g_sm.bcast[0] = old == (int)gridDim.x - 1;
        g_sm.bcast[1] = g_sm.bcast[0] ? ld_relaxed(P.ctl + CTL_ERR) : 0;
    }
    __syncthreads();
    if (!g_sm.bcast[0]) return;  // every other workgroup has left once this one gets here
    const int err = g_sm.bcast[1];
    if (err != 0 && P.heal) {
        // After a device error the event counters hold partial counts: zero every counter
        // this forward can have touched (the router tiles' events, the experts' events, the
        // row tiles' gate/up events and the split-reduction counters), then the rest state
        // below applies as after a clean forward.
        for (int i = threadIdx.x; i < P.T; i += kThreads) st_relaxed(P.ev_logit + i, 0);
        for (int i = threadIdx.x; i < P.E; i += kThreads) st_relaxed(P.ev_exp + i, 0);
        for (int i = threadIdx.x; i < P.mt_cap * kMaxSplits; i += kThreads) st_relaxed(P.ev_h + i, 0);
        for (int i = threadIdx.x; i < P.mt_cap * (P.d / kHalfBN); i += kThreads) st_relaxed(P.red_ctr + i, 0);
        for (int i = threadIdx.x; i < P.mt_cap * P.nch; i += kThreads) st_relaxed(P.ev_d + i, 0);
        wave_drain_vm();
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        if (err == 0 || P.heal) {
            st_relaxed(P.ctl + CTL_QHEAD, 0);
            st_relaxed(P.ctl + CTL_QTAIL, 0);
            st_relaxed(P.ctl + CTL_PF, 0);
            st_relaxed(P.ctl + CTL_EV_SCAN, 1);
            st_relaxed(P.ctl + CTL_CQ, 0);
            for (int x = 0; x < 8; ++x) st_relaxed(P.ctl + CTL_XQ + 32 * x, 0);
        }
        if (err != 0 && P.heal) {
            st_relaxed(P.ctl + CTL_EV_TOPK, 0);
            st_relaxed(P.ctl + CTL_EV_G1, 0);
            st_relaxed(P.ctl + CTL_ERR, 0);
        }
        if (P.err_out) st_relaxed(P.err_out, err);
        st_relaxed(P.ctl + CTL_EXIT, 0);
        st_relaxed(P.ctl + CTL_EPOCH, g_sm.epoch + 1);
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

// ------------------------------------------------------------------------------ unfused pipeline
// The same layer as one kernel per phase, for comparison with the megakernel: each kernel runs
// one task per workgroup with the megakernel's task code, and the kernel boundaries are the
// only synchronisation (what "Event Tensor", Problem, describes as the launch-per-kernel model
// with coarse synchronisation at kernel boundaries; a HIP graph of these launches removes
// the host launch cost but keeps the boundaries).  The GroupGEMM kernels are launched with
// the grid of the most row tiles the workspace allows; workgroups past the row tiles the scan
// found return at once.
__global__ void __launch_bounds__(kThreads, 1) moe_unfused_route(Params Parg) {
    const MK_C Params &P = *(const MK_C Params *)__builtin_amdgcn_kernarg_segment_ptr();
    int tg, eb;
    route_task_coords(P, uni((int)blockIdx.x), tg, eb);
    task_route_body(P, tg, eb);
}
__global__ void __launch_bounds__(kThreads, 1) moe_unfused_topk(Params Parg) {
    const MK_C Params &P = *(const MK_C Params *)__builtin_amdgcn_kernarg_segment_ptr();
    task_topk(P, uni((int)blockIdx.x));
}
__global__ void __launch_bounds__(kThreads, 1) moe_unfused_scan(Params Parg) {
    const MK_C Params &P = *(const MK_C Params *)__builtin_amdgcn_kernarg_segment_ptr();
    int mw = 0;
    task_scan(P, mw);
}
__global__ void __launch_bounds__(kThreads, 1) moe_unfused_group(Params Parg) {
    const MK_C Params &P = *(const MK_C Params *)__builtin_amdgcn_kernarg_segment_ptr();
    task_group(P, uni((int)blockIdx.x));
}
// Gate/up tile j = (row tile, column tile) of f range sp = blockIdx.y.
__global__ void __launch_bounds__(kThreads, 1) moe_unfused_gemm1(Params Parg) {
    const MK_C Params &P = *(const MK_C Params *)__builtin_amdgcn_kernarg_segment_ptr();
    const int mt_total = uni(ld_relaxed(P.ctl + CTL_MT_TOTAL));
    const int Q = P.NB1 / P.S, j = uni((int)blockIdx.x), sp = uni((int)blockIdx.y);
    const int mt = j / Q;
    if (mt >= mt_total) return;
    const int e = uni(P.mt_expert[mt]);
    const bool single = single_row_tile(e, mt > 0 ? uni(P.mt_expert[mt - 1]) : -1,
                                        mt + 1 < mt_total ? uni(P.mt_expert[mt + 1]) : -1);
    if (uni(ld_relaxed(P.ctl + CTL_MW)) > 0)
        task_gemm1<true>(P, e, uni(P.mt_row0[mt]), uni(P.mt_rows[mt]), sp * Q + (j - mt * Q), single);
    else
        task_gemm1<false>(P, e, uni(P.mt_row0[mt]), uni(P.mt_rows[mt]), sp * Q + (j - mt * Q), single);
}
// Down-projection tile j of f range sp = blockIdx.y.
__global__ void __launch_bounds__(kThreads, 1) moe_unfused_gemm2(Params Parg) {
    const MK_C Params &P = *(const MK_C Params *)__builtin_amdgcn_kernarg_segment_ptr();
    const int mt_total = uni(ld_relaxed(P.ctl + CTL_MT_TOTAL));
    const bool wide = uni(ld_relaxed(P.ctl + CTL_MW)) > 0;
    const int N2 = wide ? P.NB2w : P.NB2, j = uni((int)blockIdx.x), sp = uni((int)blockIdx.y);
    const int mt = j / N2;
    if (mt >= mt_total) return;
    const int e = uni(P.mt_expert[mt]);
    const bool single = single_row_tile(e, mt > 0 ? uni(P.mt_expert[mt - 1]) : -1,
                                        mt + 1 < mt_total ? uni(P.mt_expert[mt + 1]) : -1);
    if (wide)
        task_gemm2<true>(P, e, uni(P.mt_row0[mt]), uni(P.mt_rows[mt]), j - mt * N2, sp, mt, single);
    else
        task_gemm2<false>(P, e, uni(P.mt_row0[mt]), uni(P.mt_rows[mt]), j - mt * N2, sp, mt, single);
}
__global__ void __launch_bounds__(kThreads, 1) moe_unfused_combine(Params Parg) {
    const MK_C Params &P = *(const MK_C Params *)__builtin_amdgcn_kernarg_segment_ptr();
    unsigned long long t1;
    task_combine(P, uni((int)blockIdx.x), t1);
}

}  // namespace mk

// ------------------------------------------------------------------------------ launch glue
// The static schedule binds routing tasks to workgroups and has tasks spin-wait on events
// that other workgroups' tasks notify, so it relies on its grid being resident all at once.
// With cooperative set it is launched as a cooperative kernel, which the runtime refuses (an
// error, not a hang) when the grid cannot be co-resident.  The dynamic schedule never waits
// for a task bound to a workgroup (every task it hands out is ready) and is launched plainly.
hipError_t mk_launch(const mk::Params &p, int grid, hipStream_t stream, bool cooperative) {
    if (cooperative) {
        mk::Params arg = p;
        void *args[] = {&arg};
        return hipLaunchCooperativeKernel((const void *)mk::moe_megakernel, dim3(grid), dim3(mk::kThreads), args, 0,
                                          stream);
    }
    hipLaunchKernelGGL(mk::moe_megakernel, dim3(grid), dim3(mk::kThreads), 0, stream, p);
    return hipGetLastError();
}

// The unfused pipeline: seven launches on stream (grids from the host-known counts; the
// GroupGEMM grids cover the most row tiles the workspace holds).
hipError_t mk_launch_unfused(const mk::Params &p, hipStream_t stream) {
    const dim3 blk(mk::kThreads);
    hipLaunchKernelGGL(mk::moe_unfused_route, dim3(p.nR), blk, 0, stream, p);
    hipLaunchKernelGGL(mk::moe_unfused_topk, dim3(p.T), blk, 0, stream, p);
    hipLaunchKernelGGL(mk::moe_unfused_scan, dim3(1), blk, 0, stream, p);
    hipLaunchKernelGGL(mk::moe_unfused_group, dim3(p.T), blk, 0, stream, p);
    hipLaunchKernelGGL(mk::moe_unfused_gemm1, dim3(p.mt_cap * (p.NB1 / p.S), p.S), blk, 0, stream, p);
    hipLaunchKernelGGL(mk::moe_unfused_gemm2, dim3(p.mt_cap * p.NB2, p.S), blk, 0, stream, p);
    hipLaunchKernelGGL(mk::moe_unfused_combine, dim3(p.nC), blk, 0, stream, p);
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

// ------------------------------------------------------------------------------ static scratch
// The workspace of the allocation-free entry point: a file-scope device array, of which every
// GPU that loads this library holds its own copy (at its own address) until the process ends.
// In host code the name `scratch` is only a stand-in for the symbol: its device address is
// looked up once per device with hipGetSymbolAddress and kept, and only that address is ever
// passed to a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[mk::kScratchBytes];

constexpr int kMaxScratchDevices = 64;

// Device address and size of the current device's scratch (looked up on the first call for
// each device, with that device current).
hipError_t mk_scratch(void **ptr, size_t *bytes) {
    static std::mutex mu;
    static void *addr[kMaxScratchDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    *bytes = mk::kScratchBytes;
    return hipSuccess;
}

hipError_t mk_occupancy(int *blocks_per_cu) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, mk::moe_megakernel, mk::kThreads, 0);
}
