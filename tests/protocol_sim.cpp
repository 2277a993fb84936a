// CPU model of the megakernel's task protocol, run by host threads (tests/test_protocol_sim.py).
//
// The kernel's task graph, task numbering, event counters and both schedulers are restated
// here in plain C++ with std::atomic: worker threads stand in for the persistent
// workgroups (worker w on "XCD" w % 8), counters for the event tensors, and each task
// writes and reads plain data words in place of the arrays it produces and consumes.  Each
// task sleeps a random time, so many interleavings are tried.  Checked per forward:
//   * every task runs exactly once and every output word is written;
//   * every data word a task reads was written before it (the producer's release, i.e. its
//     notify after its stores, and the consumer's acquire after its wait); built with
//     ThreadSanitizer the same run also reports any read not ordered after its write;
//   * no wait reaches the watchdog (deadlock freedom), except in the run that drops one
//     notification on purpose, where the watchdog must end the forward;
//   * the control words and every counter are back at their rest values afterwards, and
//     the next forward (next epoch) runs on the same control block.
// Shapes marked dense run the all-token gate/up of a one-tile batch: one row tile per expert
// (possibly empty), gate/up tiles that start before the scan's result word compute over every
// token and then wait for it, later ones only if their expert has rows; the scan arms the
// gate/up events with atomic adds (the tiles may have counted them down already) and whoever
// brings one to zero fires it; in the dynamic schedule the top-k task and the gate/up tiles
// are tickets without a queue slot.
// Events follow the kernel: a counter rests at 0 (the scan event at 1); producers add
// their deltas and the consumer (static) arms it with the expected count before waiting,
// so a counter may pass through negative values; the event fires when it reaches 0.
//
// Usage: protocol_sim [seed [count [watchdog_ms]]]; prints "<n> failures".  Built with -DPLANT=1 (a
// down-projection task of the static schedule that does not wait for its event) or
// -DPLANT=2 (a gate/up task that notifies twice), the checks must fail: the tests use these
// builds to show that the checks catch such mistakes.
#ifndef PLANT
#define PLANT 0
#endif
#include <algorithm>
#include <atomic>
#include <chrono>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <thread>
#include <vector>

namespace {

constexpr int kTile = 64, kBM = 64, kWideBM = 256, kChunk = 2048;
std::atomic<int> failures{0};
#define CHECK(c)                                                             \
    do {                                                                     \
        if (!(c)) {                                                          \
            std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);         \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

struct Config {
    int B, E, k, d, tpw, reb, NB1, NB2, NB2w, S, CT, W;
    bool wide_ok;
    double zipf;  // 0: uniform routing
    bool dynamic;
    bool drop_notify;
    bool dense;  // all-token gate/up (a batch of one routing tile)
};

int cdiv(int a, int b) { return (a + b - 1) / b; }
int round8(int v) { return (v + 7) & ~7; }

// ------------------------------------------------------------------ routing (given)
struct Routing {
    std::vector<int> idx;                  // [B*k]
    std::vector<int> hist, indptr;         // [E], [E+1]
    std::vector<std::vector<int>> tcnt;    // [T][E] rows of e in tile t
    std::vector<int> mt_expert, mt_row0, mt_rows, mt_base;  // row tiles
    std::vector<int> amt;                  // [B*k] row tile of assignment a
    int mw = 0;
};

Routing make_routing(const Config &c, std::mt19937_64 &rng) {
    Routing r;
    const int T = cdiv(c.B, kTile);
    std::vector<double> wt(c.E);
    for (int e = 0; e < c.E; ++e) wt[e] = c.zipf > 0 ? 1.0 / std::pow(1.0 + e, c.zipf) : 1.0;
    r.idx.resize((size_t)c.B * c.k);
    for (int b = 0; b < c.B; ++b) {
        std::vector<double> w = wt;
        for (int i = 0; i < c.k; ++i) {  // k distinct experts, drawn by weight
            std::discrete_distribution<int> dist(w.begin(), w.end());
            const int e = dist(rng);
            r.idx[(size_t)b * c.k + i] = e;
            w[e] = 0.0;
        }
    }
    r.hist.assign(c.E, 0);
    r.tcnt.assign(T, std::vector<int>(c.E, 0));
    for (int a = 0; a < c.B * c.k; ++a) {
        r.hist[r.idx[a]]++;
        r.tcnt[(a / c.k) / kTile][r.idx[a]]++;
    }
    r.indptr.assign(c.E + 1, 0);
    for (int e = 0; e < c.E; ++e) r.indptr[e + 1] = r.indptr[e] + r.hist[e];
    // row tiles per expert: wide (256 rows) above 64 rows when allowed, a remainder of at
    // most 64 rows in one narrow tile; else 64-row tiles
    r.mt_base.assign(c.E + 1, 0);
    std::vector<int> erows(c.E, kBM);
    for (int e = 0; e < c.E; ++e) {
        r.mt_base[e] = (int)r.mt_expert.size();
        const int h = r.hist[e];
        if (c.dense) {  // row tile e: all of expert e's rows (at most 64), possibly none
            r.mt_expert.push_back(e), r.mt_row0.push_back(r.indptr[e]), r.mt_rows.push_back(h);
            continue;
        }
        int done = 0;
        if (c.wide_ok && h > kBM) {
            erows[e] = kWideBM;
            while (h - done > kBM) {
                const int n = std::min(kWideBM, h - done);
                r.mt_expert.push_back(e), r.mt_row0.push_back(r.indptr[e] + done), r.mt_rows.push_back(n);
                done += n;
                r.mw++;
            }
        }
        while (done < h) {
            const int n = std::min(kBM, h - done);
            r.mt_expert.push_back(e), r.mt_row0.push_back(r.indptr[e] + done), r.mt_rows.push_back(n);
            done += n;
        }
    }
    r.mt_base[c.E] = (int)r.mt_expert.size();
    // stable grouping: row p of expert e in token order; amt = the row tile holding p
    std::vector<int> next(r.indptr.begin(), r.indptr.end() - 1);
    r.amt.resize((size_t)c.B * c.k);
    for (int a = 0; a < c.B * c.k; ++a) {
        const int e = r.idx[a], p = next[e]++;
        r.amt[a] = r.mt_base[e] + (p - r.indptr[e]) / erows[e];
    }
    return r;
}

// ------------------------------------------------------------------ one forward's model
struct Sim {
    const Config &c;
    const Routing &r;
    int T, gpt, nTG, nEB, nR, K, Sg, G, M1, M1p, mt, q1, q2, q1p, q2p, N2, bn2, nch, Cb, nC, total, Q, nImp;
    bool wide;
    uint64_t epoch;
    long long watchdog_us;
    // control block (persists across forwards)
    struct Ctl {
        std::atomic<int> qhead{0}, qtail{0}, exit{0}, err{0}, ev_topk{0}, ev_scan{1}, ev_g1{0}, cq{0};
        std::atomic<int> xq[8];
        std::atomic<uint64_t> total64{0}, scan64{0};
        Ctl() {
            for (auto &x : xq) x.store(0);
        }
    } *ctl;
    std::vector<std::atomic<uint64_t>> *slots;
    // events of this forward
    std::vector<std::atomic<int>> ev_logit, ev_exp, ev_h, ev_d, red;
    // data words (plain): written by one task, read by others after the protocol orders them
    std::vector<int> L, TH, P, H, YP, Y, OUT;
    int TAB = 0;
    // bookkeeping
    std::vector<std::atomic<int>> runs;

    Sim(const Config &c_, const Routing &r_, Ctl *ctl_, std::vector<std::atomic<uint64_t>> *slots_, uint64_t ep,
        long long wd)
        : c(c_), r(r_), epoch(ep), watchdog_us(wd), ctl(ctl_), slots(slots_) {
        T = cdiv(c.B, kTile);
        gpt = kTile / (8 * c.tpw);
        nTG = cdiv(c.B, 8 * c.tpw);
        nEB = cdiv(c.E, c.reb);
        nR = nTG * nEB;
        K = nR, Sg = K + T, G = Sg + 1, M1 = G + T, M1p = round8(M1);
        mt = (int)r.mt_expert.size();
        wide = r.mw > 0;
        N2 = wide ? c.NB2w : c.NB2;
        bn2 = wide ? 256 : 128;
        Q = c.NB1 / c.S;
        q1 = mt * Q, q2 = mt * N2, q1p = round8(q1), q2p = round8(q2);
        if (!c.dynamic && wide) {  // static, wide: XCD lists of whole row tiles, padded alike
            const int per = (mt + 7) / 8;
            q1p = 8 * per * Q, q2p = 8 * per * N2;
        }
        Cb = M1p + c.S * (q1p + q2p);
        nch = cdiv(c.d, kChunk);
        nC = cdiv(c.B, c.CT) * nch;
        total = Cb + nC;
        nImp = nR + (c.dense ? 1 + c.E * c.NB1 : 0);
        ev_logit = std::vector<std::atomic<int>>(T);
        ev_exp = std::vector<std::atomic<int>>(c.E);
        ev_h = std::vector<std::atomic<int>>((size_t)mt * c.S);
        ev_d = std::vector<std::atomic<int>>((size_t)mt * nch);
        red = std::vector<std::atomic<int>>((size_t)mt * c.NB2);
        for (auto *v : {&ev_logit, &ev_exp, &ev_h, &ev_d, &red})
            for (auto &x : *v) x.store(0);
        L.assign((size_t)nTG * nEB, 0);
        TH.assign(T, 0);
        P.assign(T, 0);
        H.assign((size_t)mt * c.NB1, 0);
        YP.assign((size_t)c.S * mt * c.NB2, 0);
        Y.assign((size_t)mt * (c.d / 128), 0);
        OUT.assign((size_t)cdiv(c.B, c.CT) * nch, 0);
        runs = std::vector<std::atomic<int>>(total);
        for (auto &x : runs) x.store(0);
    }

    int base_g1(int s) const { return s == 0 ? M1p : M1p + q1p + (s - 1) * (q1p + q2p); }
    int base_g2(int s) const { return s < c.S - 1 ? base_g1(s + 1) + q1p : M1p + c.S * q1p + (c.S - 1) * q2p; }
    int decode_gemm(bool xcd_map, int g, int &s, int &j) const {
        int o = g - M1p, kind = 0;
        if (o < q1p) {
            s = 0, kind = 1;
        } else {
            o -= q1p;
            for (int rr = 1; rr < c.S && kind == 0; ++rr) {
                if (o < q1p) {
                    s = rr, kind = 1;
                } else {
                    o -= q1p;
                    if (o < q2p) s = rr - 1, kind = 2;
                    else o -= q2p;
                }
            }
            if (kind == 0) s = c.S - 1, kind = 2;
        }
        const int cnt = kind == 1 ? q1 : q2;
        if (xcd_map) {  // XCD o % 8 takes row tiles [mt x / 8, mt (x+1) / 8)
            const int per = kind == 1 ? Q : N2, x = o & 7, r0 = mt * x / 8, r1 = mt * (x + 1) / 8, i = o >> 3;
            j = r0 * per + i;
            return i < (r1 - r0) * per ? kind : 0;
        }
        j = o;
        return j < cnt ? kind : 0;
    }
    void route_coords(int g, int &tg, int &eb) const {
        const int full = nTG & ~7;
        if (c.B > 2 * c.E && g < full * nEB) {
            const int x = g & 7, l = g >> 3, lg = l / nEB;
            tg = 8 * lg + x, eb = l - lg * nEB;
        } else {
            tg = g / nEB, eb = g - tg * nEB;
        }
    }
    int route_tasks_of_tile(int t) const {
        const int g0 = t * gpt, g1 = std::min(g0 + gpt, nTG);
        return (g1 - g0) * nEB;
    }

    // --- event helpers
    bool wait_zero(std::atomic<int> &a) {
        const auto t0 = std::chrono::steady_clock::now();
        for (unsigned it = 0;; ++it) {
            if (a.load(std::memory_order_acquire) == 0) return true;
            if (ctl->err.load(std::memory_order_relaxed)) return false;
            if ((it & 63u) == 0 &&
                std::chrono::duration_cast<std::chrono::microseconds>(std::chrono::steady_clock::now() - t0).count() >
                    watchdog_us) {
                ctl->err.fetch_or(1);
                return false;
            }
            std::this_thread::yield();
        }
    }
    // returns whether this notification fired the event (brought it to zero)
    bool notify(std::atomic<int> &a, int delta) { return a.fetch_add(delta, std::memory_order_acq_rel) + delta == 0; }
    void push_range(int g0, int cnt) {
        if (cnt <= 0) return;
        const int s0 = ctl->qtail.fetch_add(cnt, std::memory_order_relaxed);
        if (s0 + cnt > (int)slots->size()) {
            ctl->err.fetch_or(4);
            return;
        }
        for (int i = 0; i < cnt; ++i) (*slots)[s0 + i].store((epoch << 32) | (uint32_t)(g0 + i), std::memory_order_release);
    }

    // --- the tasks
    bool run(int g, std::mt19937_64 &rng) {
        if (g < 0 || g >= total) return true;
        std::uniform_int_distribution<int> dl(0, 60);
        const int delay = dl(rng);
        if (delay > 40) std::this_thread::sleep_for(std::chrono::microseconds(delay - 40));
        else if (delay > 20) std::this_thread::yield();
        const bool dyn = c.dynamic;
        if (g < K) {  // ROUTE
            runs[g]++;
            int tg, eb;
            route_coords(g, tg, eb);
            L[(size_t)tg * nEB + eb] = 1;
            const int t = tg / gpt;
            const bool push = dyn && !c.dense;  // (dense: the top-k task has a ticket and waits)
            int delta = -1;
            if (push && tg % gpt == 0 && eb == 0) delta += route_tasks_of_tile(t);
            if (notify(ev_logit[t], delta) && push) push_range(K + t, 1);
            return true;
        }
        if (g < Sg) {  // TOPK
            runs[g]++;
            const int t = g - K;
            if (!dyn || c.dense) {
                ev_logit[t].fetch_add(route_tasks_of_tile(t), std::memory_order_relaxed);  // arm
                if (!wait_zero(ev_logit[t])) return false;
            }
            for (int tg = t * gpt; tg < std::min((t + 1) * gpt, nTG); ++tg)
                for (int eb = 0; eb < nEB; ++eb) CHECK(L[(size_t)tg * nEB + eb] == 1);
            TH[t] = 1;
            if (T == 1) return fused_scan_group(dyn);
            int delta = -1;
            if (dyn && t == 0) delta += T;
            if (notify(ctl->ev_topk, delta) && dyn) push_range(Sg, 1);
            return true;
        }
        if (g == Sg) {  // SCAN
            runs[g]++;
            if (T == 1) return true;
            if (!dyn) {
                ctl->ev_topk.fetch_add(T, std::memory_order_relaxed);
                if (!wait_zero(ctl->ev_topk)) return false;
            }
            for (int t = 0; t < T; ++t) CHECK(TH[t] == 1);
            publish_tables(true);
            for (int t = 0; t < T; ++t) ev_logit[t].store(1, std::memory_order_relaxed);  // grouped event
            notify(ctl->ev_scan, -1);
            if (!dyn) publish_scan();
            if (dyn) {
                push_range(G, T);
                const int real = M1 + c.S * (q1 + q2) + nC;
                ctl->total64.store((epoch << 32) | (uint32_t)real, std::memory_order_release);
            }
            return true;
        }
        if (g < M1p) {  // GROUP
            runs[g]++;
            const int t = g - G;
            if (t >= T || T == 1) return true;
            if (!dyn && !wait_zero(ctl->ev_scan)) return false;
            CHECK(TAB == 1);
            P[t] = 1;
            notify(ev_logit[t], -1);
            for (int e = 0; e < c.E; ++e) {
                const int cnt = r.tcnt[t][e];
                if (!cnt || (c.drop_notify && t == 0 && e == first_expert(0))) continue;
                if (notify(ev_exp[e], -cnt) && dyn) push_expert(e);
            }
            return true;
        }
        if (g < Cb) {
            int sp, j;
            const int kind = decode_gemm(!dyn && wide, g, sp, j);
            runs[g]++;
            if (kind == 0) return true;
            if (kind == 1 && c.dense) {  // GEMM1, all-token gate/up: row tile m is expert m
                const int m = j / Q, n = sp * Q + j % Q;
                if (!scan_seen()) {  // before the routing: every token, then wait for it
                    if (!wait_scan()) return false;
                }
                CHECK(TAB == 1 && P[0] == 1);  // the tables and perm/inv it keeps rows by
                H[(size_t)m * c.NB1 + n] = 1;
                if (PLANT == 2 && m == 0 && n == 0) notify(ev_h[(size_t)m * c.S + sp], -1);
                if (notify(ev_h[(size_t)m * c.S + sp], -1) && dyn) {
                    CHECK(TAB == 1);
                    if (r.mt_rows[m] > 0) push_range(base_g2(sp) + m * N2, N2);
                    if (notify(ctl->ev_g1, -1)) push_range(Cb, nC);
                }
                return true;
            }
            if (kind == 1) {  // GEMM1
                const int m = j / Q, n = sp * Q + j % Q, e = r.mt_expert[m];
                // a one-tile batch was grouped before the layout was published: no wait
                if (!dyn && (T > 1 || c.drop_notify) && !wait_zero(ev_exp[e])) return false;
                for (int t = 0; t < T; ++t)
                    if (r.tcnt[t][e]) CHECK(P[t] == 1);
                H[(size_t)m * c.NB1 + n] = 1;
                if (PLANT == 2 && m == 0 && n == 0) notify(ev_h[(size_t)m * c.S + sp], -1);
                if (notify(ev_h[(size_t)m * c.S + sp], -1) && dyn) {
                    push_range(base_g2(sp) + m * N2, N2);
                    if (notify(ctl->ev_g1, -1)) push_range(Cb, nC);
                }
                return true;
            }
            // GEMM2
            const int m = j / N2, n = j % N2;
            if (c.dense && !dyn && !wait_scan()) return false;  // the layout was known without it
            if (c.dense && r.mt_rows[m] == 0) return true;       // an expert without tokens
            if (!dyn && PLANT != 1 && !wait_zero(ev_h[(size_t)m * c.S + sp])) return false;
            for (int nn = sp * Q; nn < (sp + 1) * Q; ++nn) CHECK(H[(size_t)m * c.NB1 + nn] == 1);
            bool done = true;
            if (wide) {  // 256 columns: two 128-column y tiles
                Y[(size_t)m * (c.d / 128) + 2 * n] = 1;
                Y[(size_t)m * (c.d / 128) + 2 * n + 1] = 1;
            } else if (c.S == 1) {
                Y[(size_t)m * (c.d / 128) + n] = 1;
            } else {  // split f: partial, then the last finisher adds the partials in order
                YP[((size_t)sp * mt + m) * c.NB2 + n] = 1;
                const int old = red[(size_t)m * c.NB2 + n].fetch_add(1, std::memory_order_acq_rel);
                done = old == c.S - 1;
                if (done) {
                    red[(size_t)m * c.NB2 + n].store(0, std::memory_order_relaxed);
                    for (int q = 0; q < c.S; ++q) CHECK(YP[((size_t)q * mt + m) * c.NB2 + n] == 1);
                    Y[(size_t)m * (c.d / 128) + n] = 1;
                }
            }
            if (done) notify(ev_d[(size_t)m * nch + n * bn2 / kChunk], -1);
            return true;
        }
        // COMBINE
        runs[g]++;
        const int cc = g - Cb, grp = cc / nch, chunk = cc % nch;
        const int b_lo = grp * c.CT, nb = std::min(c.CT, c.B - b_lo);
        if (c.dense && !dyn && !wait_scan()) return false;
        if (T > 1 && !wait_zero(ev_logit[b_lo / kTile])) return false;
        CHECK(P[b_lo / kTile] == 1);
        for (int i = 0; i < nb * c.k; ++i)
            if (!wait_zero(ev_d[(size_t)r.amt[(size_t)b_lo * c.k + i] * nch + chunk])) return false;
        for (int i = 0; i < nb * c.k; ++i) {
            const int m = r.amt[(size_t)b_lo * c.k + i];
            for (int col = chunk * kChunk; col < std::min(c.d, (chunk + 1) * kChunk); col += 128)
                CHECK(Y[(size_t)m * (c.d / 128) + col / 128] == 1);
        }
        OUT[cc] = 1;
        return true;
    }
    // static: the scan's result word (epoch, row tiles, wide), stored after the scan's tables
    bool scan_seen() const { return (ctl->scan64.load(std::memory_order_acquire) >> 32) == epoch; }
    void publish_scan() {
        ctl->scan64.store((epoch << 32) | (wide ? 0x80000000ull : 0ull) | (uint32_t)mt, std::memory_order_release);
    }
    bool wait_scan() {
        const auto t0 = std::chrono::steady_clock::now();
        for (unsigned it = 0;; ++it) {
            const uint64_t v = ctl->scan64.load(std::memory_order_acquire);
            if ((v >> 32) == epoch) {
                CHECK((int)(v & 0x7fffffff) == mt && ((v >> 31) & 1) == (uint64_t)wide);
                return true;
            }
            if (ctl->err.load(std::memory_order_relaxed)) return false;
            if ((it & 63u) == 0 &&
                std::chrono::duration_cast<std::chrono::microseconds>(std::chrono::steady_clock::now() - t0).count() >
                    watchdog_us) {
                ctl->err.fetch_or(1);
                return false;
            }
            std::this_thread::yield();
        }
    }
    int first_expert(int t) const {
        for (int e = 0; e < c.E; ++e)
            if (r.tcnt[t][e]) return e;
        return -1;
    }
    void publish_tables(bool arm_exp) {
        TAB = 1;
        for (int e = 0; e < c.E; ++e)
            if (arm_exp && r.hist[e]) ev_exp[e].store(r.hist[e], std::memory_order_relaxed);
        for (int m = 0; m < mt; ++m) {
            if (c.dense && r.mt_rows[m] == 0) continue;  // no down projection, no combine reads it
            if (!c.dense)  // (dense: armed by atomic adds, see fused_scan_group)
                for (int s = 0; s < c.S; ++s) ev_h[(size_t)m * c.S + s].store(Q, std::memory_order_relaxed);
            for (int ch = 0; ch < nch; ++ch)
                ev_d[(size_t)m * nch + ch].store(std::min(kChunk, c.d - ch * kChunk) / bn2, std::memory_order_relaxed);
        }
        if (c.dynamic) ctl->ev_g1.store(c.S * mt, std::memory_order_relaxed);
    }
    void push_expert(int e) {  // the gate/up tiles of expert e's row tiles, every f range
        const int m0 = r.mt_base[e], nm = r.mt_base[e + 1] - m0;
        for (int s = 0; s < c.S; ++s) push_range(base_g1(s) + m0 * Q, nm * Q);
    }
    bool fused_scan_group(bool dyn) {  // a batch of one routing tile: scan and grouping in top-k
        publish_tables(false);  // the experts' events stay at rest: no grouping task decrements them
        P[0] = 1;
        if (c.dense) {
            int active = 0;
            for (int e = 0; e < c.E; ++e) active += r.hist[e] > 0;
            if (dyn) {
                const int real = K + 1 + c.S * (q1 + active * N2) + nC;
                ctl->total64.store((epoch << 32) | (uint32_t)real, std::memory_order_release);
            }
            const int skip = c.drop_notify ? first_expert(0) : -1;
            for (int e = 0; e < c.E; ++e)
                for (int s = 0; s < c.S; ++s) {
                    const int arm = e == skip ? Q + 1 : Q;  // (a dropped notification: never fires)
                    if (!notify(ev_h[(size_t)e * c.S + s], arm) || !dyn) continue;
                    if (r.mt_rows[e] > 0) push_range(base_g2(s) + e * N2, N2);
                    if (notify(ctl->ev_g1, -1)) push_range(Cb, nC);
                }
            if (!dyn) notify(ctl->ev_scan, -1);
            publish_scan();
            return true;
        }
        if (dyn) {
            const int real = K + 1 + c.S * (q1 + q2) + nC;
            ctl->total64.store((epoch << 32) | (uint32_t)real, std::memory_order_release);
            for (int e = 0; e < c.E; ++e)
                if (r.hist[e] && !(c.drop_notify && e == first_expert(0))) push_expert(e);
            return true;
        }
        if (c.drop_notify) ev_exp[first_expert(0)].store(1, std::memory_order_relaxed);  // a wait that never ends
        notify(ctl->ev_scan, -1);
        publish_scan();
        return true;
    }

    // --- schedulers
    struct Cursor {
        int g, phase = 0, y = 0;
        bool steal = false;
    };
    int static_next(int w, Cursor &cu) {
        if (cu.phase == 0) {
            if (cu.g < M1p) {
                const int g = cu.g;
                cu.g += c.W;
                return g;
            }
            if (!c.dense && !wait_scan()) return -2;  // (dense: the layout is known from the start)
            cu.steal = Cb - M1p >= 2 * c.W;
            cu.phase = total - M1p <= c.W ? 2 : 1;
            cu.g = M1p + w;
        }
        if (cu.phase == 2) {
            const int g = cu.g;
            cu.g = INT_MAX;
            return g >= total ? -1 : g;
        }
        const int x = w & 7;
        for (;;) {
            if (!cu.steal || cu.y < 8) {
                const int xs = (x + cu.y) & 7;
                bool take = true;
                if (cu.y != 0) {  // other XCDs' lists: wide forwards take down-projection positions only
                    const int nx = M1p + 8 * ctl->xq[xs].load() + xs;
                    take = nx < Cb && (!wide || nx >= M1p + q1p);
                }
                const int cl = take ? ctl->xq[xs].fetch_add(1) : -1;
                const int g = M1p + 8 * cl + xs;
                if (!cu.steal) return g >= total ? -1 : g;
                if (cl < 0 || g >= Cb) {
                    ++cu.y;
                    continue;
                }
                return g;
            }
            const int g = Cb + ctl->cq.fetch_add(1);
            return g >= total ? -1 : g;
        }
    }
    int pop(int &known_total) {
        const int t = ctl->qhead.fetch_add(1);
        if (t < nR) return t;
        if (t < nImp) {  // dense: the top-k task, then every gate/up tile, f range by f range
            const int u = t - nR - 1;
            if (u < 0) return t;
            const int sp = u / q1;
            return base_g1(sp) + (u - sp * q1);
        }
        if (known_total >= 0 && t >= known_total) return -1;
        const int i = t - nImp;
        const auto t0 = std::chrono::steady_clock::now();
        for (unsigned it = 0;; ++it) {
            if (i < (int)slots->size()) {
                const uint64_t v = (*slots)[i].load(std::memory_order_acquire);
                if ((v >> 32) == epoch) return (int)(uint32_t)v;
            }
            if (known_total < 0) {
                const uint64_t tot = ctl->total64.load(std::memory_order_acquire);
                if ((tot >> 32) == epoch) {
                    known_total = (int)(uint32_t)tot;
                    if (t >= known_total) return -1;
                }
            }
            if (ctl->err.load(std::memory_order_relaxed)) return -2;
            if ((it & 63u) == 0 &&
                std::chrono::duration_cast<std::chrono::microseconds>(std::chrono::steady_clock::now() - t0).count() >
                    watchdog_us) {
                ctl->err.fetch_or(1);
                return -2;
            }
            std::this_thread::yield();
        }
    }
    void worker(int w, uint64_t seed) {
        std::mt19937_64 rng(seed);
        Cursor cu;
        cu.g = w;
        int known_total = -1;
        for (;;) {
            const int g = c.dynamic ? pop(known_total) : static_next(w, cu);
            if (g < 0) break;
            if (!run(g, rng)) break;
        }
        // the last worker out puts the control block back to its rest state
        if (ctl->exit.fetch_add(1, std::memory_order_acq_rel) == c.W - 1) {
            const int err = ctl->err.load();
            if (err) {  // after an error the counters hold partial counts
                for (auto *v : {&ev_logit, &ev_exp, &ev_h, &ev_d, &red})
                    for (auto &x : *v) x.store(0);
                ctl->ev_topk.store(0), ctl->ev_g1.store(0);
            }
            ctl->qhead.store(0), ctl->qtail.store(0), ctl->ev_scan.store(1), ctl->cq.store(0);
            for (auto &x : ctl->xq) x.store(0);
            ctl->exit.store(0, std::memory_order_release);
        }
    }
};

// Runs one forward; returns the error word.
int forward(const Config &c, const Routing &r, Sim::Ctl &ctl, std::vector<std::atomic<uint64_t>> &slots, uint64_t epoch,
            uint64_t seed, long long watchdog_us, bool check) {
    Sim s(c, r, &ctl, &slots, epoch, watchdog_us);
    std::vector<std::thread> th;
    for (int w = 0; w < c.W; ++w) th.emplace_back([&s, w, seed] { s.worker(w, seed * 1315423911ull + (uint64_t)w); });
    for (auto &t : th) t.join();
    const int err = ctl.err.load();
    if (!check) return err;
    // every task exactly once, every output written.  The static schedule walks every
    // position (padding and the no-op scan/grouping positions of a one-tile batch included);
    // the dynamic one runs only what was pushed.
    for (int g = 0; g < s.total; ++g) {
        int expect = 1;
        if (c.dynamic) {
            if (g == s.Sg) expect = s.T > 1;
            else if (g >= s.G && g < s.M1p) expect = s.T > 1 && g - s.G < s.T;
            else if (g >= s.M1p && g < s.Cb) {
                int sp, j;
                const int kind = s.decode_gemm(false, g, sp, j);
                expect = kind != 0;
                if (c.dense && kind == 2) expect = r.mt_rows[j / s.N2] > 0;  // pushed only with rows
            }
        }
        if (s.runs[g].load() != expect) {
            std::printf("FAIL task %d ran %d times, expected %d (B=%d E=%d k=%d dyn=%d)\n", g, s.runs[g].load(),
                        expect, c.B, c.E, c.k, (int)c.dynamic);
            ++failures;
            break;
        }
    }
    for (size_t i = 0; i < s.OUT.size(); ++i) CHECK(s.OUT[i] == 1);
    // rest state
    for (auto *v : {&s.ev_logit, &s.ev_exp, &s.ev_h, &s.ev_d, &s.red})
        for (auto &x : *v) CHECK(x.load() == 0);
    CHECK(ctl.ev_topk.load() == 0 && ctl.ev_scan.load() == 1 && ctl.ev_g1.load() == 0);
    CHECK(ctl.qhead.load() == 0 && ctl.qtail.load() == 0 && ctl.cq.load() == 0 && ctl.exit.load() == 0);
    for (auto &x : ctl.xq) CHECK(x.load() == 0);
    return err;
}

}  // namespace

int main(int argc, char **argv) {
    const uint64_t seed0 = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
    const int count = argc > 2 ? std::atoi(argv[2]) : 1;
    const long long watchdog_us = (argc > 3 ? std::atoll(argv[3]) : 20000) * 1000;
    // shapes: one routing tile, several tiles, splits of the down projection, wide row tiles
    // with thin remainders, skewed (Zipf) routing, k = 1 and large k
    //            B     E   k   d    tpw reb NB1 NB2 NB2w S  CT  W   wide  zipf
    const Config shapes[] = {
        {1,     8,  2,  512,  1, 4,  4,  4, 2,  1, 1,  16, false, 0.0},
        {16,    8,  2,  256,  1, 4,  4,  2, 1,  1, 1,  16, true,  0.0},
        {57,   64,  6, 2048,  1, 4, 11, 16, 8,  1, 1,  16, true,  0.0},
        {32,    8,  2, 4096,  1, 4, 28, 32, 16, 4, 1,  24, false, 0.0},
        {203,  16,  4, 2048,  4, 16, 4, 16, 8,  2, 4,  16, false, 1.2},
        {700,  16,  2,  512,  4, 16, 2,  4, 2,  1, 4,  16, true,  0.0},
        {1500, 16,  8, 2304,  8, 16, 3, 18, 9,  1, 8,  24, true,  0.0},
        {600,  16,  4,  256,  4, 16, 2,  2, 1,  1, 4,  16, true,  1.2},
        {130,  64,  1,  256,  4, 16, 2,  2, 1,  1, 4,  16, true,  1.2},
        // all-token gate/up (dense): the tiny layer, the sweep at B = 57 and 16, a split down
        // projection, and Zipf routing that leaves experts without tokens
        {16,    8,  2,  256,  1, 4,  4,  2, 1,  1, 1,  16, false, 0.0, false, false, true},
        {57,   64,  6, 2048,  1, 4, 11, 16, 8,  1, 1,  16, false, 0.0, false, false, true},
        {16,   64,  6, 2048,  1, 4, 11, 16, 8,  1, 1,  24, false, 0.0, false, false, true},
        {32,    8,  2, 4096,  1, 4, 112, 32, 16, 4, 1,  16, false, 0.0, false, false, true},
        {48,   16,  6,  256,  1, 4,  3,  2, 1,  1, 1,  16, false, 2.0, false, false, true},
    };
    std::vector<std::atomic<uint64_t>> slots(1 << 16);
    for (auto &s : slots) s.store(0);
    Sim::Ctl ctl;
    uint64_t epoch = 1;
    int runs = 0;
    for (int rep = 0; rep < count; ++rep) {
        for (const Config &base : shapes) {
            for (int dyn = 0; dyn < 2; ++dyn) {
                Config c = base;
                c.dynamic = dyn != 0;
                c.drop_notify = false;
                std::mt19937_64 rng(seed0 * 7919ull + (uint64_t)rep * 104729ull + (uint64_t)c.B * 31 + (uint64_t)dyn);
                const Routing r = make_routing(c, rng);
                for (int f = 0; f < 2; ++f) {  // two forwards back to back on one control block
                    const int err = forward(c, r, ctl, slots, epoch++, rng(), watchdog_us, true);
                    if (err) {
                        std::printf("FAIL error word %d (B=%d E=%d k=%d dyn=%d)\n", err, c.B, c.E, c.k, dyn);
                        ++failures;
                        ctl.err.store(0);
                    }
                    ++runs;
                }
            }
        }
    }
    // a dropped notification must end the forward through the watchdog, then the control
    // block is usable again
    for (int dyn = 0; dyn < 2; ++dyn)
        for (const Config *bp : {&shapes[2], &shapes[4], &shapes[10]}) {
            Config c = *bp;
            c.dynamic = dyn != 0;
            c.drop_notify = true;
            std::mt19937_64 rng(seed0 + 17 + (uint64_t)dyn);
            const Routing r = make_routing(c, rng);
            const int err = forward(c, r, ctl, slots, epoch++, rng(), 200'000, false);
            CHECK(err & 1);
            ctl.err.store(0);
            c.drop_notify = false;
            CHECK(forward(c, r, ctl, slots, epoch++, rng(), watchdog_us, true) == 0);
        }
    std::printf("%d forwards, %d failures\n", runs, failures.load());
    return failures.load() != 0;
}
