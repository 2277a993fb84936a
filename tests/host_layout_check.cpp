// Host-logic check of the workspace layout (built and run by tests/test_host_layout.py with
// g++, no GPU): for a range of layer shapes and workspace capacities, the layout grows with
// the capacity, and a workspace sized for `cap` tokens holds every array of every batch
// B <= cap under adversarial routing (row tiles, task indices, queue slots, trace records,
// split partial buffers).
#include <algorithm>
#include <cstdio>
#include <vector>

#include "mk_common.h"

using namespace mk;

static int fails = 0;
#define CHECK(cond, ...)                 \
    do {                                 \
        if (!(cond)) {                   \
            ++fails;                     \
            std::printf("FAIL %s: ", #cond); \
            std::printf(__VA_ARGS__);    \
            std::printf("\n");           \
        }                                \
    } while (0)

static int64_t round8(int64_t v) { return (v + 7) / 8 * 8; }

// Row tiles of BM rows over a histogram.
static int64_t row_tiles(const std::vector<int64_t> &h, int64_t BM) {
    int64_t n = 0;
    for (int64_t v : h) n += (v + BM - 1) / BM;
    return n;
}

// Histograms of B tokens with k distinct experts each (so h[e] <= B) that stress the tile
// count: spread evenly, as many experts as possible with BM + 1 rows, all on the first k.
static std::vector<std::vector<int64_t>> histograms(int64_t B, int64_t E, int64_t k, int64_t BM) {
    std::vector<std::vector<int64_t>> out;
    const int64_t A = B * k;
    std::vector<int64_t> even(E, A / E);
    for (int64_t e = 0; e < A % E; ++e) ++even[e];
    out.push_back(even);
    std::vector<int64_t> lumpy(E, 0);
    int64_t left = A;
    for (int64_t e = 0; e < E && left > 0; ++e) {
        const int64_t v = std::min({left, B, BM + 1});
        lumpy[e] = v;
        left -= v;
    }
    for (int64_t e = 0; e < E && left > 0; ++e) {  // whatever is left, up to B per expert
        const int64_t v = std::min(left, B - lumpy[e]);
        lumpy[e] += v;
        left -= v;
    }
    out.push_back(lumpy);
    std::vector<int64_t> first(E, 0);
    for (int64_t e = 0; e < k; ++e) first[e] = B;
    out.push_back(first);
    return out;
}

int main() {
    const Shape shapes[] = {{8, 2, 4096, 14336}, {64, 6, 2048, 1408}, {256, 8, 7168, 2048}, {128, 8, 2048, 768},
                            {8, 2, 256, 512},    {1, 1, 128, 128},    {256, 16, 256, 256},  {5, 3, 128, 128},
                            {4, 2, 256, 8192},   {20, 2, 512, 128}};
    const int64_t caps[] = {1, 3, 16, 57, 64, 65, 128, 512, 513, 1024, 1025, 4096, 16384};
    int cases = 0;
    for (const Shape &s : shapes) {
        size_t prev = 0;
        for (int64_t cap : caps) {
            if (cap * s.k >= (int64_t)1 << 31) continue;
            const Layout L = make_layout(s, cap);
            CHECK(L.total >= prev, "E=%d k=%d d=%d f=%d cap=%lld: total %zu < %zu", s.E, s.k, s.d, s.f,
                  (long long)cap, L.total, prev);
            prev = L.total;
            const Counts cc = make_counts(s, cap);
            const int64_t records = cc.q_cap + cc.nR_max;  // trace records the layout holds
            const int64_t Acap = cap * s.k;
            for (int64_t B : {(int64_t)1, std::max<int64_t>(1, cap / 2), std::max<int64_t>(1, cap - 1), cap}) {
                const Counts c = make_counts(s, B);
                const Tiles t = tile_config(s, B);
                const int64_t A = B * s.k;
                CHECK(c.nR <= cc.nR_max, "nR %lld > nR_max %lld", (long long)c.nR, (long long)cc.nR_max);
                // row tiles: an expert's wide tiling never has more tiles than its narrow
                // one (nor more down-projection tiles: NB2w < NB2), so the narrow counts bound
                // every mix of shapes the kernel can choose
                for (const auto &h : histograms(B, s.E, s.k, kBM)) {
                    ++cases;
                    const int64_t mt = row_tiles(h, kBM);
                    CHECK(mt <= cc.mt_cap, "E=%d k=%d B=%lld cap=%lld: row tiles %lld > mt_cap %lld", s.E, s.k,
                          (long long)B, (long long)cap, (long long)mt, (long long)cc.mt_cap);
                    // task indices of the static layout: routing, padded GroupGEMM blocks, combine
                    const int64_t M1 = c.nR + 2 * c.T + 1;
                    const int64_t q1 = mt * (t.NB1 / t.S), q2 = mt * t.NB2;
                    const int64_t total = round8(M1) + t.S * (round8(q1) + round8(q2)) + c.nC;
                    CHECK(total <= records, "E=%d k=%d B=%lld cap=%lld: %lld tasks > %lld trace records", s.E, s.k,
                          (long long)B, (long long)cap, (long long)total, (long long)records);
                    // static schedule with wide row tiles: XCD lists of whole row tiles, each
                    // padded to ceil(mt / 8) row tiles (at most as many row tiles as narrow)
                    if (t.wide_ok) {
                        const int64_t per = (mt + 7) / 8;
                        const int64_t tw = round8(M1) + 8 * per * (t.NB1 / t.S) + 8 * per * t.NB2w + c.nC;
                        CHECK(tw <= records, "E=%d k=%d B=%lld cap=%lld: %lld wide-layout tasks > %lld trace records",
                              s.E, s.k, (long long)B, (long long)cap, (long long)tw, (long long)records);
                    }
                    // dynamic queue: every pushed task (top-k, grouping, both GEMMs, combine) has a slot
                    const int64_t pushed = 2 * c.T + 1 + t.S * (q1 + q2) + c.nC;
                    CHECK(pushed <= cc.q_cap, "E=%d k=%d B=%lld cap=%lld: %lld pushes > q_cap %lld", s.E, s.k,
                          (long long)B, (long long)cap, (long long)pushed, (long long)cc.q_cap);
                }
                // fp32 partials of a split down projection: S planes of B*k rows of d
                if (t.S > 1) {
                    const size_t need = (size_t)t.S * A * s.d * 4;
                    CHECK(t.S <= max_down_splits(s), "S %d > max %d", t.S, max_down_splits(s));
                    const size_t have = (size_t)max_down_splits(s) * std::min<int64_t>(Acap, 1024) * s.d * 4;
                    CHECK(need <= have, "E=%d B=%lld: split partials %zu > %zu", s.E, (long long)B, need, have);
                    CHECK(L.red_ctr - L.yp >= need, "yp region too small");
                }
                CHECK(L.h - L.inv >= (size_t)A * 4 && L.y - L.h >= (size_t)A * s.f * 2, "h region");
                if (all_token_gate_up(s, B)) {
                    // one row tile per expert, every expert's gate/up tiles in the static layout
                    // and the trace, down-projection tasks pushed per expert
                    ++cases;
                    CHECK(A >= s.E && s.E <= cc.mt_cap, "E=%d B=%lld cap=%lld: all-token row tiles %d > mt_cap %lld",
                          s.E, (long long)B, (long long)cap, s.E, (long long)cc.mt_cap);
                    const int64_t M1 = c.nR + 2 * c.T + 1;
                    const int64_t total = round8(M1) + t.S * (round8(s.E * (t.NB1 / t.S)) + round8(s.E * t.NB2)) + c.nC;
                    CHECK(total <= records, "E=%d B=%lld cap=%lld: all-token tasks %lld > %lld trace records", s.E,
                          (long long)B, (long long)cap, (long long)total, (long long)records);
                    const int64_t pushed = t.S * s.E * t.NB2 + c.nC;
                    CHECK(pushed <= cc.q_cap, "E=%d B=%lld cap=%lld: all-token pushes %lld > q_cap %lld", s.E,
                          (long long)B, (long long)cap, (long long)pushed, (long long)cc.q_cap);
                }
                CHECK(L.yp - L.y >= (size_t)A * s.d * 2, "y region");
            }
        }
    }
    // the requirement grows with the capacity at every step (the capacity lookup bisects it)
    for (const Shape &s : shapes) {
        size_t prev = 0;
        for (int64_t cap = 1; cap <= 2200; ++cap) {
            const size_t t = make_layout(s, cap).total;
            CHECK(t >= prev, "E=%d k=%d d=%d f=%d cap=%lld: total %zu < %zu", s.E, s.k, s.d, s.f, (long long)cap,
                  t, prev);
            prev = t;
        }
    }
    // the per-batch policies of the named workloads: which forwards run the all-token gate/up
    // (an expert idle with probability <= 1/4 in a one-tile batch), the width of the narrow
    // down-projection tasks, the down-projection splits and the half-width tiles
    {
        struct Case {
            Shape s;
            int64_t B;
            bool all_token;
            int dc, S, BN;
        };
        const Case pol[] = {
            {{8, 2, 4096, 14336}, 32, true, 256, 4, 128},    // Mixtral decode
            {{8, 2, 4096, 14336}, 4, false, 256, 4, 128},    // Mixtral, a batch of 4: idle p = 0.32
            {{64, 6, 2048, 1408}, 1, false, 64, 1, 64},      // sweep B = 1: half width
            {{64, 6, 2048, 1408}, 3, false, 128, 1, 128},    // sweep B = 3: 18 x 8 pair tasks < 256
            {{64, 6, 2048, 1408}, 16, true, 256, 1, 128},    // sweep B = 16: idle p = 0.21
            {{64, 6, 2048, 1408}, 57, true, 256, 1, 128},
            {{64, 6, 2048, 1408}, 128, false, 256, 1, 128},  // two routing tiles
            {{256, 8, 7168, 2048}, 128, false, 256, 1, 128}, // DeepSeek-shaped
            {{128, 8, 2048, 768}, 4096, false, 256, 1, 128}, // prefill
            {{8, 2, 256, 512}, 16, true, 128, 1, 128},       // tiny: 8 experts x 1 pair task < 256
        };
        for (const Case &c : pol) {
            ++cases;
            const Tiles t = tile_config(c.s, c.B);
            CHECK(all_token_gate_up(c.s, c.B) == c.all_token, "E=%d B=%lld: all-token %d", c.s.E, (long long)c.B,
                  (int)all_token_gate_up(c.s, c.B));
            CHECK(t.DC == c.dc && t.S == c.S && t.BN == c.BN, "E=%d B=%lld: DC %d S %d BN %d", c.s.E, (long long)c.B,
                  t.DC, t.S, t.BN);
        }
    }
    std::printf("%d cases, %d failures\n", cases, fails);
    return fails != 0;
}
