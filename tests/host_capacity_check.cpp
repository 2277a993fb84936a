// Host-logic check of the workspace capacity lookup (built and run by
// tests/test_host_layout.py with g++ and threads, no GPU): two threads look up the capacity
// of workspaces of alternating sizes for one plan at the same time, and every answer must
// equal the bisection done from scratch (the largest B whose requirement fits).
#include <atomic>
#include <cstdio>
#include <thread>
#include <vector>

#include "mk_capacity.h"

using namespace mk;

static int64_t brute_capacity(const Shape &s, size_t bytes) {
    int64_t lo = 0, hi = ((int64_t)1 << 31) / s.k;
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo + 1) / 2;
        if (make_layout(s, mid < 1 ? 1 : mid).total <= bytes)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

int main() {
    const Shape s{128, 8, 2048, 768};
    const uint64_t plan_id = 42;
    std::vector<size_t> sizes;
    std::vector<int64_t> expect;
    for (int64_t B : {1, 7, 64, 65, 512, 4096, 16384}) {
        sizes.push_back(workspace_bytes_for(s, B));
        sizes.push_back(workspace_bytes_for(s, B) - 1);
    }
    for (size_t b : sizes) expect.push_back(brute_capacity(s, b));
    std::atomic<int> fails{0};
    auto worker = [&](int t) {
        for (int it = 0; it < 20000; ++it) {
            const size_t i = (size_t)(it * 3 + t) % sizes.size();
            const int64_t cap = workspace_capacity(s, plan_id, sizes[i]);
            if (cap != expect[i]) fails.fetch_add(1);
            if (cap > 0 && make_layout(s, cap).total > sizes[i]) fails.fetch_add(1);
        }
    };
    std::thread a(worker, 0), b(worker, 1);
    a.join();
    b.join();
    std::printf("%zu sizes, %d failures\n", sizes.size(), fails.load());
    return fails.load() != 0;
}
