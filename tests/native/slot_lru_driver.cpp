// Test driver for the host slot manager (csrc/slot_lru.hpp), built by
// tests/test_native_sanitized.py with AddressSanitizer and UndefinedBehaviorSanitizer
// on the host compiler.  Reads "E N rule steps" then, per step, "T K" and T*K ids;
// prints per step the path and the miss list, then the map, owners, LRU order and the
// counters, for comparison with the oracle.
#include <algorithm>
#include <cstdio>
#include <vector>

#include "slot_lru.hpp"

int main() {
    int E, N, rule, steps;
    if (std::scanf("%d %d %d %d", &E, &N, &rule, &steps) != 4) return 2;
    moe::SlotLRU lru(E, N, rule);
    std::vector<moe::Miss> misses;
    for (int s = 0; s < steps; ++s) {
        int T, K;
        if (std::scanf("%d %d", &T, &K) != 2) return 2;
        std::vector<int> ids((size_t)T * K);
        for (auto& v : ids)
            if (std::scanf("%d", &v) != 1) return 2;
        std::vector<int> u(ids);
        std::sort(u.begin(), u.end());
        u.erase(std::unique(u.begin(), u.end()), u.end());
        misses.clear();
        const bool pooled = lru.step(u.data(), (int)u.size(), (long long)T * K, misses);
        std::printf("step %d %zu", pooled ? 0 : 1, misses.size());
        for (const auto& m : misses) std::printf(" %d %d %d", m.expert, m.slot, m.evicted);
        std::printf("\n");
    }
    std::printf("map");
    for (int v : lru.map()) std::printf(" %d", v);
    std::printf("\nowner");
    for (int v : lru.owner()) std::printf(" %d", v);
    std::vector<int> order(N > 0 ? N : 1);
    lru.lru_order(order.data(), N);
    std::printf("\norder");
    for (int i = 0; i < N; ++i) std::printf(" %d", order[i]);
    std::printf("\ncounters %llu %llu %llu %llu\n", (unsigned long long)lru.steps(), (unsigned long long)lru.hits(),
                (unsigned long long)lru.misses(), (unsigned long long)lru.fallbacks());
    return 0;
}
