// Per-layer slot manager: map table, slot owners, LRU order, free-slot stack, counters.
//
// Follows the prepare() of vLLM PR "Run MoE models exceeding VRAM via expert CPU
// offloading with GPU cache", section "How it works" and the review thread's
// OrderedDict form: the step's distinct expert ids, ascending, one at a time; a hit
// moves the expert to the most recently used end; a miss takes the last free slot
// (free slots start as 0..N-1 and are popped from the end) or evicts the least
// recently used expert and reuses its slot.  The route rule is the llama.cpp
// "Persistent expert slot pool" prefill rule: a step that exceeds the slots takes
// the selective-copy path and leaves this state untouched (section "Why not the
// other approaches on the table").
//
// The LRU order is an intrusive doubly linked list over expert ids, so every
// operation is O(1) and a step is O(D).  Host only; no HIP.
#pragma once

#include <cstdint>
#include <vector>

namespace moe {

struct Miss {
    int32_t expert, slot, evicted;
};

class SlotLRU {
public:
    SlotLRU() = default;
    SlotLRU(int32_t n_experts, int32_t n_slots, int32_t rule) { init(n_experts, n_slots, rule); }

    void init(int32_t n_experts, int32_t n_slots, int32_t rule) {
        E_ = n_experts;
        N_ = n_slots;
        rule_ = rule;
        reset();
    }

    void reset() {
        map_.assign(E_, -1);
        owner_.assign(N_, -1);
        free_.resize(N_);
        for (int32_t s = 0; s < N_; ++s) free_[s] = s;
        prev_.assign(E_, -1);
        next_.assign(E_, -1);
        head_ = tail_ = -1;
        steps_ = hits_ = misses_ = fallbacks_ = 0;
    }

    // Route decision for a step with D distinct ids out of n_tokens * top_k.
    bool overflows(int32_t D, int64_t n_pairs) const {
        if (rule_ == 1) return n_pairs > N_ && D > 0;
        return D > N_;
    }

    // One step over the ascending distinct ids u[0..D).  Returns true for the pooled
    // path (misses appended to `out`), false for the fallback path (nothing changes
    // except the step and fallback counters).
    bool step(const int32_t* u, int32_t D, int64_t n_pairs, std::vector<Miss>& out) {
        ++steps_;
        if (overflows(D, n_pairs)) {
            ++fallbacks_;
            return false;
        }
        for (int32_t i = 0; i < D; ++i) {
            const int32_t e = u[i];
            if (map_[e] >= 0) {
                unlink(e);
                push_mru(e);
                ++hits_;
                continue;
            }
            int32_t slot, evicted;
            if (!free_.empty()) {
                slot = free_.back();
                free_.pop_back();
                evicted = -1;
            } else {
                evicted = head_;
                unlink(evicted);
                slot = map_[evicted];
                map_[evicted] = -1;
            }
            map_[e] = slot;
            owner_[slot] = e;
            push_mru(e);
            ++misses_;
            out.push_back({e, slot, evicted});
        }
        return true;
    }

    // Accounting for a step of the all-resident mode: every distinct id is a hit.
    void count_resident(int32_t D) {
        ++steps_;
        hits_ += (uint64_t)D;
    }

    int32_t n_experts() const { return E_; }
    int32_t n_slots() const { return N_; }
    const std::vector<int32_t>& map() const { return map_; }
    const std::vector<int32_t>& owner() const { return owner_; }

    // Resident experts, least recently used first; -1 padded to n.
    void lru_order(int32_t* dst, int32_t n) const {
        int32_t i = 0;
        for (int32_t e = head_; e >= 0 && i < n; e = next_[e]) dst[i++] = e;
        for (; i < n; ++i) dst[i] = -1;
    }

    uint64_t steps() const { return steps_; }
    uint64_t hits() const { return hits_; }
    uint64_t misses() const { return misses_; }
    uint64_t fallbacks() const { return fallbacks_; }

private:
    void unlink(int32_t e) {
        const int32_t p = prev_[e], n = next_[e];
        if (p >= 0) next_[p] = n; else head_ = n;
        if (n >= 0) prev_[n] = p; else tail_ = p;
        prev_[e] = next_[e] = -1;
    }
    void push_mru(int32_t e) {
        prev_[e] = tail_;
        next_[e] = -1;
        if (tail_ >= 0) next_[tail_] = e; else head_ = e;
        tail_ = e;
    }

    int32_t E_ = 0, N_ = 0, rule_ = 0;
    std::vector<int32_t> map_, owner_, free_, prev_, next_;
    int32_t head_ = -1, tail_ = -1;
    uint64_t steps_ = 0, hits_ = 0, misses_ = 0, fallbacks_ = 0;
};

}  // namespace moe
