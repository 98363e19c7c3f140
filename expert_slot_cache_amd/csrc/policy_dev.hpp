// The slot manager's decision as device code, shared by the launches that need it
// (the prepare launch, which also copies the step's experts, and the fused decode
// step, whose workgroups each know their own expert from it).
//
// The rule is the one of vLLM PR "Run MoE models exceeding VRAM via expert CPU
// offloading with GPU cache" (section "How it works"; the eviction policies its
// review thread lists): the step's distinct ids ascending, one at a time; a hit
// records the use, a miss takes the last free slot (free slots start as 0..N-1) or
// the slot of the victim -- the resident expert, not yet processed by this step,
// with the smallest key under the layer's policy.  The route rule is the llama.cpp
// "Persistent expert slot pool" prefill rule: a step that exceeds the slots takes the
// selective-copy path and leaves the state untouched.
//
// Every workgroup that runs the decision reads the layer's current state copy into
// LDS and runs the same steps on it, so every such workgroup reaches the same
// result without waiting for another.  The policy walk runs in one wave: the ids in
// order, each touching one slot (LDS), a victim found by a wave-wide minimum over
// the slots.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace moe {

constexpr int kPolThreads = 256;
constexpr int kPolWaves = kPolThreads / 64;

// The decision's LDS arrays (int32 words): misc [16]; map, rank, list [E]; presence
// bits [E/32 + 1]; owner, free, key, use, prot, touched, evicted-by-miss [N]; and
// under EVICT_DECAY a reduction area [16], cnt, occ [E] and the copy jobs [E + N + 2].
struct PolLds {
    int32_t *map, *rank, *list, *owner, *fre, *prot, *tch, *mev, *misc;
    uint32_t *key, *use, *bits;
    float* cnt;        // decayed use counts (DECAY)
    int32_t* occ;      // the step's (token, k) selections per expert (DECAY)
    int32_t* job;      // DECAY walk output: slot copies at [0, N + 1), host reads at [N + 1, ...)
    uint64_t* red;     // DECAY: per-wave minima (8 words of 64 bits)
};

// misc words
enum { PM_NFREE = 0, PM_TICK = 1, PM_NPROT = 2, PM_POOLED = 3, PM_PATH = 4, PM_NMISS = 5, PM_HITS = 6, PM_BAD = 7,
       PM_WAVES = 8 /* 4 words: per-wave counts of the compaction */, PM_NHOST = 12, PM_NMOVE = 13 };

__host__ __device__ inline size_t pol_lds_words(int E, int N, int evict) {
    const size_t base = 16 + (size_t)3 * E + (size_t)(E / 32 + 1) + (size_t)7 * N;
    return evict == EVICT_DECAY ? base + 16 + (size_t)3 * E + N + 2 : base;
}

__device__ inline PolLds pol_lds(int32_t* w, int E, int N, int evict) {
    PolLds L;
    L.misc = w; w += 16;
    L.red = nullptr;
    if (evict == EVICT_DECAY) {
        L.red = reinterpret_cast<uint64_t*>(w);   // 64 bytes into the (aligned) block
        w += 16;
    }
    L.map = w;  w += E;
    L.rank = w; w += E;
    L.list = w; w += E;
    L.bits = reinterpret_cast<uint32_t*>(w); w += E / 32 + 1;
    L.owner = w; w += N;
    L.fre = w;  w += N;
    L.key = reinterpret_cast<uint32_t*>(w); w += N;
    L.use = reinterpret_cast<uint32_t*>(w); w += N;
    L.prot = w; w += N;
    L.tch = w;  w += N;
    L.mev = w;  w += N;
    L.cnt = nullptr;
    L.occ = L.job = nullptr;
    if (evict == EVICT_DECAY) {
        L.cnt = reinterpret_cast<float*>(w); w += E;
        L.occ = w; w += E;
        L.job = w;
    }
    return L;
}

// Pointers into one state copy.
struct SlotView {
    int32_t* map;
    int32_t* owner;
    int32_t* fre;
    uint32_t* key;
    uint32_t* use;
    int32_t* prot;
    float* cnt;
    int32_t* meta;
};

__device__ inline SlotView slot_view(char* base, int E, int N) {
    const SlotStateLayout o = slot_state_layout(E, N);
    SlotView v;
    v.map = reinterpret_cast<int32_t*>(base + o.map);
    v.owner = reinterpret_cast<int32_t*>(base + o.owner);
    v.fre = reinterpret_cast<int32_t*>(base + o.free);
    v.key = reinterpret_cast<uint32_t*>(base + o.key);
    v.use = reinterpret_cast<uint32_t*>(base + o.use);
    v.prot = reinterpret_cast<int32_t*>(base + o.prot);
    v.cnt = reinterpret_cast<float*>(base + o.cnt);
    v.meta = reinterpret_cast<int32_t*>(base + o.meta);
    return v;
}

// The wave-wide minimum of a 64-bit value (every lane gets it).
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, off, 64);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), off, 64);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o < v ? o : v;
    }
    return v;
}

// One wave (all 64 lanes, uniform control flow): the slot with the smallest key
// among the candidates.  prot_only: the protected slots (SLRU demotion); else the
// resident slots the step has not touched, ordered by the policy's key.  Keys are
// distinct (each is a tick drawn once), so the minimum is unique; with no candidate
// (which a pooled step cannot reach) slot 0 is returned so that no access leaves
// the arrays.
__device__ __forceinline__ int pol_argmin(const PolLds& L, int N, int evict, bool prot_only) {
    const int lane = threadIdx.x & 63;
    uint64_t best = ~0ull;
    int bs = -1;
    for (int s = lane; s < N; s += 64) {
        bool c;
        uint64_t k = L.key[s];
        if (prot_only) {
            c = L.prot[s] != 0;
        } else {
            c = L.owner[s] >= 0 && L.tch[s] == 0;
            if (evict == EVICT_LFU) k |= (uint64_t)L.use[s] << 32;
            if (evict == EVICT_SLRU) k |= (uint64_t)(L.prot[s] != 0) << 32;
        }
        if (c && k < best) {
            best = k;
            bs = s;
        }
    }
    const uint64_t m = wave_min_u64(best);
    const uint64_t who = __ballot(bs >= 0 && best == m);
    if (!who) return 0;
    return __shfl(bs, (int)__builtin_ctzll(who), 64);
}

struct Decision {
    int path;    // PATH_POOL, PATH_STAGE, PATH_NONE (an id outside [0, E))
    int D;       // distinct ids
    int nmiss;   // misses (pool path): experts copied into a slot
    int hits;
    int nhost;   // DECAY, pool path: experts read from the host into staging for the step
    int nmove;   // DECAY: 1 when the step's decision moved an expert (counted in nmiss)
};

// The decayed-count part of a pooled step (EVICT_DECAY), by all threads of the
// workgroup, on the LDS state with list[0, D) = the step's distinct ids ascending and
// occ = their selections.  Leaves the decision's fields in misc, and list[0, nmiss) =
// the experts copied into slots (the move first) with mev = what each evicted,
// list[nmiss, nmiss + nhost) = the host-read experts in staging order, rank[e] = N +
// staging entry for a host-read expert.
__device__ inline void pol_decay(const PolicyArgs& a, const PolLds& L, int D) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int E = a.E, N = a.N;
    const int pooled = L.misc[PM_POOLED] + 1;
    const bool decide = pooled % kDecayEvery == 0;
    const float decay = 0x1.fa7c18p-1f;   // 2^(-1/64) rounded to float32 (half-life 512 steps)
    if (decide)
        for (int e = tid; e < E; e += kPolThreads) L.cnt[e] = __fmul_rn(L.cnt[e], decay);
    __syncthreads();
    int nmove = 0;
    if (decide && L.misc[PM_NFREE] == 0) {
        // the most used host expert (largest count, then lowest id) and the least used
        // resident one (smallest count, then lowest id), as 64-bit minima: counts are
        // non-negative, so their bit patterns order like their values
        uint64_t bh = ~0ull, bg = ~0ull;
        for (int e = tid; e < E; e += kPolThreads) {
            const uint32_t c = __float_as_uint(L.cnt[e]);
            const uint64_t kh = ((uint64_t)(~c) << 32) | (uint32_t)e;
            const uint64_t kg = ((uint64_t)c << 32) | (uint32_t)e;
            if (L.map[e] < 0) bh = kh < bh ? kh : bh;
            else bg = kg < bg ? kg : bg;
        }
        bh = wave_min_u64(bh);
        bg = wave_min_u64(bg);
        if (lane == 0) {
            L.red[wave] = bh;
            L.red[kPolWaves + wave] = bg;
        }
        __syncthreads();
        for (int w = 0; w < kPolWaves; ++w) {
            bh = L.red[w] < bh ? L.red[w] : bh;
            bg = L.red[kPolWaves + w] < bg ? L.red[kPolWaves + w] : bg;
        }
        if (bh != ~0ull && bg != ~0ull) {
            const int h = (int)(uint32_t)bh, g = (int)(uint32_t)bg;
            if (__fsub_rn(L.cnt[h], L.cnt[g]) > kDecayThreshold) {
                nmove = 1;
                __syncthreads();   // every thread has read map before it changes
                if (tid == 0) {
                    const int s = L.map[g];
                    L.map[g] = -1;
                    L.map[h] = s;
                    L.owner[s] = h;
                    L.job[0] = h;
                    L.mev[0] = g;
                }
            }
        }
    }
    __syncthreads();
    // the distinct ids in order (wave 0, 64 at a time): resident -> hit; the j-th
    // non-resident one takes free slot fre[nfree - 1 - j] while there is one, else it
    // is read from the host into staging entry j - nfree
    if (wave == 0) {
        const int nfree = L.misc[PM_NFREE];
        int j0 = 0, hits = 0;
        for (int c0 = 0; c0 < D; c0 += 64) {
            const int i = c0 + lane;
            const int e = i < D ? L.list[i] : 0;
            const bool in = i < D;
            const bool res = in && L.map[e] >= 0;
            const uint64_t m = __ballot(in && !res);
            hits += __popcll(__ballot(res));
            const int j = j0 + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (in && !res) {
                if (j < nfree) {
                    const int s = L.fre[nfree - 1 - j];
                    L.map[e] = s;
                    L.owner[s] = e;
                    L.job[nmove + j] = e;
                    L.mev[nmove + j] = -1;
                    L.rank[e] = -1;
                } else {
                    L.job[N + 1 + (j - nfree)] = e;
                    L.rank[e] = N + (j - nfree);
                }
            }
            j0 += __popcll(m);
        }
        if (lane == 0) {
            const int ins = j0 < nfree ? j0 : nfree;
            L.misc[PM_NFREE] = nfree - ins;
            L.misc[PM_NMISS] = nmove + ins;
            L.misc[PM_NHOST] = j0 - ins;
            L.misc[PM_HITS] = hits;
            L.misc[PM_NMOVE] = nmove;
            L.misc[PM_POOLED] = pooled;
        }
    }
    __syncthreads();
    // the step's selections join the counts (one float add per expert); the copy jobs
    // go to list (its distinct ids are no longer needed)
    for (int e = tid; e < E; e += kPolThreads) L.cnt[e] = __fadd_rn(L.cnt[e], (float)L.occ[e]);
    const int nmiss = L.misc[PM_NMISS], nhost = L.misc[PM_NHOST];
    for (int j = tid; j < nmiss + nhost; j += kPolThreads) L.list[j] = j < nmiss ? L.job[j] : L.job[N + 1 + j - nmiss];
    __syncthreads();
}

// The decision of one step, by all kPolThreads threads of the workgroup.  Leaves in
// LDS: the state after the step (map, owner, free, key, use, prot, misc
// nfree/tick/nprot), list[0, nmiss) = the missed experts in order with mev[j] = the
// expert each evicted (-1: a free slot), rank[e] = position of e among the distinct
// ids (-1 for a missed expert on the pool path); on the staging path list[0, D) =
// the distinct ids (the staging order).
__device__ inline Decision pol_decide(const PolicyArgs& a, const SlotView& cur, const PolLds& L) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int E = a.E, N = a.N;
    const int nwords = (E + 31) >> 5;

    // the first 8 * kPolThreads ids, requested before the state so that the reads overlap
    int e0[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int i = tid + q * kPolThreads;
        e0[q] = i < a.n ? a.ids[i] : 0;
    }

    // 0. the state the step starts from; a thread's loads of the first two rounds
    // (E, N <= 512) are all issued before it writes any of them to LDS
    if (!a.resident) {
        constexpr int R = 2;
        int vm[R] = {}, vo[R] = {}, vf[R] = {}, vp[R] = {};
        uint32_t vk[R] = {}, vu[R] = {};
        int vmeta = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int e = tid + r * kPolThreads;
            if (e < E) vm[r] = cur.map[e];
            if (e < N) {
                vo[r] = cur.owner[e];
                vf[r] = cur.fre[e];
                vk[r] = cur.key[e];
                vu[r] = cur.use[e];
                vp[r] = cur.prot[e];
            }
        }
        if (tid < 4) vmeta = cur.meta[tid];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int e = tid + r * kPolThreads;
            if (e < E) L.map[e] = vm[r];
            if (e < N) {
                L.owner[e] = vo[r];
                L.fre[e] = vf[r];
                L.key[e] = vk[r];
                L.use[e] = vu[r];
                L.prot[e] = vp[r];
            }
        }
        if (tid < 4) L.misc[tid] = vmeta;
        for (int e = tid + R * kPolThreads; e < E; e += kPolThreads) L.map[e] = cur.map[e];
        for (int s = tid + R * kPolThreads; s < N; s += kPolThreads) {
            L.owner[s] = cur.owner[s];
            L.fre[s] = cur.fre[s];
            L.key[s] = cur.key[s];
            L.use[s] = cur.use[s];
            L.prot[s] = cur.prot[s];
        }
        if (a.evict == EVICT_DECAY)
            for (int e = tid; e < E; e += kPolThreads) {
                L.cnt[e] = cur.cnt[e];
                L.occ[e] = 0;
            }
    }
    for (int i = tid; i < nwords; i += kPolThreads) L.bits[i] = 0u;
    if (tid == 0) L.misc[PM_BAD] = 0;
    __syncthreads();

    // 1. distinct ids: presence bitmap, then ordered compaction (ballot + mbcnt).  With
    // at most 64 experts the marks go into a 64-bit mask per lane, OR-ed across the
    // wave, and one lane sets the two bitmap words.
    if (E <= 64) {
        uint64_t m = 0;
        bool bad = false;
        for (int i0 = tid; i0 < a.n; i0 += 8 * kPolThreads) {
            int e[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int i = i0 + q * kPolThreads;
                e[q] = i0 == tid ? e0[q] : (i < a.n ? a.ids[i] : 0);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if (i0 + q * kPolThreads >= a.n) break;
                if ((unsigned)e[q] < (unsigned)E)
                    m |= 1ull << e[q];
                else
                    bad = true;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const uint32_t lo = (uint32_t)m, hi = (uint32_t)(m >> 32);
            m |= (uint64_t)(uint32_t)__shfl_xor((int)lo, off, 64) |
                 ((uint64_t)(uint32_t)__shfl_xor((int)hi, off, 64) << 32);
        }
        if (bad) L.misc[PM_BAD] = 1;
        if (lane == 0) {
            if ((uint32_t)m) atomicOr(&L.bits[0], (uint32_t)m);
            if (E > 32 && (uint32_t)(m >> 32)) atomicOr(&L.bits[1], (uint32_t)(m >> 32));
        }
    } else {
        for (int i0 = tid; i0 < a.n; i0 += 8 * kPolThreads) {
            int e[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int i = i0 + q * kPolThreads;
                e[q] = i0 == tid ? e0[q] : (i < a.n ? a.ids[i] : 0);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if (i0 + q * kPolThreads >= a.n) break;
                if ((unsigned)e[q] < (unsigned)E)
                    atomicOr(&L.bits[e[q] >> 5], 1u << (e[q] & 31));
                else
                    L.misc[PM_BAD] = 1;
            }
        }
    }
    __syncthreads();
    int base = 0;
    if (E <= 64) {
        // the id set is one 64-bit mask: an expert's rank is the number of set bits below it
        const uint64_t all = (uint64_t)L.bits[0] | (E > 32 ? (uint64_t)L.bits[1] << 32 : 0ull);
        if (tid < E && ((all >> tid) & 1ull)) {
            const int pos = __popcll(all & ((1ull << tid) - 1ull));
            L.list[pos] = tid;
            L.rank[tid] = pos;
        }
        base = __popcll(all);
    } else {
        for (int c0 = 0; c0 < E; c0 += kPolThreads) {
            const int e = c0 + tid;
            const bool present = e < E && ((L.bits[e >> 5] >> (e & 31)) & 1u);
            const uint64_t m = __ballot(present);
            const uint32_t below =
                __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (lane == 0) L.misc[PM_WAVES + wave] = __popcll(m);
            __syncthreads();
            int off = 0, total = 0;
#pragma unroll
            for (int w = 0; w < kPolWaves; ++w) {
                const int cnt = L.misc[PM_WAVES + w];
                off += (w < wave) ? cnt : 0;
                total += cnt;
            }
            if (present) {
                const int pos = base + off + (int)below;
                L.list[pos] = e;
                L.rank[e] = pos;
            }
            base += total;
            __syncthreads();
        }
    }
    __syncthreads();
    Decision d{};
    d.D = base;
    if (L.misc[PM_BAD]) {
        d.path = PATH_NONE;
        return d;
    }
    if (a.resident) {
        d.path = PATH_POOL;
        d.hits = d.D;
        return d;
    }
    if (a.rule == 1 ? (a.n > N && d.D > 0) : (d.D > N)) {
        d.path = PATH_STAGE;
        return d;
    }

    d.path = PATH_POOL;
    if (a.evict == EVICT_DECAY) {
        for (int i = tid; i < a.n; i += kPolThreads) atomicAdd(&L.occ[a.ids[i]], 1);
        __syncthreads();
        pol_decay(a, L, d.D);
        d.nmiss = L.misc[PM_NMISS];
        d.hits = L.misc[PM_HITS];
        d.nhost = L.misc[PM_NHOST];
        d.nmove = L.misc[PM_NMOVE];
        return d;
    }
    // 2a. a step whose ids all hit (most decode steps) under LRU, FIFO or LFU: id i of
    // the ascending list takes tick + i as its key, so every id is updated at once
    // (the order of the walk below fixes nothing else; SLRU promotions do, and walk)
    if (tid == 0) L.misc[PM_PATH] = 0;
    __syncthreads();
    for (int i = tid; i < d.D; i += kPolThreads)
        if (L.map[L.list[i]] < 0) L.misc[PM_PATH] = 1;
    __syncthreads();
    if (L.misc[PM_PATH] == 0 && a.evict != EVICT_SLRU) {
        const uint32_t tick = (uint32_t)L.misc[PM_TICK];
        for (int i = tid; i < d.D; i += kPolThreads) {
            const int s = L.map[L.list[i]];
            if (a.evict != EVICT_FIFO) L.key[s] = tick + (uint32_t)i;
            if (a.evict == EVICT_LFU) L.use[s] = L.use[s] + 1u;
        }
        __syncthreads();
        if (tid == 0) {
            L.misc[PM_TICK] = (int32_t)(tick + (uint32_t)d.D);
            L.misc[PM_NMISS] = 0;
            L.misc[PM_HITS] = d.D;
        }
        __syncthreads();
        d.nmiss = 0;
        d.hits = d.D;
        return d;
    }

    // 2b. the policy, one distinct id at a time in ascending order, in wave 0.  Miss j's
    // expert goes to list[j] (j <= the id being processed, so nothing unread is
    // overwritten).
    if (wave == 0) {
        const int evict = a.evict;
        const int cap = (4 * N) / 5;              // SLRU: protected segment capacity
        int nfree = L.misc[PM_NFREE];
        int nprot = L.misc[PM_NPROT];
        uint32_t tick = (uint32_t)L.misc[PM_TICK];
        for (int s = lane; s < N; s += 64) L.tch[s] = 0;
        int hits = 0, nm = 0;
        for (int i = 0; i < d.D; ++i) {
            const int e = L.list[i];
            int s = L.map[e];
            if (s >= 0) {
                ++hits;
                const uint32_t t = tick++;
                const int was_prot = L.prot[s];
                if (lane == 0) {
                    if (evict != EVICT_FIFO) L.key[s] = t;
                    if (evict == EVICT_LFU) L.use[s] = L.use[s] + 1u;
                    if (evict == EVICT_SLRU && !was_prot) L.prot[s] = 1;
                    L.tch[s] = 1;
                }
                if (evict == EVICT_SLRU && !was_prot && ++nprot > cap) {
                    // the protected segment is over its share: its oldest place is demoted
                    const int dm = pol_argmin(L, N, evict, true);
                    if (lane == 0) {
                        L.prot[dm] = 0;
                        L.key[dm] = tick;
                    }
                    ++tick;
                    --nprot;
                }
            } else {
                int ev = -1;
                if (nfree > 0) {
                    s = L.fre[--nfree];
                } else {
                    s = pol_argmin(L, N, evict, false);
                    ev = L.owner[s];
                    if (evict == EVICT_SLRU && L.prot[s]) --nprot;
                    if (lane == 0 && ev >= 0) L.map[ev] = -1;
                }
                const uint32_t t = tick++;
                if (lane == 0) {
                    L.map[e] = s;
                    L.owner[s] = e;
                    L.key[s] = t;
                    L.use[s] = 1u;
                    L.prot[s] = 0;
                    L.tch[s] = 1;
                    L.list[nm] = e;
                    L.mev[nm] = ev;
                    L.rank[e] = -1;
                }
                ++nm;
            }
        }
        if (lane == 0) {
            L.misc[PM_NFREE] = nfree;
            L.misc[PM_TICK] = (int32_t)tick;
            L.misc[PM_NPROT] = nprot;
            L.misc[PM_NMISS] = nm;
            L.misc[PM_HITS] = hits;
        }
    }
    __syncthreads();
    d.nmiss = L.misc[PM_NMISS];
    d.hits = L.misc[PM_HITS];
    return d;
}

// The device-mapped store address of expert e.
__device__ __forceinline__ const char* pol_store_at(const PolicyArgs& a, int e) {
    return a.pieces[e / a.per_piece] + (size_t)(e % a.per_piece) * a.eb;
}

// The prefetch entry holding expert e, or -1.  All lanes of a wave call it with the
// same e.
__device__ __forceinline__ int pol_pf_entry(const PolicyArgs& a, int e) {
    if (a.pf_n <= 0) return -1;
    const int lane = threadIdx.x & 63;
    const int t = lane < a.pf_n ? a.pf_tag[lane] : -1;
    const uint64_t m = __ballot(t == e);
    return m ? (int)__builtin_ctzll(m) : -1;
}

// Where a missed or staged expert's bytes are read from: its prefetch entry (HBM) if
// it has one, else the pinned store over the host link.  Wave-uniform e.
__device__ __forceinline__ const char* pol_src(const PolicyArgs& a, int e) {
    const int j = pol_pf_entry(a, e);
    return j >= 0 ? a.pf_buf + (size_t)j * a.eb : pol_store_at(a, e);
}

// Counters without a read-back (the lead's thread 0 does not wait for old values).
__device__ __forceinline__ void pol_bump(unsigned long long* c, unsigned long long v) {
    __hip_atomic_fetch_add(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The lead workgroup's write-out of a decision: the state after the step into the
// other copy, the counters, the step record and the layer's path word.
__device__ inline void pol_publish(const PolicyArgs& a, const SlotView& nxt, const PolLds& L, const Decision& d) {
    const int tid = threadIdx.x;
    const int E = a.E, N = a.N;
    for (int e = tid; !a.resident && e < E; e += kPolThreads) nxt.map[e] = L.map[e];
    for (int s = tid; !a.resident && s < N; s += kPolThreads) {
        nxt.owner[s] = L.owner[s];
        nxt.fre[s] = L.fre[s];
        nxt.key[s] = L.key[s];
        nxt.use[s] = L.use[s];
        nxt.prot[s] = L.prot[s];
    }
    if (tid < 4 && !a.resident) nxt.meta[tid] = L.misc[tid];
    if (a.evict == EVICT_DECAY && !a.resident)
        for (int e = tid; e < E; e += kPolThreads) nxt.cnt[e] = L.cnt[e];
    // experts the step moves (into slots, then staging), and those of them read from
    // the prefetch buffer (wave 0, one expert at a time)
    const int njobs = d.path == PATH_STAGE ? d.D : (d.path == PATH_POOL ? d.nmiss + d.nhost : 0);
    int npf = 0;
    if (a.pf_n > 0 && tid < 64) {
        const int nj = njobs;
        for (int j = 0; j < nj; ++j) npf += pol_pf_entry(a, L.list[j]) >= 0 ? 1 : 0;
    }
    for (int j = tid; d.path == PATH_POOL && j < d.nmiss; j += kPolThreads) {
        const int e = L.list[j];
        a.ds.rec[4 + 3 * j] = e;
        a.ds.rec[5 + 3 * j] = L.map[e];
        a.ds.rec[6 + 3 * j] = L.mev[j];
    }
    if (tid == 0) {
        *a.path = d.path;
        a.ds.rec[0] = d.path;
        a.ds.rec[1] = d.D;
        a.ds.rec[2] = d.path == PATH_POOL ? d.nmiss : 0;
        a.ds.rec[3] = d.path == PATH_NONE ? 1 : 0;
        unsigned long long* ctr = a.ds.ctr;
        if (d.path == PATH_NONE) {
            __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        } else if (d.path == PATH_STAGE) {
            pol_bump(ctr + 0, 1);
            pol_bump(ctr + 3, 1);
            pol_bump(ctr + 4, (unsigned long long)(d.D - npf) * a.eb);
            pol_bump(ctr + 5, (unsigned long long)d.D);
        } else {
            pol_bump(ctr + 0, 1);
            pol_bump(ctr + 1, (unsigned long long)d.hits);
            if (d.nmiss) pol_bump(ctr + 2, (unsigned long long)d.nmiss);
            if (njobs) pol_bump(ctr + 4, (unsigned long long)(njobs - npf) * a.eb);
            if (d.nhost) pol_bump(ctr + 5, (unsigned long long)d.nhost);
            if (d.nmove) pol_bump(ctr + 8, (unsigned long long)d.nmove);
        }
        if (npf) pol_bump(ctr + 6, (unsigned long long)npf);
        if (a.timed_jobs) __hip_atomic_store(a.timed_jobs, njobs - npf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

// An all-hit step of at most 64 ids under LRU, FIFO or LFU, by the lead workgroup of
// the fused step or of a prepare launch (wave 0; every id valid and resident; repeated
// ids count once).  Such a step changes only the keys (LFU: also the uses) of its slots
// and the tick, as the all-hit path of pol_decide does (distinct id i, ascending, gets
// key tick + i; tick += D), and nothing else in the launch reads keys or uses on such a
// step, so the lead applies the changes to the current state copy in place and marks
// that the copies keep their roles (ctl[2] = 0: no flip after a fused step; a prepare
// launch flips only after its readers have counted themselves in, which this one's do
// not).  Results, record and counters are those of the decision.
__device__ inline void pol_hit_in_place(const PolicyArgs& a, const SlotView& cur, int K) {
    const int lane = threadIdx.x;
    if (lane >= 64) return;
    const int id = lane < K ? a.ids[lane] : 0x7fffffff;
    const int s = lane < K ? cur.map[id] : -1;
    const uint32_t tick = (uint32_t)cur.meta[1];
    // the first occurrence of each id, then its rank among the distinct ids
    bool first = lane < K;
    for (int j = 0; j < K; ++j) {
        const int idj = __shfl(id, j, 64);
        first = first && !(j < lane && idj == id);
    }
    int rank = 0, D = 0;
    for (int j = 0; j < K; ++j) {
        const int fj = __shfl((int)first, j, 64);
        const int idj = __shfl(id, j, 64);
        D += fj;
        rank += (fj && idj < id) ? 1 : 0;
    }
    if (first) {
        if (a.evict != EVICT_FIFO) cur.key[s] = tick + (uint32_t)rank;
        if (a.evict == EVICT_LFU) cur.use[s] = cur.use[s] + 1u;
    }
    if (lane < K) a.out[lane] = s;
    if (lane == 0) {
        cur.meta[1] = (int32_t)(tick + (uint32_t)D);
        *a.path = PATH_POOL;
        a.ds.rec[0] = PATH_POOL;
        a.ds.rec[1] = D;
        a.ds.rec[2] = 0;
        a.ds.rec[3] = 0;
        pol_bump(a.ds.ctr + 0, 1);
        pol_bump(a.ds.ctr + 1, (unsigned long long)D);
        if (a.timed_jobs) __hip_atomic_store(a.timed_jobs, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        a.ds.ctl[2] = 0;
    }
}

// A workgroup of a prepare launch has read everything it reads of the current state
// copy: it counts itself in (one thread, after the workgroup's reads have returned);
// pol_last_reader, called at the end of the workgroup with the returned count, lets
// the last one of the launch make the other copy current.  Nothing of the launch
// reads the current copy after that, and the lead's writes to the other copy are
// complete when the launch is.  (The count is read back only at the end, so its
// round trip overlaps the workgroup's work.)  The count is relaxed: the reads it
// stands for have returned (the wait below; their values fed the decision), which is
// all it orders, and a release at agent scope would write back the XCD's L2 in every
// workgroup.
__device__ __forceinline__ int pol_reader_arrive(int32_t* ctl) {
    __builtin_amdgcn_s_waitcnt(0);
    return __hip_atomic_fetch_add(&ctl[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void pol_last_reader(int32_t* ctl, int old, int nblocks) {
    if (old == nblocks - 1) {
        __hip_atomic_store(&ctl[1], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int par = __hip_atomic_load(&ctl[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ctl[0], par ^ 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace moe
