// The slot manager on the GPU (policy = MOE_POLICY_DEVICE): one launch per step
// computes the step's distinct expert ids, applies the route rule, runs the LRU on
// the layer's state in HBM, remaps the ids, and pulls the missed (or staged)
// experts from the pinned store.  Nothing waits for the host, so a whole decode
// step can be queued at once.
//
// The LRU is the one of vLLM PR "Run MoE models exceeding VRAM via expert CPU
// offloading with GPU cache" (section "How it works" and the review thread's
// OrderedDict form) -- the distinct ids ascending, one at a time: a hit moves the
// expert to the most recently used end; a miss takes the last free slot (free
// slots start as 0..N-1) or evicts the least recently used expert -- and the route
// rule is the llama.cpp "Persistent expert slot pool" prefill rule (a step that
// exceeds the slots takes the selective-copy path and leaves the state untouched).
// It is the same state machine as the host slot manager, kept as the same arrays:
// map[E], owner[N], a free stack, and a doubly linked LRU list over expert ids.
//
// Every workgroup of the launch runs the same decision on its own copy of the state
// in LDS (a few microseconds of latency, the same in each), so that each knows the
// step's copies without waiting for another workgroup; the first one also writes the
// results.  It writes the state back in place once every other workgroup has its
// copy: those count themselves in an arrival word and never wait for anything, so
// the first workgroup's (bounded) wait always ends.  Nothing in a step depends on
// the host, so a decode step can be captured in a graph and replayed.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace moe {

constexpr int kPolicyThreads = 256;
constexpr int kPolicyWaves = kPolicyThreads / 64;
constexpr size_t kFillUnit = (size_t)64 << 10;   // bytes of one copy work unit
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// Dynamic LDS: map, prev, next, rank, list [E] and owner, free [N] (int32), then the
// presence bits [E/32 + 1].
__global__ __launch_bounds__(kPolicyThreads) void k_policy(PolicyArgs a) {
    extern __shared__ int32_t sm[];
    const int E = a.E, N = a.N;
    int32_t* map = sm;
    int32_t* prv = map + E;
    int32_t* nxt = prv + E;
    int32_t* rank = nxt + E;
    int32_t* list = rank + E;
    int32_t* own = list + E;
    int32_t* fre = own + N;
    uint32_t* bits = reinterpret_cast<uint32_t*>(fre + N);
    __shared__ int32_t wave_cnt[kPolicyWaves];
    __shared__ int32_t s_bad, s_njobs;
    __shared__ int32_t s_meta[3];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nwords = (E + 31) >> 5;
    const bool lead = blockIdx.x == 0;
    // The arguments span four 64-byte lines of the scalar cache and the grid size (a
    // hidden argument) a fifth: one field of each is read here, so that all lines are
    // requested together instead of one miss at a time where each field is first used
    // (the state pointers, for one, are needed right after the ids).
    const int nblocks = (int)gridDim.x;
    __asm__ volatile("" ::"s"(nblocks), "s"(a.st.map), "s"(a.st.meta), "s"(a.err), "s"(a.tab));
    unsigned long long* ctr = a.ctr;   // steps, hits, misses, fallbacks, bytes_h2d, staged
    int32_t* rec = a.rec;
    // counter updates are additions nothing in the launch reads back: atomics without a
    // return value, so that the lead thread does not wait for a read of the old values
    auto bump = [](unsigned long long* c, unsigned long long v) {
        __hip_atomic_fetch_add(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };

    // the first 8 * kPolicyThreads ids (every workgroup reads them for the decision),
    // and the one id this thread writes an output for first (index blockIdx.x *
    // kPolicyThreads + tid, below), requested before the state so that the reads overlap
    int e0[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int i = tid + q * kPolicyThreads;
        e0[q] = i < a.n ? a.ids[i] : 0;
    }
    const int gid0 = blockIdx.x * kPolicyThreads + tid;
    const int mine = gid0 < a.n ? a.ids[gid0] : 0;
    auto id_at = [&](int i) { return i == gid0 ? mine : a.ids[i]; };

    // 0. the state the step starts from (loaded first: its latency overlaps the
    // distinct-id pass), and an empty presence bitmap
    if (!a.resident) {
        // a thread's loads for the first two rounds (E, N <= 512) are all issued before
        // it writes any of them to LDS: one round trip, not one per array group
        constexpr int R = 2;
        int vm[R] = {}, vp[R] = {}, vn[R] = {}, vo[R] = {}, vf[R] = {};
        int vmeta = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int e = tid + r * kPolicyThreads;
            if (e < E) {
                vm[r] = a.st.map[e];
                vp[r] = a.st.prev[e];
                vn[r] = a.st.next[e];
            }
            if (e < N) {
                vo[r] = a.st.owner[e];
                vf[r] = a.st.free[e];
            }
        }
        if (tid < 3) vmeta = a.st.meta[tid];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int e = tid + r * kPolicyThreads;
            if (e < E) {
                map[e] = vm[r];
                prv[e] = vp[r];
                nxt[e] = vn[r];
            }
            if (e < N) {
                own[e] = vo[r];
                fre[e] = vf[r];
            }
        }
        if (tid < 3) s_meta[tid] = vmeta;
        for (int e = tid + R * kPolicyThreads; e < E; e += kPolicyThreads) {
            map[e] = a.st.map[e];
            prv[e] = a.st.prev[e];
            nxt[e] = a.st.next[e];
        }
        for (int s = tid + R * kPolicyThreads; s < N; s += kPolicyThreads) {
            own[s] = a.st.owner[s];
            fre[s] = a.st.free[s];
        }
    }
    for (int i = tid; i < nwords; i += kPolicyThreads) bits[i] = 0u;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    // the copy is in LDS: this workgroup no longer reads the state in HBM
    if (!a.resident && !lead && tid == 0) __hip_atomic_fetch_add(a.arrive, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // 1. distinct ids: presence bitmap, then ordered compaction (ballot + mbcnt).  A
    // thread reads eight ids before it marks any, so that their loads are in flight
    // together (a prefill step has thousands of ids per workgroup).  With at most 64
    // experts the marks go into a 64-bit mask per lane, OR-ed across the wave, and
    // one lane sets the (two) bitmap words: thousands of LDS atomics on two words
    // would serialise.
    if (E <= 64) {
        uint64_t m = 0;
        bool bad = false;
        for (int i0 = tid; i0 < a.n; i0 += 8 * kPolicyThreads) {
            int e[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int i = i0 + q * kPolicyThreads;
                e[q] = i0 == tid ? e0[q] : (i < a.n ? a.ids[i] : 0);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if (i0 + q * kPolicyThreads >= a.n) break;
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
        if (bad) s_bad = 1;
        if (lane == 0) {
            if ((uint32_t)m) atomicOr(&bits[0], (uint32_t)m);
            if (E > 32 && (uint32_t)(m >> 32)) atomicOr(&bits[1], (uint32_t)(m >> 32));
        }
    } else {
        for (int i0 = tid; i0 < a.n; i0 += 8 * kPolicyThreads) {
            int e[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int i = i0 + q * kPolicyThreads;
                e[q] = i0 == tid ? e0[q] : (i < a.n ? a.ids[i] : 0);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if (i0 + q * kPolicyThreads >= a.n) break;
                if ((unsigned)e[q] < (unsigned)E)
                    atomicOr(&bits[e[q] >> 5], 1u << (e[q] & 31));
                else
                    s_bad = 1;
            }
        }
    }
    __syncthreads();
    int base = 0;
    if (E <= 64) {
        // the id set is one 64-bit mask: an expert's rank is the number of set bits below it
        const uint64_t all = (uint64_t)bits[0] | (E > 32 ? (uint64_t)bits[1] << 32 : 0ull);
        if (tid < E && ((all >> tid) & 1ull)) {
            const int pos = __popcll(all & ((1ull << tid) - 1ull));
            list[pos] = tid;
            rank[tid] = pos;
        }
        base = __popcll(all);
        __syncthreads();
    }
    for (int c0 = 0; E > 64 && c0 < E; c0 += kPolicyThreads) {
        const int e = c0 + tid;
        const bool present = e < E && ((bits[e >> 5] >> (e & 31)) & 1u);
        const uint64_t m = __ballot(present);
        const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (lane == 0) wave_cnt[wave] = __popcll(m);
        __syncthreads();
        int off = 0, total = 0;
        for (int w = 0; w < kPolicyWaves; ++w) {
            const int cnt = wave_cnt[w];
            off += (w < wave) ? cnt : 0;
            total += cnt;
        }
        if (present) {
            const int pos = base + off + (int)below;
            list[pos] = e;
            rank[e] = pos;
        }
        base += total;
        __syncthreads();
    }
    const int D = base;

    if (a.resident) {
        // every expert lives at slot = id: count the hits, the ids are the slots
        // (nothing to copy; the ids are spread over the launch's workgroups)
        const int gtid = blockIdx.x * kPolicyThreads + tid;
        const int gthreads = nblocks * kPolicyThreads;
        for (int i = gtid; i < a.n; i += gthreads) a.out[i] = s_bad ? -1 : id_at(i);
        if (lead && tid == 0) {
            *a.path = s_bad ? PATH_NONE : PATH_POOL;
            rec[0] = s_bad ? PATH_NONE : PATH_POOL;
            rec[1] = D;
            rec[2] = 0;
            rec[3] = s_bad;
            if (s_bad) {
                __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            } else {
                bump(ctr + 0, 1);
                bump(ctr + 1, (unsigned long long)D);
            }
        }
        return;
    }

    // 2. the step's outcome; every branch leaves the copies in list[0, njobs) with
    // their destinations (pool: the expert's slot; staging: the list position).
    // With a pair table (read-through) nothing is copied here: the table tells the
    // forward which pairs read their expert from the store, and for a miss, which
    // slot it writes the expert to on the way.
    int njobs = 0;
    int nlink = 0;   // experts the step moves over the host link
    bool pool = true;
    const size_t eb = a.eb;
    auto store_at = [&](int e) { return a.pieces[e / a.per_piece] + (size_t)(e % a.per_piece) * eb; };
    // every workgroup holds the decision, so the per-id outputs are spread over all
    // of them (each id is written by exactly one thread of the launch)
    const int gtid = blockIdx.x * kPolicyThreads + tid;
    const int gthreads = nblocks * kPolicyThreads;
    if (s_bad) {
        // an id outside [0, E): nothing changes, the step produces no expert
        for (int i = gtid; i < a.n; i += gthreads) {
            a.out[i] = -1;
            if (a.tab) a.tab[i] = PairSrc{nullptr, nullptr};
        }
        if (lead) {
            if (tid == 0) {
                *a.path = PATH_NONE;
                rec[0] = PATH_NONE;
                rec[1] = D;
                rec[2] = 0;
                rec[3] = 1;
                __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            }
        }
    } else if (a.rule == 1 ? (a.n > N && D > 0) : (D > N)) {
        // route rule ([llama-pool] prefill rule): selective copy -- the step's experts
        // go to staging in rank order; the pool state is untouched
        pool = false;
        nlink = D;
        njobs = a.tab ? 0 : D;
        for (int i = gtid; i < a.n; i += gthreads) {
            const int e = id_at(i);
            a.out[i] = rank[e];
            if (a.tab) a.tab[i] = PairSrc{store_at(e), nullptr};
        }
        if (lead) {
            if (tid == 0) {
                *a.path = PATH_STAGE;
                rec[0] = PATH_STAGE;
                rec[1] = D;
                rec[2] = 0;
                rec[3] = 0;
                bump(ctr + 0, 1);
                bump(ctr + 3, 1);
                bump(ctr + 4, (unsigned long long)D * a.eb);
                bump(ctr + 5, (unsigned long long)D);
            }
        }
    } else {
        // 3. the LRU, one id at a time in ascending order.  Miss j's expert is written to
        // list[j] (j <= the id being processed, so nothing unread is overwritten), and a
        // missed expert's rank entry becomes -1 (rank is not needed on this path).
        if (E <= 64 && N <= 64) {
            // the lists in registers of wave 0: lane e holds expert e's map entry and
            // neighbours, lane s slot s's owner and free-list entry; the wave walks the ids
            // with scalar control flow, reading single lanes (readlane) and writing them
            // (a select on the lane id); a chain of dependent LDS accesses costs ~0.3 us
            // per id, these a few cycles each
            if (wave == 0) {
                int vmap = lane < E ? map[lane] : -1;
                int vprv = lane < E ? prv[lane] : -1;
                int vnxt = lane < E ? nxt[lane] : -1;
                int vown = lane < N ? own[lane] : -1;
                int vfre = lane < N ? fre[lane] : -1;
                int head = __builtin_amdgcn_readfirstlane(s_meta[0]);
                int tail = __builtin_amdgcn_readfirstlane(s_meta[1]);
                int nfree = __builtin_amdgcn_readfirstlane(s_meta[2]);
                const uint32_t lo = __builtin_amdgcn_readfirstlane(bits[0]);
                const uint32_t hi = E > 32 ? __builtin_amdgcn_readfirstlane(bits[1]) : 0u;
                uint64_t todo = (uint64_t)lo | ((uint64_t)hi << 32);
                int hits = 0, misses = 0;
                auto get = [](int v, int l) { return __builtin_amdgcn_readlane(v, l); };
                auto put = [lane](int& v, int l, int x) { v = lane == l ? x : v; };
                auto unlink = [&](int e) {
                    const int p = get(vprv, e), q = get(vnxt, e);
                    if (p >= 0) put(vnxt, p, q); else head = q;
                    if (q >= 0) put(vprv, q, p); else tail = p;
                    put(vprv, e, -1);
                    put(vnxt, e, -1);
                };
                auto push_mru = [&](int e) {
                    put(vprv, e, tail);
                    put(vnxt, e, -1);
                    if (tail >= 0) put(vnxt, tail, e); else head = e;
                    tail = e;
                };
                // A step whose ids all hit (most decode steps): its experts leave the list
                // and rejoin at the tail in ascending order, the others keep their order --
                // what the walk below ends with, computed by all lanes at once.  Each lane
                // finds its nearest neighbours outside the step by pointer doubling (a list
                // of at most 64 needs 6 rounds; the bound keeps a damaged state from looping).
                const bool mine = lane < E && ((todo >> lane) & 1ull);
                if (todo && !__ballot(mine && vmap < 0)) {
                    const uint64_t S = todo;
                    auto in_step = [S](int x) { return x >= 0 && ((S >> x) & 1ull) != 0; };
                    int jp = vprv, jn = vnxt;
                    for (int r = 0; r < 7 && __ballot(in_step(jp) || in_step(jn)); ++r) {
                        const int pp = __shfl(jp, jp < 0 ? lane : jp, 64);
                        const int nn = __shfl(jn, jn < 0 ? lane : jn, 64);
                        if (in_step(jp)) jp = pp;
                        if (in_step(jn)) jn = nn;
                    }
                    const int s_min = (int)__builtin_ctzll(S), s_max = 63 - (int)__builtin_clzll(S);
                    const int r_tail = in_step(tail) ? get(jp, tail) : tail;   // last one staying
                    const int r_head = in_step(head) ? get(jn, head) : head;   // first one staying
                    if (mine) {
                        const uint64_t below = S & ((1ull << lane) - 1ull);
                        const uint64_t above = lane < 63 ? S >> (lane + 1) : 0ull;
                        vprv = lane == s_min ? r_tail : 63 - (int)__builtin_clzll(below);
                        vnxt = above ? lane + 1 + (int)__builtin_ctzll(above) : -1;
                    } else if (vmap >= 0) {
                        vprv = jp;
                        vnxt = jn >= 0 ? jn : s_min;
                    }
                    head = r_head >= 0 ? r_head : s_min;
                    tail = s_max;
                    hits = __popcll(S);
                    todo = 0ull;
                }
                while (todo) {
                    const int e = (int)__builtin_ctzll(todo);
                    todo &= todo - 1ull;
                    if (get(vmap, e) >= 0) {
                        unlink(e);
                        push_mru(e);
                        ++hits;
                        continue;
                    }
                    int slot, evicted;
                    if (nfree > 0) {
                        slot = get(vfre, --nfree);
                        evicted = -1;
                    } else {
                        evicted = head;
                        unlink(evicted);
                        slot = get(vmap, evicted);
                        put(vmap, evicted, -1);
                    }
                    put(vmap, e, slot);
                    put(vown, slot, e);
                    push_mru(e);
                    if (lane == 0) {
                        if (lead) {
                            rec[4 + 3 * misses] = e;
                            rec[5 + 3 * misses] = slot;
                            rec[6 + 3 * misses] = evicted;
                        }
                        list[misses] = e;
                        rank[e] = -1;
                    }
                    ++misses;
                }
                if (lane < E) {
                    map[lane] = vmap;
                    prv[lane] = vprv;
                    nxt[lane] = vnxt;
                }
                if (lane < N) {
                    own[lane] = vown;
                    fre[lane] = vfre;
                }
                if (lane == 0) {
                    s_meta[0] = head;
                    s_meta[1] = tail;
                    s_meta[2] = nfree;
                    s_njobs = misses;
                    if (lead) {
                        *a.path = PATH_POOL;
                        rec[0] = PATH_POOL;
                        rec[1] = D;
                        rec[2] = misses;
                        rec[3] = 0;
                        bump(ctr + 0, 1);
                        bump(ctr + 1, (unsigned long long)hits);
                        bump(ctr + 2, (unsigned long long)misses);
                        bump(ctr + 4, (unsigned long long)misses * a.eb);
                    }
                }
            }
        } else if (tid == 0) {
            int head = s_meta[0], tail = s_meta[1], nfree = s_meta[2];
            int hits = 0, misses = 0;
            auto unlink = [&](int e) {
                const int p = prv[e], q = nxt[e];
                if (p >= 0) nxt[p] = q; else head = q;
                if (q >= 0) prv[q] = p; else tail = p;
                prv[e] = nxt[e] = -1;
            };
            auto push_mru = [&](int e) {
                prv[e] = tail;
                nxt[e] = -1;
                if (tail >= 0) nxt[tail] = e; else head = e;
                tail = e;
            };
            for (int i = 0; i < D; ++i) {
                const int e = list[i];
                if (map[e] >= 0) {
                    unlink(e);
                    push_mru(e);
                    ++hits;
                    continue;
                }
                int slot, evicted;
                if (nfree > 0) {
                    slot = fre[--nfree];
                    evicted = -1;
                } else {
                    evicted = head;
                    unlink(evicted);
                    slot = map[evicted];
                    map[evicted] = -1;
                }
                map[e] = slot;
                own[slot] = e;
                push_mru(e);
                if (lead) {
                    rec[4 + 3 * misses] = e;
                    rec[5 + 3 * misses] = slot;
                    rec[6 + 3 * misses] = evicted;
                }
                list[misses] = e;
                rank[e] = -1;
                ++misses;
            }
            s_meta[0] = head;
            s_meta[1] = tail;
            s_meta[2] = nfree;
            s_njobs = misses;
            if (lead) {
                *a.path = PATH_POOL;
                rec[0] = PATH_POOL;
                rec[1] = D;
                rec[2] = misses;
                rec[3] = 0;
                bump(ctr + 0, 1);
                bump(ctr + 1, (unsigned long long)hits);
                bump(ctr + 2, (unsigned long long)misses);
                bump(ctr + 4, (unsigned long long)misses * a.eb);
            }
        }
        __syncthreads();
        nlink = s_njobs;
        njobs = a.tab ? 0 : nlink;
        // the remap, through the fresh table
        for (int i = gtid; i < a.n; i += gthreads) {
            const int e = id_at(i);
            const int slot = map[e];
            a.out[i] = slot;
            if (a.tab)
                a.tab[i] = rank[e] < 0 ? PairSrc{store_at(e), a.slots + (size_t)slot * eb}
                                       : PairSrc{nullptr, nullptr};
        }
    }

    // 4. the state the step leaves (unchanged unless the LRU ran), written in place
    // once every other workgroup has its copy; the arrival word goes back to 0
    if (lead) {
        if (tid == 0) {
            const int others = nblocks - 1;
            unsigned long long polls = 0;
            while (__hip_atomic_load(a.arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < others) {
                if (++polls > a.spin_limit) {
                    __hip_atomic_store(a.err, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
            __hip_atomic_store(a.arrive, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        for (int e = tid; e < E; e += kPolicyThreads) {
            a.st.map[e] = map[e];
            a.st.prev[e] = prv[e];
            a.st.next[e] = nxt[e];
        }
        for (int s = tid; s < N; s += kPolicyThreads) {
            a.st.owner[s] = own[s];
            a.st.free[s] = fre[s];
        }
        if (tid < 3) a.st.meta[tid] = s_meta[tid];
        if (tid == 0 && a.timed_jobs)
            __hip_atomic_store(a.timed_jobs, nlink, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }

    // 5. the copies: 64 KiB work units over the launch, store -> slot / staging
    const size_t upj = (eb + kFillUnit - 1) / kFillUnit;
    const size_t units = upj * (size_t)njobs;
    for (size_t u = blockIdx.x; u < units; u += (size_t)nblocks) {
        const int j = (int)(u / upj);
        const int e = list[j];
        const size_t off = (u - (size_t)j * upj) * kFillUnit;
        const size_t nvec = (eb - off < kFillUnit ? eb - off : kFillUnit) / 16;
        const char* src = store_at(e) + off;
        char* dst = (pool ? a.slots + (size_t)map[e] * eb : a.staging + (size_t)j * eb) + off;
        const u32x4v* __restrict__ s4 = reinterpret_cast<const u32x4v*>(src);
        u32x4v* __restrict__ d4 = reinterpret_cast<u32x4v*>(dst);
        for (size_t i0 = tid; i0 < nvec; i0 += 4 * kPolicyThreads) {
            u32x4v v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const size_t i = i0 + (size_t)q * kPolicyThreads;
                if (i < nvec) v[q] = s4[i];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const size_t i = i0 + (size_t)q * kPolicyThreads;
                if (i < nvec) __builtin_nontemporal_store(v[q], d4 + i);
            }
        }
    }
}

size_t policy_lds_bytes(int E, int N) { return ((size_t)5 * E + 2 * N + E / 32 + 1) * sizeof(int32_t); }

hipError_t launch_policy(const PolicyArgs& a, int grid, hipEvent_t start, hipEvent_t stop, hipStream_t s) {
    if (a.n < 1 || a.n > (1 << 24) || grid < 1 || a.eb % 16 ||
        (!a.resident && a.per_piece < 1))
        return hipErrorInvalidValue;
    const size_t lds = policy_lds_bytes(a.E, a.N);
    if (start)
        hipExtLaunchKernelGGL(k_policy, dim3(grid), dim3(kPolicyThreads), lds, s, start, stop, 0, a);
    else
        hipLaunchKernelGGL(k_policy, dim3(grid), dim3(kPolicyThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace moe
