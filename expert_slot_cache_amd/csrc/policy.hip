// The slot manager on the GPU (policy = MOE_POLICY_DEVICE): one kernel per step
// computes the step's distinct expert ids, applies the route rule, runs the LRU on
// the layer's state in HBM, remaps the ids, and writes the step's copy jobs; a copy
// kernel then pulls the missed (or staged) experts from the pinned store.  Nothing
// waits for the host, so a whole decode step can be queued at once.
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
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace moe {

constexpr int kPolicyThreads = 1024;

// The step.  Dynamic LDS: map, prev, next, rank, list [E] and owner, free [N]
// (int32), then the presence bits [E/32 + 1].
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
    __shared__ int32_t wave_cnt[kPolicyThreads / 64];
    __shared__ int32_t s_bad;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nwords = (E + 31) >> 5;
    DevState st = a.st;

    // 1. distinct ids: presence bitmap, then ordered compaction (ballot + mbcnt)
    for (int i = tid; i < nwords; i += kPolicyThreads) bits[i] = 0u;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    for (int i = tid; i < a.n; i += kPolicyThreads) {
        const int e = a.ids[i];
        if ((unsigned)e < (unsigned)E)
            atomicOr(&bits[e >> 5], 1u << (e & 31));
        else
            s_bad = 1;
    }
    __syncthreads();
    int base = 0;
    for (int c0 = 0; c0 < E; c0 += kPolicyThreads) {
        const int e = c0 + tid;
        const bool present = e < E && ((bits[e >> 5] >> (e & 31)) & 1u);
        const uint64_t m = __ballot(present);
        const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (lane == 0) wave_cnt[wave] = __popcll(m);
        __syncthreads();
        int off = 0, total = 0;
        for (int w = 0; w < kPolicyThreads / 64; ++w) {
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
    int32_t* rec = st.rec;
    int32_t* jobs = st.jobs;
    if (s_bad) {
        // an id outside [0, E): nothing changes, the step produces no expert
        for (int i = tid; i < a.n; i += kPolicyThreads) a.out[i] = -1;
        if (tid == 0) {
            *a.path = PATH_NONE;
            rec[0] = PATH_NONE;
            rec[1] = D;
            rec[2] = 0;
            rec[3] = 1;
            jobs[0] = 0;
            __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
        return;
    }
    unsigned long long* ctr = st.ctr;   // steps, hits, misses, fallbacks, bytes_h2d, staged
    if (a.resident) {
        // every expert lives at slot = id: count the hits, the ids are the slots
        for (int i = tid; i < a.n; i += kPolicyThreads) a.out[i] = a.ids[i];
        if (tid == 0) {
            *a.path = PATH_POOL;
            rec[0] = PATH_POOL;
            rec[1] = D;
            rec[2] = 0;
            rec[3] = 0;
            jobs[0] = 0;
            ctr[0] += 1;
            ctr[1] += (unsigned long long)D;
        }
        return;
    }
    // 2. route rule ([llama-pool] prefill rule): distinct ids above the slots, or
    // (static rule) pairs above the slots
    const bool fallback = a.rule == 1 ? (a.n > N && D > 0) : (D > N);
    if (fallback) {
        // selective copy: the step's experts go to staging in rank order; the pool
        // state is untouched
        for (int i = tid; i < a.n; i += kPolicyThreads) a.out[i] = rank[a.ids[i]];
        for (int r = tid; r < D; r += kPolicyThreads) {
            jobs[1 + 2 * r] = list[r];
            jobs[2 + 2 * r] = -(r + 1);
        }
        if (tid == 0) {
            *a.path = PATH_STAGE;
            rec[0] = PATH_STAGE;
            rec[1] = D;
            rec[2] = 0;
            rec[3] = 0;
            jobs[0] = D;
            ctr[0] += 1;
            ctr[3] += 1;
            ctr[4] += (unsigned long long)D * a.eb;
            ctr[5] += (unsigned long long)D;
        }
        return;
    }
    // 3. the LRU, in LDS
    for (int e = tid; e < E; e += kPolicyThreads) {
        map[e] = st.map[e];
        prv[e] = st.prev[e];
        nxt[e] = st.next[e];
    }
    for (int s = tid; s < N; s += kPolicyThreads) {
        own[s] = st.owner[s];
        fre[s] = st.free[s];
    }
    __syncthreads();
    if (tid == 0) {
        int head = st.meta[0], tail = st.meta[1], nfree = st.meta[2];
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
            rec[4 + 3 * misses] = e;
            rec[5 + 3 * misses] = slot;
            rec[6 + 3 * misses] = evicted;
            jobs[1 + 2 * misses] = e;
            jobs[2 + 2 * misses] = slot;
            ++misses;
        }
        st.meta[0] = head;
        st.meta[1] = tail;
        st.meta[2] = nfree;
        *a.path = PATH_POOL;
        rec[0] = PATH_POOL;
        rec[1] = D;
        rec[2] = misses;
        rec[3] = 0;
        jobs[0] = misses;
        ctr[0] += 1;
        ctr[1] += (unsigned long long)hits;
        ctr[2] += (unsigned long long)misses;
        ctr[4] += (unsigned long long)misses * a.eb;
    }
    __syncthreads();
    // 4. write the state back and remap through the fresh table
    for (int e = tid; e < E; e += kPolicyThreads) {
        st.map[e] = map[e];
        st.prev[e] = prv[e];
        st.next[e] = nxt[e];
    }
    for (int s = tid; s < N; s += kPolicyThreads) {
        st.owner[s] = own[s];
        st.free[s] = fre[s];
    }
    for (int i = tid; i < a.n; i += kPolicyThreads) a.out[i] = map[a.ids[i]];
}

size_t policy_lds_bytes(int E, int N) { return ((size_t)5 * E + 2 * N + E / 32 + 1) * sizeof(int32_t); }

hipError_t launch_policy(const PolicyArgs& a, hipStream_t s) {
    if (a.n < 1 || a.n > (1 << 24)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_policy, dim3(1), dim3(kPolicyThreads), policy_lds_bytes(a.E, a.N), s, a);
    return hipGetLastError();
}

// The step's copy jobs (written by k_policy): job j copies expert jobs[1 + 2j]
// from the pinned store to slot jobs[2 + 2j] (>= 0) or staging entry
// -jobs[2 + 2j] - 1.  Work unit u: job u / units_per_job, 64 KiB of it.  When
// `timed_jobs` is set, one thread records the launch's job count there (host-mapped)
// so that event timings of launches without copies can be told apart.
constexpr int kFillDevThreads = 256;
constexpr size_t kFillDevUnit = (size_t)64 << 10;
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kFillDevThreads) void k_fill_dev(FillDevArgs a) {
    const int njobs = a.jobs[0];
    if (blockIdx.x == 0 && threadIdx.x == 0 && a.timed_jobs)
        __hip_atomic_store(a.timed_jobs, njobs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const size_t upj = (a.eb + kFillDevUnit - 1) / kFillDevUnit;
    const size_t total = upj * (size_t)njobs;
    for (size_t u = blockIdx.x; u < total; u += gridDim.x) {
        const int j = (int)(u / upj);
        const int e = a.jobs[1 + 2 * j];
        const int d = a.jobs[2 + 2 * j];
        const size_t off = (u - (size_t)j * upj) * kFillDevUnit;
        const size_t nvec = (a.eb - off < kFillDevUnit ? a.eb - off : kFillDevUnit) / 16;
        const char* src = a.pieces[e / a.per_piece] + (size_t)(e % a.per_piece) * a.eb + off;
        char* dst = (d >= 0 ? a.slots + (size_t)d * a.eb : a.staging + (size_t)(-d - 1) * a.eb) + off;
        const u32x4v* __restrict__ s4 = reinterpret_cast<const u32x4v*>(src);
        u32x4v* __restrict__ d4 = reinterpret_cast<u32x4v*>(dst);
        for (size_t i0 = threadIdx.x; i0 < nvec; i0 += 4 * kFillDevThreads) {
            u32x4v v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const size_t i = i0 + (size_t)q * kFillDevThreads;
                if (i < nvec) v[q] = s4[i];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const size_t i = i0 + (size_t)q * kFillDevThreads;
                if (i < nvec) __builtin_nontemporal_store(v[q], d4 + i);
            }
        }
    }
}

hipError_t launch_fill_dev(const FillDevArgs& a, int grid, hipEvent_t start, hipEvent_t stop, hipStream_t s) {
    if (grid < 1 || a.eb % 16) return hipErrorInvalidValue;
    if (start)
        hipExtLaunchKernelGGL(k_fill_dev, dim3(grid), dim3(kFillDevThreads), 0, s, start, stop, 0, a);
    else
        hipLaunchKernelGGL(k_fill_dev, dim3(grid), dim3(kFillDevThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
