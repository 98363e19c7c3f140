// The slot manager on the GPU (policy = MOE_POLICY_DEVICE), prepare form: one launch
// per step computes the step's distinct expert ids, applies the route rule, runs the
// eviction policy on the layer's state in HBM, remaps the ids, and pulls the missed
// (or staged) experts from the pinned store.  Nothing waits for the host, so a whole
// decode step can be queued at once, and nothing waits for another workgroup.
//
// The decision itself (policy_dev.hpp) follows vLLM PR "Run MoE models exceeding VRAM
// with expert CPU offloading with GPU cache", section "How it works", and the
// llama.cpp "Persistent expert slot pool" prefill rule.  Every workgroup of the launch
// runs it on its own LDS copy of the state (a few microseconds of latency, the same
// in each), so that each knows the step's copies; the first one also writes the
// results and the state after the step, into the layer's other state copy.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"
#include "policy_dev.hpp"

namespace moe {

constexpr size_t kFillUnit = (size_t)128 << 10;  // bytes of one copy work unit (16-256 KiB measured; 128 best by ~1 %)
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// The step's copies: 128 KiB work units over the launch, store -> slot (misses, in
// order), then -> staging (the distinct ids in rank order on the staging path, the
// host-read experts on a pooled step under EVICT_DECAY).
__device__ __forceinline__ void copy_step(const PolicyArgs& a, const PolLds& L, const Decision& d) {
    const int tid = threadIdx.x;
    const int nblocks = (int)gridDim.x;
    const bool pool = d.path == PATH_POOL;
    const int njobs = pool ? d.nmiss + d.nhost : d.D;
    const int nslot = pool ? d.nmiss : 0;     // jobs [0, nslot) go to slots, the rest to staging
    const size_t eb = a.eb;
    const size_t upj = (eb + kFillUnit - 1) / kFillUnit;
    const size_t units = upj * (size_t)njobs;
    for (size_t u = blockIdx.x; u < units; u += (size_t)nblocks) {
        const int j = (int)(u / upj);
        const int e = L.list[j];
        const size_t off = (u - (size_t)j * upj) * kFillUnit;
        const size_t nvec = (eb - off < kFillUnit ? eb - off : kFillUnit) / 16;
        const char* src = pol_src(a, e) + off;
        char* dst = (j < nslot ? a.slots + (size_t)L.map[e] * eb : a.staging + (size_t)(j - nslot) * eb) + off;
        const u32x4v* __restrict__ s4 = reinterpret_cast<const u32x4v*>(src);
        u32x4v* __restrict__ d4 = reinterpret_cast<u32x4v*>(dst);
        for (size_t i0 = tid; i0 < nvec; i0 += 4 * kPolThreads) {
            u32x4v v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const size_t i = i0 + (size_t)q * kPolThreads;
                if (i < nvec) v[q] = s4[i];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const size_t i = i0 + (size_t)q * kPolThreads;
                if (i < nvec) __builtin_nontemporal_store(v[q], d4 + i);
            }
        }
    }
}

__global__ __launch_bounds__(kPolThreads) void k_policy(PolicyArgs a) {
    extern __shared__ int32_t sm[];
    const PolLds L = pol_lds(sm, a.E, a.N, a.evict);
    const int tid = threadIdx.x;
    const bool lead = blockIdx.x == 0;
    const int nblocks = (int)gridDim.x;
    const int par = a.ds.ctl[0] & 1;
    const SlotView cur = slot_view(a.ds.copy[par], a.E, a.N);
    if (a.n <= 64 && !a.resident && a.evict != EVICT_SLRU && a.evict != EVICT_DECAY) {
        // a decode step whose ids are all valid and resident (and the static rule quiet)
        // changes keys only: the lead updates the current copy in place, the copies keep
        // their roles, and no other workgroup has anything to do
        __shared__ int allhit;
        if (tid < 64) {
            const int id = tid < a.n ? a.ids[tid] : 0;
            const bool ok = tid >= a.n || ((unsigned)id < (unsigned)a.E && cur.map[id] >= 0);
            const bool all = __all(ok);
            if (tid == 0) allhit = all && (a.rule == 0 || a.n <= a.N);
        }
        __syncthreads();
        if (allhit) {
            if (lead) pol_hit_in_place(a, cur, a.n);
            return;
        }
    }
    const Decision d = pol_decide(a, cur, L);
    // the workgroup's reads of the current copy returned before the decision's barriers
    int arrived = -1;
    if (tid == 0) arrived = pol_reader_arrive(a.ds.ctl);
    if (lead) pol_publish(a, slot_view(a.ds.copy[par ^ 1], a.E, a.N), L, d);

    // the remap, through the fresh table (each id written by one thread of the launch)
    const int gtid = blockIdx.x * kPolThreads + tid;
    const int gthreads = nblocks * kPolThreads;
    for (int i = gtid; i < a.n; i += gthreads) {
        const int e = a.ids[i];
        int v = -1;
        if (d.path == PATH_POOL) v = a.resident ? e : (L.map[e] >= 0 ? L.map[e] : L.rank[e]);
        else if (d.path == PATH_STAGE) v = L.rank[e];
        a.out[i] = v;
    }
    if (!a.resident && d.path != PATH_NONE) copy_step(a, L, d);
    if (tid == 0) pol_last_reader(a.ds.ctl, arrived, nblocks);
}

// ---- prefetch ------------------------------------------------------------------------
// One launch: every workgroup finds the same plan -- the predicted experts that the
// layer's current state copy does not hold, ascending, at most pf_n, to entries 0, 1,
// ... -- and copies its share of them (128 KiB units); workgroup 0 writes the entries'
// tags (entries past the plan keep theirs: their bytes are untouched).  Nothing in the
// launch reads the tags, and a step reads them only after the launch is complete.
__global__ __launch_bounds__(kPolThreads) void k_prefetch(PrefetchArgs a) {
    __shared__ uint32_t bits[kMaxExperts / 32];
    __shared__ int32_t list[64];
    __shared__ int32_t cnt[kPolWaves];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int E = a.E;
    const int nwords = (E + 31) >> 5;
    const int par = a.ds.ctl[0] & 1;
    const int32_t* map = reinterpret_cast<const int32_t*>(a.ds.copy[par] + slot_state_layout(E, a.N).map);
    for (int i = tid; i < nwords; i += kPolThreads) bits[i] = 0u;
    __syncthreads();
    if (tid < a.n) {
        const int e = a.ids[tid];
        if ((unsigned)e < (unsigned)E && map[e] < 0) atomicOr(&bits[e >> 5], 1u << (e & 31));
    }
    __syncthreads();
    int base = 0;
    for (int c0 = 0; c0 < E && base < a.pf_n; c0 += kPolThreads) {
        const int e = c0 + tid;
        const bool present = e < E && ((bits[e >> 5] >> (e & 31)) & 1u);
        const uint64_t m = __ballot(present);
        const uint32_t below =
            __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (lane == 0) cnt[wave] = __popcll(m);
        __syncthreads();
        int off = 0, total = 0;
        for (int w = 0; w < kPolWaves; ++w) {
            off += w < wave ? cnt[w] : 0;
            total += cnt[w];
        }
        const int pos = base + off + (int)below;
        if (present && pos < a.pf_n) list[pos] = e;
        base += total;
        __syncthreads();
    }
    const int njobs = base < a.pf_n ? base : a.pf_n;
    if (blockIdx.x == 0) {
        if (tid < njobs) a.tag[tid] = list[tid];
        if (tid == 0 && njobs) pol_bump(a.ds.ctr + 7, (unsigned long long)njobs * a.eb);
    }
    const size_t eb = a.eb;
    const size_t upj = (eb + kFillUnit - 1) / kFillUnit;
    const size_t units = upj * (size_t)njobs;
    for (size_t u = blockIdx.x; u < units; u += gridDim.x) {
        const int j = (int)(u / upj);
        const int e = list[j];
        const size_t off = (u - (size_t)j * upj) * kFillUnit;
        const size_t nvec = (eb - off < kFillUnit ? eb - off : kFillUnit) / 16;
        const u32x4v* __restrict__ s4 =
            reinterpret_cast<const u32x4v*>(a.pieces[e / a.per_piece] + (size_t)(e % a.per_piece) * eb + off);
        u32x4v* __restrict__ d4 = reinterpret_cast<u32x4v*>(a.buf + (size_t)j * eb + off);
        for (size_t i0 = tid; i0 < nvec; i0 += 4 * kPolThreads) {
            u32x4v v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const size_t i = i0 + (size_t)q * kPolThreads;
                if (i < nvec) v[q] = s4[i];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const size_t i = i0 + (size_t)q * kPolThreads;
                if (i < nvec) __builtin_nontemporal_store(v[q], d4 + i);
            }
        }
    }
}

hipError_t launch_prefetch(const PrefetchArgs& a, int copy_grid, hipStream_t s) {
    if (a.n < 1 || a.n > kPolThreads || a.pf_n < 1 || a.pf_n > 64 || a.E > kMaxExperts || a.eb % 16 ||
        a.per_piece < 1 || copy_grid < 1)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_prefetch, dim3(copy_grid), dim3(kPolThreads), 0, s, a);
    return hipGetLastError();
}

size_t policy_lds_bytes(int E, int N, int evict) { return pol_lds_words(E, N, evict) * sizeof(int32_t); }

hipError_t launch_policy(const PolicyArgs& a, int grid, hipEvent_t start, hipEvent_t stop, hipStream_t s) {
    if (a.n < 1 || a.n > (1 << 24) || grid < 1 || a.eb % 16 || a.evict < EVICT_LRU || a.evict > EVICT_DECAY ||
        (!a.resident && a.per_piece < 1))
        return hipErrorInvalidValue;
    const size_t lds = policy_lds_bytes(a.E, a.N, a.evict);
    if (start)
        hipExtLaunchKernelGGL(k_policy, dim3(grid), dim3(kPolThreads), lds, s, start, stop, 0, a);
    else
        hipLaunchKernelGGL(k_policy, dim3(grid), dim3(kPolThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace moe
