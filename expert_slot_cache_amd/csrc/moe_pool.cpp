// C-ABI runtime of the expert slot cache: pinned host store, fixed-address HBM slot
// pools, copy streams, the per-layer slot manager, prepare/forward/step.
//
// Step order per layer (llama.cpp "Persistent expert slot pool", section "Design"
// item 3: read ids back, update the LRU, issue async H2D for misses and rewrite the
// map table before the remap consumes it):
//   1. k_distinct on the compute stream -> distinct ids in pinned host memory;
//      wait for it (the one host sync of a step).
//   2. host: range check, route rule, LRU update (SlotLRU) -> miss list.
//   3. hipMemcpyAsync store -> slot for each miss on the copy streams, optionally
//      in chunks.  No write-after-read wait is needed: every kernel that reads a
//      slot or the staging area runs on the compute stream, and the readback of
//      step 1 has seen k_distinct finish -- so every kernel queued before it,
//      the last reader of any destination included, has finished too.
//   4. the step's map changes go to a small pinned list that k_remap reads: it
//      applies them to the persistent HBM table and remaps through the fresh table.
//      The compute stream waits for the copies (an event per copy stream).  No
//      kernel ever waits for the host or for another stream: streams can share a
//      hardware queue, and a kernel spinning on work queued behind it would only
//      end at its time limit.
//   5. forward kernels on the compute stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "moe_pool.h"
#include "kernels.hpp"
#include "layout.hpp"
#include "slot_lru.hpp"

namespace {

thread_local char g_err[512] = "";

void set_err(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

}  // namespace

namespace moe {
// The calling thread's last error message (moe_last_error), for the library's other
// translation units.
void set_last_error(const char* msg) { snprintf(g_err, sizeof(g_err), "%s", msg); }
}  // namespace moe

namespace {

#define FAIL(code, ...)        \
    do {                       \
        set_err(__VA_ARGS__);  \
        return (code);         \
    } while (0)

#define HIPCHK(call)                                                                     \
    do {                                                                                 \
        hipError_t e_ = (call);                                                          \
        if (e_ != hipSuccess) {                                                          \
            set_err("%s failed: %s (%s:%d)", #call, hipGetErrorString(e_), __FILE__, __LINE__); \
            return MOE_EHIP;                                                             \
        }                                                                                \
    } while (0)

constexpr size_t kAlign = 256;
size_t round_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

using moe::Layout;
using moe::make_layout;

struct Timing {
    hipEvent_t a = nullptr, b = nullptr;   // start, stop
    bool pending = false;
    uint64_t bytes = 0;                    // copies: bytes between the two events
};

// Pinned allocations are made in pieces of at most this many bytes (whole experts).
constexpr size_t kStorePiece = (size_t)1 << 30;
// Workgroups of one device-policy step: each runs the decision, then the copies
// (128 KiB units) spread over all of them.
constexpr int kPolicyGrid = 128;
// Copy workers of a fused one-token step (the part of each missed expert past its w13
// rows, 64 KiB units).
constexpr int kStepCopyWorkers = 64;
// Workgroups of a prefetch's copy launch.
constexpr int kPrefetchGrid = 64;

struct LayerState {
    moe::SlotLRU lru;
    std::vector<char*> store;    // pinned host pieces holding the E experts in order
    std::vector<char*> store_dev;// the same pieces' device addresses (mapped)
    int32_t per_piece = 1;       // experts per piece
    char* slots = nullptr;       // HBM: nslot_alloc experts + zeroed tail
    int32_t* map_dev = nullptr;  // HBM int32 [E]: the persistent map table
    int32_t* upd_host = nullptr; // pinned int32 [2E]: this step's (entry, value) changes
    int32_t* upd_dev = nullptr;  // device view of upd_host
    int32_t* path_dev = nullptr; // HBM int32: the path the last remap chose
    bool prepared = false;
    char* expert(int32_t e, size_t eb) const { return store[e / per_piece] + (size_t)(e % per_piece) * eb; }
    const char* expert_dev(int32_t e, size_t eb) const {
        return store_dev[e / per_piece] + (size_t)(e % per_piece) * eb;
    }
    int32_t prep_tokens = 0;
    int32_t prep_path = MOE_PATH_POOL;
    uint64_t bytes_h2d = 0;
    uint64_t staged = 0;
    std::vector<Timing> copy_t;  // one per copy stream
    Timing w13_t, w2_t;
    // last step, as prepare returned it (MOE_POLICY_HOST) or as the host knows it
    bool has_last = false;
    int32_t last_path = MOE_PATH_POOL;
    std::vector<moe::Miss> last_misses;
    // MOE_POLICY_DEVICE: the slot manager's state in HBM, the store pieces' device
    // addresses (device array), and the fill timing of this layer
    char* dev_block = nullptr;
    moe::DevState ds{};
    bool rt_sample = false;      // the pending w13/w2 timing sample is a read-through step
    // prefetch buffer (prefetch_slots entries), its tags and job list (device), and the
    // event the next step of the layer waits for
    char* pf_buf = nullptr;
    int32_t* pf_tag = nullptr;
    hipEvent_t pf_done = nullptr;
    bool pf_pending = false;
    hipEvent_t step_done = nullptr;   // after the layer's last prepare or step
    bool stepped = false;
    const char** pieces_dev = nullptr;
    bool last_empty = false;     // the last step had no tokens (not seen by the GPU)
    uint64_t empty_steps = 0;    // steps with no tokens (counted on the host)
    Timing fill_t;
};

}  // namespace

struct moe_pool {
    moe_pool_config_t cfg{};
    Layout lay;
    moe::Geom geom{};
    int32_t nslot_alloc = 0;
    int32_t timing_alloc = 0;     // config.timing at create: > 0 if the timing events exist
    hipStream_t compute = nullptr;
    std::vector<hipStream_t> copy;
    std::vector<hipEvent_t> copy_done;
    hipEvent_t pf_issue = nullptr;  // compute-stream point a prefetch starts after
    std::vector<LayerState> layers;
    char* staging = nullptr;
    int32_t staging_cap = 0;
    int32_t staging_owner = -1;
    uint32_t* rb_host = nullptr;  // pinned [1 + E] tagged words, written by k_distinct
    uint32_t* rb_dev = nullptr;   // device view of rb_host
    uint32_t rb_tag = 0;          // tag of the last readback (1 .. 2^18 - 1)
    int32_t rb_used = 0;          // words of rb_host written by the last readback
    std::vector<int32_t> ulist;   // the last readback's distinct ids
    int32_t* rank_dev = nullptr;  // HBM [E]
    int32_t* ident_dev = nullptr; // HBM [E] identity table (resident mode)
    int32_t* paths_dev = nullptr; // HBM [n_layers]
    void* act = nullptr;          // HBM [max_tokens * K][I] SwiGLU output
    float* y = nullptr;           // HBM [max_tokens * K][H] per-pair w2 output
    int32_t* grp = nullptr;       // HBM grouped-path index buffer
    int32_t grp_slots = 0;        // largest slot count a forward can address
    std::vector<moe::Miss> misses;
    // MOE_POLICY_DEVICE
    uint32_t* errs_host = nullptr;      // pinned coherent [n_layers]: set by the GPU on an id outside [0,E)
    uint32_t* errs_dev = nullptr;
    int32_t* timed_jobs_host = nullptr; // pinned coherent [n_layers]: jobs of the last timed fill
    int32_t* timed_jobs_dev = nullptr;
    int32_t* rt_jobs_host = nullptr;    // pinned coherent [n_layers]: experts read through by the
    int32_t* rt_jobs_dev = nullptr;     //   last timed read-through step
    int32_t last_prepared = -1;         // the layer of the latest prepare (device policy)
    std::vector<char> used_copy;
    int copy_rr = 0;
    // timing totals (sampled calls)
    double copy_ms = 0, w13_ms = 0, w2_ms = 0, sync_ms = 0;
    uint64_t copy_calls = 0, copy_bytes = 0, kern_calls = 0;
    uint64_t n_copy_batches = 0, n_forwards = 0;   // all calls, for the sampling period
};

struct moe_lru {
    moe::SlotLRU lru;
    std::vector<moe::Miss> misses;
    std::vector<int32_t> u;
};

namespace {

void destroy_pool(moe_pool* p) {
    if (!p) return;
    if (p->compute || !p->copy.empty()) (void)hipDeviceSynchronize();
    for (auto& L : p->layers) {
        for (char* piece : L.store)
            if (piece) (void)hipHostFree(piece);
        if (L.slots) (void)hipFree(L.slots);
        if (L.map_dev) (void)hipFree(L.map_dev);
        if (L.upd_host) (void)hipHostFree(L.upd_host);
        if (L.dev_block) (void)hipFree(L.dev_block);
        if (L.pieces_dev) (void)hipFree(L.pieces_dev);
        if (L.pf_buf) (void)hipFree(L.pf_buf);
        if (L.pf_tag) (void)hipFree(L.pf_tag);
        if (L.pf_done) (void)hipEventDestroy(L.pf_done);
        if (L.step_done) (void)hipEventDestroy(L.step_done);
        if (L.fill_t.a) (void)hipEventDestroy(L.fill_t.a);
        if (L.fill_t.b) (void)hipEventDestroy(L.fill_t.b);
        for (auto& t : L.copy_t) {
            if (t.a) (void)hipEventDestroy(t.a);
            if (t.b) (void)hipEventDestroy(t.b);
        }
        for (Timing* t : {&L.w13_t, &L.w2_t}) {
            if (t->a) (void)hipEventDestroy(t->a);
            if (t->b) (void)hipEventDestroy(t->b);
        }
    }
    for (auto s : p->copy) (void)hipStreamDestroy(s);
    for (auto e : p->copy_done) (void)hipEventDestroy(e);
    if (p->pf_issue) (void)hipEventDestroy(p->pf_issue);
    if (p->staging) (void)hipFree(p->staging);
    if (p->rb_host) (void)hipHostFree(p->rb_host);
    if (p->rank_dev) (void)hipFree(p->rank_dev);
    if (p->paths_dev) (void)hipFree(p->paths_dev);
    if (p->ident_dev) (void)hipFree(p->ident_dev);
    if (p->act) (void)hipFree(p->act);
    if (p->y) (void)hipFree(p->y);
    if (p->grp) (void)hipFree(p->grp);
    if (p->errs_host) (void)hipHostFree(p->errs_host);
    if (p->timed_jobs_host) (void)hipHostFree(p->timed_jobs_host);
    if (p->rt_jobs_host) (void)hipHostFree(p->rt_jobs_host);
    delete p;
}

moe_status_t check_layer(const moe_pool* p, int32_t layer) {
    if (!p) FAIL(MOE_EINVAL, "null pool");
    if (layer < 0 || layer >= p->cfg.n_layers) FAIL(MOE_EINVAL, "layer %d outside [0,%d)", layer, p->cfg.n_layers);
    return MOE_OK;
}

// Harvest finished timing event pairs (all work before the last readback sync).
bool done(const Timing& t) { return t.pending && hipEventQuery(t.b) == hipSuccess; }

bool harvest(moe_pool* p, Timing& t, double* acc) {
    if (!t.pending) return false;
    float ms = 0;
    const bool ok = hipEventElapsedTime(&ms, t.a, t.b) == hipSuccess;
    if (ok) *acc += ms;
    t.pending = false;
    return ok;
}

void harvest_layer(moe_pool* p, LayerState& L, int32_t l) {
    if (!p->cfg.timing) return;
    // the copy span of a step: earliest start to latest stop over the copy streams
    bool any = false, ready = true;
    for (auto& t : L.copy_t)
        if (t.pending) {
            any = true;
            ready = ready && done(t);
        }
    if (any && ready) {
        int ref = -1;
        for (size_t i = 0; i < L.copy_t.size(); ++i)
            if (L.copy_t[i].pending) {
                ref = (int)i;
                break;
            }
        float lo = 0, hi = 0;
        uint64_t bytes = 0;
        for (auto& t : L.copy_t) {
            if (!t.pending) continue;
            float s = 0, e = 0;
            (void)hipEventElapsedTime(&s, L.copy_t[ref].a, t.a);
            (void)hipEventElapsedTime(&e, L.copy_t[ref].a, t.b);
            lo = std::min(lo, s);
            hi = std::max(hi, e);
            bytes += t.bytes;
            t.pending = false;
        }
        p->copy_ms += hi - lo;
        p->copy_calls++;
        p->copy_bytes += bytes;
    }
    if (L.w13_t.pending && L.w2_t.pending && (!done(L.w13_t) || !done(L.w2_t))) return;
    if (L.rt_sample && L.w13_t.pending && L.w2_t.pending) {
        // a read-through step: with experts read over the link its two launches are
        // the step's transfer span; without, a forward like any other
        L.rt_sample = false;
        const int32_t jobs = ((volatile int32_t*)p->rt_jobs_host)[l];
        if (jobs > 0) {
            double ms = 0;
            const bool a = harvest(p, L.w13_t, &ms);
            const bool b = harvest(p, L.w2_t, &ms);
            if (a && b) {
                p->copy_ms += ms;
                p->copy_calls++;
                p->copy_bytes += (uint64_t)jobs * p->lay.total;
            }
            return;
        }
    }
    const bool a = harvest(p, L.w13_t, &p->w13_ms);
    const bool b = harvest(p, L.w2_t, &p->w2_ms);
    if (a && b) p->kern_calls++;
}

// A timed fill (device policy) counts only when it copied something; the kernel
// leaves its job count in host memory for this.
void harvest_fill(moe_pool* p, int32_t l) {
    LayerState& L = p->layers[l];
    if (!L.fill_t.pending || !done(L.fill_t)) return;
    const int32_t jobs = ((volatile int32_t*)p->timed_jobs_host)[l];
    if (jobs > 0) {
        float ms = 0;
        if (hipEventElapsedTime(&ms, L.fill_t.a, L.fill_t.b) == hipSuccess) {
            p->copy_ms += ms;
            p->copy_calls++;
            p->copy_bytes += (uint64_t)jobs * p->lay.total;
        }
    }
    L.fill_t.pending = false;
}

void harvest_all(moe_pool* p) {
    for (int32_t l = 0; l < p->cfg.n_layers; ++l) harvest_layer(p, p->layers[l], l);
    if (p->cfg.policy == MOE_POLICY_DEVICE)
        for (int32_t l = 0; l < p->cfg.n_layers; ++l) harvest_fill(p, l);
}

// The copy-kernel engine: the experts go in batches of up to kFillMaxJobs per launch,
// batches round-robin over the copy streams; each used stream records its copy_done
// event (joined into the compute stream), as with the DMA engine.
moe_status_t issue_copy_kernels(moe_pool* p, LayerState& L, const std::vector<std::pair<char*, int32_t>>& jobs) {
    const int ns = (int)p->copy.size();
    const size_t eb = p->lay.total;
    std::fill(p->used_copy.begin(), p->used_copy.end(), 0);
    bool timed = p->cfg.timing > 0 && (p->n_copy_batches++ % (uint64_t)p->cfg.timing) == 0;
    for (const auto& t : L.copy_t) timed = timed && !t.pending;
    const int nb = (int)((jobs.size() + moe::kFillMaxJobs - 1) / moe::kFillMaxJobs);
    const int streams_needed = std::min(ns, nb);
    for (int i = 0; i < streams_needed; ++i) {
        const int s = (p->copy_rr + i) % ns;
        if (timed) {
            HIPCHK(hipEventRecord(L.copy_t[s].a, p->copy[s]));
            L.copy_t[s].bytes = 0;
        }
        p->used_copy[s] = 1;
    }
    int rr = p->copy_rr;
    for (size_t j0 = 0; j0 < jobs.size(); j0 += moe::kFillMaxJobs) {
        moe::FillBatch b{};
        b.bytes = eb;
        b.n = (int)std::min<size_t>(moe::kFillMaxJobs, jobs.size() - j0);
        for (int i = 0; i < b.n; ++i) b.job[i] = moe::FillJob{L.expert_dev(jobs[j0 + i].second, eb), jobs[j0 + i].first};
        HIPCHK(moe::launch_fill(b, p->copy[rr]));
        if (timed) L.copy_t[rr].bytes += (uint64_t)b.n * eb;
        rr = (rr + 1) % ns;
    }
    p->copy_rr = rr;
    for (int s = 0; s < ns; ++s) {
        if (!p->used_copy[s]) continue;
        if (timed) {
            HIPCHK(hipEventRecord(L.copy_t[s].b, p->copy[s]));
            L.copy_t[s].pending = true;
        }
        HIPCHK(hipEventRecord(p->copy_done[s], p->copy[s]));
        HIPCHK(hipStreamWaitEvent(p->compute, p->copy_done[s], 0));
    }
    L.bytes_h2d += (uint64_t)eb * jobs.size();
    return MOE_OK;
}

// Enqueue host->HBM copies of the experts (src -> dst pairs) on the copy streams,
// record each used stream's copy_done event, and make the compute stream wait
// for those events.
// jobs: (destination in HBM, source expert index in the layer's store).
moe_status_t issue_copies(moe_pool* p, LayerState& L, const std::vector<std::pair<char*, int32_t>>& jobs) {
    if (jobs.empty()) return MOE_OK;
    const int ns = (int)p->copy.size();
    const size_t eb = p->lay.total;
    if (p->cfg.copy_engine == MOE_COPY_KERNEL) return issue_copy_kernels(p, L, jobs);
    const size_t chunk = p->cfg.copy_chunk_bytes ? p->cfg.copy_chunk_bytes : eb;
    std::fill(p->used_copy.begin(), p->used_copy.end(), 0);
    bool timed = p->cfg.timing > 0 && (p->n_copy_batches++ % (uint64_t)p->cfg.timing) == 0;
    for (const auto& t : L.copy_t) timed = timed && !t.pending;
    const int streams_needed = std::min<size_t>(ns, jobs.size() * ((eb + chunk - 1) / chunk));
    for (int i = 0; i < streams_needed; ++i) {
        const int s = (p->copy_rr + i) % ns;
        if (timed) {
            HIPCHK(hipEventRecord(L.copy_t[s].a, p->copy[s]));
            L.copy_t[s].bytes = 0;
        }
        p->used_copy[s] = 1;
    }
    int rr = p->copy_rr;
    for (const auto& j : jobs) {
        const char* src = L.expert(j.second, eb);
        for (size_t off = 0; off < eb; off += chunk) {
            const size_t n = std::min(chunk, eb - off);
            HIPCHK(hipMemcpyAsync(j.first + off, src + off, n, hipMemcpyHostToDevice, p->copy[rr]));
            if (timed) L.copy_t[rr].bytes += n;
            rr = (rr + 1) % ns;
        }
    }
    p->copy_rr = rr;
    for (int s = 0; s < ns; ++s) {
        if (!p->used_copy[s]) continue;
        if (timed) {
            HIPCHK(hipEventRecord(L.copy_t[s].b, p->copy[s]));
            L.copy_t[s].pending = true;
        }
        HIPCHK(hipEventRecord(p->copy_done[s], p->copy[s]));
        HIPCHK(hipStreamWaitEvent(p->compute, p->copy_done[s], 0));
    }
    L.bytes_h2d += (uint64_t)eb * jobs.size();
    return MOE_OK;
}

// ---- the steps of prepare -----------------------------------------------------------

// The next readback: zero the words the last one used and take a new tag.
void next_readback(moe_pool* p) {
    std::memset(p->rb_host, 0, (size_t)p->rb_used * 4);
    p->rb_tag = p->rb_tag % ((1u << 18) - 1) + 1;
    p->rb_used = 0;
}

// Distinct ids of the step, written by the kernel as tagged words into pinned host
// memory (zeroed here beforehand) and rank[] on the device.
moe_status_t launch_distinct_ids(moe_pool* p, const int32_t* ids_dev, int n) {
    next_readback(p);
    HIPCHK(moe::launch_distinct(ids_dev, n, p->cfg.n_experts, p->rb_dev, p->rank_dev, p->rb_tag, p->compute));
    return MOE_OK;
}

// The readback: the step's one host sync.  The host spins until each word it needs
// carries this step's tag, checking the stream now and then so that a failed launch
// cannot leave it spinning.  Fills p->ulist[0..D).
moe_status_t read_distinct(moe_pool* p, int32_t layer, int32_t* D_out) {
    const uint32_t tag = p->rb_tag;
    const int32_t E = p->cfg.n_experts;
    const auto t0 = std::chrono::steady_clock::now();
    const volatile uint32_t* rbv = p->rb_host;
    auto wait_word = [&](int i) -> moe_status_t {
        for (uint64_t it = 1;; ++it) {
            const uint32_t w = rbv[i];
            if ((w >> 14) == tag) return MOE_OK;
            if ((it & 255) == 0) {
                const hipError_t q = hipStreamQuery(p->compute);
                if (q == hipSuccess) {
                    // everything queued has finished, the distinct kernel included
                    if ((rbv[i] >> 14) == tag) return MOE_OK;
                    FAIL(MOE_EHIP, "distinct-id readback word %d missing after the stream drained", i);
                }
                if (q != hipErrorNotReady) FAIL(MOE_EHIP, "hipStreamQuery failed: %s", hipGetErrorString(q));
            }
            __builtin_ia32_pause();
        }
    };
    p->rb_used = 1;
    moe_status_t st = wait_word(0);
    if (st) return st;
    const uint32_t w0 = rbv[0];
    const int32_t D = (int32_t)(w0 & 0x1FFFu);
    const bool bad = (w0 >> 13) & 1u;
    if (D > E) FAIL(MOE_EHIP, "distinct-id readback returned D=%d", D);
    p->rb_used = 1 + D;
    for (int32_t i = 0; i < D; ++i) {
        st = wait_word(1 + i);
        if (st) return st;
        p->ulist[i] = (int32_t)(rbv[1 + i] & 0x3FFFu);
    }
    if (p->cfg.timing)
        p->sync_ms += std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    if (bad) FAIL(MOE_ERANGE, "layer %d: an expert id is outside [0,%d)", layer, E);
    if (D < 1) FAIL(MOE_EHIP, "distinct-id readback returned D=%d", D);
    *D_out = D;
    return MOE_OK;
}

// The LRU step over p->ulist[0..D), the map-change list and the miss copies (the
// compute stream waits for them).
moe_status_t route(moe_pool* p, LayerState& L, int32_t layer, int32_t D, int n, int32_t* the_path,
                   int32_t* n_upd_out) {
    const size_t eb = p->lay.total;
    const int32_t* u = p->ulist.data();
    moe_status_t st;
    p->misses.clear();
    *the_path = MOE_PATH_POOL;
    *n_upd_out = 0;
    // The readback has seen this step's distinct kernel finish, and with it every
    // earlier kernel of the compute stream: no reads of a destination are pending,
    // so the copies wait for nothing.
    if (p->cfg.resident) {
        L.lru.count_resident(D);
    } else if (L.lru.step(u, D, (int64_t)n, p->misses)) {
        // The map changes, applied by the remap kernel before it reads the table.
        // Each touched entry carries its value after the whole step: an expert can
        // be evicted by an earlier (lower-id) miss of the step and re-inserted by
        // its own miss later in the same step, so an entry may appear twice -- with
        // the same final value, which makes the kernel's unordered writes safe.
        // (The previous step's list was consumed before this step's readback.)
        const std::vector<int32_t>& fmap = L.lru.map();
        int n_upd = 0;
        for (const auto& m : p->misses) {
            if (m.evicted >= 0) {
                L.upd_host[2 * n_upd] = m.evicted;
                L.upd_host[2 * n_upd + 1] = fmap[m.evicted];
                ++n_upd;
            }
            L.upd_host[2 * n_upd] = m.expert;
            L.upd_host[2 * n_upd + 1] = fmap[m.expert];
            ++n_upd;
        }
        *n_upd_out = n_upd;
        if (!p->misses.empty()) {
            std::vector<std::pair<char*, int32_t>> jobs;
            jobs.reserve(p->misses.size());
            for (const auto& m : p->misses) jobs.emplace_back(L.slots + (size_t)m.slot * eb, m.expert);
            st = issue_copies(p, L, jobs);
            if (st) return st;
        }
    } else {
        // selective-copy fallback: the step's experts go to staging in rank order;
        // the pool is untouched
        *the_path = MOE_PATH_FALLBACK;
        std::vector<std::pair<char*, int32_t>> jobs;
        jobs.reserve(D);
        for (int32_t r = 0; r < D; ++r) jobs.emplace_back(p->staging + (size_t)r * eb, u[r]);
        st = issue_copies(p, L, jobs);
        if (st) return st;
        L.staged += (uint64_t)D;
        p->staging_owner = layer;
    }
    return MOE_OK;
}

void finish_prepare(moe_pool* p, LayerState& L, int32_t n_tokens, int32_t the_path, moe_miss_t* miss_host,
                    int32_t miss_cap, int32_t* n_miss, int32_t* path) {
    L.prepared = true;
    L.prep_tokens = n_tokens;
    L.prep_path = the_path;
    const int32_t nm = (int32_t)p->misses.size();
    if (miss_host) {
        for (int32_t i = 0; i < std::min(nm, miss_cap); ++i)
            miss_host[i] = moe_miss_t{p->misses[i].expert, p->misses[i].slot, p->misses[i].evicted};
    }
    if (n_miss) *n_miss = nm;
    if (path) *path = the_path;
    L.has_last = true;
    L.last_path = the_path;
    L.last_misses = p->misses;
}

// Staging entries a pooled step addresses past the pool (slot ids N + r): the
// experts that placement by decayed counts reads from the host for one step (at most
// the step's distinct ids, so at most N and at most the staging capacity).
int32_t mixed_entries(const moe_pool_config_t& c, int32_t staging_cap) {
    return c.evict == MOE_EVICT_DECAY && !c.resident ? std::min(c.n_slots, staging_cap) : 0;
}

moe::Slots layer_slots(const moe_pool* p, const LayerState& L) {
    const int32_t nmix = mixed_entries(p->cfg, p->staging_cap);
    // with mixed ids the pool's valid ids end at the current n_slots (slot ids from N on
    // are staging entries)
    return moe::Slots{L.slots, p->staging, nmix ? p->cfg.n_slots : p->nslot_alloc, p->staging_cap, nmix,
                      L.path_dev};
}

moe::ForwardArgs forward_args(const moe_pool* p, const LayerState& L, const void* x_dev, const int32_t* slot_ids_dev,
                              const float* topk_w_dev, const void* resid_dev, int32_t n_tokens, void* out_dev) {
    moe::ForwardArgs a{};
    a.sl = layer_slots(p, L);
    a.slot_ids = slot_ids_dev;
    a.x = x_dev;
    a.topk_w = topk_w_dev;
    a.resid = resid_dev;
    a.out = out_dev;
    a.T = n_tokens;
    a.act = p->act;
    a.y = p->y;
    a.grp = p->grp;
    a.nslots_alloc = std::max(1, p->grp_slots);
    a.max_pairs = p->cfg.max_tokens * p->cfg.top_k;
    return a;
}

moe_status_t launch_layer_forward(moe_pool* p, LayerState& L, const void* x_dev, const int32_t* slot_ids_dev,
                                  const float* topk_w_dev, const void* resid_dev, int32_t n_tokens, void* out_dev) {
    const moe::ForwardArgs a = forward_args(p, L, x_dev, slot_ids_dev, topk_w_dev, resid_dev, n_tokens, out_dev);
    moe::StageEvents ev;
    const bool timed = p->cfg.timing > 0 && (p->n_forwards++ % (uint64_t)p->cfg.timing) == 0 && !L.w13_t.pending &&
                       !L.w2_t.pending;
    if (timed) {
        ev.w13_start = L.w13_t.a;
        ev.w13_stop = L.w13_t.b;
        ev.w2_start = L.w2_t.a;
        ev.w2_stop = L.w2_t.b;
    }
    HIPCHK(moe::launch_forward(p->geom, a, timed ? &ev : nullptr, p->compute));
    if (timed) {
        L.w13_t.pending = true;
        L.w2_t.pending = true;
    }
    return MOE_OK;
}

// ---- MOE_POLICY_DEVICE ------------------------------------------------------------
// Byte layout of one layer's device state block: the two state copies
// (moe::slot_state_layout), the control words {par, readers}, the counters and the
// last step's record.
struct DevLayout {
    size_t copy0, copy1, ctl, ctr, rec, total;
};

DevLayout dev_layout(int32_t E, int32_t N) {
    DevLayout d{};
    const size_t one = moe::slot_state_layout(E, N).total;
    d.copy0 = 0;
    d.copy1 = one;
    d.ctl = 2 * one;
    d.ctr = d.ctl + kAlign;
    d.rec = d.ctr + kAlign;
    d.total = round_up(d.rec + (size_t)(4 + 3 * N) * 4);
    return d;
}

// The cold state image: in both copies map -1, owners -1, free slots 0..N-1 (popped
// from the end), keys and uses 0, nothing protected, meta {nfree = N, tick 0,
// nprot 0}; par 0, no readers, counters and record zero.
std::vector<char> dev_cold_image(const moe_pool* p) {
    const int32_t E = p->cfg.n_experts, N = p->cfg.resident ? 0 : p->cfg.n_slots;
    const DevLayout d = dev_layout(E, N);
    const moe::SlotStateLayout o = moe::slot_state_layout(E, N);
    std::vector<char> img(d.total, 0);
    for (size_t base : {d.copy0, d.copy1}) {
        auto w = [&](size_t off) { return reinterpret_cast<int32_t*>(img.data() + base + off); };
        std::fill(w(o.map), w(o.map) + E, -1);
        std::fill(w(o.owner), w(o.owner) + N, -1);
        for (int32_t s2 = 0; s2 < N; ++s2) w(o.free)[s2] = s2;
        w(o.meta)[0] = N;
    }
    return img;
}

moe_status_t dev_init_layers(moe_pool* p) {
    const std::vector<char> img = dev_cold_image(p);
    for (auto& L : p->layers) {
        HIPCHK(hipMemcpy(L.dev_block, img.data(), img.size(), hipMemcpyHostToDevice));
        L.rt_sample = false;
        L.has_last = false;
        L.last_empty = false;
        L.empty_steps = 0;
    }
    std::memset(p->errs_host, 0, sizeof(uint32_t) * p->cfg.n_layers);
    return MOE_OK;
}

// An id outside [0,E) found by a layer's earlier device step.
moe_status_t check_dev_err(moe_pool* p, int32_t layer) {
    volatile uint32_t* e = p->errs_host + layer;
    if (*e) {
        *e = 0;
        FAIL(MOE_ERANGE, "layer %d: an earlier step had an expert id outside [0,%d); it changed nothing and its"
                         " output is undefined", layer, p->cfg.n_experts);
    }
    return MOE_OK;
}

// The decision's arguments for one step of layer `layer` (n_tokens >= 1).
moe::PolicyArgs policy_args(moe_pool* p, LayerState& L, int32_t layer, const int32_t* ids_dev, int32_t n_tokens,
                            int32_t* slot_ids_dev) {
    const bool resident = p->cfg.resident != 0;
    moe::PolicyArgs a{};
    a.ids = ids_dev;
    a.n = n_tokens * p->cfg.top_k;
    a.E = p->cfg.n_experts;
    a.N = resident ? 0 : p->cfg.n_slots;
    a.rule = p->cfg.rule;
    a.evict = p->cfg.evict;
    a.resident = p->cfg.resident;
    a.eb = p->lay.total;
    a.ds = L.ds;
    a.out = slot_ids_dev;
    a.path = L.path_dev;
    a.err = p->errs_dev + layer;
    a.pieces = L.pieces_dev;
    a.per_piece = L.per_piece;
    a.slots = L.slots;
    a.staging = p->staging;
    a.pf_tag = L.pf_tag;
    a.pf_buf = L.pf_buf;
    a.pf_n = L.pf_buf ? p->cfg.prefetch_slots : 0;
    return a;
}

// A step of the layer starts after the layer's last prefetch (the join of the copy
// stream into the compute stream).
moe_status_t join_prefetch(moe_pool* p, LayerState& L) {
    if (!L.pf_pending) return MOE_OK;
    HIPCHK(hipStreamWaitEvent(p->compute, L.pf_done, 0));
    L.pf_pending = false;
    return MOE_OK;
}

// Every prefetch tag of the layer back to "nothing held".
moe_status_t clear_prefetch(moe_pool* p, LayerState& L) {
    if (!L.pf_tag) return MOE_OK;
    L.stepped = false;
    const std::vector<int32_t> none(p->cfg.prefetch_slots, -1);
    HIPCHK(hipMemcpy(L.pf_tag, none.data(), none.size() * 4, hipMemcpyHostToDevice));
    L.pf_pending = false;
    return MOE_OK;
}

// Queue the slot manager with its copies for one step (n_tokens >= 1).
moe_status_t dev_prepare(moe_pool* p, LayerState& L, int32_t layer, const int32_t* ids_dev, int32_t n_tokens,
                         int32_t* slot_ids_dev) {
    const bool resident = p->cfg.resident != 0;
    moe_status_t st = join_prefetch(p, L);
    if (st) return st;
    moe::PolicyArgs a = policy_args(p, L, layer, ids_dev, n_tokens, slot_ids_dev);
    // the copy span of a timed step is the launch's (its decision takes a few us)
    const bool timed = !resident && p->cfg.timing > 0 &&
                       (p->n_copy_batches++ % (uint64_t)p->cfg.timing) == 0 && !L.fill_t.pending;
    a.timed_jobs = timed ? p->timed_jobs_dev + layer : nullptr;
    // resident: no copies, so only as many workgroups as the ids need (256 per)
    const int grid = resident ? std::max(1, std::min(kPolicyGrid, a.n / 256)) : kPolicyGrid;
    HIPCHK(moe::launch_policy(a, grid, timed ? L.fill_t.a : nullptr, timed ? L.fill_t.b : nullptr, p->compute));
    if (timed) L.fill_t.pending = true;
    if (L.step_done) {
        HIPCHK(hipEventRecord(L.step_done, p->compute));
        L.stepped = true;
    }
    L.prepared = true;
    L.prep_tokens = n_tokens;
    L.prep_path = -1;            // known on the GPU only
    L.has_last = true;
    L.last_empty = false;
    return MOE_OK;
}

template <class T>
moe_status_t dev_read(const moe_pool* p, T* dst, const void* src, size_t n) {
    for (auto s : p->copy) HIPCHK(hipStreamSynchronize(s));   // a prefetch counts its bytes
    HIPCHK(hipStreamSynchronize(p->compute));
    HIPCHK(hipMemcpy(dst, src, n * sizeof(T), hipMemcpyDeviceToHost));
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_strerror(moe_status_t s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_EINVAL: return "invalid argument";
        case MOE_ENOMEM: return "out of memory";
        case MOE_EHIP: return "HIP runtime error";
        case MOE_ERANGE: return "expert id out of range";
        case MOE_ESTATE: return "forward without a matching prepare";
    }
    return "unknown status";
}

const char* moe_last_error(void) { return g_err; }

size_t moe_expert_bytes(int32_t wtype, int32_t hidden, int32_t inter) {
    Layout L;
    return make_layout(wtype, hidden, inter, &L) ? L.total : 0;
}

moe_status_t moe_pool_create(const moe_pool_config_t* cfg, void* stream, moe_pool_t** out) {
    if (!cfg || !out) FAIL(MOE_EINVAL, "null argument");
    *out = nullptr;
    const moe_pool_config_t& c = *cfg;
    if (c.n_layers < 1) FAIL(MOE_EINVAL, "n_layers %d < 1", c.n_layers);
    if (c.n_experts < 1 || c.n_experts > moe::kMaxExperts) FAIL(MOE_EINVAL, "n_experts %d outside [1,%d]", c.n_experts, moe::kMaxExperts);
    if (c.top_k < 1 || c.top_k > c.n_experts || c.top_k > moe::kMaxTopK) FAIL(MOE_EINVAL, "top_k %d invalid", c.top_k);
    if (c.n_slots < 0 || c.n_slots > moe::kMaxExperts)
        FAIL(MOE_EINVAL, "n_slots %d outside [0,%d]", c.n_slots, moe::kMaxExperts);
    if (c.atype != MOE_A_F32 && c.atype != MOE_A_BF16) FAIL(MOE_EINVAL, "atype %d invalid", c.atype);
    if (c.rule != MOE_RULE_DISTINCT && c.rule != MOE_RULE_STATIC) FAIL(MOE_EINVAL, "rule %d invalid", c.rule);
    if (c.max_tokens < 1) FAIL(MOE_EINVAL, "max_tokens %d < 1", c.max_tokens);
    if (c.timing < 0) FAIL(MOE_EINVAL, "timing %d < 0", c.timing);
    if (c.n_copy_streams < 1 || c.n_copy_streams > 8) FAIL(MOE_EINVAL, "n_copy_streams %d outside [1,8]", c.n_copy_streams);
    if (c.copy_engine != MOE_COPY_DMA && c.copy_engine != MOE_COPY_KERNEL) FAIL(MOE_EINVAL, "copy_engine %d invalid", c.copy_engine);
    if (c.policy != MOE_POLICY_HOST && c.policy != MOE_POLICY_DEVICE) FAIL(MOE_EINVAL, "policy %d invalid", c.policy);
    if (c.read_through != 0 && c.read_through != 1) FAIL(MOE_EINVAL, "read_through %d invalid", c.read_through);
    if (c.read_through && c.policy != MOE_POLICY_DEVICE) FAIL(MOE_EINVAL, "read_through needs the device policy");
    if (c.evict < MOE_EVICT_LRU || c.evict > MOE_EVICT_DECAY) FAIL(MOE_EINVAL, "evict %d invalid", c.evict);
    if (c.evict == MOE_EVICT_DECAY && c.read_through)
        FAIL(MOE_EINVAL, "placement by decayed counts changes the state on every pooled step; it runs with"
                         " read_through 0 (copy, then compute)");
    if (c.evict == MOE_EVICT_DECAY && (int64_t)c.n_slots * 2 > moe::kMaxExperts)
        FAIL(MOE_EINVAL, "placement by decayed counts addresses n_slots slots plus as many staging entries: "
                         "n_slots %d > %d", c.n_slots, moe::kMaxExperts / 2);
    if (c.prefetch_slots < 0 || c.prefetch_slots > 64) FAIL(MOE_EINVAL, "prefetch_slots %d outside [0,64]", c.prefetch_slots);
    if (c.prefetch_slots && (c.policy != MOE_POLICY_DEVICE || c.resident))
        FAIL(MOE_EINVAL, "prefetch needs the device policy and a pool (not the all-resident mode)");
    if (c.evict != MOE_EVICT_LRU && c.policy != MOE_POLICY_DEVICE)
        FAIL(MOE_EINVAL, "the host slot manager implements LRU only; evict %d needs the device policy", c.evict);
    if (c.policy == MOE_POLICY_DEVICE && c.n_experts > 2048)
        FAIL(MOE_EINVAL, "the device policy keeps a layer's state in LDS: n_experts %d > 2048", c.n_experts);
    if (c.policy == MOE_POLICY_DEVICE &&
        moe::policy_lds_bytes(c.n_experts, c.resident ? 0 : c.n_slots, c.evict) + (size_t)(c.hidden / 32) * 80 + 16 >
            65536)
        FAIL(MOE_EINVAL, "the device policy keeps a layer's state in LDS (64 KiB per workgroup): %d experts and %d"
                         " slots do not fit", c.n_experts, c.n_slots);
    if ((size_t)c.max_tokens * c.top_k > (size_t)1 << 24) FAIL(MOE_EINVAL, "max_tokens * top_k too large");
    Layout lay;
    if (!make_layout(c.wtype, c.hidden, c.inter, &lay)) FAIL(MOE_EINVAL, "unsupported shape/format (wtype %d, H %d, I %d)", c.wtype, c.hidden, c.inter);
    if (!moe::decode_shape_supported(c.wtype, c.atype, c.hidden, c.inter))
        FAIL(MOE_EINVAL, "shape not supported by the kernels (wtype %d, atype %d, H %d, I %d)", c.wtype, c.atype,
             c.hidden, c.inter);

    moe_pool* p = new (std::nothrow) moe_pool();
    if (!p) FAIL(MOE_ENOMEM, "host allocation failed");
    p->cfg = c;
    p->timing_alloc = c.timing;
    p->lay = lay;
    p->compute = static_cast<hipStream_t>(stream);
    p->geom.H = c.hidden;
    p->geom.I = c.inter;
    p->geom.K = c.top_k;
    p->geom.E = c.n_experts;
    p->geom.wtype = c.wtype;
    p->geom.atype = c.atype;
    p->geom.slot_stride = lay.total;
    p->geom.off_w13 = lay.off_w13;
    p->geom.off_w2 = lay.off_w2;
    p->geom.off_s13 = lay.off_s13;
    p->geom.off_s2 = lay.off_s2;
    const int32_t E = c.n_experts;
    p->nslot_alloc = c.resident ? E : c.n_slots;
    p->staging_cap = c.resident ? 0 : (int32_t)std::min<int64_t>(E, (int64_t)c.top_k * c.max_tokens);

    const size_t eb = lay.total;
    const size_t slot_bytes = (size_t)p->nslot_alloc * eb + kAlign;
    const size_t act_bytes = (size_t)c.max_tokens * c.top_k * moe::act_bytes_per_pair(c.wtype, c.inter);
    const size_t y_bytes = (size_t)c.max_tokens * c.top_k * c.hidden * sizeof(float);
    // (room for the staging entries a decayed-count step addresses past the pool, so
    // that the policy can be switched later)
    p->grp_slots = std::max(p->nslot_alloc + (c.resident ? 0 : std::min(p->nslot_alloc, p->staging_cap)),
                            p->staging_cap);
    const size_t grp_bytes = moe::grouped_index_bytes(c.max_tokens, c.top_k, std::max(1, p->grp_slots));
    const size_t hbm = (size_t)c.n_layers * (slot_bytes + (size_t)E * 4 + (size_t)c.prefetch_slots * eb) +
                       (size_t)p->staging_cap * eb + act_bytes + y_bytes + grp_bytes + (size_t)E * 8;
    if (c.hbm_budget_bytes && hbm > c.hbm_budget_bytes) {
        delete p;
        FAIL(MOE_ENOMEM, "pool needs %zu HBM bytes, budget is %zu", hbm, c.hbm_budget_bytes);
    }

#define CREATE_HIP(call)                                                                            \
    do {                                                                                            \
        hipError_t e_ = (call);                                                                     \
        if (e_ != hipSuccess) {                                                                     \
            set_err("%s failed: %s", #call, hipGetErrorString(e_));                                 \
            destroy_pool(p);                                                                        \
            return (e_ == hipErrorOutOfMemory || e_ == hipErrorMemoryAllocation) ? MOE_ENOMEM : MOE_EHIP; \
        }                                                                                           \
    } while (0)

    p->copy.resize(c.n_copy_streams, nullptr);
    p->copy_done.resize(c.n_copy_streams, nullptr);
    p->used_copy.assign(c.n_copy_streams, 0);
    for (int i = 0; i < c.n_copy_streams; ++i) {
        CREATE_HIP(hipStreamCreateWithFlags(&p->copy[i], hipStreamNonBlocking));
        CREATE_HIP(hipEventCreateWithFlags(&p->copy_done[i], hipEventDisableTiming));
    }
    const unsigned tflag = c.timing ? hipEventDefault : hipEventDisableTiming;
    p->layers.resize(c.n_layers);
    size_t pinned_total = 0;
    for (int32_t l = 0; l < c.n_layers; ++l) {
        LayerState& L = p->layers[l];
        L.lru.init(E, c.resident ? 0 : c.n_slots, c.rule);
        // The all-resident mode keeps every expert in HBM and never copies from a
        // store, so it has none.
        L.per_piece = (int32_t)std::max<size_t>(1, std::min<size_t>(E, kStorePiece / eb));
        for (int32_t e0 = 0; !c.resident && e0 < E; e0 += L.per_piece) {
            const size_t bytes = (size_t)std::min(L.per_piece, E - e0) * eb;
            char* piece = nullptr;
            // coherent: the copy kernels read the store through its device mapping,
            // and a GPU-cached line of host memory can outlive the allocation (a
            // later pinned allocation at the same place then reads stale on the GPU)
            const hipError_t he = hipHostMalloc((void**)&piece, bytes, hipHostMallocMapped | hipHostMallocCoherent);
            if (he != hipSuccess) {
                set_err("hipHostMalloc of %zu bytes (layer %d, experts %d..) failed after %zu pinned bytes: %s", bytes, l,
                        e0, pinned_total, hipGetErrorString(he));
                destroy_pool(p);
                return MOE_ENOMEM;
            }
            L.store.push_back(piece);
            pinned_total += bytes;
            char* piece_dev = nullptr;
            CREATE_HIP(hipHostGetDevicePointer((void**)&piece_dev, piece, 0));
            L.store_dev.push_back(piece_dev);
        }
        CREATE_HIP(hipMalloc((void**)&L.slots, slot_bytes));
        CREATE_HIP(hipMemset(L.slots + (size_t)p->nslot_alloc * eb, 0, kAlign));
        CREATE_HIP(hipMalloc((void**)&L.map_dev, (size_t)E * 4));
        CREATE_HIP(hipMemset(L.map_dev, 0xFF, (size_t)E * 4));   // all -1
        CREATE_HIP(hipHostMalloc((void**)&L.upd_host, (size_t)E * 8, hipHostMallocCoherent | hipHostMallocMapped));
        CREATE_HIP(hipHostGetDevicePointer((void**)&L.upd_dev, L.upd_host, 0));
        L.copy_t.resize(c.n_copy_streams);
        if (c.timing) {
            for (auto& t : L.copy_t) {
                CREATE_HIP(hipEventCreateWithFlags(&t.a, tflag));
                CREATE_HIP(hipEventCreateWithFlags(&t.b, tflag));
            }
            for (Timing* t : {&L.w13_t, &L.w2_t}) {
                CREATE_HIP(hipEventCreateWithFlags(&t->a, tflag));
                CREATE_HIP(hipEventCreateWithFlags(&t->b, tflag));
            }
        }
    }
    if (p->staging_cap > 0) CREATE_HIP(hipMalloc((void**)&p->staging, (size_t)p->staging_cap * eb));
    CREATE_HIP(hipHostMalloc((void**)&p->rb_host, (size_t)(E + 1) * 4, hipHostMallocCoherent | hipHostMallocMapped));
    std::memset(p->rb_host, 0, (size_t)(E + 1) * 4);
    CREATE_HIP(hipHostGetDevicePointer((void**)&p->rb_dev, p->rb_host, 0));
    p->ulist.resize(E);
    CREATE_HIP(hipMalloc((void**)&p->rank_dev, (size_t)E * 4));
    CREATE_HIP(hipMalloc((void**)&p->ident_dev, (size_t)E * 4));
    {
        std::vector<int32_t> id(E);
        for (int32_t e = 0; e < E; ++e) id[e] = e;
        CREATE_HIP(hipMemcpy(p->ident_dev, id.data(), (size_t)E * 4, hipMemcpyHostToDevice));
    }
    CREATE_HIP(hipMalloc((void**)&p->paths_dev, sizeof(int32_t) * c.n_layers));
    CREATE_HIP(hipMemset(p->paths_dev, 0, sizeof(int32_t) * c.n_layers));
    for (int32_t l = 0; l < c.n_layers; ++l) p->layers[l].path_dev = p->paths_dev + l;
    if (c.policy == MOE_POLICY_DEVICE) {
        const DevLayout d = dev_layout(E, c.resident ? 0 : c.n_slots);
        for (auto& L : p->layers) {
            CREATE_HIP(hipMalloc((void**)&L.dev_block, d.total));
            L.ds.copy[0] = L.dev_block + d.copy0;
            L.ds.copy[1] = L.dev_block + d.copy1;
            L.ds.ctl = reinterpret_cast<int32_t*>(L.dev_block + d.ctl);
            L.ds.ctr = reinterpret_cast<unsigned long long*>(L.dev_block + d.ctr);
            L.ds.rec = reinterpret_cast<int32_t*>(L.dev_block + d.rec);
            if (!L.store_dev.empty()) {
                CREATE_HIP(hipMalloc((void**)&L.pieces_dev, sizeof(char*) * L.store_dev.size()));
                CREATE_HIP(hipMemcpy(L.pieces_dev, L.store_dev.data(), sizeof(char*) * L.store_dev.size(),
                                     hipMemcpyHostToDevice));
            }
            if (c.timing) {
                CREATE_HIP(hipEventCreateWithFlags(&L.fill_t.a, tflag));
                CREATE_HIP(hipEventCreateWithFlags(&L.fill_t.b, tflag));
            }
            if (c.prefetch_slots) {
                CREATE_HIP(hipMalloc((void**)&L.pf_buf, (size_t)c.prefetch_slots * eb));
                CREATE_HIP(hipMalloc((void**)&L.pf_tag, (size_t)c.prefetch_slots * 4));
                CREATE_HIP(hipEventCreateWithFlags(&L.pf_done, hipEventDisableTiming));
                CREATE_HIP(hipEventCreateWithFlags(&L.step_done, hipEventDisableTiming));
                const moe_status_t cst = clear_prefetch(p, L);
                if (cst) {
                    destroy_pool(p);
                    return cst;
                }
            }
        }
        if (c.prefetch_slots) CREATE_HIP(hipEventCreateWithFlags(&p->pf_issue, hipEventDisableTiming));
        CREATE_HIP(hipHostMalloc((void**)&p->errs_host, sizeof(uint32_t) * c.n_layers,
                                 hipHostMallocCoherent | hipHostMallocMapped));
        CREATE_HIP(hipHostGetDevicePointer((void**)&p->errs_dev, p->errs_host, 0));
        CREATE_HIP(hipHostMalloc((void**)&p->timed_jobs_host, sizeof(int32_t) * c.n_layers,
                                 hipHostMallocCoherent | hipHostMallocMapped));
        std::memset(p->timed_jobs_host, 0, sizeof(int32_t) * c.n_layers);
        CREATE_HIP(hipHostGetDevicePointer((void**)&p->timed_jobs_dev, p->timed_jobs_host, 0));
        if (c.read_through) {
            CREATE_HIP(hipHostMalloc((void**)&p->rt_jobs_host, sizeof(int32_t) * c.n_layers,
                                     hipHostMallocCoherent | hipHostMallocMapped));
            std::memset(p->rt_jobs_host, 0, sizeof(int32_t) * c.n_layers);
            CREATE_HIP(hipHostGetDevicePointer((void**)&p->rt_jobs_dev, p->rt_jobs_host, 0));
        }
        const moe_status_t ist = dev_init_layers(p);
        if (ist) {
            destroy_pool(p);
            return ist;
        }
    }
    CREATE_HIP(hipMalloc((void**)&p->act, act_bytes));
    CREATE_HIP(hipMalloc((void**)&p->y, y_bytes));
    CREATE_HIP(hipMalloc((void**)&p->grp, grp_bytes));
#undef CREATE_HIP
    p->misses.reserve(E);
    *out = p;
    return MOE_OK;
}

void moe_pool_destroy(moe_pool_t* pool) { destroy_pool(pool); }

moe_status_t moe_pool_load_expert(moe_pool_t* p, int32_t layer, int32_t expert, const void* host_src,
                                  size_t nbytes) {
    moe_status_t st = check_layer(p, layer);
    if (st) return st;
    if (expert < 0 || expert >= p->cfg.n_experts) FAIL(MOE_EINVAL, "expert %d outside [0,%d)", expert, p->cfg.n_experts);
    if (!host_src || nbytes != p->lay.total) FAIL(MOE_EINVAL, "need %zu bytes, got %zu", p->lay.total, nbytes);
    LayerState& L = p->layers[layer];
    // the store may be the source of a queued copy: let those finish first
    for (auto s : p->copy) HIPCHK(hipStreamSynchronize(s));
    if (p->cfg.resident)
        HIPCHK(hipMemcpy(L.slots + (size_t)expert * p->lay.total, host_src, nbytes, hipMemcpyHostToDevice));
    else
        std::memcpy(L.expert(expert, p->lay.total), host_src, nbytes);
    // a prefetched copy of the old bytes must not be used
    if (L.pf_tag) {
        HIPCHK(hipStreamSynchronize(p->compute));
        const moe_status_t st2 = clear_prefetch(p, L);
        if (st2) return st2;
    }
    return MOE_OK;
}

moe_status_t moe_pool_reset(moe_pool_t* p) {
    if (!p) FAIL(MOE_EINVAL, "null pool");
    HIPCHK(hipStreamSynchronize(p->compute));
    for (auto s : p->copy) HIPCHK(hipStreamSynchronize(s));
    for (auto& L : p->layers) {
        L.lru.init(p->cfg.n_experts, p->cfg.resident ? 0 : p->cfg.n_slots, p->cfg.rule);
        HIPCHK(hipMemset(L.map_dev, 0xFF, (size_t)p->cfg.n_experts * 4));
        L.prepared = false;
        L.bytes_h2d = 0;
        L.staged = 0;
        L.has_last = false;
    }
    p->staging_owner = -1;
    p->last_prepared = -1;
    for (auto& L : p->layers) {
        const moe_status_t cst = clear_prefetch(p, L);
        if (cst) return cst;
    }
    if (p->cfg.policy == MOE_POLICY_DEVICE) return dev_init_layers(p);
    return MOE_OK;
}

moe_status_t moe_pool_prepare(moe_pool_t* p, int32_t layer, const int32_t* topk_ids_dev, int32_t n_tokens,
                              int32_t* slot_ids_dev, moe_miss_t* miss_host, int32_t miss_cap, int32_t* n_miss,
                              int32_t* path) {
    moe_status_t st = check_layer(p, layer);
    if (st) return st;
    if (n_tokens < 0 || n_tokens > p->cfg.max_tokens) FAIL(MOE_EINVAL, "n_tokens %d outside [0,%d]", n_tokens, p->cfg.max_tokens);
    if (n_tokens > 0 && (!topk_ids_dev || !slot_ids_dev)) FAIL(MOE_EINVAL, "null ids");
    if (miss_cap < 0) FAIL(MOE_EINVAL, "miss_cap < 0");
    LayerState& L = p->layers[layer];
    const int32_t E = p->cfg.n_experts;
    const int n = n_tokens * p->cfg.top_k;
    // from here on a failure leaves no prepared step (a forward then needs a new
    // prepare); the cache state is unchanged
    L.prepared = false;
    if (p->cfg.policy == MOE_POLICY_DEVICE) {
        st = check_dev_err(p, layer);
        if (st) return st;
        if (n_miss) *n_miss = -1;
        if (path) *path = -1;
        if (n_tokens == 0) {
            L.prepared = true;
            L.prep_tokens = 0;
            L.prep_path = MOE_PATH_POOL;
            L.has_last = true;
            L.last_empty = true;
            L.empty_steps++;
            return MOE_OK;
        }
        st = dev_prepare(p, L, layer, topk_ids_dev, n_tokens, slot_ids_dev);
        if (st) return st;
        p->last_prepared = layer;
        if (p->cfg.timing) harvest_all(p);
        return MOE_OK;
    }

    if (n_tokens == 0) {
        p->misses.clear();
        if (p->cfg.resident) L.lru.count_resident(0); else L.lru.step(nullptr, 0, 0, p->misses);
        finish_prepare(p, L, 0, MOE_PATH_POOL, miss_host, miss_cap, n_miss, path);
        return MOE_OK;
    }

    st = launch_distinct_ids(p, topk_ids_dev, n);
    if (st) return st;
    int32_t D = 0;
    st = read_distinct(p, layer, &D);
    if (st) return st;

    // 2. route + LRU; 3. misses: store -> slot on the copy streams, after this
    // layer's last reads; 4. the remap (map changes applied first)
    int32_t the_path = MOE_PATH_POOL, n_upd = 0;
    st = route(p, L, layer, D, n, &the_path, &n_upd);
    if (st) return st;
    int32_t* table = p->cfg.resident ? p->ident_dev : L.map_dev;
    const int status = the_path == MOE_PATH_FALLBACK ? moe::PATH_STAGE : moe::PATH_POOL;
    HIPCHK(moe::launch_remap(topk_ids_dev, n, E, table, p->rank_dev, L.upd_dev, n_upd, status,
                             slot_ids_dev, L.path_dev, p->compute));
    finish_prepare(p, L, n_tokens, the_path, miss_host, miss_cap, n_miss, path);
    if (p->cfg.timing) harvest_all(p);   // event queries stay off the path to the remap
    return MOE_OK;
}

moe_status_t moe_pool_forward(moe_pool_t* p, int32_t layer, const void* x_dev, const int32_t* slot_ids_dev,
                              const float* topk_w_dev, const void* resid_dev, int32_t n_tokens, void* out_dev) {
    moe_status_t st = check_layer(p, layer);
    if (st) return st;
    LayerState& L = p->layers[layer];
    if (!L.prepared || L.prep_tokens != n_tokens)
        FAIL(MOE_ESTATE, "layer %d: forward(n_tokens=%d) without a matching prepare", layer, n_tokens);
    const bool fb = L.prep_path == MOE_PATH_FALLBACK;
    if (fb && p->staging_owner != layer)
        FAIL(MOE_ESTATE, "layer %d: its staged experts were replaced by layer %d's fallback", layer, p->staging_owner);
    if (p->cfg.policy == MOE_POLICY_DEVICE && n_tokens > 0 && p->last_prepared != layer)
        FAIL(MOE_ESTATE, "layer %d: layer %d was prepared after it (under the device policy a forward must follow its"
                         " own prepare: staging is shared and the host does not know which steps fell back)",
             layer, p->last_prepared);
    if (n_tokens == 0) return MOE_OK;
    if (!x_dev || !slot_ids_dev || !topk_w_dev || !out_dev) FAIL(MOE_EINVAL, "null buffer");
    return launch_layer_forward(p, L, x_dev, slot_ids_dev, topk_w_dev, resid_dev, n_tokens, out_dev);
}

moe_status_t moe_pool_step(moe_pool_t* p, int32_t layer, const int32_t* topk_ids_dev, int32_t n_tokens,
                           int32_t* slot_ids_dev, const void* x_dev, const float* topk_w_dev, const void* resid_dev,
                           void* out_dev, moe_miss_t* miss_host, int32_t miss_cap, int32_t* n_miss, int32_t* path) {
    if (n_tokens > 0 && (!x_dev || !topk_w_dev || !out_dev)) FAIL(MOE_EINVAL, "null buffer");
    if (p && p->cfg.policy == MOE_POLICY_DEVICE && p->cfg.read_through && n_tokens == 1) {
        // The fused one-token step (device policy): the decision runs inside the w13
        // launch, a missed expert's w13 rows are read from the store and written through
        // to its slot by the GEMV blocks while copy workers of the same launch move the
        // rest of it, and the hit experts' GEMVs run alongside.  Everything the forward
        // needs is checked before anything is queued.
        moe_status_t st = check_layer(p, layer);
        if (st) return st;
        if (!topk_ids_dev || !slot_ids_dev) FAIL(MOE_EINVAL, "null ids");
        if (miss_cap < 0) FAIL(MOE_EINVAL, "miss_cap < 0");
        LayerState& L = p->layers[layer];
        st = check_dev_err(p, layer);
        if (st) return st;
        if (n_miss) *n_miss = -1;
        if (path) *path = -1;
        const bool timed = p->cfg.timing > 0 && (p->n_forwards++ % (uint64_t)p->cfg.timing) == 0 &&
                           !L.w13_t.pending && !L.w2_t.pending;
        st = join_prefetch(p, L);
        if (st) return st;
        moe::PolicyArgs pa = policy_args(p, L, layer, topk_ids_dev, 1, slot_ids_dev);
        pa.timed_jobs = timed && p->rt_jobs_dev ? p->rt_jobs_dev + layer : nullptr;
        moe::ForwardArgs a = forward_args(p, L, x_dev, slot_ids_dev, topk_w_dev, resid_dev, 1, out_dev);
        moe::StageEvents ev;
        if (timed) {
            ev.w13_start = L.w13_t.a;
            ev.w13_stop = L.w13_t.b;
            ev.w2_start = L.w2_t.a;
            ev.w2_stop = L.w2_t.b;
        }
        HIPCHK(moe::launch_step_decode(p->geom, pa, a, kStepCopyWorkers, timed ? &ev : nullptr, p->compute));
        if (L.step_done) {
            HIPCHK(hipEventRecord(L.step_done, p->compute));
            L.stepped = true;
        }
        if (timed) {
            L.w13_t.pending = true;
            L.w2_t.pending = true;
            L.rt_sample = true;
        }
        p->last_prepared = layer;
        // the step is complete: a forward needs a prepare of its own
        L.prepared = false;
        L.has_last = true;
        L.last_empty = false;
        if (p->cfg.timing) harvest_all(p);
        return MOE_OK;
    }
    moe_status_t st = moe_pool_prepare(p, layer, topk_ids_dev, n_tokens, slot_ids_dev, miss_host, miss_cap, n_miss,
                                       path);
    if (st) return st;
    return moe_pool_forward(p, layer, x_dev, slot_ids_dev, topk_w_dev, resid_dev, n_tokens, out_dev);
}

moe_status_t moe_pool_prefetch(moe_pool_t* p, int32_t layer, const int32_t* predicted_ids_dev, int32_t n_tokens,
                               int32_t after) {
    moe_status_t st = check_layer(p, layer);
    if (st) return st;
    LayerState& L = p->layers[layer];
    if (!L.pf_buf) FAIL(MOE_EINVAL, "the pool has no prefetch buffer (prefetch_slots = 0)");
    const int64_t n = (int64_t)n_tokens * p->cfg.top_k;
    if (n_tokens < 1 || n > 256) FAIL(MOE_EINVAL, "prefetch of %d tokens x top_k %d: need 1..256 ids", n_tokens, p->cfg.top_k);
    if (!predicted_ids_dev) FAIL(MOE_EINVAL, "null ids");
    if (after < MOE_PREFETCH_AFTER_LAYER || after > MOE_PREFETCH_AFTER_PREVIOUS) FAIL(MOE_EINVAL, "after %d invalid", after);
    moe::PrefetchArgs a{};
    a.ids = predicted_ids_dev;
    a.n = (int)n;
    a.E = p->cfg.n_experts;
    a.N = p->cfg.n_slots;
    a.ds = L.ds;
    a.tag = L.pf_tag;
    a.buf = L.pf_buf;
    a.pf_n = p->cfg.prefetch_slots;
    a.pieces = L.pieces_dev;
    a.per_piece = L.per_piece;
    a.eb = p->lay.total;
    hipStream_t cs = p->copy[0];
    // when it may start (see moe_pool.h); the layer's next step joins it
    if (after == MOE_PREFETCH_AFTER_QUEUED) {
        HIPCHK(hipEventRecord(p->pf_issue, p->compute));
        HIPCHK(hipStreamWaitEvent(cs, p->pf_issue, 0));
    } else if (after == MOE_PREFETCH_AFTER_LAYER && L.stepped) {
        HIPCHK(hipStreamWaitEvent(cs, L.step_done, 0));
    }
    HIPCHK(moe::launch_prefetch(a, kPrefetchGrid, cs));
    HIPCHK(hipEventRecord(L.pf_done, cs));
    L.pf_pending = true;
    return MOE_OK;
}

moe_status_t moe_pool_last_step(moe_pool_t* p, int32_t layer, int32_t* path, moe_miss_t* miss_host,
                                int32_t miss_cap, int32_t* n_miss) {
    moe_status_t st = check_layer(p, layer);
    if (st) return st;
    if (miss_cap < 0) FAIL(MOE_EINVAL, "miss_cap < 0");
    LayerState& L = p->layers[layer];
    if (!L.has_last) FAIL(MOE_ESTATE, "layer %d: no step since create or reset", layer);
    std::vector<moe::Miss> ms;
    int32_t the_path = L.last_path;
    if (p->cfg.policy == MOE_POLICY_DEVICE) {
        if (L.last_empty) {
            the_path = MOE_PATH_POOL;
        } else {
            const int32_t N = p->cfg.resident ? 0 : p->cfg.n_slots;
            std::vector<int32_t> rec(4 + 3 * (size_t)N);
            if ((st = dev_read(p, rec.data(), L.ds.rec, rec.size()))) return st;
            if (rec[3]) {
                p->errs_host[layer] = 0;
                FAIL(MOE_ERANGE, "layer %d: the step had an expert id outside [0,%d); it changed nothing", layer,
                     p->cfg.n_experts);
            }
            the_path = rec[0] == moe::PATH_STAGE ? MOE_PATH_FALLBACK : MOE_PATH_POOL;
            for (int32_t i = 0; i < rec[2]; ++i) ms.push_back({rec[4 + 3 * i], rec[5 + 3 * i], rec[6 + 3 * i]});
        }
    } else {
        ms = L.last_misses;
    }
    const int32_t nm = (int32_t)ms.size();
    if (miss_host)
        for (int32_t i = 0; i < std::min(nm, miss_cap); ++i) miss_host[i] = moe_miss_t{ms[i].expert, ms[i].slot, ms[i].evicted};
    if (n_miss) *n_miss = nm;
    if (path) *path = the_path;
    return MOE_OK;
}

moe_status_t moe_pool_sync(moe_pool_t* p) {
    if (!p) FAIL(MOE_EINVAL, "null pool");
    for (auto s : p->copy) HIPCHK(hipStreamSynchronize(s));
    HIPCHK(hipStreamSynchronize(p->compute));
    if (p->cfg.policy == MOE_POLICY_DEVICE)
        for (int32_t l = 0; l < p->cfg.n_layers; ++l) {
            const moe_status_t st = check_dev_err(p, l);
            if (st) return st;
        }
    return MOE_OK;
}

moe_status_t moe_pool_get_stats(const moe_pool_t* p, int32_t layer, moe_pool_stats_t* out) {
    if (!p || !out) FAIL(MOE_EINVAL, "null argument");
    if (layer < -1 || layer >= p->cfg.n_layers) FAIL(MOE_EINVAL, "layer %d invalid", layer);
    std::memset(out, 0, sizeof(*out));
    for (int32_t l = 0; l < p->cfg.n_layers; ++l) {
        if (layer >= 0 && l != layer) continue;
        const LayerState& L = p->layers[l];
        if (p->cfg.policy == MOE_POLICY_DEVICE) {
            unsigned long long c[9];
            const moe_status_t st = dev_read(p, c, L.ds.ctr, 9);
            if (st) return st;
            out->steps += c[0] + L.empty_steps;
            out->hits += c[1];
            out->misses += c[2];
            out->fallbacks += c[3];
            out->bytes_h2d += c[4];
            out->staged += c[5];
            out->prefetched += c[6];
            out->prefetch_bytes += c[7];
            out->moves += c[8];
            continue;
        }
        out->steps += L.lru.steps();
        out->hits += L.lru.hits();
        out->misses += L.lru.misses();
        out->fallbacks += L.lru.fallbacks();
        out->bytes_h2d += L.bytes_h2d;
        out->staged += L.staged;
    }
    return MOE_OK;
}

moe_status_t moe_pool_get_state(const moe_pool_t* p, int32_t layer, int32_t* map_E, int32_t* owner_N,
                                int32_t* lru_N) {
    moe_status_t st = check_layer(p, layer);
    if (st) return st;
    if (p->cfg.policy == MOE_POLICY_DEVICE) {
        const LayerState& L = p->layers[layer];
        const int32_t E = p->cfg.n_experts, N = p->cfg.resident ? 0 : p->cfg.n_slots;
        int32_t ctl[2] = {0, 0};
        if ((st = dev_read(p, ctl, L.ds.ctl, 2))) return st;
        const moe::SlotStateLayout o = moe::slot_state_layout(E, N);
        const char* cur = L.ds.copy[ctl[0] & 1];
        std::vector<int32_t> map(E), owner(N), prot(N);
        std::vector<uint32_t> key(N), use(N);
        std::vector<float> cnt(E);
        if ((st = dev_read(p, map.data(), cur + o.map, E))) return st;
        if (p->cfg.evict == MOE_EVICT_DECAY && (st = dev_read(p, cnt.data(), cur + o.cnt, E))) return st;
        if (N && (st = dev_read(p, owner.data(), cur + o.owner, N))) return st;
        if (N && (st = dev_read(p, key.data(), cur + o.key, N))) return st;
        if (N && (st = dev_read(p, use.data(), cur + o.use, N))) return st;
        if (N && (st = dev_read(p, prot.data(), cur + o.prot, N))) return st;
        if (map_E) std::copy(map.begin(), map.end(), map_E);
        if (owner_N) std::copy(owner.begin(), owner.end(), owner_N);
        if (lru_N) {
            // the eviction order: resident slots by the policy's key (SLRU: the
            // probationary segment first; DECAY: by use count, then expert id)
            std::vector<int32_t> res;
            for (int32_t q = 0; q < N; ++q)
                if (owner[q] >= 0) res.push_back(q);
            const int32_t ev = p->cfg.evict;
            auto k = [&](int32_t q) {
                uint64_t v = key[q];
                if (ev == MOE_EVICT_LFU) v |= (uint64_t)use[q] << 32;
                if (ev == MOE_EVICT_SLRU) v |= (uint64_t)(prot[q] != 0) << 32;
                if (ev == MOE_EVICT_DECAY) {
                    uint32_t cb;
                    std::memcpy(&cb, &cnt[owner[q]], 4);   // non-negative: bits order like values
                    v = ((uint64_t)cb << 32) | (uint32_t)owner[q];
                }
                return v;
            };
            std::sort(res.begin(), res.end(), [&](int32_t a, int32_t b) { return k(a) < k(b); });
            int32_t i = 0;
            for (int32_t q : res) lru_N[i++] = owner[q];
            for (; i < N; ++i) lru_N[i] = -1;
        }
        return MOE_OK;
    }
    const moe::SlotLRU& s = p->layers[layer].lru;
    if (map_E) std::copy(s.map().begin(), s.map().end(), map_E);
    if (owner_N) std::copy(s.owner().begin(), s.owner().end(), owner_N);
    if (lru_N) s.lru_order(lru_N, s.n_slots());
    return MOE_OK;
}

moe_status_t moe_pool_read_slot(moe_pool_t* p, int32_t layer, int32_t slot, void* host_dst, size_t n) {
    moe_status_t st = check_layer(p, layer);
    if (st) return st;
    if (!host_dst || n > p->lay.total) FAIL(MOE_EINVAL, "bad destination or size");
    const char* src;
    if (slot >= 0) {
        if (slot >= p->nslot_alloc) FAIL(MOE_EINVAL, "slot %d outside [0,%d)", slot, p->nslot_alloc);
        src = p->layers[layer].slots + (size_t)slot * p->lay.total;
    } else {
        const int32_t r = -slot - 1;
        if (r >= p->staging_cap) FAIL(MOE_EINVAL, "staging entry %d outside [0,%d)", r, p->staging_cap);
        src = p->staging + (size_t)r * p->lay.total;
    }
    st = moe_pool_sync(p);
    if (st) return st;
    HIPCHK(hipMemcpy(host_dst, src, n, hipMemcpyDeviceToHost));
    return MOE_OK;
}

moe_status_t moe_pool_slot_ptr(const moe_pool_t* p, int32_t layer, int32_t slot, void** dev_ptr) {
    moe_status_t st = check_layer(p, layer);
    if (st) return st;
    if (!dev_ptr || slot < 0 || slot >= p->nslot_alloc) FAIL(MOE_EINVAL, "bad slot %d", slot);
    *dev_ptr = p->layers[layer].slots + (size_t)slot * p->lay.total;
    return MOE_OK;
}

moe_status_t moe_pool_store_ptr(const moe_pool_t* p, int32_t layer, int32_t expert, void** host_ptr) {
    moe_status_t st = check_layer(p, layer);
    if (st) return st;
    if (!host_ptr || expert < 0 || expert >= p->cfg.n_experts) FAIL(MOE_EINVAL, "bad expert %d", expert);
    if (p->cfg.resident) FAIL(MOE_EINVAL, "the all-resident mode has no host store");
    *host_ptr = p->layers[layer].expert(expert, p->lay.total);
    return MOE_OK;
}

moe_status_t moe_ptr_is_pinned_host(const void* ptr, int32_t* is_pinned) {
    if (!ptr || !is_pinned) FAIL(MOE_EINVAL, "null argument");
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof(attr));
    hipError_t e = hipPointerGetAttributes(&attr, ptr);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        *is_pinned = 0;
        return MOE_OK;
    }
    *is_pinned = attr.type == hipMemoryTypeHost ? 1 : 0;
    return MOE_OK;
}

moe_status_t moe_pool_get_timing(moe_pool_t* p, moe_pool_timing_t* out) {
    if (!p || !out) FAIL(MOE_EINVAL, "null argument");
    moe_status_t st = moe_pool_sync(p);
    if (st) return st;
    harvest_all(p);
    out->copy_ms = p->copy_ms;
    out->copy_calls = p->copy_calls;
    out->copy_bytes = p->copy_bytes;
    out->w13_ms = p->w13_ms;
    out->w2_ms = p->w2_ms;
    out->kernel_calls = p->kern_calls;
    out->sync_wait_ms = p->sync_ms;
    return MOE_OK;
}

moe_status_t moe_pool_set_timing(moe_pool_t* p, int32_t every) {
    if (!p) FAIL(MOE_EINVAL, "null pool");
    if (every < 0) FAIL(MOE_EINVAL, "timing period %d < 0", every);
    if (every > 0 && p->timing_alloc <= 0) FAIL(MOE_EINVAL, "the pool was created without timing events");
    moe_status_t st = moe_pool_sync(p);
    if (st) return st;
    harvest_all(p);   // under the old period: nothing stays pending
    p->cfg.timing = every;
    return MOE_OK;
}

moe_status_t moe_pool_reset_timing(moe_pool_t* p) {
    if (!p) FAIL(MOE_EINVAL, "null pool");
    moe_status_t st = moe_pool_sync(p);
    if (st) return st;
    harvest_all(p);
    p->copy_ms = p->w13_ms = p->w2_ms = p->sync_ms = 0;
    p->copy_calls = p->copy_bytes = p->kern_calls = 0;
    return MOE_OK;
}

moe_status_t moe_read_calibration(const void* buf_dev, size_t buf_bytes, size_t bytes, int32_t reps, void* stream,
                                  double* avg_us) {
    if (!buf_dev || !avg_us || reps < 1 || bytes < 16 || bytes % 16 || bytes > buf_bytes)
        FAIL(MOE_EINVAL, "bad calibration arguments");
    hipStream_t s = static_cast<hipStream_t>(stream);
    unsigned* sink = nullptr;
    hipEvent_t a = nullptr, b = nullptr;
    moe_status_t st = MOE_OK;
    double total = 0;
    auto fail = [&](hipError_t e, const char* what) {
        set_err("%s failed: %s", what, hipGetErrorString(e));
        st = MOE_EHIP;
    };
    hipError_t e;
    if ((e = hipMalloc((void**)&sink, 1024)) != hipSuccess) fail(e, "hipMalloc");
    if (!st && (e = hipEventCreate(&a)) != hipSuccess) fail(e, "hipEventCreate");
    if (!st && (e = hipEventCreate(&b)) != hipSuccess) fail(e, "hipEventCreate");
    const size_t regions = buf_bytes / bytes;
    const char* base = static_cast<const char*>(buf_dev);
    for (int32_t i = -2; !st && i < reps; ++i) {   // two untimed launches first
        const char* p = base + (size_t)((i + 2) % regions) * bytes;
        if ((e = moe::launch_read_probe(p, bytes, sink, a, b, s)) != hipSuccess) { fail(e, "read probe launch"); break; }
        if ((e = hipEventSynchronize(b)) != hipSuccess) { fail(e, "hipEventSynchronize"); break; }
        float ms = 0;
        if ((e = hipEventElapsedTime(&ms, a, b)) != hipSuccess) { fail(e, "hipEventElapsedTime"); break; }
        if (i >= 0) total += ms * 1e3;
    }
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
    if (sink) (void)hipFree(sink);
    if (st) return st;
    *avg_us = total / reps;
    return MOE_OK;
}

moe_status_t moe_link_calibration(size_t bytes, int32_t reps, int32_t engine, int32_t n_streams, void* stream,
                                  double* avg_us) {
    if (!avg_us || reps < 1 || bytes < 16 || bytes % 16 || (engine != MOE_COPY_KERNEL && engine != MOE_COPY_DMA) ||
        n_streams < 1 || n_streams > 8)
        FAIL(MOE_EINVAL, "bad calibration arguments");
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* host = nullptr;
    char* host_dev = nullptr;
    char* dev = nullptr;
    hipEvent_t a = nullptr, b = nullptr;
    std::vector<hipStream_t> side(n_streams, nullptr);   // side[0] stays `stream`
    std::vector<hipEvent_t> done(n_streams, nullptr);
    moe_status_t st = MOE_OK;
    double total = 0;
    auto fail = [&](hipError_t err, const char* what) {
        set_err("%s failed: %s", what, hipGetErrorString(err));
        st = (err == hipErrorOutOfMemory || err == hipErrorMemoryAllocation) ? MOE_ENOMEM : MOE_EHIP;
    };
    hipError_t e;
    // the same kind of memory as the store (coherent, device-mapped)
    if ((e = hipHostMalloc((void**)&host, bytes, hipHostMallocMapped | hipHostMallocCoherent)) != hipSuccess)
        fail(e, "hipHostMalloc");
    if (!st) std::memset(host, 0x5A, bytes);
    if (!st && (e = hipHostGetDevicePointer((void**)&host_dev, host, 0)) != hipSuccess) fail(e, "hipHostGetDevicePointer");
    if (!st && (e = hipMalloc((void**)&dev, bytes)) != hipSuccess) fail(e, "hipMalloc");
    if (!st && (e = hipEventCreate(&a)) != hipSuccess) fail(e, "hipEventCreate");
    if (!st && (e = hipEventCreate(&b)) != hipSuccess) fail(e, "hipEventCreate");
    side[0] = s;
    for (int i = 1; !st && i < n_streams; ++i)
        if ((e = hipStreamCreateWithFlags(&side[i], hipStreamNonBlocking)) != hipSuccess) fail(e, "hipStreamCreate");
    for (int i = 0; !st && i < n_streams; ++i)
        if ((e = hipEventCreateWithFlags(&done[i], hipEventDisableTiming)) != hipSuccess) fail(e, "hipEventCreate");
    // the transfer split into n_streams parts of 16-byte multiples, one per stream
    const size_t part = (bytes / 16 + n_streams - 1) / n_streams * 16;
    for (int32_t i = -1; !st && i < reps; ++i) {
        if ((e = hipEventRecord(a, s)) != hipSuccess) { fail(e, "hipEventRecord"); break; }
        for (int k = 0; !st && k < n_streams; ++k) {
            const size_t off = (size_t)k * part;
            if (off >= bytes) break;
            const size_t n = std::min(part, bytes - off);
            if (k > 0 && (e = hipStreamWaitEvent(side[k], a, 0)) != hipSuccess) { fail(e, "hipStreamWaitEvent"); break; }
            if (engine == MOE_COPY_KERNEL) {
                moe::FillBatch fb{};
                fb.n = 1;
                fb.bytes = n;
                fb.job[0] = moe::FillJob{host_dev + off, dev + off};
                e = moe::launch_fill(fb, side[k]);
            } else {
                e = hipMemcpyAsync(dev + off, host + off, n, hipMemcpyHostToDevice, side[k]);
            }
            if (e != hipSuccess) { fail(e, "copy"); break; }
            if (k > 0) {
                if ((e = hipEventRecord(done[k], side[k])) != hipSuccess) { fail(e, "hipEventRecord"); break; }
                if ((e = hipStreamWaitEvent(s, done[k], 0)) != hipSuccess) { fail(e, "hipStreamWaitEvent"); break; }
            }
        }
        if (st) break;
        if ((e = hipEventRecord(b, s)) != hipSuccess) { fail(e, "hipEventRecord"); break; }
        if ((e = hipEventSynchronize(b)) != hipSuccess) { fail(e, "hipEventSynchronize"); break; }
        float ms = 0;
        if ((e = hipEventElapsedTime(&ms, a, b)) != hipSuccess) { fail(e, "hipEventElapsedTime"); break; }
        if (i >= 0) total += ms * 1e3;
    }
    for (int i = 1; i < n_streams; ++i)
        if (side[i]) {
            (void)hipStreamSynchronize(side[i]);
            (void)hipStreamDestroy(side[i]);
        }
    for (auto ev : done)
        if (ev) (void)hipEventDestroy(ev);
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
    if (dev) (void)hipFree(dev);
    if (host) (void)hipHostFree(host);
    if (st) return st;
    *avg_us = total / reps;
    return MOE_OK;
}

moe_status_t moe_pool_set_slots(moe_pool_t* p, int32_t n_slots) {
    if (!p) FAIL(MOE_EINVAL, "null pool");
    if (p->cfg.resident) FAIL(MOE_EINVAL, "the all-resident mode has no slot pool");
    if (n_slots < 0 || n_slots > p->nslot_alloc)
        FAIL(MOE_EINVAL, "n_slots %d outside [0,%d] (the slots allocated at create)", n_slots, p->nslot_alloc);
    if (p->cfg.policy == MOE_POLICY_DEVICE &&
        moe::policy_lds_bytes(p->cfg.n_experts, n_slots, p->cfg.evict) + (size_t)(p->cfg.hidden / 32) * 80 + 16 >
            65536)
        FAIL(MOE_EINVAL, "%d slots do not fit the device slot manager's LDS", n_slots);
    moe_status_t st = moe_pool_sync(p);
    if (st) return st;
    if (p->cfg.policy == MOE_POLICY_DEVICE) {
        const DevLayout d = dev_layout(p->cfg.n_experts, n_slots);
        for (auto& L : p->layers) {
            char* blk = nullptr;
            HIPCHK(hipMalloc((void**)&blk, d.total));
            HIPCHK(hipFree(L.dev_block));
            L.dev_block = blk;
            L.ds.copy[0] = blk + d.copy0;
            L.ds.copy[1] = blk + d.copy1;
            L.ds.ctl = reinterpret_cast<int32_t*>(blk + d.ctl);
            L.ds.ctr = reinterpret_cast<unsigned long long*>(blk + d.ctr);
            L.ds.rec = reinterpret_cast<int32_t*>(blk + d.rec);
        }
    }
    p->cfg.n_slots = n_slots;
    return moe_pool_reset(p);
}

moe_status_t moe_pool_set_eviction(moe_pool_t* p, int32_t evict) {
    if (!p) FAIL(MOE_EINVAL, "null pool");
    const moe_pool_config_t& c = p->cfg;
    if (evict < MOE_EVICT_LRU || evict > MOE_EVICT_DECAY) FAIL(MOE_EINVAL, "evict %d invalid", evict);
    if (evict != MOE_EVICT_LRU && c.policy != MOE_POLICY_DEVICE)
        FAIL(MOE_EINVAL, "the host slot manager implements LRU only; evict %d needs the device policy", evict);
    if (evict == MOE_EVICT_DECAY && c.read_through)
        FAIL(MOE_EINVAL, "placement by decayed counts runs with read_through 0");
    if (evict == MOE_EVICT_DECAY && (int64_t)p->nslot_alloc * 2 > moe::kMaxExperts)
        FAIL(MOE_EINVAL, "placement by decayed counts: %d slots > %d", p->nslot_alloc, moe::kMaxExperts / 2);
    if (c.policy == MOE_POLICY_DEVICE &&
        moe::policy_lds_bytes(c.n_experts, c.resident ? 0 : c.n_slots, evict) + (size_t)(c.hidden / 32) * 80 + 16 >
            65536)
        FAIL(MOE_EINVAL, "the decision's state under evict %d does not fit its LDS", evict);
    moe_status_t st = moe_pool_sync(p);
    if (st) return st;
    p->cfg.evict = evict;
    return moe_pool_reset(p);
}

// ---- host-only slot manager ---------------------------------------------------
moe_status_t moe_lru_create(int32_t n_experts, int32_t n_slots, int32_t rule, moe_lru_t** out) {
    if (!out) FAIL(MOE_EINVAL, "null out");
    *out = nullptr;
    if (n_experts < 1 || n_experts > moe::kMaxExperts || n_slots < 0) FAIL(MOE_EINVAL, "bad sizes");
    if (rule != MOE_RULE_DISTINCT && rule != MOE_RULE_STATIC) FAIL(MOE_EINVAL, "bad rule");
    moe_lru* l = new (std::nothrow) moe_lru();
    if (!l) FAIL(MOE_ENOMEM, "host allocation failed");
    l->lru.init(n_experts, n_slots, rule);
    l->u.reserve(n_experts);
    *out = l;
    return MOE_OK;
}

void moe_lru_destroy(moe_lru_t* l) { delete l; }

moe_status_t moe_lru_step(moe_lru_t* l, const int32_t* ids, int32_t n_tokens, int32_t top_k, int32_t* slot_ids,
                          moe_miss_t* miss_host, int32_t miss_cap, int32_t* n_miss, int32_t* path) {
    if (!l) FAIL(MOE_EINVAL, "null lru");
    if (n_tokens < 0 || top_k < 1 || miss_cap < 0) FAIL(MOE_EINVAL, "bad sizes");
    const int64_t n = (int64_t)n_tokens * top_k;
    if (n > 0 && (!ids || !slot_ids)) FAIL(MOE_EINVAL, "null ids");
    const int32_t E = l->lru.n_experts();
    std::vector<char> seen(E, 0);
    for (int64_t i = 0; i < n; ++i) {
        if (ids[i] < 0 || ids[i] >= E) FAIL(MOE_ERANGE, "expert id %d outside [0,%d)", ids[i], E);
        seen[ids[i]] = 1;
    }
    l->u.clear();
    std::vector<int32_t> rank(E, -1);
    for (int32_t e = 0; e < E; ++e)
        if (seen[e]) {
            rank[e] = (int32_t)l->u.size();
            l->u.push_back(e);
        }
    l->misses.clear();
    const bool pooled = l->lru.step(l->u.data(), (int32_t)l->u.size(), n, l->misses);
    for (int64_t i = 0; i < n; ++i) slot_ids[i] = pooled ? l->lru.map()[ids[i]] : rank[ids[i]];
    const int32_t nm = (int32_t)l->misses.size();
    if (miss_host)
        for (int32_t i = 0; i < std::min(nm, miss_cap); ++i)
            miss_host[i] = moe_miss_t{l->misses[i].expert, l->misses[i].slot, l->misses[i].evicted};
    if (n_miss) *n_miss = nm;
    if (path) *path = pooled ? MOE_PATH_POOL : MOE_PATH_FALLBACK;
    return MOE_OK;
}

moe_status_t moe_lru_get_state(const moe_lru_t* l, int32_t* map_E, int32_t* owner_N, int32_t* lru_N) {
    if (!l) FAIL(MOE_EINVAL, "null lru");
    if (map_E) std::copy(l->lru.map().begin(), l->lru.map().end(), map_E);
    if (owner_N) std::copy(l->lru.owner().begin(), l->lru.owner().end(), owner_N);
    if (lru_N) l->lru.lru_order(lru_N, l->lru.n_slots());
    return MOE_OK;
}

moe_status_t moe_lru_get_stats(const moe_lru_t* l, moe_pool_stats_t* out) {
    if (!l || !out) FAIL(MOE_EINVAL, "null argument");
    std::memset(out, 0, sizeof(*out));
    out->steps = l->lru.steps();
    out->hits = l->lru.hits();
    out->misses = l->lru.misses();
    out->fallbacks = l->lru.fallbacks();
    return MOE_OK;
}

}  // extern "C"
