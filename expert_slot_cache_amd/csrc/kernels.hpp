// Launchers of the gfx950 kernels (C++ linkage, used by the C-ABI runtime only).
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace moe {

enum WType { W_F32 = 0, W_BF16 = 1, W_INT4 = 2 };
enum AType { A_F32 = 0, A_BF16 = 1 };

constexpr int kMaxExperts = 4096;
constexpr int kMaxTopK = 64;
constexpr int kDecodeMaxTokens = 8;   // n_tokens above this use the grouped GEMM path

// Shape and byte layout of one expert as stored in a slot.
struct Geom {
    int H, I, K;
    int E;                          // experts per layer
    int wtype, atype;
    size_t slot_stride;             // bytes per slot (= bytes per expert)
    size_t off_w13, off_w2, off_s13, off_s2;
};

// Distinct ids of ids[0..n), written to host-mapped rb with a tag (1..2^18-1) in
// bits 14..31 of every word: rb[0] = tag<<14 | bad<<13 | D (bad: an id outside
// [0,E)), rb[1+i] = tag<<14 | i-th ascending distinct id.  rank[e] (device) =
// position of e in that list.
hipError_t launch_distinct(const int32_t* ids, int n, int E, uint32_t* rb, int32_t* rank, uint32_t tag,
                           hipStream_t stream);

enum { PATH_POOL = 0, PATH_STAGE = 1, PATH_NONE = 2 };

// The remap of one step, with the decision status/n_upd:
//   PATH_POOL : apply upd[2u] -> upd[2u+1] (u < n_upd) to `table` in place, then
//               out[i] = table[ids[i]]
//   PATH_STAGE: out[i] = rank[ids[i]]
//   PATH_NONE : out[i] = -1
// ids outside [0,E) give -1.  The path is also written to *path (device), which
// the forward kernels read to pick the slot base.  upd may be host-mapped.
hipError_t launch_remap(const int32_t* ids, int n, int E, int32_t* table, const int32_t* rank, const int32_t* upd,
                        int n_upd, int status, int32_t* out, int32_t* path, hipStream_t stream);

// Optional event pairs around the two projection stages (any may be null).
struct StageEvents {
    hipEvent_t w13_start = nullptr, w13_stop = nullptr;
    hipEvent_t w2_start = nullptr, w2_stop = nullptr;
};

// The two places a layer's experts can be read from; *path (written by the
// step's decision or remap) picks one: PATH_POOL -> pool, PATH_STAGE -> stage,
// PATH_NONE -> none.
// On the pool path, slot ids npool .. npool + nmix - 1 name staging entries 0 ..
// nmix - 1 (experts a step reads from the host without placing them: the placement by
// decayed use counts); nmix is 0 under the other policies.
struct Slots {
    const char* pool;
    const char* stage;
    int npool;              // valid slot ids in the pool: [0, npool)
    int nstage;             // valid staging ranks: [0, nstage)
    int nmix;               // staging entries the pool path also addresses
    const int32_t* path;    // device word
};

struct ForwardArgs {
    Slots sl;
    const int32_t* slot_ids;// [T][K]
    const void* x;          // [T][H]
    const float* topk_w;    // [T][K]
    const void* resid;      // [T][H] or null
    void* out;              // [T][H]
    int T;
    // scratch
    void* act;              // [T*K][I]: SwiGLU output (fp32 for f32 weights, else bf16)
    float* y;               // [T*K][H] fp32: per-(token, expert) w2 output
    int32_t* grp;           // grouped-path index buffer (grouped_index_bytes)
    int nslots_alloc;       // slot count the grp buffer was sized for
    int max_pairs;          // max_tokens * K the scratch was sized for
    int32_t* flip_par;      // decode w2 launch of a fused step: the layer's ctl words (else null)
};

// The slot-indexed fused MoE for one layer.
hipError_t launch_forward(const Geom& g, const ForwardArgs& a, const StageEvents* ev,
                          hipStream_t stream);

// Whether the decode kernels support this shape (row chunk counts they can split).
bool decode_shape_supported(int wtype, int atype, int H, int I);

// Bytes of one (token, expert) pair's SwiGLU output in the act scratch.
size_t act_bytes_per_pair(int wtype, int I);

// Bytes of the grouped-path index buffer for max_tokens tokens and nslots slots.
size_t grouped_index_bytes(int max_tokens, int K, int nslots);

// Whole-expert copies by a kernel (the miss path's copy engine when it is not the
// DMA engine): job i copies `bytes` from src (a device-mapped pointer into pinned
// host memory) to dst (HBM).  Jobs travel in the kernel arguments.
constexpr int kFillMaxJobs = 16;
struct FillJob {
    const char* src;
    char* dst;
};
struct FillBatch {
    FillJob job[kFillMaxJobs];
    int n;
    size_t bytes;   // per job, a multiple of 16
};
hipError_t launch_fill(const FillBatch& b, hipStream_t s);

// ---- the slot manager on the GPU -----------------------------------------------------
// Eviction policies (the victim among the resident experts the step has not yet
// processed is the one with the smallest key):
//   LRU : key = tick of the last touch
//   FIFO: key = tick of the insertion
//   LFU : (use = touches since insertion, key = tick of the last touch)
//   SLRU: (prot = protected segment, key = tick of taking its place in the segment);
//         the probationary segment (prot 0) gives the victim while it has a candidate
// DECAY is placement by decayed use counts instead ("Running 125B MoE on Two 32 GB
// Cards", sections 4.3-4.4): a miss on a full pool is read from the host for the
// step (staging entry r, slot id N + r) and evicts nothing; every 8th pooled step
// first multiplies every count by 2^(-1/64) and, with the pool full, moves the most
// used host expert into the slot of the least used resident one when its count is
// larger by more than 2; each pooled step then adds its (token, k) selections.
enum { EVICT_LRU = 0, EVICT_FIFO = 1, EVICT_LFU = 2, EVICT_SLRU = 3, EVICT_DECAY = 4 };
constexpr int kDecayEvery = 8;          // pooled steps between decisions
constexpr float kDecayThreshold = 2.0f; // the count gap a move needs

// One copy of a layer's slot-manager state, all slot-indexed except map:
// map[E] (slot or -1), owner[N] (expert or -1), free[N] (a stack, meta[0] entries
// valid, popped from the top), key[N], use[N] (u32), prot[N], cnt[E] (f32 decayed use
// counts), meta = {nfree, tick, nprot, pooled steps}.  Each layer holds two copies: a
// launch reads copy ctl[0] and its lead workgroup writes the state after the step
// into the other copy.
struct SlotStateLayout {
    size_t map, owner, free, key, use, prot, cnt, meta, total;
};
__host__ __device__ inline size_t slot_state_align(size_t n) { return (n + 255) / 256 * 256; }
__host__ __device__ inline SlotStateLayout slot_state_layout(int E, int N) {
    SlotStateLayout L{};
    size_t o = 0;
    L.map = o;   o = slot_state_align(o + (size_t)E * 4);
    L.owner = o; o = slot_state_align(o + (size_t)N * 4);
    L.free = o;  o = slot_state_align(o + (size_t)N * 4);
    L.key = o;   o = slot_state_align(o + (size_t)N * 4);
    L.use = o;   o = slot_state_align(o + (size_t)N * 4);
    L.prot = o;  o = slot_state_align(o + (size_t)N * 4);
    L.cnt = o;   o = slot_state_align(o + (size_t)E * 4);
    L.meta = o;  o = slot_state_align(o + 16 * 4);
    L.total = o;
    return L;
}

// A layer's device-side slot manager: the two state copies, the control words
// ctl = {par: the current copy, readers: workgroups of the running launch that have
// read it (0 between launches), wrote: the fused step's lead wrote the other copy},
// counters ctr = u64 {steps, hits, misses, fallbacks, bytes_h2d, staged, prefetched,
// prefetch bytes, moves} and the last step's record rec = {path, D, n_miss, bad, then
// (expert, slot, evicted) per miss}.  A prepare launch's last reader flips par; after a
// fused step the w2 launch flips it when `wrote` is set.  No workgroup ever waits for
// another.
struct DevState {
    char* copy[2];
    int32_t* ctl;
    unsigned long long* ctr;
    int32_t* rec;
};

struct PolicyArgs {
    const int32_t* ids;      // [n] this step's top-k ids
    int n;                   // n_tokens * top_k (>= 1)
    int E, N;
    int rule;                // 0: fallback iff D > N; 1: iff n > N (and D > 0)
    int evict;               // EVICT_*
    int resident;            // 1: every expert at slot = id (count hits only)
    unsigned long long eb;   // bytes per expert (bytes_h2d counter; a multiple of 16)
    DevState ds;
    int32_t* out;            // [n] slot ids (or staging ranks)
    int32_t* path;           // the layer's path word
    uint32_t* err;           // host-mapped: 1 = an id outside [0, E)
    // the copies (unused when resident)
    const char* const* pieces;  // device array: device-mapped base of each store piece
    int per_piece;           // experts per piece
    char* slots;             // the layer's slot pool
    char* staging;           // the staging area
    int32_t* timed_jobs;     // host-mapped, or null: experts the step moves over the link
    // the layer's prefetch buffer (pf_n = 0: none): pf_n entries of eb bytes at pf_buf,
    // entry j holding an exact copy of expert pf_tag[j] (-1: nothing); a missed or staged
    // expert found there is read from it instead of over the host link
    const int32_t* pf_tag;
    char* pf_buf;
    int pf_n;
};
// Dynamic LDS of the decision for E experts and N slots under policy evict.
size_t policy_lds_bytes(int E, int N, int evict);
// grid: workgroups of the launch (the per-id outputs and the copies spread over them).
hipError_t launch_policy(const PolicyArgs& a, int grid, hipEvent_t start, hipEvent_t stop, hipStream_t s);

// Prefetch of predicted experts for a layer's next step ([vLLM-cache] planned async
// H2D with cross-layer prediction; [prefetch]: copies on a copy stream, joined by an
// event before the layer runs), one launch: the predicted ids' distinct experts that
// the layer's current state copy does not hold, ascending, at most pf_n, are copied
// into entries 0, 1, ... and tagged.
struct PrefetchArgs {
    const int32_t* ids;      // [n] predicted top-k ids (1 <= n <= 256)
    int n;
    int E, N;
    DevState ds;             // the layer's slot-manager state (map of the current copy)
    int32_t* tag;            // [pf_n]
    char* buf;               // pf_n entries of eb bytes
    int pf_n;                // 1..64
    const char* const* pieces;
    int per_piece;
    unsigned long long eb;
};
hipError_t launch_prefetch(const PrefetchArgs& a, int copy_grid, hipStream_t s);

// The one-token decode step in two launches (read-through misses): the first runs the
// decision in every workgroup that needs it, the w13 GEMV + SwiGLU (a missed expert's
// rows read from the pinned store and written through to its slot, a staged one's
// read from the store), and copies the rest of each missed or staged expert (from its
// w2 region on) into the slot or staging entry; the second is the w2 GEMV + combine.
// fw.slot_ids must be pol.out; n_copy: workgroups that copy.
hipError_t launch_step_decode(const Geom& g, const PolicyArgs& pol, const ForwardArgs& fw, int n_copy,
                              const StageEvents* ev, hipStream_t s);

// One launch of the streaming-read calibration kernel over [p, p + bytes) (bytes a
// multiple of 16), timed by the event pair; sink: 1 KiB of device scratch.
hipError_t launch_read_probe(const void* p, size_t bytes, unsigned* sink, hipEvent_t start, hipEvent_t stop,
                             hipStream_t s);

// Whether n_tokens above kDecodeMaxTokens take the grouped MFMA path for this shape.
bool grouped_shape(int wtype, int H, int I);

}  // namespace moe
