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
// step's remap) picks one: PATH_POOL -> pool, PATH_STAGE -> stage, PATH_NONE -> none.
// Where a (token, expert) pair's expert is read from when it is not its slot: the
// expert in the device-mapped pinned store (`from`), and the slot it is written
// through to as it is read (`to`, or null).
struct PairSrc {
    const char* from;
    char* to;
};

struct Slots {
    const char* pool;
    const char* stage;
    int npool;              // valid slot ids in the pool: [0, npool)
    int nstage;             // valid staging ranks: [0, nstage)
    const int32_t* path;    // device word
    const PairSrc* src;     // null, or per pair: a non-null `from` replaces the slot (decode GEMVs)
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
// One layer's LRU state (HBM, int32): map[E] (slot or -1), owner[N] (expert or -1),
// free[N] (stack of free slots; meta[2] entries valid), prev/next[E] (the LRU list
// over expert ids, -1 terminated), meta = {head, tail, nfree}.
struct LruState {
    int32_t* map;
    int32_t* owner;
    int32_t* free;
    int32_t* prev;
    int32_t* next;
    int32_t* meta;
};

// The state plus ctr = u64 {steps, hits, misses, fallbacks, bytes_h2d, staged},
// rec = the last step {path, D, n_miss, bad, then (expert, slot, evicted) per miss}
// and arrive = the step's count of workgroups holding their copy of the state (0
// between steps).
struct DevState {
    LruState s;
    unsigned long long* ctr;
    int32_t* rec;
    int32_t* arrive;
};

struct PolicyArgs {
    const int32_t* ids;      // [n] this step's top-k ids
    int n;                   // n_tokens * top_k (>= 1)
    int E, N;
    int rule;                // 0: fallback iff D > N; 1: iff n > N (and D > 0)
    int resident;            // 1: every expert at slot = id (count hits only)
    unsigned long long eb;   // bytes per expert (bytes_h2d counter; a multiple of 16)
    LruState st;             // the layer's state, updated in place
    unsigned long long* ctr;
    int32_t* rec;
    int32_t* arrive;         // 0 at launch; left 0
    int32_t* out;            // [n] slot ids (or staging ranks)
    int32_t* path;           // the layer's path word
    uint32_t* err;           // host-mapped: 1 = an id outside [0, E); 2 = the write-back's
                             // wait for the other workgroups timed out
    unsigned long long spin_limit;  // bound on that wait (polls)
    // the copies (unused when resident)
    const char* const* pieces;  // device array: device-mapped base of each store piece
    int per_piece;           // experts per piece
    char* slots;             // the layer's slot pool
    char* staging;           // the staging area
    int32_t* timed_jobs;     // host-mapped, or null: experts the step moves over the link
    PairSrc* tab;            // null: copy the step's experts; else [n]: the forward reads them
                             // through (misses are written to their slots on the way)
};
size_t policy_lds_bytes(int E, int N);
// grid: workgroups of the launch (the per-id outputs and the copies spread over them).
hipError_t launch_policy(const PolicyArgs& a, int grid, hipEvent_t start, hipEvent_t stop, hipStream_t s);

// One launch of the streaming-read calibration kernel over [p, p + bytes) (bytes a
// multiple of 16), timed by the event pair; sink: 1 KiB of device scratch.
hipError_t launch_read_probe(const void* p, size_t bytes, unsigned* sink, hipEvent_t start, hipEvent_t stop,
                             hipStream_t s);

// Whether n_tokens above kDecodeMaxTokens take the grouped MFMA path for this shape.
bool grouped_shape(int wtype, int H, int I);

}  // namespace moe
