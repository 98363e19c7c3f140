/*
 * moe_pool.h -- MoE expert offload with a fixed-size HBM expert-slot cache (C ABI).
 *
 * All experts of every layer live in one pinned host store.  Each layer owns a
 * pool of N fixed-address HBM slots; each step the router's topk_ids are reduced
 * to their distinct experts, hits and misses are counted, the least recently used
 * slot is evicted for each miss, misses are copied host -> HBM on copy streams,
 * and topk_ids are remapped to slot ids through the layer's map table.  A step
 * that touches more distinct experts than there are slots bypasses the pool:
 * its experts are copied into a staging area and the pool is left untouched.
 * The experts then run as a slot-indexed fused MoE (w13 projection, SwiGLU, w2
 * projection, top-k weighted sum).
 *
 * Sources (the pages this library implements):
 *  [vLLM-cache]  vLLM PR "Run MoE models exceeding VRAM via expert CPU offloading
 *                with GPU cache (--moe-expert-cache-size)": sections "Architecture",
 *                "How it works", "torch.compile compatibility", the test list, and the
 *                review thread (OrderedDict LRU, persistent int32 mapping, async H2D).
 *  [llama-pool]  llama.cpp discussion "RFC: Persistent expert slot pool for MoE CPU
 *                offload (--moe-expert-cache)": sections "Summary", "Design" (items
 *                1-4), "Why not the other approaches on the table" (prefill rule),
 *                "Validation" (stale map table).
 *  [flash-2x32]  "Running 125B MoE on Two 32 GB Cards": section 1 (INT4 g128 expert
 *                shape and bytes), section 3.4 (an id of -1 must never reach a kernel),
 *                sections 4.3-4.4 (placement by decayed use counts).
 *  [prefetch]    article on vLLM PR #51710 (layer prefetch): copy stream joined back to
 *                the compute stream with events; large copies split into chunks.
 *
 * Conventions for every entry point:
 *  - Every call returns a moe_status_t; nothing throws or aborts across the ABI.
 *    moe_last_error() gives a message for the calling thread's last failure.
 *  - A failing call leaves the pool's cache state (map, owners, LRU order,
 *    counters, slot bytes) unchanged.
 *  - "dev" pointers are device (HBM) addresses owned by the caller; "host"
 *    pointers are ordinary host memory owned by the caller.  The library owns the
 *    pinned store, the slot pools, the staging area, its scratch buffers, its
 *    copy streams and events.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    kernels of a pool run on that one compute stream.
 *  - One host thread per pool at a time ([vLLM-cache] review thread: prepare()
 *    assumes a single-threaded forward).  Different pools are independent.
 */
#ifndef MOE_POOL_H
#define MOE_POOL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status_t;
#define MOE_OK       0
#define MOE_EINVAL  (-1)  /* bad argument or configuration */
#define MOE_ENOMEM  (-2)  /* host or device allocation failed, or over hbm_budget_bytes */
#define MOE_EHIP    (-3)  /* a HIP runtime call failed */
#define MOE_ERANGE  (-4)  /* an expert id outside [0, n_experts) */
#define MOE_ESTATE  (-5)  /* forward without a matching prepare, or staging reused */

/* weight formats; the byte layout of one expert is given at moe_pool_load_expert */
#define MOE_W_F32        0
#define MOE_W_BF16       1
#define MOE_W_INT4_G128  2
/* activation / output formats */
#define MOE_A_F32   0
#define MOE_A_BF16  1
/* route rule: when a step bypasses the pool ([llama-pool] prefill rule) */
#define MOE_RULE_DISTINCT 0  /* distinct experts of the step > n_slots (default) */
#define MOE_RULE_STATIC   1  /* top_k * n_tokens > n_slots (the ubatch could reach more
                                experts than there are slots) */
/* copy engine of the miss path (host store -> HBM) */
#define MOE_COPY_KERNEL 0  /* a copy kernel on the copy streams, reading the pinned store
                              through its device mapping (default: on MI355X it moves a
                              12 MiB expert ~3 % and a 2.4 MiB one ~15 % faster) */
#define MOE_COPY_DMA    1  /* hipMemcpyAsync on the copy streams */
/* where the slot manager runs */
#define MOE_POLICY_HOST   0  /* on the host: prepare reads the step's distinct ids back
                                (one sync per layer) and returns the path and misses */
#define MOE_POLICY_DEVICE 1  /* on the GPU: prepare and step only queue work (a kernel runs
                                the same slot manager on device-resident state and pulls
                                the misses); the path and misses of a step are read later
                                with moe_pool_last_step */
/* eviction policy: which resident expert a miss replaces ([vLLM-cache] review thread:
   the four policies it lists).  The victim is always a resident expert the step has
   not yet processed; among those: */
#define MOE_EVICT_LRU  0  /* the least recently used (default; the policy the PR ships) */
#define MOE_EVICT_FIFO 1  /* the earliest inserted */
#define MOE_EVICT_LFU  2  /* the fewest uses since insertion, then the least recently used */
#define MOE_EVICT_SLRU 3  /* segmented LRU: a miss enters a probationary segment, a hit there
                             promotes to a protected segment of (4 N) / 5 experts (its
                             oldest is demoted back when it overflows); victims come from
                             the probationary segment first */
#define MOE_EVICT_DECAY 4 /* placement by decayed use counts ([flash-2x32] sections 4.3 and
                             4.4, moving experts at run time): the pool fills from
                             free slots; on a full pool a miss is read from the host into
                             staging for that step only (its slot id is n_slots + the
                             staging entry) and evicts nothing.  Every 8th pooled step first
                             multiplies every expert's count by 2^(-1/64) (float32) and,
                             with the pool full, moves the host expert of largest count
                             into the slot of the resident expert of smallest count (lowest
                             id on ties) when the gap exceeds 2 (a miss, and a move); each
                             pooled step then adds its (token, k) selections to the counts.
                             Needs read_through 0 and n_slots <= 2048. */
/* path a step took */
#define MOE_PATH_POOL     0
#define MOE_PATH_FALLBACK 1

typedef struct moe_pool moe_pool_t;
typedef struct moe_lru moe_lru_t;

typedef struct {
    int32_t n_layers;
    int32_t n_experts;      /* E per layer, 1..4096 */
    int32_t top_k;          /* K, 1..min(E, 64) */
    int32_t hidden;         /* H */
    int32_t inter;          /* I (w13 has 2I rows: gate rows [0,I), up rows [I,2I)) */
    int32_t n_slots;        /* N slots per layer; 0 = no pool, every step falls back */
    int32_t wtype;          /* MOE_W_* */
    int32_t atype;          /* MOE_A_* */
    int32_t rule;           /* MOE_RULE_* */
    int32_t resident;       /* 1 = every expert lives in HBM at slot = expert id and the
                               map is the identity: the all-resident reference mode
                               ([vLLM-cache] "FullGPUProvider"); n_slots is ignored and
                               there is no host store (nothing is ever copied in) */
    int32_t max_tokens;     /* largest n_tokens accepted by prepare/forward (>= 1) */
    int32_t n_copy_streams; /* copy streams for host -> HBM copies, 1..8 */
    size_t copy_chunk_bytes;/* split each copy into pieces of at most this size
                               (0 = one hipMemcpyAsync per expert) */
    size_t hbm_budget_bytes;/* 0 = no limit; else slots + staging + scratch must fit */
    int32_t timing;         /* 0 = off; N >= 1 = time every Nth forward's two kernels
                               and every Nth prepare's copies with HIP events
                               (moe_pool_get_timing).  The events cost a few us per
                               timed call, so a period > 1 keeps them off most calls. */
    int32_t copy_engine;    /* MOE_COPY_KERNEL (0) or MOE_COPY_DMA (1); the same bytes land
                               in the same places either way.  copy_chunk_bytes applies
                               to the DMA engine only. */
    int32_t policy;         /* MOE_POLICY_HOST (0) or MOE_POLICY_DEVICE (1, n_experts <=
                               2048, copies by the copy kernel on the compute stream).
                               Both give the same slot ids, misses, counters and bits. */
    int32_t read_through;   /* 1 (device policy): a one-token moe_pool_step is two launches.
                               The first runs the decision in its own workgroups and the
                               w13 GEMV: a missed expert's w13 rows are read from the
                               pinned store and written through to its slot by the GEMV
                               blocks, while copy workers of the same launch move the
                               rest of it (a staged expert likewise goes to staging), so
                               the hit experts' compute and the miss transfers overlap.
                               The second is the w2 GEMV + combine.  Slot bytes, counters
                               and outputs are those of the copying step.  0: the step's
                               experts are copied first (prepare + forward always copy). */
    int32_t evict;          /* MOE_EVICT_* (non-LRU policies need MOE_POLICY_DEVICE) */
    int32_t prefetch_slots; /* 0 = none; 1..64 (device policy, not resident): HBM entries per
                               layer that moe_pool_prefetch fills with predicted experts */
} moe_pool_config_t;

typedef struct {
    int32_t expert;   /* the expert copied in */
    int32_t slot;     /* the slot it now occupies */
    int32_t evicted;  /* the expert evicted from that slot, or -1 if the slot was free */
} moe_miss_t;

typedef struct {
    uint64_t steps;      /* accepted prepare calls (pooled or not) */
    uint64_t hits;       /* distinct experts found resident, per step */
    uint64_t misses;     /* distinct experts copied into a slot, per step */
    uint64_t fallbacks;  /* steps that bypassed the pool */
    uint64_t bytes_h2d;  /* bytes steps copied host -> HBM (misses and staging not served
                            from a prefetch buffer) */
    uint64_t staged;     /* experts copied into staging by fallback steps (and by the
                            host reads of pooled steps under MOE_EVICT_DECAY) */
    uint64_t prefetched; /* missed or staged experts a step took from its prefetch buffer */
    uint64_t prefetch_bytes; /* bytes moved host -> HBM by moe_pool_prefetch */
    uint64_t moves;      /* MOE_EVICT_DECAY: experts its decisions moved into the pool
                            (counted in misses); host reads count in staged */
} moe_pool_stats_t;

typedef struct {
    double copy_ms;       /* sum, over timed prepare calls, of the span of their copies */
    uint64_t copy_calls;  /* timed prepare calls that issued copies */
    uint64_t copy_bytes;  /* bytes those timed copies moved */
    double w13_ms;        /* sum of durations of the timed w13 (+ SwiGLU) kernels */
    double w2_ms;         /* sum of durations of the timed w2 (+ combine) kernels */
    uint64_t kernel_calls;/* timed forward calls (each times both kernels) */
    double sync_wait_ms;  /* host time blocked on the distinct-id readbacks (all calls) */
} moe_pool_timing_t;

/* ---- errors -------------------------------------------------------------- */
/* A fixed message for a status code (overflow is not one of them: it is the
 * fallback path, [llama-pool] "Why not the other approaches on the table"). */
const char* moe_strerror(moe_status_t s);
/* Message for the calling thread's most recent failing call (static storage). */
const char* moe_last_error(void);

/* ---- layout -------------------------------------------------------------- */
/* Bytes of one expert in format `wtype` with hidden H and intermediate I, or 0 if
 * the shape is not supported (f32: H, I multiples of 4; bf16: multiples of 8;
 * int4: multiples of 128).  Layout: see moe_pool_load_expert. */
size_t moe_expert_bytes(int32_t wtype, int32_t hidden, int32_t inter);

/* ---- pool lifetime ---------------------------------------------------------- */
/* Allocates the pinned store (n_layers * n_experts experts; contents undefined
 * until moe_pool_load_expert writes them), one HBM
 * pool per layer (n_slots experts plus a zeroed 256-byte tail, allocated once so
 * slot addresses never change: [vLLM-cache] Architecture, the slot pool allocated
 * once at fixed addresses; [llama-pool] Design item 1), a staging area of min(E, K*max_tokens)
 * experts, the per-layer map tables (int32 [E], all -1) and scratch buffers.
 * hbm_budget_bytes, when set, caps the HBM part ([llama-pool] Design item 4).
 * Errors: EINVAL (bad config), ENOMEM, EHIP. */
moe_status_t moe_pool_create(const moe_pool_config_t* cfg, void* stream, moe_pool_t** out);
/* Frees everything moe_pool_create allocated, after the pool's queued work; NULL is
 * accepted.  The caller's buffers are not touched. */
void moe_pool_destroy(moe_pool_t* pool);

/* Copies one expert's bytes from `host_src` (moe_expert_bytes bytes) into the
 * pinned store ([vLLM-cache] "Architecture": the pinned host backing store that
 * holds every expert of the layer).
 * In resident mode the bytes go straight to HBM slot `expert` instead.  If the expert
 * is currently resident in a slot, that slot is not refreshed: load experts before
 * the first prepare.  Byte layout (regions in order, each on a 256-byte boundary):
 *   f32 : w13 [2I][H] fp32 row-major, w2 [H][I] fp32 row-major
 *   bf16: w13 [2I][H] bf16, w2 [H][I] bf16
 *   int4: w13 codes [2I][H/8] u32, w2 codes [H][I/8] u32, s13 [2I][H/128] bf16,
 *         s2 [H][I/128] bf16; element j of a row is bits 4*(j%8) of word j/8 and
 *         decodes to (q - 8) * s[row][j/128] ([flash-2x32] section 1: codes plus
 *         bf16 scales, no zero point).
 * Errors: EINVAL (bad layer/expert/size), EHIP. */
moe_status_t moe_pool_load_expert(moe_pool_t* pool, int32_t layer, int32_t expert,
                                  const void* host_src, size_t nbytes);

/* The pool-size knob of [llama-pool] "Summary" (the -mec sweep): from now on each layer
 * keeps at most n_slots experts, 0 <= n_slots <= the n_slots given at create (0: every
 * step falls back), and the pool is returned to cold as by moe_pool_reset.  The store
 * and the slot memory stay as they are, so one filled store serves every point of a
 * sweep.  Errors: EINVAL (resident mode, n_slots out of range), EHIP. */
moe_status_t moe_pool_set_slots(moe_pool_t* pool, int32_t n_slots);

/* The eviction policy knob ([vLLM-cache] review thread: the policies it lists; and
 * [flash-2x32] sections 4.3-4.4): from now on the layers use MOE_EVICT_* `evict`, and
 * the pool is returned to cold as by moe_pool_reset; the store and the slot memory
 * stay as they are, so one filled store serves a comparison of the policies.
 * Errors: EINVAL (evict out of range, a non-LRU policy with the host slot manager,
 * MOE_EVICT_DECAY with read_through, the state not fitting the decision's LDS), EHIP. */
moe_status_t moe_pool_set_eviction(moe_pool_t* pool, int32_t evict);

/* Returns the pool to cold ([vLLM-cache] "How it works": the cache state the first
 * prepare starts from): every map entry -1, all slots free, eviction order empty,
 * counters zero (resident mode: counters only).  Slot bytes are not cleared.
 * Errors: EINVAL, EHIP. */
moe_status_t moe_pool_reset(moe_pool_t* pool);

/* ---- the step --------------------------------------------------------------- */
/* prepare ([vLLM-cache] "How it works": unique ids, hit -> move to MRU, miss ->
 * evict LRU + H2D copy + update mapping, remap through the persistent mapping;
 * [llama-pool] Design items 2-3: route rule, then ids readback, LRU update, async
 * H2D for misses and a map-table rewrite before the remap reads it).
 *
 *  topk_ids_dev  int32 [n_tokens][top_k], device.  0 <= n_tokens <= max_tokens.
 *  slot_ids_dev  int32 [n_tokens][top_k], device, written: the slot of each id
 *                (POOL) or the id's rank among the step's distinct ids, which is its
 *                staging index (FALLBACK).
 *  miss_host     optional host array of miss_cap entries; receives the misses in
 *                processing order (ascending expert id).  *n_miss is the full count
 *                even when it exceeds miss_cap.  A FALLBACK step has no misses.
 *  path          MOE_PATH_POOL or MOE_PATH_FALLBACK.
 *
 * The distinct ids are found on the GPU and written straight into pinned host
 * memory: prepare spins until that kernel has published them (one sync per layer
 * per step, as in [llama-pool] "Limitations").
 * It returns once the copies (on the copy streams), the map upload and the remap
 * are enqueued; the compute stream waits for the copies through events.
 * Distinct ids are processed in ascending order; free slots are taken from the
 * highest index down; a non-resident expert maps to -1.
 * Errors: EINVAL, ERANGE (an id outside [0,E): nothing changes), EHIP.
 *
 * Under MOE_POLICY_DEVICE prepare is asynchronous: it queues one launch on the compute
 * stream (the decision, the remap and the copies; [llama-pool] "Limitations" names the
 * per-layer readback as the cost this removes) and returns at once.  The step's path
 * and miss list -- the same values the host policy returns here -- are a record the
 * launch leaves in device memory: *n_miss and *path are set to -1, miss_host is not
 * written, and moe_pool_last_step returns the record after waiting for the step.  An id outside
 * [0,E) is found on the GPU: that step changes nothing and writes -1 slot ids;
 * moe_pool_last_step and moe_pool_sync report it as ERANGE, and so does any later
 * prepare/step on the layer that runs after the GPU has flagged it.  A forward must
 * follow its own prepare with no other layer's prepare in between (else ESTATE):
 * staging is shared and the host does not know which steps fell back. */
moe_status_t moe_pool_prepare(moe_pool_t* pool, int32_t layer, const int32_t* topk_ids_dev,
                              int32_t n_tokens, int32_t* slot_ids_dev,
                              moe_miss_t* miss_host, int32_t miss_cap, int32_t* n_miss,
                              int32_t* path);

/* forward: the slot-indexed fused MoE on the layer's last prepare.
 *  x_dev        [n_tokens][H] activations (MOE_A_F32: float, MOE_A_BF16: bf16).
 *  slot_ids_dev int32 [n_tokens][top_k] from that prepare.  A slot id outside the
 *               prepared range contributes nothing (never dereferenced;
 *               [flash-2x32] section 3.4).
 *  topk_w_dev   float [n_tokens][top_k] gate weights.
 *  resid_dev    optional [n_tokens][H] in the activation format, added to the result.
 *  out_dev      [n_tokens][H] in the activation format:
 *               out[t] = resid[t] + sum_k w[t][k] * W2[s] (silu(W13g[s] x[t]) * W13u[s] x[t])
 *               with fp32 accumulation and the k sum in k order.
 * Batch-1 to small-batch decode uses two GEMV kernels; larger n_tokens use a
 * grouped GEMM over slot-sorted tokens.  The kernel choice depends only on
 * (n_tokens, top_k, H, I, formats), so the pooled and the all-resident pools give
 * bit-identical outputs.
 * Errors: EINVAL, ESTATE (no prepare of this layer with this n_tokens since the
 * last reset, or its staging area was reused by another layer's fallback), EHIP. */
moe_status_t moe_pool_forward(moe_pool_t* pool, int32_t layer, const void* x_dev,
                              const int32_t* slot_ids_dev, const float* topk_w_dev,
                              const void* resid_dev, int32_t n_tokens, void* out_dev);

/* prepare + forward of one layer in one call (same arguments, same semantics,
 * same errors and the same bits), for callers that run the two back to back.
 * No kernel of the step waits for the host or for another stream: streams can
 * share a hardware queue, so such a wait could sit behind the very work it waits
 * for.  With the host policy the host reads the distinct ids back, runs the LRU,
 * queues the copies (the compute stream waits for them) and then the remap and
 * the forward; with the device policy nothing is read back.  See `read_through`
 * for the one-token variant that copies nothing before the forward. */
moe_status_t moe_pool_step(moe_pool_t* pool, int32_t layer, const int32_t* topk_ids_dev, int32_t n_tokens,
                           int32_t* slot_ids_dev, const void* x_dev, const float* topk_w_dev,
                           const void* resid_dev, void* out_dev, moe_miss_t* miss_host, int32_t miss_cap,
                           int32_t* n_miss, int32_t* path);

/* Cross-layer prefetch ([vLLM-cache] "Planned follow-ups": async H2D with cross-layer
 * prediction; [prefetch] "how the prefetch enters forward": after one layer runs, a
 * later layer's weights are copied on a copy stream, and that layer waits for them
 * through an event before it runs).  A hint that the next step of `layer` will use
 * the experts in predicted_ids_dev (int32 [n_tokens][top_k], device, 1 <= n_tokens *
 * top_k <= 256): on a copy stream, starting as `after` says (AFTER_LAYER: the ids
 * must already be in place; AFTER_QUEUED: the ids may come from work queued on the
 * compute stream; AFTER_PREVIOUS: the caller guarantees that the layer's last step
 * is done when the copy stream gets there), the predicted experts the layer does not
 * hold (ascending, at most prefetch_slots of them) are copied from the pinned store
 * into the layer's prefetch buffer entries 0, 1, ....  The layer's next prepare or step waits for
 * that copy (an event joins the streams; no kernel waits) and takes a missed or staged
 * expert found in the buffer from HBM instead of over the host link.  The cache is
 * unchanged by a prefetch: slot ids, misses, evictions, counters other than
 * prefetched / prefetch_bytes / bytes_h2d, and outputs are those of the same steps
 * without it.  Invalid ids are ignored.  predicted_ids_dev is read on the copy
 * stream: keep it unchanged until the layer's next prepare or step has been queued
 * (later work on the compute stream is ordered after the prefetch from then on).
 * Errors: EINVAL (no prefetch buffer, bad sizes), EHIP. */
#define MOE_PREFETCH_AFTER_LAYER    0  /* once the layer's last prepare or step is done */
#define MOE_PREFETCH_AFTER_QUEUED   1  /* once everything queued on the compute stream is done */
#define MOE_PREFETCH_AFTER_PREVIOUS 2  /* after the pool's previous prefetch only (for a
                                          captured graph, whose replays run one after another:
                                          the first prefetch of the capture waits for the
                                          queued work, the rest follow it) */
moe_status_t moe_pool_prefetch(moe_pool_t* pool, int32_t layer, const int32_t* predicted_ids_dev,
                               int32_t n_tokens, int32_t after);

/* The path and misses of the layer's last prepare (or step), as that call would have
 * returned them under MOE_POLICY_HOST; under MOE_POLICY_DEVICE the call first waits
 * for the layer's queued work.  miss_host/n_miss/path as in moe_pool_prepare.
 * Errors: EINVAL, ESTATE (no step yet since create or reset), ERANGE (that step had
 * an id outside [0,E): it changed nothing), EHIP. */
moe_status_t moe_pool_last_step(moe_pool_t* pool, int32_t layer, int32_t* path, moe_miss_t* miss_host,
                                int32_t miss_cap, int32_t* n_miss);

/* Waits until all of the pool's copies and kernels issued so far are complete
 * ([prefetch]: the compute stream joins the copy stream before results are used).
 * Under MOE_POLICY_DEVICE it then reports (and clears) an out-of-range id found by
 * a queued step (ERANGE).  Errors: EINVAL, EHIP, ERANGE. */
moe_status_t moe_pool_sync(moe_pool_t* pool);

/* ---- introspection (tests, benchmarks) ------------------------------------ */
/* The hit / miss counters of [vLLM-cache] "How it works" (hits and misses counted per
 * distinct expert of a step) and the fallback count of [llama-pool] "Design" item 2.
 * layer = -1 sums over layers.  Under MOE_POLICY_DEVICE it waits for queued work.
 * Errors: EINVAL, EHIP. */
moe_status_t moe_pool_get_stats(const moe_pool_t* pool, int32_t layer, moe_pool_stats_t* out);
/* The slot manager's state ([vLLM-cache] review thread: the persistent expert -> slot
 * mapping and the cache's eviction order).  map_E: int32[E] expert -> slot or -1;
 * owner_N: int32[N] slot -> expert or -1; lru_N: int32[N] resident experts in the
 * order the layer's policy would evict them (LRU: least recently used first), -1
 * padded.  Any pointer may be NULL.  Under MOE_POLICY_DEVICE it waits for queued
 * work.  Errors: EINVAL, EHIP. */
moe_status_t moe_pool_get_state(const moe_pool_t* pool, int32_t layer, int32_t* map_E,
                                int32_t* owner_N, int32_t* lru_N);
/* Test hook for the slot-contents check of [vLLM-cache] "Test results" (a slot holds
 * its expert's bytes after eviction and reload): synchronously copies n bytes
 * (<= one expert) of HBM slot `slot` of `layer` (slot < 0: staging entry -slot-1)
 * into host_dst, after the pool's queued work.  Errors: EINVAL, EHIP. */
moe_status_t moe_pool_read_slot(moe_pool_t* pool, int32_t layer, int32_t slot,
                                void* host_dst, size_t n);
/* Device address of slot `slot` of `layer` (constant for the pool's lifetime). */
moe_status_t moe_pool_slot_ptr(const moe_pool_t* pool, int32_t layer, int32_t slot, void** dev_ptr);
/* Host address of expert `expert` of `layer` in the pinned store (EINVAL in the
 * all-resident mode, which has no store).  The store is allocated in pieces of at
 * most 1 GiB; one expert never straddles two pieces. */
moe_status_t moe_pool_store_ptr(const moe_pool_t* pool, int32_t layer, int32_t expert, void** host_ptr);
/* *is_pinned = 1 if `p` lies in page-locked host memory known to HIP. */
moe_status_t moe_ptr_is_pinned_host(const void* p, int32_t* is_pinned);
/* Accumulated event timings (config.timing = 1); waits for queued work first. */
moe_status_t moe_pool_get_timing(moe_pool_t* pool, moe_pool_timing_t* out);
moe_status_t moe_pool_reset_timing(moe_pool_t* pool);
/* The event-timing period from now on (config.timing's meaning).  0 stops the sampling,
 * so that the pool's steps can be captured in a HIP graph (a capture cannot hold the
 * timed launches); every >= 1 needs a pool created with timing >= 1, which owns the
 * events.  Waits for queued work and keeps what was accumulated.
 * Errors: EINVAL (every < 0, or >= 1 on a pool created without timing), EHIP. */
moe_status_t moe_pool_set_timing(moe_pool_t* pool, int32_t every);

/* ---- calibration (benchmarks) ----------------------------------------------- */
/* What one kernel launch of `bytes` can read on this GPU: a plain streaming read
 * (each wave 4 KiB contiguous), launched reps times (after two untimed launches)
 * on `stream`, each launch over the next `bytes`-sized region of the caller's
 * device buffer [buf_dev, buf_dev + buf_bytes) so that a repeat does not hit the
 * on-chip caches, each timed with a HIP event pair around the dispatch (the way
 * the forward kernels are timed).  *avg_us = mean duration.  bytes: a positive
 * multiple of 16, at most buf_bytes.  The call synchronizes on each launch.
 * Errors: EINVAL, EHIP. */
moe_status_t moe_read_calibration(const void* buf_dev, size_t buf_bytes, size_t bytes, int32_t reps,
                                  void* stream, double* avg_us);

/* The host link's rate: `bytes` (a positive multiple of 16) from pinned, device-mapped
 * host memory to HBM (both allocated by the call and freed before it returns), reps
 * times after one untimed copy, with the given engine (MOE_COPY_KERNEL or MOE_COPY_DMA),
 * split into n_streams (1..8) equal parts copied side by side on `stream` and
 * n_streams - 1 streams of the call's own, each copy timed with events on `stream`
 * around all parts.  *avg_us = mean duration.  Errors: EINVAL, ENOMEM, EHIP. */
moe_status_t moe_link_calibration(size_t bytes, int32_t reps, int32_t engine, int32_t n_streams, void* stream,
                                  double* avg_us);

/* ---- a forward that allocates nothing ---------------------------------------- */
/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same fused MoE as
 * moe_pool_forward (the same kernels, so the same bits for the same slot bytes and
 * slot ids), over n_slots experts the caller holds contiguously at slots_dev (expert
 * s at slots_dev + s * moe_expert_bytes(wtype, hidden, inter), the byte layout of
 * moe_pool_load_expert), without a pool.  slot_ids_dev, x_dev, topk_w_dev, resid_dev
 * (optional), out_dev and n_tokens as in moe_pool_forward; a slot id outside
 * [0, n_slots) contributes nothing.  Its scratch lives in a device array of 64 MiB
 * per GPU that the library holds until the process ends; a call needing more
 * (decode: n_tokens * top_k * inter * 2 bytes; more than 8 tokens with bf16 weights:
 * also n_tokens * top_k * hidden * 4 and the index lists) is refused with EINVAL.
 * Calls on one GPU share that array: calls that overlap on one GPU race.  The call
 * makes no allocation (its first call on a device looks up the array's address).
 * Errors: EINVAL, EHIP. */
moe_status_t moe_forward_slots(int32_t wtype, int32_t atype, int32_t hidden, int32_t inter, int32_t top_k,
                               const void* slots_dev, int32_t n_slots, const int32_t* slot_ids_dev,
                               const void* x_dev, const float* topk_w_dev, const void* resid_dev,
                               int32_t n_tokens, void* out_dev, void* stream);

/* ---- the slot manager alone (host only, no GPU) ----------------------------- */
/* The same per-layer LRU state machine prepare() runs, driven from host ids, for
 * pool-size planning and for checking the bookkeeping without a GPU.  Semantics
 * as moe_pool_prepare (ids host int32 [n_tokens][top_k]; slot_ids host). */
moe_status_t moe_lru_create(int32_t n_experts, int32_t n_slots, int32_t rule, moe_lru_t** out);
void moe_lru_destroy(moe_lru_t* lru);
moe_status_t moe_lru_step(moe_lru_t* lru, const int32_t* ids_host, int32_t n_tokens,
                          int32_t top_k, int32_t* slot_ids_host, moe_miss_t* miss_host,
                          int32_t miss_cap, int32_t* n_miss, int32_t* path);
moe_status_t moe_lru_get_state(const moe_lru_t* lru, int32_t* map_E, int32_t* owner_N,
                               int32_t* lru_N);
moe_status_t moe_lru_get_stats(const moe_lru_t* lru, moe_pool_stats_t* out);

#ifdef __cplusplus
}
#endif
#endif /* MOE_POOL_H */
