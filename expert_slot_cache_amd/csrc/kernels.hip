// gfx950 kernels of the expert slot cache: distinct ids, remap, and the
// slot-indexed fused MoE for decode (GEMV) shapes.
//
// Wave size is 64 throughout (CDNA).  All floating point accumulates in fp32, and
// every reduction has a fixed order, so a result depends only on the values it
// reads -- never on which slot an expert sits in.  That is what makes a pooled
// layer bit-identical to the same layer with every expert resident.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"
#include "policy_dev.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)0x7FC0;  // NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Butterfly sum over the 64 lanes: every lane ends with the same value, and the
// association order is fixed.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------------------
// K-distinct: presence bitmap in LDS, then ordered compaction with a wave64
// ballot + mbcnt lane prefix and a per-wave offset.  One workgroup.
//   [vLLM-cache "How it works": unique ids of topk_ids, ascending]
//
// The result goes straight to host memory, each 32-bit word carrying the step's
// tag in its top bits: rb[0] = tag<<14 | bad<<13 | D, rb[1 + i] = tag<<14 | id_i.
// The host zeroes the words before the launch and waits for each word it needs
// to show the tag, so no store ordering or cache flush is needed.
// ---------------------------------------------------------------------------
constexpr int kDistinctThreads = 1024;

// The body of k_distinct.  Writes rb (host) and, for each present id e,
// rank_out[e] = its position.  Returns D.  The rb words are system-scope stores,
// which no cache holds back: the host reads them while the kernel runs.
__device__ __forceinline__ int distinct_block(const int32_t* __restrict__ ids, int n, int E,
                                              uint32_t* __restrict__ rb, int32_t* __restrict__ rank_out,
                                              uint32_t tag, uint32_t* bits, int32_t* wave_cnt, int32_t& bad) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nwords = (E + 31) >> 5;
    const uint32_t hi = tag << 14;
    for (int i = tid; i < nwords; i += kDistinctThreads) bits[i] = 0u;
    if (tid == 0) bad = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kDistinctThreads) {
        const int e = ids[i];
        if ((unsigned)e < (unsigned)E)
            atomicOr(&bits[e >> 5], 1u << (e & 31));
        else
            bad = 1;
    }
    __syncthreads();
    int base = 0;
    for (int c0 = 0; c0 < E; c0 += kDistinctThreads) {
        const int e = c0 + tid;
        const bool present = e < E && ((bits[e >> 5] >> (e & 31)) & 1u);
        const uint64_t m = __ballot(present);
        const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (lane == 0) wave_cnt[wave] = __popcll(m);
        __syncthreads();
        int off = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kDistinctThreads / 64; ++w) {
            const int c = wave_cnt[w];
            off += (w < wave) ? c : 0;
            total += c;
        }
        if (present) {
            const int pos = base + off + (int)below;
            __hip_atomic_store(&rb[1 + pos], hi | (uint32_t)e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            rank_out[e] = pos;
        }
        base += total;
        __syncthreads();
    }
    if (tid == 0)
        __hip_atomic_store(&rb[0], hi | ((uint32_t)(bad != 0) << 13) | (uint32_t)base, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_SYSTEM);
    return base;
}

__global__ __launch_bounds__(kDistinctThreads) void k_distinct(const int32_t* __restrict__ ids, int n,
                                                               int E, uint32_t* __restrict__ rb,
                                                               int32_t* __restrict__ rank, uint32_t tag) {
    __shared__ uint32_t bits[kMaxExperts / 32];
    __shared__ int32_t wave_cnt[kDistinctThreads / 64];
    __shared__ int32_t bad;
    distinct_block(ids, n, E, rb, rank, tag, bits, wave_cnt, bad);
}

hipError_t launch_distinct(const int32_t* ids, int n, int E, uint32_t* rb, int32_t* rank, uint32_t tag,
                           hipStream_t stream) {
    hipLaunchKernelGGL(k_distinct, dim3(1), dim3(kDistinctThreads), 0, stream, ids, n, E, rb, rank, tag);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// K-remap: slot_ids[i] = table[ids[i]]  [vLLM-cache: remap topk_ids through the
// persistent mapping, updated in place at each miss; llama-pool: get_rows(table,
// ids) on a table rewritten before the remap reads it].
//
// The step's table changes (pairs (expert, entry after the step)) are applied
// inside the kernel: every workgroup copies the table into LDS and applies the
// list there, and workgroup 0 also writes the changes back to the persistent
// table.  So the remap can only read the fresh table.  An entry may be listed
// twice, always with the same value, so the order of the writes does not matter.
// Ids outside [0,E) give -1, which the forward kernels never dereference.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_remap(const int32_t* __restrict__ ids, int n, int E,
                                               int32_t* __restrict__ table, const int32_t* __restrict__ rank,
                                               const int32_t* __restrict__ upd, int n_upd, int status,
                                               int32_t* __restrict__ out, int32_t* __restrict__ path) {
    __shared__ int32_t tab[kMaxExperts];
    const int tid = threadIdx.x;
    const int i = blockIdx.x * 256 + tid;
    if (status == PATH_POOL) {
        for (int e = tid; e < E; e += 256) tab[e] = table[e];
        __syncthreads();
        for (int u = tid; u < n_upd; u += 256) {
            const int32_t e = upd[2 * u];
            const int32_t v = upd[2 * u + 1];
            tab[e] = v;
            if (blockIdx.x == 0) table[e] = v;
        }
        __syncthreads();
        if (i < n) {
            const int e = ids[i];
            out[i] = ((unsigned)e < (unsigned)E) ? tab[e] : -1;
        }
    } else if (i < n) {
        const int e = ids[i];
        out[i] = (status == PATH_STAGE && (unsigned)e < (unsigned)E) ? rank[e] : -1;
    }
    if (blockIdx.x == 0 && tid == 0) *path = status;
}

hipError_t launch_remap(const int32_t* ids, int n, int E, int32_t* table, const int32_t* rank, const int32_t* upd,
                        int n_upd, int status, int32_t* out, int32_t* path, hipStream_t stream) {
    const int blocks = n > 0 ? (n + 255) / 256 : 1;
    hipLaunchKernelGGL(k_remap, dim3(blocks), dim3(256), 0, stream, ids, n, E, table, rank, upd, n_upd, status, out,
                       path);
    return hipGetLastError();
}

// Elements per 16-byte chunk of a weight row.
template <int WT>
struct WTraits;
template <>
struct WTraits<W_F32> {
    static constexpr int EPC = 4;
};
template <>
struct WTraits<W_BF16> {
    static constexpr int EPC = 8;
};
template <>
struct WTraits<W_INT4> {
    static constexpr int EPC = 32;
};

// Element i of an activation array as fp32.
template <int AT>
__device__ __forceinline__ float load_act(const void* __restrict__ p, size_t i) {
    if (AT == A_F32) return static_cast<const float*>(p)[i];
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

// ---------------------------------------------------------------------------
// Decode GEMV kernels.
//
// A weight row is a run of 16-byte chunks (f32: 4 elements, bf16: 8, int4: 32).
// G lanes share a row (G = the largest power of two <= 64 dividing the chunk
// count), each lane taking CPL = chunks / G chunks at stride G, so one load
// instruction of a lane group covers G * 16 contiguous bytes of the row and a
// wave reads 64 / G rows side by side.  The activation vector stays in registers
// for the whole wave ("lane-stationary"): lane j of a group always owns the same
// chunk columns, loads their activations once (from L2) and reuses them for
// every row it streams.  All weight loads of a lane are issued before any math.
//
// Products:
//   bf16 x bf16 : v_dot2c_f32_bf16 over packed pairs (fp32 accumulate)
//   int4 x bf16 : code q becomes the bf16 value 128 + q by OR-ing it into the
//                 mantissa of 0x4300 (exact); sum (128+q) x with dot2, minus
//                 136 * sum(x) of the chunk, times the group's bf16 scale
//   otherwise   : fp32 FMAs
// Every reduction (in-lane chunk order, the butterfly over G lanes, the k order
// of the combine) is fixed, so results depend only on the bytes read.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

__device__ __forceinline__ uint4 load16(const char* p) { return *reinterpret_cast<const uint4*>(p); }

// Reads of one slot's bytes through a buffer resource, with system-coherent cache
// policy (sc0 sc1): a slot refilled by a host -> HBM DMA is always read from
// memory, never from a stale cache line, whatever the ordering between the copy
// and the kernel's launch.  Offsets are bytes within the slot; the hardware
// returns zeros past the slot's end.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kCoherent = 1 | 16;   // sc0 | sc1

struct SlotReader {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ SlotReader(const char* base, size_t bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)bytes, 0x00020000)) {}
    __device__ __forceinline__ uint4 load16(size_t off) const {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCoherent);
        return make_uint4(v.x, v.y, v.z, v.w);
    }
    // a per-lane offset plus a wave-uniform one (held in a scalar register): a lane keeps
    // one offset per row instead of one per chunk
    __device__ __forceinline__ uint4 load16(uint32_t voff, uint32_t soff) const {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kCoherent);
        return make_uint4(v.x, v.y, v.z, v.w);
    }
    __device__ __forceinline__ float scale(size_t off) const {
        return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, kCoherent));
    }
    // the scale's bf16 bits, widened only where they are used (widening here would make
    // the wave wait for this load, and every load issued before it, right away)
    __device__ __forceinline__ uint16_t scale_bits(size_t off) const {
        return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, kCoherent);
    }
};

// Vector stores into a slot: the write-through of an expert that a kernel reads from
// the pinned store (the bytes land in the slot exactly as read; a scale goes back
// to its bf16 bits, which the widening above keeps exactly).
struct SlotWriter {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ SlotWriter(char* base, size_t bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000)) {}
    __device__ __forceinline__ void store16(size_t off, uint4 v) const {
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{v.x, v.y, v.z, v.w}, r, (int)off, 0, 0);
    }
    __device__ __forceinline__ void store16(uint32_t voff, uint32_t soff, uint4 v) const {
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{v.x, v.y, v.z, v.w}, r, (int)voff, (int)soff, 0);
    }
    __device__ __forceinline__ void store_scale(size_t off, float v) const {
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(__float_as_uint(v) >> 16), r, (int)off, 0, 0);
    }
    __device__ __forceinline__ void store_scale_bits(size_t off, uint16_t b) const {
        __builtin_amdgcn_raw_buffer_store_b16(b, r, (int)off, 0, 0);
    }
};

// Where one (token, expert) pair reads its expert: a slot or staging entry, or (a
// read-through step) the expert in the device-mapped pinned store, which a missed
// expert's lanes also write through to its slot (`to`).
struct PairIn {
    const char* ebase;
    char* to;
    bool valid;     // the pair has an expert (else it contributes zeros)
};

// Activation-sized reads of a buffer, by byte offset (data written by an earlier
// kernel).
struct PlainMem {
    const char* p;
    __device__ __forceinline__ explicit PlainMem(const void* base) : p(static_cast<const char*>(base)) {}
    __device__ __forceinline__ uint4 ld16(size_t off) const { return *reinterpret_cast<const uint4*>(p + off); }
    __device__ __forceinline__ uint2 ld8(size_t off) const { return *reinterpret_cast<const uint2*>(p + off); }
};

// The slot ids of the step's path (see Slots): ids [0, na) at a, ids [na, na + nb) at
// b (the staging entries a pooled step addresses past the pool).
struct SlotSpan {
    const char* a;
    const char* b;
    int na, nb;
    __device__ __forceinline__ int n() const { return na + nb; }
    __device__ __forceinline__ const char* at(int slot, size_t stride) const {
        return slot < na ? a + (size_t)slot * stride : b + (size_t)(slot - na) * stride;
    }
};

__device__ __forceinline__ SlotSpan pick_slots(const Slots& sl) {
    const int p = *sl.path;
    SlotSpan r;
    r.a = p == PATH_STAGE ? sl.stage : sl.pool;
    r.na = p == PATH_POOL ? sl.npool : (p == PATH_STAGE ? sl.nstage : 0);
    r.b = sl.stage;
    r.nb = p == PATH_POOL ? sl.nmix : 0;
    return r;
}

// The wave's index in its workgroup, as a value the compiler knows is uniform
// across the wave: addresses derived from it (slot ids, buffer resources) stay in
// scalar registers instead of forcing a per-lane loop around every buffer load.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Sum over the G lanes of a group (G a power of two) of N values at once; every
// lane of the group ends with the same values, in a fixed butterfly order (G/2,
// G/4, ..., 1).  The offsets are constants and the N exchanges of a step are
// independent, so the steps' cross-lane round trips overlap instead of running one
// reduction after another (the guard on G is uniform across the wave).
template <int N>
__device__ __forceinline__ void group_sum_n(float (&v)[N], int G) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        if (off < G) {
            float o[N];
#pragma unroll
            for (int i = 0; i < N; ++i) o[i] = __shfl_xor(v[i], off, 64);
#pragma unroll
            for (int i = 0; i < N; ++i) v[i] += o[i];
        }
    }
}

// ---- activation chunks held in registers ------------------------------------
// XT_F32: fp32 values; XT_BF16: the chunk's 8 bf16 as loaded; XT_I4: pairs for
// the int4 dot (x_m, x_{m+4}) of each 8-element word, plus the chunk's sum.
enum { XT_F32 = 0, XT_BF16 = 1, XT_I4 = 2 };

template <int WT, int AT>
struct XSel {
    static constexpr int XT = (WT == W_INT4) ? XT_I4 : ((WT == W_BF16 && AT == A_BF16) ? XT_BF16 : XT_F32);
};

template <int WT, int XT>
struct XChunk;

template <int WT>
struct XChunk<WT, XT_F32> {
    static constexpr int N = WTraits<WT>::EPC;
    float v[N];
    // element e0 .. e0+N-1 of a vector of type AT, read through m (byte offsets)
    template <int AT, class M>
    __device__ __forceinline__ void load(const M& m, size_t e0) {
        if (AT == A_F32) {
#pragma unroll
            for (int q = 0; q < N / 4; ++q) {
                const uint4 f = m.ld16((e0 + 4 * q) * 4);
                v[4 * q] = __uint_as_float(f.x);
                v[4 * q + 1] = __uint_as_float(f.y);
                v[4 * q + 2] = __uint_as_float(f.z);
                v[4 * q + 3] = __uint_as_float(f.w);
            }
        } else {
#pragma unroll
            for (int q = 0; q < N / 4; ++q) {
                const uint2 u = m.ld8((e0 + 4 * q) * 2);
                v[4 * q] = bf16_lo(u.x);
                v[4 * q + 1] = bf16_hi(u.x);
                v[4 * q + 2] = bf16_lo(u.y);
                v[4 * q + 3] = bf16_hi(u.y);
            }
        }
    }
};

template <>
struct XChunk<W_BF16, XT_BF16> {
    uint4 v;
    template <int AT, class M>
    __device__ __forceinline__ void load(const M& m, size_t e0) {
        v = m.ld16(e0 * 2);
    }
};

// Activation chunks of an INT4 GEMV already repacked (XChunk<W_INT4> below) and stored
// in LDS by the workgroup, 80 bytes per 32 elements: the 16 words, then the sum.
// Element e0 of the packed vectors is chunk (e0 - e_base) / 32.
constexpr int kPackedChunkBytes = 80;
struct PackedX {
    const char* base;
    size_t e_base;
};

template <>
struct XChunk<W_INT4, XT_I4> {
    uint32_t p[16];
    float sx;
    template <int AT>
    __device__ __forceinline__ void load(const PackedX& m, size_t e0) {
        const char* d = m.base + ((e0 - m.e_base) >> 5) * kPackedChunkBytes;
        const uint4* q = reinterpret_cast<const uint4*>(d);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 v = q[i];
            p[4 * i + 0] = v.x;
            p[4 * i + 1] = v.y;
            p[4 * i + 2] = v.z;
            p[4 * i + 3] = v.w;
        }
        sx = *reinterpret_cast<const float*>(d + 64);
    }
    __device__ __forceinline__ void store_packed(char* d) const {
        uint4* q = reinterpret_cast<uint4*>(d);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = make_uint4(p[4 * i], p[4 * i + 1], p[4 * i + 2], p[4 * i + 3]);
        *reinterpret_cast<float*>(d + 64) = sx;
    }
    // the chunk's 32 bf16 activations as read (four 16-byte loads), before repacking
    struct Raw {
        uint4 u[4];
    };
    template <class M>
    __device__ __forceinline__ static Raw fetch(const M& m, size_t e0) {
        Raw r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r.u[i] = m.ld16((e0 + 8 * i) * 2);
        return r;
    }
    template <int AT, class M>
    __device__ __forceinline__ void load(const M& m, size_t e0) {
        pack(fetch(m, e0));
    }
    __device__ __forceinline__ void pack(const Raw& r) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {        // word i: elements 8i .. 8i+7
            const uint4 u = r.u[i];
            p[4 * i + 0] = (u.x & 0xFFFFu) | (u.z << 16);          // (x0, x4)
            p[4 * i + 1] = (u.x >> 16) | (u.z & 0xFFFF0000u);      // (x1, x5)
            p[4 * i + 2] = (u.y & 0xFFFFu) | (u.w << 16);          // (x2, x6)
            p[4 * i + 3] = (u.y >> 16) | (u.w & 0xFFFF0000u);      // (x3, x7)
            s += ((bf16_lo(u.x) + bf16_hi(u.x)) + (bf16_lo(u.y) + bf16_hi(u.y))) +
                 ((bf16_lo(u.z) + bf16_hi(u.z)) + (bf16_lo(u.w) + bf16_hi(u.w)));
        }
        sx = s;
    }
};

// ---- chunk dot products -------------------------------------------------------
__device__ __forceinline__ float cdot(const uint4 w, const XChunk<W_F32, XT_F32>& x) {
    float acc = __uint_as_float(w.x) * x.v[0];
    acc = fmaf(__uint_as_float(w.y), x.v[1], acc);
    acc = fmaf(__uint_as_float(w.z), x.v[2], acc);
    acc = fmaf(__uint_as_float(w.w), x.v[3], acc);
    return acc;
}

__device__ __forceinline__ float cdot(const uint4 w, const XChunk<W_BF16, XT_F32>& x) {
    float acc = bf16_lo(w.x) * x.v[0];
    acc = fmaf(bf16_hi(w.x), x.v[1], acc);
    acc = fmaf(bf16_lo(w.y), x.v[2], acc);
    acc = fmaf(bf16_hi(w.y), x.v[3], acc);
    acc = fmaf(bf16_lo(w.z), x.v[4], acc);
    acc = fmaf(bf16_hi(w.z), x.v[5], acc);
    acc = fmaf(bf16_lo(w.w), x.v[6], acc);
    acc = fmaf(bf16_hi(w.w), x.v[7], acc);
    return acc;
}

__device__ __forceinline__ float cdot(const uint4 w, const XChunk<W_BF16, XT_BF16>& x) {
    float acc = dot2_bf16(w.x, x.v.x, 0.0f);
    acc = dot2_bf16(w.y, x.v.y, acc);
    acc = dot2_bf16(w.z, x.v.z, acc);
    acc = dot2_bf16(w.w, x.v.w, acc);
    return acc;
}

__device__ __forceinline__ float cdot(const uint4 w, const XChunk<W_INT4, XT_I4>& x) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t q2 = ((ws[i] >> (4 * m)) & 0x000F000Fu) | 0x43004300u;   // (128+q_m, 128+q_{m+4})
            acc = dot2_bf16(q2, x.p[4 * i + m], acc);
        }
    }
    return acc - 136.0f * x.sx;
}

// act element type written by the w13 stage: bf16 for bf16 / int4 weights
template <int WT>
struct ActOf {
    static constexpr int AT = (WT == W_F32) ? A_F32 : A_BF16;
};

template <int AT>
__device__ __forceinline__ void store_act(void* __restrict__ p, size_t i, float v) {
    if (AT == A_F32)
        static_cast<float*>(p)[i] = v;
    else
        static_cast<uint16_t*>(p)[i] = f32_to_bf16_rne(v);
}

// ---- w13 + SwiGLU --------------------------------------------------------------
// A row's nc chunks are split over WPR waves ("parts") of G lanes (WPR > 1 only
// when G == 64), CPL chunks per lane: part q takes chunks [(q*CPL + j)*G + gl].
// A lane group covers RP gate/up row pairs.  With WPR > 1 the parts' sums meet in
// LDS (red) and are added in part order.  One call covers row block `rblk` of
// pair `pair` with the workgroup's 4 waves:
// act[pair][i] = silu(W13[s][i] . x[t]) * (W13[s][I + i] . x[t])
// G = 1 << gs lanes share a row.  The slot id and the path word are read first, side by
// side: they are the only loads the weight addresses depend on.
// MULTI (bf16 / fp32 weights, WPR == 1): `later` holds the pairs after `pair` that use
// the same slot (pair q = token q / K, k = q % K); each is computed, in pair order, from
// the weight registers of this one read, exactly as its own block would compute it.
template <int WT, int AT, int CPL, int RP, int WPR, bool MULTI = false>
__device__ __forceinline__ void w13_rows(const PairIn& pin, size_t stride, const void* __restrict__ x, int H, int I,
                                         int gs, size_t off_w, size_t off_s, void* __restrict__ act, int t, int pair,
                                         int rblk, float (*red)[2][RP], char* xs, uint64_t later = 0, int K = 1) {
    static_assert(!MULTI || (WT != W_INT4 && WPR == 1), "one read for several pairs: bf16 / fp32, one wave per row");
    using X = XChunk<WT, XSel<WT, AT>::XT>;
    constexpr int EPC = WTraits<WT>::EPC;
    constexpr int ACT = ActOf<WT>::AT;
    const int G = 1 << gs;
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int gl = lane & (G - 1);
    const int groups = 64 >> gs;
    const int grp = lane >> gs;
    const int part = wave % WPR;
    const int i0 = ((rblk * (4 / WPR) + wave / WPR) * groups + grp) * RP;
    // lane groups past the last row skip their loads; no early return, which would
    // let the compiler sink the pair's loads below it
    const bool ok = pin.valid && i0 < I;
    const int nc = CPL * G * WPR;
    const size_t row_bytes = (size_t)nc * 16;
    // INT4: this thread's activation chunk is requested before anything that depends on
    // the expert.  Loads complete in the order they are issued, so the repacking below
    // waits for these loads only, not for the weights issued after them.
    using XI4 = XChunk<W_INT4, XT_I4>;
    [[maybe_unused]] XI4::Raw xr;
    [[maybe_unused]] const int nxc = H / 32;
    if constexpr (WT == W_INT4)
        xr = XI4::fetch(PlainMem(x), (size_t)t * H + (size_t)min((int)threadIdx.x, nxc - 1) * 32);
    __builtin_amdgcn_sched_barrier(0);
    // the expert's address in scalar registers before the branch, so that the
    // arguments it needs are loaded with the others (one round trip, not two)
    const char* ebase = pin.ebase;
    __asm__ volatile("" ::"s"(ebase), "s"(stride), "s"(off_w));

    float pg[RP], pu[RP];
    if constexpr (WT == W_INT4) {
        // Every lane issues all of its weight and scale loads with no branch between them
        // and the activation loads: a lane group past the last row reads a clamped row and
        // drops the result, and a pair without a valid slot gets a buffer of length zero,
        // whose loads return zeros without touching memory.  The activation vector is then
        // repacked once per workgroup into LDS (xs) while the weights are in flight, and
        // each lane reads its chunks from there.
        const SlotReader rd(ebase, pin.valid ? stride : 0);
        uint4 wg[RP][CPL], wu[RP][CPL];
        uint16_t sg[RP][CPL], su[RP][CPL];
        const int spr = H / 128;
        uint32_t og[RP], ou[RP];   // per lane one offset per row; the chunk steps are wave-uniform
#pragma unroll
        for (int p = 0; p < RP; ++p) {
            const int i = min(i0 + p, I - 1);
            og[p] = (uint32_t)(off_w + (size_t)i * row_bytes) + (uint32_t)gl * 16u;
            ou[p] = (uint32_t)(off_w + (size_t)(I + i) * row_bytes) + (uint32_t)gl * 16u;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const uint32_t so = (uint32_t)((part * CPL + j) * G) * 16u;
                wg[p][j] = rd.load16(og[p], so);
                wu[p][j] = rd.load16(ou[p], so);
            }
        }
#pragma unroll
        for (int p = 0; p < RP; ++p) {
            const int i = min(i0 + p, I - 1);
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = (part * CPL + j) * G + gl;
                sg[p][j] = rd.scale_bits(off_s + ((size_t)i * spr + (c >> 2)) * 2);
                su[p][j] = rd.scale_bits(off_s + ((size_t)(I + i) * spr + (c >> 2)) * 2);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        {
            // every thread repacks, and the chunk's sum (which reads all of it) is taken as
            // used before the branch: the compiler would otherwise sink the activation loads
            // into the branch, after the weights, and the repacking would wait for the
            // weights too
            XI4 xc;
            xc.pack(xr);
            __asm__ volatile("" ::"v"(xc.sx));
            if ((int)threadIdx.x < nxc) xc.store_packed(xs + threadIdx.x * kPackedChunkBytes);
        }
        for (int c = threadIdx.x + blockDim.x; c < nxc; c += blockDim.x) {
            XI4 xc;
            xc.template load<AT>(PlainMem(x), (size_t)t * H + (size_t)c * 32);
            xc.store_packed(xs + c * kPackedChunkBytes);
        }
        __syncthreads();
        if (pin.to && ok) {
            // a miss read from the store: the lane writes what it read to the slot
            const SlotWriter wr(pin.to, stride);
#pragma unroll
            for (int p = 0; p < RP; ++p) {
                const int i = min(i0 + p, I - 1);
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    const int c = (part * CPL + j) * G + gl;
                    const uint32_t so = (uint32_t)((part * CPL + j) * G) * 16u;
                    wr.store16(og[p], so, wg[p][j]);
                    wr.store16(ou[p], so, wu[p][j]);
                    if ((c & 3) == 0) {
                        wr.store_scale_bits(off_s + ((size_t)i * spr + (c >> 2)) * 2, sg[p][j]);
                        wr.store_scale_bits(off_s + ((size_t)(I + i) * spr + (c >> 2)) * 2, su[p][j]);
                    }
                }
            }
        }
        // each packed chunk is read from LDS where it is used (holding all CPL of them
        // would cost 17 registers each); every row still sums its chunks in j order
#pragma unroll
        for (int p = 0; p < RP; ++p) pg[p] = pu[p] = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            X xv;
            xv.template load<AT>(PackedX{xs, (size_t)t * H}, (size_t)t * H + (size_t)((part * CPL + j) * G + gl) * EPC);
#pragma unroll
            for (int p = 0; p < RP; ++p) {
                pg[p] += cdot(wg[p][j], xv) * bf16_to_f32(sg[p][j]);
                pu[p] += cdot(wu[p][j], xv) * bf16_to_f32(su[p][j]);
            }
        }
        float gu[2 * RP];
#pragma unroll
        for (int p = 0; p < RP; ++p) {
            gu[2 * p] = pg[p];
            gu[2 * p + 1] = pu[p];
        }
        group_sum_n<2 * RP>(gu, G);
#pragma unroll
        for (int p = 0; p < RP; ++p) {
            pg[p] = gu[2 * p];
            pu[p] = gu[2 * p + 1];
        }
    } else {
        if (ok) {
            const SlotReader rd(ebase, stride);
            uint4 wg[RP][CPL], wu[RP][CPL];
            // per lane one offset per row (its gate and up rows, its first chunk); the
            // chunk steps are wave-uniform
            uint32_t og[RP], ou[RP];
#pragma unroll
            for (int p = 0; p < RP; ++p) {
                const int i = min(i0 + p, I - 1);
                og[p] = (uint32_t)(off_w + (size_t)i * row_bytes) + (uint32_t)gl * 16u;
                ou[p] = (uint32_t)(off_w + (size_t)(I + i) * row_bytes) + (uint32_t)gl * 16u;
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    const uint32_t so = (uint32_t)((part * CPL + j) * G) * 16u;
                    wg[p][j] = rd.load16(og[p], so);
                    wu[p][j] = rd.load16(ou[p], so);
                }
            }
            float sg[RP][CPL], su[RP][CPL];
            if (WT == W_INT4) {
                const int spr = H / 128;
#pragma unroll
                for (int p = 0; p < RP; ++p) {
                    const int i = min(i0 + p, I - 1);
#pragma unroll
                    for (int j = 0; j < CPL; ++j) {
                        const int c = (part * CPL + j) * G + gl;
                        sg[p][j] = rd.scale(off_s + ((size_t)i * spr + (c >> 2)) * 2);
                        su[p][j] = rd.scale(off_s + ((size_t)(I + i) * spr + (c >> 2)) * 2);
                    }
                }
            }
            X xv[CPL];
#pragma unroll
            for (int j = 0; j < CPL; ++j)
                xv[j].template load<AT>(PlainMem(x), (size_t)t * H + (size_t)((part * CPL + j) * G + gl) * EPC);
            // every load of the lane is in flight before the first use: the scheduler
            // would otherwise hold some back to save registers (two round trips)
            __builtin_amdgcn_sched_barrier(0);
            if (pin.to) {
                // a miss read from the store: the lane writes what it read to the slot
                const SlotWriter wr(pin.to, stride);
#pragma unroll
                for (int p = 0; p < RP; ++p) {
#pragma unroll
                    for (int j = 0; j < CPL; ++j) {
                        const uint32_t so = (uint32_t)((part * CPL + j) * G) * 16u;
                        wr.store16(og[p], so, wg[p][j]);
                        wr.store16(ou[p], so, wu[p][j]);
                    }
                }
                if (WT == W_INT4) {
                    const int spr = H / 128;
#pragma unroll
                    for (int p = 0; p < RP; ++p) {
                        const int i = min(i0 + p, I - 1);
#pragma unroll
                        for (int j = 0; j < CPL; ++j) {
                            const int c = (part * CPL + j) * G + gl;
                            if ((c & 3) == 0) {
                                wr.store_scale(off_s + ((size_t)i * spr + (c >> 2)) * 2, sg[p][j]);
                                wr.store_scale(off_s + ((size_t)(I + i) * spr + (c >> 2)) * 2, su[p][j]);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int p = 0; p < RP; ++p) {
                float a = 0.0f, b = 0.0f;
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    float dg = cdot(wg[p][j], xv[j]);
                    float du = cdot(wu[p][j], xv[j]);
                    if (WT == W_INT4) {
                        dg *= sg[p][j];
                        du *= su[p][j];
                    }
                    a += dg;
                    b += du;
                }
                pg[p] = a;
                pu[p] = b;
            }
            float gu[2 * RP];
#pragma unroll
            for (int p = 0; p < RP; ++p) {
                gu[2 * p] = pg[p];
                gu[2 * p + 1] = pu[p];
            }
            group_sum_n<2 * RP>(gu, G);
#pragma unroll
            for (int p = 0; p < RP; ++p) {
                pg[p] = gu[2 * p];
                pu[p] = gu[2 * p + 1];
            }
            if constexpr (MULTI) {
                for (uint64_t m = later; m; m &= m - 1) {
                    const int q = __builtin_ctzll(m);
                    const int tq = q / K;
#pragma unroll
                    for (int j = 0; j < CPL; ++j)
                        xv[j].template load<AT>(PlainMem(x), (size_t)tq * H + (size_t)((part * CPL + j) * G + gl) * EPC);
                    float hq[2 * RP];
#pragma unroll
                    for (int p = 0; p < RP; ++p) {
                        float a = 0.0f, b = 0.0f;
#pragma unroll
                        for (int j = 0; j < CPL; ++j) {
                            a += cdot(wg[p][j], xv[j]);
                            b += cdot(wu[p][j], xv[j]);
                        }
                        hq[2 * p] = a;
                        hq[2 * p + 1] = b;
                    }
                    group_sum_n<2 * RP>(hq, G);
                    if (gl == 0)
#pragma unroll
                        for (int p = 0; p < RP; ++p)
                            if (i0 + p < I) store_act<ACT>(act, (size_t)q * I + i0 + p, silu(hq[2 * p]) * hq[2 * p + 1]);
                }
            }
        } else {
#pragma unroll
            for (int p = 0; p < RP; ++p) pg[p] = pu[p] = 0.0f;
        }
    }
    if (WPR > 1) {
        if (lane == 0)
#pragma unroll
            for (int p = 0; p < RP; ++p) {
                red[wave][0][p] = pg[p];
                red[wave][1][p] = pu[p];
            }
        __syncthreads();
        if (part != 0) return;
#pragma unroll
        for (int p = 0; p < RP; ++p) {
            float a = 0.0f, b = 0.0f;
            for (int q = 0; q < WPR; ++q) {
                a += red[wave + q][0][p];
                b += red[wave + q][1][p];
            }
            pg[p] = a;
            pu[p] = b;
        }
    }
    if (gl == 0)
#pragma unroll
        for (int p = 0; p < RP; ++p)
            if (i0 + p < I) store_act<ACT>(act, (size_t)pair * I + i0 + p, ok ? silu(pg[p]) * pu[p] : 0.0f);
}

// grid.x: row blocks; grid.y: k; grid.z: tokens.
template <int WT, int AT, int CPL, int RP, int WPR>
__global__ __launch_bounds__(256) void k_w13_gemv(Slots sl, size_t stride, const int32_t* __restrict__ slot_ids,
                                                  const void* __restrict__ x, int H, int I, int gs,
                                                  size_t off_w, size_t off_s, void* __restrict__ act) {
    __shared__ float red[4][2][RP];
    extern __shared__ __attribute__((aligned(16))) char xs_packed[];   // INT4: the packed activations
    // the slot id and the path word, side by side before any branch: they are the only
    // loads the weight addresses depend on
    const int pair = blockIdx.z * gridDim.y + blockIdx.y;
    const int slot = slot_ids[pair];
    const SlotSpan sp = pick_slots(sl);
    const bool valid = slot >= 0 && slot < sp.n();
    const PairIn pin{valid ? sp.at(slot, stride) : sp.a, nullptr, valid};
    if constexpr (WT != W_INT4 && WPR == 1) {
        // several tokens (at most 64 pairs): the block of the first pair on a slot computes
        // every pair on it from one read of its rows; the other blocks on it have no work
        const int TK = (int)(gridDim.y * gridDim.z);
        if (gridDim.z > 1 && TK <= 64 && valid) {
            const int lane = threadIdx.x & 63;
            const int sq = slot_ids[min(lane, TK - 1)];
            const uint64_t same = __ballot(lane < TK && sq == slot);
            if (same & ((1ull << pair) - 1)) return;
            const uint64_t later = pair == 63 ? 0 : same & (~0ull << (pair + 1));
            w13_rows<WT, AT, CPL, RP, WPR, true>(pin, stride, x, H, I, gs, off_w, off_s, act, blockIdx.z, pair,
                                                 blockIdx.x, red, xs_packed, later, (int)gridDim.y);
            return;
        }
    }
    w13_rows<WT, AT, CPL, RP, WPR>(pin, stride, x, H, I, gs, off_w, off_s, act, blockIdx.z, pair, blockIdx.x, red,
                                   xs_packed);
}

// INT4 w13 with a row's gate and up halves on two neighbouring lane groups (G <= 32
// lanes each) instead of one: twice the waves for the same bytes, so more loads are in
// flight per SIMD at batch 1.  Each group sums its row's chunks in chunk order and
// butterflies over its G lanes exactly as w13_rows does for the gate and up sums, the
// gate group takes the up sum from its neighbour (lane + G), and the result has the
// same bits as w13_rows'.  grid.x: blocks of 4 * (32 / G) rows; grid.y: k; grid.z: tokens.
template <int AT, int CPL>
__global__ __launch_bounds__(256) void k_w13_i4s(Slots sl, size_t stride, const int32_t* __restrict__ slot_ids,
                                                 const void* __restrict__ x, int H, int I, int gs, size_t off_w,
                                                 size_t off_s, void* __restrict__ act) {
    using X = XChunk<W_INT4, XSel<W_INT4, AT>::XT>;
    using XI4 = XChunk<W_INT4, XT_I4>;
    constexpr int EPC = WTraits<W_INT4>::EPC;
    extern __shared__ __attribute__((aligned(16))) char xs[];   // the packed activations
    const int t = blockIdx.z;
    const int pair = blockIdx.z * gridDim.y + blockIdx.y;
    const int slot = slot_ids[pair];
    const SlotSpan sp = pick_slots(sl);
    const bool valid = slot >= 0 && slot < sp.n();
    const char* ebase = valid ? sp.at(slot, stride) : sp.a;
    const int G = 1 << gs;
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int gl = lane & (G - 1);
    const int grp = lane >> gs;
    const int half = grp & 1;                       // 0: the gate row, 1: the up row
    const int i0 = ((int)blockIdx.x * 4 + wave) * (32 >> gs) + (grp >> 1);
    const bool ok = valid && i0 < I;
    const int nxc = H / 32;
    // the activation chunk first (see w13_rows)
    const XI4::Raw xr = XI4::fetch(PlainMem(x), (size_t)t * H + (size_t)min((int)threadIdx.x, nxc - 1) * 32);
    __builtin_amdgcn_sched_barrier(0);
    __asm__ volatile("" ::"s"(ebase), "s"(stride), "s"(off_w));
    const SlotReader rd(ebase, valid ? stride : 0);
    const size_t row_bytes = (size_t)CPL * G * 16;
    const int wrow = (half ? I : 0) + min(i0, I - 1);
    const uint32_t ow = (uint32_t)(off_w + (size_t)wrow * row_bytes) + (uint32_t)gl * 16u;
    const int spr = H / 128;
    uint4 w[CPL];
    uint16_t sc[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) w[j] = rd.load16(ow, (uint32_t)(j * G) * 16u);
#pragma unroll
    for (int j = 0; j < CPL; ++j) sc[j] = rd.scale_bits(off_s + ((size_t)wrow * spr + ((j * G + gl) >> 2)) * 2);
    __builtin_amdgcn_sched_barrier(0);
    {
        XI4 xc;
        xc.pack(xr);
        __asm__ volatile("" ::"v"(xc.sx));
        if ((int)threadIdx.x < nxc) xc.store_packed(xs + threadIdx.x * kPackedChunkBytes);
    }
    for (int c = threadIdx.x + blockDim.x; c < nxc; c += blockDim.x) {
        XI4 xc;
        xc.template load<AT>(PlainMem(x), (size_t)t * H + (size_t)c * 32);
        xc.store_packed(xs + c * kPackedChunkBytes);
    }
    __syncthreads();
    float v[1] = {0.0f};
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        X xv;
        xv.template load<AT>(PackedX{xs, (size_t)t * H}, (size_t)t * H + (size_t)(j * G + gl) * EPC);
        v[0] += cdot(w[j], xv) * bf16_to_f32(sc[j]);
    }
    group_sum_n<1>(v, G);
    const float up = __shfl_xor(v[0], G, 64);
    if (gl == 0 && half == 0 && i0 < I)
        store_act<ActOf<W_INT4>::AT>(act, (size_t)pair * I + i0, ok ? silu(v[0]) * up : 0.0f);
}

// ---- the fused one-token decode step: decision + w13 + tail copies ----------------------
// Workgroup roles by index: 0 = the lead (the decision, the state after the step, the
// counters, the step's slot ids and path word); 1 .. n_copy = copy workers (the part
// of each missed or staged expert from its w2 region on: store -> slot or staging);
// the rest = the w13 GEMV blocks (row block, k).  Every workgroup first reads the
// step's ids and their entries in the current map: when each id is valid and
// resident (and the static rule does not fire) every id hits, the map stays as it is
// and the GEMV blocks start at once from it; otherwise every workgroup runs the
// decision on its own LDS copy of the state.  A missed expert's w13 rows are read
// from the pinned store and written through to its slot by the GEMV blocks that use
// them; a staged expert's are read from the store.  No workgroup waits for another.
template <int WT, int AT, int CPL, int RP, int WPR>
__global__ __launch_bounds__(256) void k_step_w13(PolicyArgs pa, size_t stride, const void* __restrict__ x, int H,
                                                  int I, int gs, size_t off_w, size_t off_s, size_t tail_off,
                                                  void* __restrict__ act, int n_copy, int nrb, int xs_off) {
    extern __shared__ __attribute__((aligned(16))) char dyn[];
    __shared__ float red[4][2][RP];
    const int b = blockIdx.x;
    const int K = pa.n;                    // one token: n == top_k
    const int tid = threadIdx.x;
    const int E = pa.E, N = pa.N;
    // the slot base with the first kernel-argument loads, not after the lookups below
    __asm__ volatile("" ::"s"(pa.slots));
    const bool lead = b == 0;
    const int g = b - 1 - n_copy;              // GEMV block index (when >= 0)
    const int k = max(g, 0) / nrb;             // (no branch before the loads below)
    const int rblk = g - k * nrb;
    // The step's ids and their entries in the current map, through the scalar cache
    // (uniform addresses; neither the ids, the control word nor the current copy's map
    // is written during this launch): the control word is read with the first eight
    // ids and the copy picked from the kernel arguments, so that the chain before the
    // weight loads is arguments -> ids -> map.  Eight ids per round, with no branch
    // between the loads of a round.
    typedef const __attribute__((address_space(4))) int32_t cint4;
    cint4* ids4 = (cint4*)pa.ids;
    int bad = 0, myslot = -1;
    auto load_ids = [&](int k0, int (&idv)[8]) {
#pragma unroll
        for (int q = 0; q < 8; ++q) idv[q] = ids4[min(k0 + q, K - 1)];
    };
    auto lookup = [&](cint4* map4, int k0, const int (&idv)[8]) {
        int mv[8], nres = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const bool ok = (unsigned)idv[q] < (unsigned)E;
            bad |= !ok;
            mv[q] = map4[ok ? idv[q] : 0];      // (also in the all-resident mode: a select, not a branch)
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int m = pa.resident ? idv[q] : mv[q];
            nres |= m;
            myslot = k0 + q == k ? m : myslot;
        }
        bad |= nres < 0;                         // some entry was -1 (not resident)
    };
    int id0[8];
    load_ids(0, id0);
    const int par = *(cint4*)pa.ds.ctl & 1;
    char* cur_base = par ? pa.ds.copy[1] : pa.ds.copy[0];
    cint4* map4 = (cint4*)(cur_base + slot_state_layout(E, N).map);
    lookup(map4, 0, id0);
    for (int k0 = 8; k0 < K; k0 += 8) {
        int idn[8];
        load_ids(k0, idn);
        lookup(map4, k0, idn);
    }
    const bool fast = !bad && (pa.resident || pa.rule == 0 || K <= N);
    if (g >= 0 && fast) {
        // every id hits: the map stays as it is, and this block's expert is at myslot
        const PairIn pin{pa.slots + (size_t)myslot * stride, nullptr, true};
        w13_rows<WT, AT, CPL, RP, WPR>(pin, stride, x, H, I, gs, off_w, off_s, act, 0, k, rblk, red, dyn + xs_off);
        return;
    }
    if (lead && fast && !pa.resident && pa.evict != EVICT_SLRU) {
        // an all-hit step changes keys only: in place, and the copies keep their roles
        pol_hit_in_place(pa, slot_view(cur_base, E, N), K);
        return;
    }
    const PolLds L = pol_lds(reinterpret_cast<int32_t*>(dyn), E, N, pa.evict);
    Decision d{};
    if (lead || !fast) d = pol_decide(pa, slot_view(cur_base, E, N), L);
    // (the w2 launch that follows makes the lead's copy current, ctl[2] = 1: every read
    // of the current copy is in this launch)
    if (lead) {
        pol_publish(pa, slot_view(pa.ds.copy[par ^ 1], E, N), L, d);
        if (tid == 0) pa.ds.ctl[2] = 1;
        if (tid < K) {
            const int id = pa.ids[tid];
            int v = -1;
            if (d.path == PATH_POOL) v = pa.resident ? id : L.map[id];
            else if (d.path == PATH_STAGE) v = L.rank[id];
            pa.out[tid] = v;
        }
        return;
    }
    if (b <= n_copy) {
        if (fast || pa.resident || d.path == PATH_NONE) return;
        const bool pool = d.path == PATH_POOL;
        const int njobs = pool ? d.nmiss : d.D;
        const size_t eb = pa.eb;
        constexpr size_t kUnit = (size_t)64 << 10;
        const size_t upj = (eb - tail_off + kUnit - 1) / kUnit;
        const size_t units = upj * (size_t)njobs;
        typedef unsigned int u32x4c __attribute__((ext_vector_type(4)));
        for (size_t u = (size_t)(b - 1); u < units; u += (size_t)n_copy) {
            const int j = (int)(u / upj);
            const int e = L.list[j];
            const size_t off = tail_off + (u - (size_t)j * upj) * kUnit;
            const size_t nvec = (eb - off < kUnit ? eb - off : kUnit) / 16;
            const u32x4c* __restrict__ s4 = reinterpret_cast<const u32x4c*>(pol_src(pa, e) + off);
            u32x4c* __restrict__ d4 =
                reinterpret_cast<u32x4c*>((pool ? pa.slots + (size_t)L.map[e] * eb : pa.staging + (size_t)j * eb) + off);
            for (size_t i0 = tid; i0 < nvec; i0 += 4 * 256) {
                u32x4c v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const size_t i = i0 + (size_t)q * 256;
                    if (i < nvec) v[q] = s4[i];
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const size_t i = i0 + (size_t)q * 256;
                    if (i < nvec) __builtin_nontemporal_store(v[q], d4 + i);
                }
            }
        }
        return;
    }
    const int e = ids4[k];
    PairIn pin{pa.slots, nullptr, false};
    if (d.path == PATH_POOL) {
        const int slot = __builtin_amdgcn_readfirstlane(pa.resident ? e : L.map[e]);
        const bool miss = !pa.resident && __builtin_amdgcn_readfirstlane(L.rank[e]) < 0;
        pin = miss ? PairIn{pol_src(pa, e), pa.slots + (size_t)slot * stride, true}
                   : PairIn{pa.slots + (size_t)slot * stride, nullptr, true};
    } else if (d.path == PATH_STAGE) {
        pin = PairIn{pol_src(pa, e), nullptr, true};
    }
    w13_rows<WT, AT, CPL, RP, WPR>(pin, stride, x, H, I, gs, off_w, off_s, act, 0, k, rblk, red, dyn + xs_off);
}

// ---- w2 + ordered top-k combine ------------------------------------------------
// A workgroup owns RB = RP * (64 / G) output rows of one token.  Its waves take the
// K * WPR (expert, part) tasks in turn: y_k[r] = W2[s_k][r] . act[t*K + k] (part
// sums) goes to LDS, then
// out[t][r] = resid[t][r] + sum_{k = 0..K-1} w[t][k] * y_k[r]   (k in order).
// A task is split into its weight fetch (which does not depend on act) and the
// rest, so that the weight loads are in flight while the workgroup repacks act.

// Weight registers of one (expert, part) task of a lane: RP rows x CPL chunks.
template <int WT, int CPL, int RP>
struct W2Task {
    uint4 w[RP][CPL];
    uint16_t sc[RP][CPL];   // int4 group scales, bf16 bits (unused otherwise)
    int pair;            // t * K + k
    int part;
    bool ok;             // the pair's slot id is valid
};

// Lane geometry of a w2 workgroup.
struct W2Lane {
    int gl, grp, RB, r0;
};

__device__ __forceinline__ W2Lane w2_lane(int gs, int RP, int rb0) {
    const int lane = threadIdx.x & 63;
    W2Lane g;
    g.gl = lane & ((1 << gs) - 1);
    g.grp = lane >> gs;
    g.RB = RP * (64 >> gs);
    g.r0 = rb0 + g.grp * RP;
    return g;
}

// `slot` is slot_ids[t * K + task / WPR], loaded by the caller (so that it can be
// read together with the path word, before any branch).  INT4 tasks issue their loads
// with no branch even for an invalid slot (a buffer of length zero, whose loads return
// zeros without touching memory), so that a caller's activation loads issued earlier
// can be waited for alone.
template <int WT, int CPL, int RP, int WPR>
__device__ __forceinline__ void w2_fetch(W2Task<WT, CPL, RP>& tk, const SlotSpan& sp, size_t stride,
                                         int slot, int t, int K, int H, int I, int gs,
                                         const W2Lane& ln, int task, size_t off_w, size_t off_s) {
    const int G = 1 << gs;
    const int k = task / WPR;
    tk.part = task - k * WPR;
    tk.pair = t * K + k;
    tk.ok = slot >= 0 && slot < sp.n();
    const char* ebase = tk.ok ? sp.at(slot, stride) : sp.a;
    __asm__ volatile("" ::"s"(ebase), "s"(stride), "s"(off_w));
    if (WT != W_INT4 && !tk.ok) return;
    const size_t row_bytes = (size_t)CPL * G * WPR * 16;
    const int spr = I / 128;
    const SlotReader rd(ebase, tk.ok ? stride : 0);
#pragma unroll
    for (int p = 0; p < RP; ++p) {
        const size_t row = off_w + (size_t)min(ln.r0 + p, H - 1) * row_bytes;
#pragma unroll
        for (int j = 0; j < CPL; ++j) tk.w[p][j] = rd.load16(row + (size_t)((tk.part * CPL + j) * G + ln.gl) * 16);
    }
    if (WT == W_INT4) {
#pragma unroll
        for (int p = 0; p < RP; ++p)
#pragma unroll
            for (int j = 0; j < CPL; ++j)
                tk.sc[p][j] = rd.scale_bits(off_s + ((size_t)min(ln.r0 + p, H - 1) * spr +
                                                     (((tk.part * CPL + j) * G + ln.gl) >> 2)) * 2);
    }
}

// The dot products of a fetched task against its act row (read through m); the
// RP results go to ys[task][grp * RP + p].
template <int WT, int CPL, int RP, int WPR, class M>
__device__ __forceinline__ void w2_finish(const W2Task<WT, CPL, RP>& tk, const M& m, int H, int I, int gs,
                                          const W2Lane& ln, size_t stride, size_t off_w, size_t off_s,
                                          float* __restrict__ yk) {
    const int G = 1 << gs;
    constexpr int ACT = ActOf<WT>::AT;
    using X = XChunk<WT, XSel<WT, ACT>::XT>;
    constexpr int EPC = WTraits<WT>::EPC;
    if (!tk.ok) {
        if (ln.gl == 0)
            for (int p = 0; p < RP; ++p) yk[p] = 0.0f;
        return;
    }
    // activations read from global memory are all requested before the first use; packed
    // ones (LDS) are read where they are used, which saves their registers
    constexpr bool kLds = std::is_same<M, PackedX>::value;
    X av[kLds ? 1 : CPL];
    if constexpr (!kLds) {
#pragma unroll
        for (int j = 0; j < CPL; ++j)
            av[j].template load<ACT>(m, (size_t)tk.pair * I + (size_t)((tk.part * CPL + j) * G + ln.gl) * EPC);
    }
    __builtin_amdgcn_sched_barrier(0);
    float acc[RP];
#pragma unroll
    for (int p = 0; p < RP; ++p) acc[p] = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        if constexpr (kLds)
            av[0].template load<ACT>(m, (size_t)tk.pair * I + (size_t)((tk.part * CPL + j) * G + ln.gl) * EPC);
        const X& a = av[kLds ? 0 : j];
#pragma unroll
        for (int p = 0; p < RP; ++p) {
            float d = cdot(tk.w[p][j], a);
            if (WT == W_INT4) d *= bf16_to_f32(tk.sc[p][j]);
            acc[p] += d;
        }
    }
    group_sum_n<RP>(acc, G);
    if (ln.gl == 0)
#pragma unroll
        for (int p = 0; p < RP; ++p) yk[p] = acc[p];
}

// The ordered top-k sum of the workgroup's RB rows (after a barrier on ys).
template <int AT>
__device__ __forceinline__ void w2_combine(const float* __restrict__ ys, int RB, int WPR, int rb0, int t, int K,
                                           int H, const float* __restrict__ topk_w, const void* __restrict__ resid,
                                           void* __restrict__ out) {
    const float* wt = topk_w + (size_t)t * K;
    for (int i = threadIdx.x; i < RB; i += blockDim.x) {
        const int r = rb0 + i;
        if (r >= H) continue;
        float acc = 0.0f;
        for (int k = 0; k < K; ++k) {
            float y = 0.0f;
            for (int q = 0; q < WPR; ++q) y += ys[(size_t)(k * WPR + q) * RB + i];
            acc = fmaf(wt[k], y, acc);
        }
        const size_t o = (size_t)t * H + r;
        if (resid) acc += load_act<AT>(resid, o);
        if (AT == A_F32)
            static_cast<float*>(out)[o] = acc;
        else
            static_cast<uint16_t*>(out)[o] = f32_to_bf16_rne(acc);
    }
}

// grid.x: blocks of RB output rows; grid.y: tokens.  ONE: the block has one wave
// per (expert, part) task (K * WPR <= NWMAX), so a wave's slot is known before any
// branch.  xcd_T > 1 (several tokens, row blocks a multiple of 8): a 1-D grid in which
// the blocks of one row block for tokens 0..T-1 are 8 apart, so they run on the same
// XCD one after another and an expert shared by several tokens is served from that
// XCD's L2 after its first read (workgroups go to the 8 XCDs round robin).
template <int WT, int AT, int CPL, int RP, int WPR, int NWMAX, bool ONE>
__global__ __launch_bounds__(NWMAX * 64) void k_w2_combine(Slots sl, size_t stride,
                                                           const int32_t* __restrict__ slot_ids,
                                                           const float* __restrict__ topk_w,
                                                           const void* __restrict__ act,
                                                           const void* __restrict__ resid, void* __restrict__ out,
                                                           int K, int H, int I, int gs, size_t off_w, size_t off_s,
                                                           int32_t* __restrict__ flip, int xcd_T) {
    extern __shared__ float ys[];               // [K][WPR][RB]
    int bx = blockIdx.x, t = blockIdx.y;
    if (xcd_T > 1) {
        const int j = (int)blockIdx.x >> 3;
        t = j % xcd_T;
        bx = (j / xcd_T) * 8 + ((int)blockIdx.x & 7);
    }
    // after a fused step whose lead wrote the other state copy (ctl[2]): that copy becomes
    // current (nothing here reads the state)
    if (flip && bx == 0 && t == 0 && threadIdx.x == 0 && flip[2]) flip[0] ^= 1;
    const int nw = blockDim.x >> 6;
    const int wave = wave_id();
    const W2Lane ln = w2_lane(gs, RP, bx * (RP * (64 >> gs)));
    const int rb0 = bx * ln.RB;
    if (ONE) {
        // the wave's slot and the path word, side by side, before any branch
        const int slot = slot_ids[t * K + wave / WPR];
        const SlotSpan sp = pick_slots(sl);
        // INT4: the token's K act vectors are repacked once per workgroup (each lane
        // would otherwise repack every chunk it uses).  A thread's first chunk is
        // requested before the weights, so that the repacking waits for it alone.
        using XI4 = XChunk<W_INT4, XT_I4>;
        [[maybe_unused]] XI4::Raw xr;
        [[maybe_unused]] const int nxc = K * (I >> 5);
        [[maybe_unused]] const size_t e0 = (size_t)t * K * I;
        if constexpr (WT == W_INT4)
            xr = XI4::fetch(PlainMem(act), e0 + (size_t)min((int)threadIdx.x, nxc - 1) * 32);
        __builtin_amdgcn_sched_barrier(0);
        W2Task<WT, CPL, RP> tk;
        w2_fetch<WT, CPL, RP, WPR>(tk, sp, stride, slot, t, K, H, I, gs, ln, wave, off_w, off_s);
        if constexpr (WT == W_INT4) {
            __builtin_amdgcn_sched_barrier(0);
            char* xs = reinterpret_cast<char*>(ys) + ((K * WPR * ln.RB * 4 + 15) & ~15);
            if ((int)threadIdx.x < nxc) {
                XI4 xc;
                xc.pack(xr);
                xc.store_packed(xs + threadIdx.x * kPackedChunkBytes);
            }
            for (int c = threadIdx.x + blockDim.x; c < nxc; c += blockDim.x) {
                XI4 xc;
                xc.template load<A_BF16>(PlainMem(act), e0 + (size_t)c * 32);
                xc.store_packed(xs + c * kPackedChunkBytes);
            }
            __syncthreads();
            w2_finish<WT, CPL, RP, WPR>(tk, PackedX{xs, e0}, H, I, gs, ln, stride, off_w, off_s,
                                        ys + (size_t)wave * ln.RB + ln.grp * RP);
        } else {
            w2_finish<WT, CPL, RP, WPR>(tk, PlainMem(act), H, I, gs, ln, stride, off_w, off_s,
                                        ys + (size_t)wave * ln.RB + ln.grp * RP);
        }
    } else {
        const SlotSpan sp = pick_slots(sl);
        for (int task = wave; task < K * WPR; task += nw) {
            W2Task<WT, CPL, RP> tk;
            w2_fetch<WT, CPL, RP, WPR>(tk, sp, stride, slot_ids[t * K + task / WPR], t, K, H, I, gs, ln,
                                       task, off_w, off_s);
            w2_finish<WT, CPL, RP, WPR>(tk, PlainMem(act), H, I, gs, ln, stride, off_w, off_s,
                                        ys + (size_t)task * ln.RB + ln.grp * RP);
        }
    }
    __syncthreads();
    w2_combine<AT>(ys, ln.RB, WPR, rb0, t, K, H, topk_w, resid, out);
}

// ---------------------------------------------------------------------------
// Grouped path (n_tokens above the decode limit, bf16 weights): the (token, k)
// pairs are grouped by slot, and each slot's group runs as a dense bf16 GEMM on
// the matrix cores against that slot's weights, read once per 32-row tile.
// ---------------------------------------------------------------------------
constexpr int kGroupThreads = 1024;
constexpr int kGBM = 32;        // rows of one 32x32 MFMA block; a tile has kGBM * MT rows
constexpr int kGBN = 128;       // output columns per workgroup: 4 waves x 32

// a6: per-slot counts, exclusive offsets, slot-sorted pair list and the tile list.
// grp layout (int32): [0] = n_tiles; [16 + t] = slot of tile t;
// [16 + S + t] = first sorted row of tile t; [16 + 2S + t] = rows in tile t;
// [16 + 3S + pos] = pair index at sorted position pos   (S = tile stride).
// A tile has at most `tile_rows` rows (a multiple of 32: the grouped GEMMs give each
// wave tile_rows / 32 blocks of 32 rows against the same weight loads).
// Pairs of one slot are contiguous; their order inside the group is unspecified
// (each GEMM row depends only on its own inputs, so results do not depend on it).
__global__ __launch_bounds__(kGroupThreads) void k_group_build(Slots sl, const int32_t* __restrict__ slot_ids,
                                                               int n, int tile_stride, int tile_rows,
                                                               int32_t* __restrict__ grp) {
    const int nslots = pick_slots(sl).n();
    __shared__ int32_t cnt[kMaxExperts];
    __shared__ int32_t off[kMaxExperts];
    __shared__ int32_t toff[kMaxExperts];
    __shared__ int32_t wsum[2][kGroupThreads / 64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    for (int i = tid; i < nslots; i += kGroupThreads) cnt[i] = 0;
    __syncthreads();
    for (int p = tid; p < n; p += kGroupThreads) {
        const int sl = slot_ids[p];
        if (sl >= 0 && sl < nslots) atomicAdd(&cnt[sl], 1);
    }
    __syncthreads();
    // exclusive scans of counts and tile counts; thread tid owns slots 4*tid .. 4*tid+3
    int c[4], tc[4], sc = 0, st = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int sl = 4 * tid + i;
        c[i] = sl < nslots ? cnt[sl] : 0;
        tc[i] = (c[i] + tile_rows - 1) / tile_rows;
        sc += c[i];
        st += tc[i];
    }
    int ic = sc, it = st;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int vc = __shfl_up(ic, o, 64);
        const int vt = __shfl_up(it, o, 64);
        if (lane >= o) {
            ic += vc;
            it += vt;
        }
    }
    if (lane == 63) {
        wsum[0][wave] = ic;
        wsum[1][wave] = it;
    }
    __syncthreads();
    int pc = 0, pt = 0, total_t = 0;
    for (int w = 0; w < kGroupThreads / 64; ++w) {
        if (w < wave) {
            pc += wsum[0][w];
            pt += wsum[1][w];
        }
        total_t += wsum[1][w];
    }
    int ec = pc + ic - sc, et = pt + it - st;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int sl = 4 * tid + i;
        if (sl < nslots) {
            off[sl] = ec;
            toff[sl] = et;
        }
        ec += c[i];
        et += tc[i];
    }
    if (tid == 0) grp[0] = total_t;
    __syncthreads();
    int32_t* t_slot = grp + 16;
    int32_t* t_row0 = grp + 16 + tile_stride;
    int32_t* t_rows = grp + 16 + 2 * tile_stride;
    int32_t* perm = grp + 16 + 3 * tile_stride;
    for (int sl = tid; sl < nslots; sl += kGroupThreads) {
        const int cs = cnt[sl];
        for (int j = 0; j * tile_rows < cs; ++j) {
            const int t = toff[sl] + j;
            t_slot[t] = sl;
            t_row0[t] = off[sl] + j * tile_rows;
            t_rows[t] = min(tile_rows, cs - j * tile_rows);
        }
    }
    __syncthreads();
    for (int i = tid; i < nslots; i += kGroupThreads) cnt[i] = 0;
    __syncthreads();
    for (int p = tid; p < n; p += kGroupThreads) {
        const int sl = slot_ids[p];
        if (sl >= 0 && sl < nslots) perm[off[sl] + atomicAdd(&cnt[sl], 1)] = p;
    }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_t mfma_32x32x16(const uint4 a, const uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                    c, 0, 0, 0);
}

// 8 bf16 activations at element e0 of an fp32 or bf16 row, as MFMA operand bits
template <int AT>
__device__ __forceinline__ uint4 load_a8(const void* __restrict__ p, size_t e0) {
    if (AT == A_BF16) return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + e0);
    const float4* f = reinterpret_cast<const float4*>(static_cast<const float*>(p) + e0);
    const float4 a = f[0], b = f[1];
    uint4 r;
    r.x = (uint32_t)f32_to_bf16_rne(a.x) | ((uint32_t)f32_to_bf16_rne(a.y) << 16);
    r.y = (uint32_t)f32_to_bf16_rne(a.z) | ((uint32_t)f32_to_bf16_rne(a.w) << 16);
    r.z = (uint32_t)f32_to_bf16_rne(b.x) | ((uint32_t)f32_to_bf16_rne(b.y) << 16);
    r.w = (uint32_t)f32_to_bf16_rne(b.z) | ((uint32_t)f32_to_bf16_rne(b.w) << 16);
    return r;
}

// One wave computes a 32 x 32 block C = A (32 rows x Kd) . B^T (32 weight rows x Kd)
// with B rows streamed from HBM straight into operand registers.  The k range is
// walked in spans of 64: lane half h (= lane / 32) supplies elements
// [span + 32h + 8j, +8) of its row to MFMA j (j = 0..3), for A and B alike, so each
// lane reads 64 contiguous bytes of its row per span and the four MFMAs together
// cover the span once.
// ---- staged activation tiles ---------------------------------------------------------
// The grouped GEMMs stage the tile's rows of activations in LDS, 64 elements (one k
// span) at a time, double-buffered: all 256 threads load the next span (two threads
// per row, 32 elements each) while the MFMAs read the current one, and the four waves
// of a workgroup share it instead of each loading its own copy.  Rows are padded to
// 144 bytes so that the 32 rows read by one MFMA operand load spread over the banks.
constexpr int kARowBytes = 144;

// A thread's share of a staged row: 32 bf16 (64 bytes), kept as four named
// registers (as an array the compiler left it in scratch memory).
struct Row32 {
    uint4 q0, q1, q2, q3;
};
template <int AT>
__device__ __forceinline__ Row32 load_row32(const void* __restrict__ p, size_t e0) {
    return Row32{load_a8<AT>(p, e0), load_a8<AT>(p, e0 + 8), load_a8<AT>(p, e0 + 16), load_a8<AT>(p, e0 + 24)};
}
__device__ __forceinline__ void store_row32(char* d, const Row32& r) {
    uint4* q = reinterpret_cast<uint4*>(d);
    q[0] = r.q0;
    q[1] = r.q1;
    q[2] = r.q2;
    q[3] = r.q3;
}

// One MFMA operand (8 bf16) of row `row`, elements [hl * 32 + 8 j, +8) of the span.
__device__ __forceinline__ uint4 lds_a8(const char* buf, int row, int hl, int j) {
    return *reinterpret_cast<const uint4*>(buf + row * kARowBytes + hl * 64 + 16 * j);
}

// ---- grouped w13 + SwiGLU ------------------------------------------------------
// grid.x: tiles (blocks past n_tiles exit); grid.y: blocks of 128 columns of I.
// act_sorted[pos][j] = silu(x[t(pos)] . W13[s][j]) * (x[t(pos)] . W13[s][I + j])
// A wave owns 32 columns of the gate and of the up half for the tile's MT blocks of
// 32 rows: every weight chunk it loads feeds MT MFMAs (blocks past the tile's rows
// are skipped; rows past the end repeat the last row and are never stored).
// (256, 2): two waves per SIMD; the accumulators then stay in VGPRs (no AGPRs)
// and the MT = 4 kernel fits without spilling.
template <int AT, int MT>
__global__ __launch_bounds__(256, 2) void k_grouped_w13(Slots sl, size_t stride,
                                                     const int32_t* __restrict__ grp, int tile_stride,
                                                     const void* __restrict__ x, int K, int H, int I,
                                                     size_t off_w, uint16_t* __restrict__ act_sorted, int ncbp) {
    __shared__ __attribute__((aligned(16))) char As[2][MT * kGBM * kARowBytes];
    // column block fastest, with ncbp (a multiple of 8) blocks per tile: consecutive
    // workgroups go to different XCDs round-robin, so a column block of every tile of a
    // slot group lands on the same XCD close in time and the group's weights are read
    // from HBM once and then from that XCD's L2
    const int cbk = blockIdx.x % ncbp;
    const int tile = blockIdx.x / ncbp;
    if (tile >= grp[0] || cbk * kGBN >= I) return;
    const SlotSpan sp = pick_slots(sl);
    const int slot = grp[16 + tile];
    const int row0 = grp[16 + tile_stride + tile];
    const int rows = grp[16 + 2 * tile_stride + tile];
    const int32_t* perm = grp + 16 + 3 * tile_stride;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int hl = lane >> 5;
    const int l32 = lane & 31;
    const int j0 = cbk * kGBN + (tid >> 6) * 32;
    const bool cols = j0 < I;                    // the wave has columns (uniform per wave)
    const int nb = (rows + kGBM - 1) / kGBM;     // row blocks present (uniform)
    // staging: thread tid covers half `sh` of row `sr`
    const int sr = tid >> 1, sh = tid & 1;
    const bool srow = sr < nb * kGBM;
    const size_t sx = srow ? (size_t)(perm[row0 + min(sr, rows - 1)] / K) * H + sh * 32 : 0;
    const int n = min(j0 + l32, I - 1);
    const size_t rb = (size_t)H * 2;
    const char* ex = sp.at(slot, stride) + off_w;
    const char* gr = ex + (size_t)n * rb + hl * 64;
    const char* ur = ex + (size_t)(I + n) * rb + hl * 64;
    f32x16_t cg[MT], cu[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) cg[m] = cu[m] = f32x16_t{};
    uint4 bg[4], bu[4];
    Row32 sa{};
    if (cols)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bg[j] = load16(gr + 16 * j);
            bu[j] = load16(ur + 16 * j);
        }
    if (srow) store_row32(As[0] + sr * kARowBytes + sh * 64, load_row32<AT>(x, sx));
    __syncthreads();
    int cur = 0;
    for (int k0 = 64; k0 <= H; k0 += 64) {
        const bool more = k0 < H;
        uint4 nbg[4], nbu[4];
        if (more) {
            if (cols)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    nbg[j] = load16(gr + (size_t)k0 * 2 + 16 * j);
                    nbu[j] = load16(ur + (size_t)k0 * 2 + 16 * j);
                }
            if (srow) sa = load_row32<AT>(x, sx + k0);
        }
        if (cols) {
            const char* buf = As[cur];
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (m < nb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint4 a = lds_a8(buf, m * kGBM + l32, hl, j);
                        cg[m] = mfma_32x32x16(a, bg[j], cg[m]);
                        cu[m] = mfma_32x32x16(a, bu[j], cu[m]);
                    }
        }
        if (more) {
            if (srow) store_row32(As[cur ^ 1] + sr * kARowBytes + sh * 64, sa);
            if (cols)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    bg[j] = nbg[j];
                    bu[j] = nbu[j];
                }
            __syncthreads();
            cur ^= 1;
        }
    }
    const int col = j0 + l32;
    if (cols && col < I) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m >= nb) break;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = m * kGBM + 8 * (i >> 2) + 4 * hl + (i & 3);
                if (r < rows) act_sorted[(size_t)(row0 + r) * I + col] = f32_to_bf16_rne(silu(cg[m][i]) * cu[m][i]);
            }
        }
    }
}

// ---- grouped w2 ------------------------------------------------------------------
// grid.x: tiles; grid.y: blocks of 128 output columns of H.
// y[pair(pos)][h] = act_sorted[pos] . W2[s][h]   (MT blocks of 32 rows per wave, the
// act rows staged in LDS as above)
template <int MT>
__global__ __launch_bounds__(256) void k_grouped_w2(Slots sl, size_t stride,
                                                    const int32_t* __restrict__ grp, int tile_stride,
                                                    const uint16_t* __restrict__ act_sorted, int H, int I,
                                                    size_t off_w, float* __restrict__ y, int ncbp) {
    __shared__ __attribute__((aligned(16))) char As[2][MT * kGBM * kARowBytes];
    const int cbk = blockIdx.x % ncbp;        // column block fastest (see k_grouped_w13)
    const int tile = blockIdx.x / ncbp;
    if (tile >= grp[0] || cbk * kGBN >= H) return;
    const SlotSpan spn = pick_slots(sl);
    const int slot = grp[16 + tile];
    const int row0 = grp[16 + tile_stride + tile];
    const int rows = grp[16 + 2 * tile_stride + tile];
    const int32_t* perm = grp + 16 + 3 * tile_stride;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int hl = lane >> 5;
    const int l32 = lane & 31;
    const int h0 = cbk * kGBN + (tid >> 6) * 32;
    const bool cols = h0 < H;
    const int nb = (rows + kGBM - 1) / kGBM;
    const int sr = tid >> 1, sh = tid & 1;
    const bool srow = sr < nb * kGBM;
    const uint16_t* sp = act_sorted + (size_t)(row0 + min(sr, rows - 1)) * I + sh * 32;
    const int n = min(h0 + l32, H - 1);
    const char* br = spn.at(slot, stride) + off_w + (size_t)n * I * 2 + hl * 64;
    f32x16_t c[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) c[m] = f32x16_t{};
    uint4 b[4];
    Row32 sa{};
    if (cols)
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = load16(br + 16 * j);
    if (srow) store_row32(As[0] + sr * kARowBytes + sh * 64, load_row32<A_BF16>(sp, 0));
    __syncthreads();
    int cur = 0;
    for (int k0 = 64; k0 <= I; k0 += 64) {
        const bool more = k0 < I;
        uint4 nb4[4];
        if (more) {
            if (cols)
#pragma unroll
                for (int j = 0; j < 4; ++j) nb4[j] = load16(br + (size_t)k0 * 2 + 16 * j);
            if (srow) sa = load_row32<A_BF16>(sp, k0);
        }
        if (cols) {
            const char* buf = As[cur];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 bj = b[j];
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    if (m < nb) {
                        const uint4 a = lds_a8(buf, m * kGBM + l32, hl, j);
                        c[m] = mfma_32x32x16(a, bj, c[m]);
                    }
            }
        }
        if (more) {
            if (srow) store_row32(As[cur ^ 1] + sr * kARowBytes + sh * 64, sa);
            if (cols)
#pragma unroll
                for (int j = 0; j < 4; ++j) b[j] = nb4[j];
            __syncthreads();
            cur ^= 1;
        }
    }
    const int col = h0 + l32;
    if (cols && col < H) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m >= nb) break;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = m * kGBM + 8 * (i >> 2) + 4 * hl + (i & 3);
                if (r < rows) y[(size_t)perm[row0 + r] * H + col] = c[m][i];
            }
        }
    }
}

// ---- grouped GEMMs for large slot groups: both operands through LDS -------------------
// A workgroup of WGR x WGC waves computes a tile of 32*WR*WGR rows x 32*WC*WGC weight
// rows (w13: the gate rows of half as many columns and the matching up rows; w2: as many
// output columns); each wave owns WR row blocks x WC weight blocks of 32 (WR*WC
// accumulators).  Each
// 64-element k span of both operands is loaded into registers two spans ahead (two
// register sets), then written into one of two LDS buffers the span before its MFMAs
// read it.  A tile row is 128 bytes in LDS with its 16-byte chunk c at position
// c ^ (row & 7), so the 32 rows one MFMA operand reads hit distinct banks.
// The library uses WR = WC = 2 with 2 x 2 waves (128-row tiles of 128 weight rows, 64 KiB
// of LDS, two workgroups per CU: one computes while the other waits for memory) or, for
// large groups, 2 x 4 waves (128 x 256, 96 KiB, one workgroup of 8 waves per CU: each
// activation row is read by half as many workgroups).  (Measured and not used: three spans ahead
// needed more than the 256 registers of two workgroups per CU and spilled; one 128-row
// workgroup per CU with three spans ahead was 1.3x slower; WR = WC = 4, 256-row tiles
// with half an LDS operand read per MFMA but one workgroup per CU, 1.4x slower.)
// Per accumulator the k order (spans in order, then MFMA j = 0..3 with the lane-half
// element split of the staged kernels) is the one of k_grouped_w13 / k_grouped_w2, so
// every output row has the same bits whichever kernel computed it.

// The span's copies of one thread: NA chunks of A rows, NB of weight rows.
template <int NA, int NB>
struct GgRegs {
    uint4 a[NA], b[NB];
};

template <bool W13, int WR, int WC, int WGR, int WGC>
__global__ __launch_bounds__(64 * WGR * WGC, (WGR * WGC > 4 ? 1 : 2)) void k_gg(Slots sl, size_t stride,
        const int32_t* __restrict__ grp, int tile_stride, const uint16_t* __restrict__ a_src, int K, int Kd,
        int ncols, size_t off_w, void* __restrict__ out, int ncbp) {
    constexpr int NW = WGR * WGC;                     // waves: WGR along rows x WGC along columns
    constexpr int RA = 32 * WR * WGR, RB = 32 * WC * WGC;   // tile rows of A and of the weights
    constexpr int NA = RA / (8 * NW), NB = RB / (8 * NW);   // chunks per thread and span
    constexpr int TA = RA * 128, TB = RB * 128;      // LDS bytes of one span
    __shared__ __attribute__((aligned(1024))) char lds[2][TA + TB];
    constexpr int cspan = W13 ? RB / 2 : RB;        // output columns per workgroup
    int cbk, tile;
    if constexpr (NW == 4) {
        cbk = blockIdx.x % ncbp;
        tile = blockIdx.x / ncbp;
        if (tile >= grp[0] || cbk * cspan >= ncols) return;
    } else {
        // ncbp = column blocks per tile.  The hardware hands workgroup b to XCD b % 8;
        // each XCD takes one contiguous run of the (tile, column block) list, column block
        // fastest, so the few column blocks of a tile (which read the same A rows) run
        // side by side on one XCD
        const int nwork = grp[0] * ncbp;
        const int per = (nwork + 7) >> 3;
        const int jx = (int)(blockIdx.x >> 3);
        if (jx >= per) return;
        const int wk = (int)(blockIdx.x & 7) * per + jx;
        if (wk >= nwork) return;
        tile = wk / ncbp;
        cbk = wk - tile * ncbp;
    }
    const SlotSpan sp = pick_slots(sl);
    const int slot = grp[16 + tile];
    const int row0 = grp[16 + tile_stride + tile];
    const int rows = grp[16 + 2 * tile_stride + tile];
    const int32_t* perm = grp + 16 + 3 * tile_stride;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = wave_id();
    const int hl = lane >> 5;
    const int l32 = lane & 31;
    const int wr = w / WGC, wc = w % WGC;
    const int c0 = cbk * cspan;
    const char* wbase = sp.at(slot, stride) + off_w;
    const size_t rowb = (size_t)Kd * 2;
    // this thread copies chunk lane % 8 of A rows w*RA/NW + q*8 + lane/8 (q < NA) and of
    // weight rows w*RB/NW + q*8 + lane/8 (q < NB).  Weight rows are consecutive within a
    // wave's share (the column blocks never pass the end: the shapes are multiples of
    // 256, and a wave's share lies in one of the w13 gate / up halves), so are A rows for
    // w2; w13 gathers its A rows.  In LDS the chunk goes to position (lane % 8) ^ (lane / 8)
    // of its row.
    const int ck = lane & 7;
    const int ra0 = w * (RA / NW) + (lane >> 3);
    const int rb0 = w * (RB / NW) + (lane >> 3);
    const int swz = (ck ^ (lane >> 3)) * 16;
    const int wrow0 = W13 ? (rb0 < RB / 2 ? c0 + rb0 : ncols + c0 + rb0 - RB / 2) : c0 + rb0;
    const char* bsrc = wbase + (size_t)wrow0 * rowb + ck * 16;
    const char* abase = reinterpret_cast<const char*>(a_src) + ck * 16;
    uint32_t aoff[W13 ? NA : 1];                    // w13: byte offsets of the gathered rows
    size_t arow0 = 0;
    if constexpr (W13) {
#pragma unroll
        for (int q = 0; q < NA; ++q)
            aoff[q] = (uint32_t)((size_t)(perm[row0 + min(ra0 + q * 8, rows - 1)] / K) * rowb);
    } else {
        arow0 = (size_t)(row0 + ra0);
    }
    const int nsp = Kd / 64;                        // even
    using Regs = GgRegs<NA, NB>;
    auto fetch = [&](Regs& g, int sn) {
        const size_t kb = (size_t)sn * 128;
#pragma unroll
        for (int q = 0; q < NB; ++q) g.b[q] = load16(bsrc + (size_t)q * 8 * rowb + kb);
#pragma unroll
        for (int q = 0; q < NA; ++q) {
            // w2: rows past the tile's end read the clamped last row: never stored
            size_t ar;
            if constexpr (W13) ar = (size_t)aoff[q];
            else ar = (size_t)min((int)arow0 + q * 8, row0 + rows - 1) * rowb;
            g.a[q] = load16(abase + ar + kb);
        }
    };
    auto put = [&](const Regs& g, char* buf) {
#pragma unroll
        for (int q = 0; q < NA; ++q)
            *reinterpret_cast<uint4*>(buf + (ra0 + q * 8) * 128 + swz) = g.a[q];
#pragma unroll
        for (int q = 0; q < NB; ++q)
            *reinterpret_cast<uint4*>(buf + TA + (rb0 + q * 8) * 128 + swz) = g.b[q];
    };
    const int nb = (rows + kGBM - 1) / kGBM;        // row blocks present (uniform)
    const int mfirst = wr * WR;                      // the wave's first row block
    // the wave's weight blocks: w13 gate blocks 0 .. WC/2-1 of its 32*WC/2 columns, then
    // the matching up blocks; w2 WC consecutive column blocks
    int nbk[WC];
#pragma unroll
    for (int bi = 0; bi < WC; ++bi) {
        if (W13) nbk[bi] = bi < WC / 2 ? wc * (WC / 2) * 32 + bi * 32 : RB / 2 + wc * (WC / 2) * 32 + (bi - WC / 2) * 32;
        else nbk[bi] = wc * WC * 32 + bi * 32;
    }
    f32x16_t acc[WR][WC];
#pragma unroll
    for (int mi = 0; mi < WR; ++mi)
#pragma unroll
        for (int bi = 0; bi < WC; ++bi) acc[mi][bi] = f32x16_t{};
    auto compute = [&](const char* A) {
        const char* B = A + TA;
        if (mfirst >= nb) return;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int pos = ((4 * hl + j) ^ (l32 & 7)) * 16;
            uint4 bf[WC];
#pragma unroll
            for (int bi = 0; bi < WC; ++bi) bf[bi] = *reinterpret_cast<const uint4*>(B + (nbk[bi] + l32) * 128 + pos);
#pragma unroll
            for (int mi = 0; mi < WR; ++mi) {
                if (mfirst + mi >= nb) break;
                const uint4 af = *reinterpret_cast<const uint4*>(A + ((mfirst + mi) * 32 + l32) * 128 + pos);
#pragma unroll
                for (int bi = 0; bi < WC; ++bi) acc[mi][bi] = mfma_32x32x16(af, bf[bi], acc[mi][bi]);
            }
        }
    };
    // span s: request span s + 2 (into the set span s came from), the MFMAs of span s
    // (LDS buffer s % 2), then span s + 1 into the other buffer (last read by span s - 1,
    // before the previous barrier).  The requests are never inside a branch, so the
    // compiler's wait before a write to LDS counts exactly the loads issued after that
    // span's: the last two spans run from a copy of the loop without the requests.
    Regs rx, ry;
    auto step = [&](int s, Regs& ahead, const Regs& next, bool fetch_ahead, bool put_next) {
        if (fetch_ahead) fetch(ahead, s + 2);
        compute(lds[s & 1]);
        if (put_next) put(next, lds[(s + 1) & 1]);
        __syncthreads();
    };
    fetch(rx, 0);
    fetch(ry, 1);
    put(rx, lds[0]);
    __syncthreads();
    int sn = 0;
    for (; sn + 2 < nsp; sn += 2) {
        step(sn, rx, ry, true, true);
        step(sn + 1, ry, rx, true, true);
    }
    step(sn, rx, ry, false, true);
    step(sn + 1, ry, rx, false, false);
    // epilogue: accumulator element i of row block m is tile row m*32 + 8(i/4) + 4 hl + i%4
#pragma unroll
    for (int mi = 0; mi < WR; ++mi) {
        const int m = mfirst + mi;
        if (m >= nb) break;
        if (W13) {
#pragma unroll
            for (int p = 0; p < WC / 2; ++p) {
                const int col = c0 + wc * (WC / 2) * 32 + p * 32 + l32;
                if (col < ncols)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int r = m * kGBM + 8 * (i >> 2) + 4 * hl + (i & 3);
                        if (r < rows)
                            static_cast<uint16_t*>(out)[(size_t)(row0 + r) * ncols + col] =
                                f32_to_bf16_rne(silu(acc[mi][p][i]) * acc[mi][WC / 2 + p][i]);
                    }
            }
        } else {
#pragma unroll
            for (int bi = 0; bi < WC; ++bi) {
                const int col = c0 + wc * WC * 32 + bi * 32 + l32;
                if (col < ncols)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int r = m * kGBM + 8 * (i >> 2) + 4 * hl + (i & 3);
                        if (r < rows) static_cast<float*>(out)[(size_t)perm[row0 + r] * ncols + col] = acc[mi][bi][i];
                    }
            }
        }
    }
}

// ---- ordered top-k combine (grouped path) -------------------------------------------
// out[t][h] = resid[t][h] + sum_{k = 0..K-1} w[t][k] * y[t*K + k][h]   (k in order;
// pairs whose slot id is out of range contribute nothing).  grid.y walks the tokens
// (a token's weights and slot ids are read once, into scalar registers); a thread
// owns 4 consecutive h (H is a multiple of 64 on this path) and issues the loads of
// y for eight k at a time before it adds them in order.
template <int AT>
__global__ __launch_bounds__(256) void k_combine(Slots sl, const float* __restrict__ y,
                                                 const float* __restrict__ topk_w,
                                                 const int32_t* __restrict__ slot_ids,
                                                 const void* __restrict__ resid, void* __restrict__ out, int T,
                                                 int K, int H) {
    const int nslots = pick_slots(sl).n();
    const int h = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (h >= H) return;
    for (int t = blockIdx.y; t < T; t += gridDim.y) {
        float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
        for (int k0 = 0; k0 < K; k0 += 8) {
            float4 v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int k = k0 + q;
                const int s = k < K ? slot_ids[t * K + k] : -1;
                v[q] = (s >= 0 && s < nslots) ? *reinterpret_cast<const float4*>(y + ((size_t)t * K + k) * H + h)
                                              : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int k = k0 + q;
                if (k >= K) break;
                const float w = topk_w[(size_t)t * K + k];
                a0 = fmaf(w, v[q].x, a0);
                a1 = fmaf(w, v[q].y, a1);
                a2 = fmaf(w, v[q].z, a2);
                a3 = fmaf(w, v[q].w, a3);
            }
        }
        const size_t o = (size_t)t * H + h;
        if (resid) {
            a0 += load_act<AT>(resid, o);
            a1 += load_act<AT>(resid, o + 1);
            a2 += load_act<AT>(resid, o + 2);
            a3 += load_act<AT>(resid, o + 3);
        }
        if (AT == A_F32) {
            *reinterpret_cast<float4*>(static_cast<float*>(out) + o) = make_float4(a0, a1, a2, a3);
        } else {
            uint2 u;
            u.x = (uint32_t)f32_to_bf16_rne(a0) | ((uint32_t)f32_to_bf16_rne(a1) << 16);
            u.y = (uint32_t)f32_to_bf16_rne(a2) | ((uint32_t)f32_to_bf16_rne(a3) << 16);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + o) = u;
        }
    }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
namespace {

// Launch shape when a whole wave shares a row (G == 64): waves per row (WPR) and
// rows per lane group (RP); otherwise one wave part and one row (pair) per group.
// Measured on the OLMoE shapes: w13 with one row per wave (the fused one-token step
// 14.7 vs 15.2 us with two), w2 with four rows per wave (8.2-8.4 vs 8.3-8.6 us at one
// token, 29.6 vs 33.2 us at eight; 9.1-9.7 / 43.0 us with one).
#ifndef MOE_W13_WPR
#define MOE_W13_WPR 1
#endif
#ifndef MOE_W13_I4_SPLIT
#define MOE_W13_I4_SPLIT 1
#endif
#ifndef MOE_W13_RP64
#define MOE_W13_RP64 1
#endif
#ifndef MOE_W2_WPR
#define MOE_W2_WPR 1
#endif
#ifndef MOE_W2_RP64
#define MOE_W2_RP64 4
#endif

int log2_of(int g) {
    int s = 0;
    while ((1 << s) < g) ++s;
    return s;
}

int chunks_of(int wtype, int n) {
    const int epc = wtype == W_F32 ? 4 : (wtype == W_BF16 ? 8 : 32);
    return n / epc;
}

int group_lanes(int nc) {
    int g = 64;
    while (g > 1 && nc % g) g >>= 1;
    return g;
}

// waves per row for a row of nc chunks split over G lanes: the largest of
// {want, want/2, ..., 1} that divides nc / G (only for G == 64)
int waves_per_row(int nc, int G, int want) {
    if (G != 64) return 1;
    int w = want;
    while (w > 1 && (nc / G) % w) w >>= 1;
    return w;
}

bool cpl_ok(int cpl) {
    switch (cpl) {
        case 1: case 2: case 3: case 4: case 5: case 6: case 8: case 12: case 16: return true;
    }
    return false;
}

template <int WT, int AT, int CPL, int RP, int WPR>
hipError_t launch_w13(const Geom& g, const ForwardArgs& a, int G, const StageEvents* ev, hipStream_t s) {
    const int rows_per_block = (4 / WPR) * (64 / G) * RP;
    const dim3 grid((g.I + rows_per_block - 1) / rows_per_block, g.K, a.T);
    const size_t lds = WT == W_INT4 ? (size_t)(g.H / 32) * kPackedChunkBytes : 0;
    if (ev && ev->w13_start)
        hipExtLaunchKernelGGL((k_w13_gemv<WT, AT, CPL, RP, WPR>), grid, dim3(256), (uint32_t)lds, s, ev->w13_start,
                              ev->w13_stop, 0, a.sl, g.slot_stride, a.slot_ids, a.x, g.H, g.I, log2_of(G), g.off_w13,
                              g.off_s13, a.act);
    else
        hipLaunchKernelGGL((k_w13_gemv<WT, AT, CPL, RP, WPR>), grid, dim3(256), lds, s, a.sl, g.slot_stride,
                           a.slot_ids, a.x, g.H, g.I, log2_of(G), g.off_w13, g.off_s13, a.act);
    return hipGetLastError();
}

template <int AT, int CPL>
hipError_t launch_w13_i4s(const Geom& g, const ForwardArgs& a, int G, const StageEvents* ev, hipStream_t s) {
    const int rows_per_block = 4 * (32 / G);
    const dim3 grid((g.I + rows_per_block - 1) / rows_per_block, g.K, a.T);
    const size_t lds = (size_t)(g.H / 32) * kPackedChunkBytes;
    if (ev && ev->w13_start)
        hipExtLaunchKernelGGL((k_w13_i4s<AT, CPL>), grid, dim3(256), (uint32_t)lds, s, ev->w13_start, ev->w13_stop, 0,
                              a.sl, g.slot_stride, a.slot_ids, a.x, g.H, g.I, log2_of(G), g.off_w13, g.off_s13, a.act);
    else
        hipLaunchKernelGGL((k_w13_i4s<AT, CPL>), grid, dim3(256), lds, s, a.sl, g.slot_stride, a.slot_ids, a.x, g.H,
                           g.I, log2_of(G), g.off_w13, g.off_s13, a.act);
    return hipGetLastError();
}

template <int WT, int AT, int CPL, int RP, int WPR>
hipError_t launch_w2(const Geom& g, const ForwardArgs& a, int G, const StageEvents* ev, hipStream_t s) {
    constexpr int NWMAX = 16;
    const int RB = (64 / G) * RP;
    const int tasks = g.K * WPR;
    const int nw = tasks < NWMAX ? tasks : NWMAX;
    size_t lds = (size_t)tasks * RB * sizeof(float);
    if (WT == W_INT4 && tasks <= NWMAX)   // the token's packed act vectors
        lds = ((lds + 15) & ~(size_t)15) + (size_t)g.K * (g.I / 32) * kPackedChunkBytes;
    const int nrb = (g.H + RB - 1) / RB;
    const int xcd_T = a.T > 1 && nrb % 8 == 0 ? a.T : 0;
    const dim3 grid = xcd_T ? dim3(nrb * a.T) : dim3(nrb, a.T);
    auto go = [&](auto kern) {
        if (ev && ev->w2_start)
            hipExtLaunchKernelGGL(kern, grid, dim3(64 * nw), (uint32_t)lds, s, ev->w2_start, ev->w2_stop, 0, a.sl,
                                  g.slot_stride, a.slot_ids, a.topk_w, a.act, a.resid, a.out, g.K, g.H, g.I,
                                  log2_of(G), g.off_w2, g.off_s2, a.flip_par, xcd_T);
        else
            hipLaunchKernelGGL(kern, grid, dim3(64 * nw), lds, s, a.sl, g.slot_stride, a.slot_ids, a.topk_w, a.act,
                               a.resid, a.out, g.K, g.H, g.I, log2_of(G), g.off_w2, g.off_s2, a.flip_par, xcd_T);
    };
    if (tasks <= NWMAX)
        go(k_w2_combine<WT, AT, CPL, RP, WPR, NWMAX, true>);
    else
        go(k_w2_combine<WT, AT, CPL, RP, WPR, NWMAX, false>);
    return hipGetLastError();
}

#define MOE_CPL_SWITCH(cpl, CALL)                       \
    switch (cpl) {                                      \
        case 1: { constexpr int C = 1; return CALL; }   \
        case 2: { constexpr int C = 2; return CALL; }   \
        case 3: { constexpr int C = 3; return CALL; }   \
        case 4: { constexpr int C = 4; return CALL; }   \
        case 5: { constexpr int C = 5; return CALL; }   \
        case 6: { constexpr int C = 6; return CALL; }   \
        case 8: { constexpr int C = 8; return CALL; }   \
        case 12: { constexpr int C = 12; return CALL; } \
        case 16: { constexpr int C = 16; return CALL; } \
    }                                                   \
    return hipErrorInvalidValue;

template <int WT, int AT>
hipError_t run_w13(const Geom& g, const ForwardArgs& a, const StageEvents* ev, hipStream_t s) {
    const int nc = chunks_of(WT, g.H);
    const int G = group_lanes(nc);
    const int wpr = waves_per_row(nc, G, MOE_W13_WPR);
    const int cpl = nc / (G * wpr);
    if (WT == W_INT4 && G != 64 && MOE_W13_I4_SPLIT) {
        MOE_CPL_SWITCH(cpl, (launch_w13_i4s<AT, C>(g, a, G, ev, s)))
    }
    if (G != 64) {
        MOE_CPL_SWITCH(cpl, (launch_w13<WT, AT, C, 1, 1>(g, a, G, ev, s)))
    }
    if (wpr == 4) {
        MOE_CPL_SWITCH(cpl, (launch_w13<WT, AT, C, MOE_W13_RP64, 4>(g, a, G, ev, s)))
    }
    if (wpr == 2) {
        MOE_CPL_SWITCH(cpl, (launch_w13<WT, AT, C, MOE_W13_RP64, 2>(g, a, G, ev, s)))
    }
    MOE_CPL_SWITCH(cpl, (launch_w13<WT, AT, C, MOE_W13_RP64, 1>(g, a, G, ev, s)))
}

template <int WT, int AT>
hipError_t run_w2(const Geom& g, const ForwardArgs& a, const StageEvents* ev, hipStream_t s) {
    const int nc = chunks_of(WT, g.I);
    const int G = group_lanes(nc);
    const int wpr = waves_per_row(nc, G, MOE_W2_WPR);
    const int cpl = nc / (G * wpr);
    if (G != 64) {
        MOE_CPL_SWITCH(cpl, (launch_w2<WT, AT, C, 1, 1>(g, a, G, ev, s)))
    }
    if (wpr == 4) {
        MOE_CPL_SWITCH(cpl, (launch_w2<WT, AT, C, MOE_W2_RP64, 4>(g, a, G, ev, s)))
    }
    if (wpr == 2) {
        MOE_CPL_SWITCH(cpl, (launch_w2<WT, AT, C, MOE_W2_RP64, 2>(g, a, G, ev, s)))
    }
    MOE_CPL_SWITCH(cpl, (launch_w2<WT, AT, C, MOE_W2_RP64, 1>(g, a, G, ev, s)))
}

template <int WT, int AT>
hipError_t run_decode(const Geom& g, const ForwardArgs& a, const StageEvents* ev, hipStream_t s) {
    hipError_t e = run_w13<WT, AT>(g, a, ev, s);
    if (e != hipSuccess) return e;
    return run_w2<WT, AT>(g, a, ev, s);
}

template <int WT, int AT, int CPL, int RP, int WPR>
hipError_t launch_step_w13(const Geom& g, const PolicyArgs& pa, const ForwardArgs& a, int G, int n_copy,
                           const StageEvents* ev, hipStream_t s) {
    const int rows_per_block = (4 / WPR) * (64 / G) * RP;
    const int nrb = (g.I + rows_per_block - 1) / rows_per_block;
    const size_t pol = (policy_lds_bytes(g.E, pa.N, pa.evict) + 15) / 16 * 16;
    const size_t lds = pol + (WT == W_INT4 ? (size_t)(g.H / 32) * kPackedChunkBytes : 0);
    const size_t tail = (size_t)2 * g.I * g.H * (WT == W_F32 ? 4 : (WT == W_BF16 ? 2 : 1)) / (WT == W_INT4 ? 2 : 1);
    const dim3 grid(1 + n_copy + nrb * g.K);
    if (ev && ev->w13_start)
        hipExtLaunchKernelGGL((k_step_w13<WT, AT, CPL, RP, WPR>), grid, dim3(256), (uint32_t)lds, s, ev->w13_start,
                              ev->w13_stop, 0, pa, g.slot_stride, a.x, g.H, g.I, log2_of(G), g.off_w13, g.off_s13, tail,
                              a.act, n_copy, nrb, (int)pol);
    else
        hipLaunchKernelGGL((k_step_w13<WT, AT, CPL, RP, WPR>), grid, dim3(256), lds, s, pa, g.slot_stride, a.x, g.H,
                           g.I, log2_of(G), g.off_w13, g.off_s13, tail, a.act, n_copy, nrb, (int)pol);
    return hipGetLastError();
}

template <int WT, int AT>
hipError_t run_step(const Geom& g, const PolicyArgs& pa, const ForwardArgs& a, int n_copy, const StageEvents* ev,
                    hipStream_t s) {
    const int nc = chunks_of(WT, g.H);
    const int G = group_lanes(nc);
    const int wpr = waves_per_row(nc, G, MOE_W13_WPR);
    const int cpl = nc / (G * wpr);
    hipError_t e = hipErrorInvalidValue;
    auto pick = [&]() -> hipError_t {
        if (G != 64) {
            MOE_CPL_SWITCH(cpl, (launch_step_w13<WT, AT, C, 1, 1>(g, pa, a, G, n_copy, ev, s)))
        }
        if (wpr == 4) {
            MOE_CPL_SWITCH(cpl, (launch_step_w13<WT, AT, C, MOE_W13_RP64, 4>(g, pa, a, G, n_copy, ev, s)))
        }
        if (wpr == 2) {
            MOE_CPL_SWITCH(cpl, (launch_step_w13<WT, AT, C, MOE_W13_RP64, 2>(g, pa, a, G, n_copy, ev, s)))
        }
        MOE_CPL_SWITCH(cpl, (launch_step_w13<WT, AT, C, MOE_W13_RP64, 1>(g, pa, a, G, n_copy, ev, s)))
    };
    if ((e = pick()) != hipSuccess) return e;
    ForwardArgs a2 = a;
    a2.flip_par = pa.ds.ctl;
    return run_w2<WT, AT>(g, a2, ev, s);
}

bool split_ok(int nc, int want) {
    const int G = group_lanes(nc);
    return cpl_ok(nc / (G * waves_per_row(nc, G, want)));
}

}  // namespace

bool decode_shape_supported(int wtype, int atype, int H, int I) {
    if (wtype == W_INT4 && atype != A_BF16) return false;
    const int n13 = chunks_of(wtype, H), n2 = chunks_of(wtype, I);
    if (n13 < 1 || n2 < 1) return false;
    return split_ok(n13, MOE_W13_WPR) && split_ok(n2, MOE_W2_WPR);
}

size_t act_bytes_per_pair(int wtype, int I) { return (size_t)I * (wtype == W_F32 ? 4 : 2); }

int grouped_tile_stride(int max_pairs, int nslots) {
    return max_pairs / kGBM + (nslots < max_pairs ? nslots : max_pairs) + 1;
}

size_t grouped_index_bytes(int max_tokens, int K, int nslots) {
    const int mp = max_tokens * K;
    return (size_t)(16 + 3 * grouped_tile_stride(mp, nslots) + mp) * sizeof(int32_t);
}

bool grouped_shape(int wtype, int H, int I) { return wtype == W_BF16 && H % 64 == 0 && I % 64 == 0; }

namespace {

// Rows per tile of the grouped GEMMs (MT blocks of 32), from the average pairs per
// expert (the weights of a slot are read once per tile; small groups keep one block).
// Measured on OLMoE-shaped prefill (skewed routing, 64 and 256 pairs per expert on
// average): 4 blocks match 1 at 64 and run the layer 1.4x faster at 256; 2 blocks
// were slower than either for w2, so they are not chosen.  (256-row tiles through the
// LDS-staged kernels, one workgroup per CU, were 1.4x slower than 128-row tiles at 256
// pairs per expert.)
#ifndef MOE_GROUPED_MT
#define MOE_GROUPED_MT 0
#endif
#ifndef MOE_GG_WIDE
#define MOE_GG_WIDE 1
#endif
int grouped_mt(int n_pairs, int n_experts) {
    if (MOE_GROUPED_MT > 0) return MOE_GROUPED_MT;
    const int per = n_pairs / (n_pairs < n_experts ? n_pairs : n_experts);
    return per >= 40 ? 4 : 1;
}

template <int AT>
hipError_t launch_grouped_combine(const Geom& g, const ForwardArgs& a, const StageEvents* ev, hipStream_t s) {
    const dim3 gc((unsigned)((g.H / 4 + 255) / 256), (unsigned)(a.T < 65535 ? a.T : 65535));
    if (ev && ev->w2_stop)
        hipExtLaunchKernelGGL((k_combine<AT>), gc, dim3(256), 0, s, nullptr, ev->w2_stop, 0, a.sl, a.y, a.topk_w,
                              a.slot_ids, a.resid, a.out, a.T, g.K, g.H);
    else
        hipLaunchKernelGGL((k_combine<AT>), gc, dim3(256), 0, s, a.sl, a.y, a.topk_w, a.slot_ids, a.resid, a.out,
                           a.T, g.K, g.H);
    return hipGetLastError();
}

// Whether the LDS-staged grouped kernels (k_gg) take this shape: hidden and intermediate
// multiples of 256 (whole column blocks, an even number of k spans) and byte offsets of
// the activation rows within 32 bits.
bool gg_shape(const Geom& g, const ForwardArgs& a) {
    return g.H % 256 == 0 && g.I % 256 == 0 && (size_t)a.T * g.H * 2 < ((size_t)1 << 32);
}

template <int AT, int MT>
hipError_t run_grouped_mt(const Geom& g, const ForwardArgs& a, const StageEvents* ev, hipStream_t s) {
    const int n = a.T * g.K;
    const int stride_t = grouped_tile_stride(a.max_pairs, a.nslots_alloc);
    const int nsl = a.sl.npool + a.sl.nmix > a.sl.nstage ? a.sl.npool + a.sl.nmix : a.sl.nstage;
    const int tiles = n / (kGBM * MT) + (nsl < n ? nsl : n) + 1;   // bound on this call's tiles
    hipLaunchKernelGGL(k_group_build, dim3(1), dim3(kGroupThreads), 0, s, a.sl, a.slot_ids, n, stride_t, kGBM * MT,
                       a.grp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    uint16_t* act = static_cast<uint16_t*>(a.act);
    if (gg_shape(g, a) && MT == 4) {
        // tiles of 128 rows: both operands through LDS (k_gg); fp32 activations keep the
        // staged w13 kernel, which converts them while staging.  With bf16 activations and
        // 128 or more pairs per expert on average: 8 waves per workgroup over 256 weight
        // rows (half the column blocks, one workgroup per CU); else 4 waves over 128.
        // (Measured on OLMoE-shaped prefill, 64 slots: at 256 pairs per expert the wide
        // form runs w2 in 181 us instead of 193, w13 alike; at 64 pairs it is 1-3 % slower.)
        const int per = n / (n < g.E ? n : g.E);
        const bool wide = MOE_GG_WIDE && AT == A_BF16 && per >= 128;
        auto go = [&](auto kern, bool w13, int nthreads, unsigned nblocks, int cb) {
            if (w13) {
                if (ev && ev->w13_start)
                    hipExtLaunchKernelGGL(kern, dim3(nblocks), dim3(nthreads), 0, s, ev->w13_start, ev->w13_stop, 0,
                                          a.sl, g.slot_stride, a.grp, stride_t, static_cast<const uint16_t*>(a.x),
                                          g.K, g.H, g.I, g.off_w13, (void*)act, cb);
                else
                    hipLaunchKernelGGL(kern, dim3(nblocks), dim3(nthreads), 0, s, a.sl, g.slot_stride, a.grp,
                                       stride_t, static_cast<const uint16_t*>(a.x), g.K, g.H, g.I, g.off_w13,
                                       (void*)act, cb);
            } else {
                if (ev && ev->w2_start)
                    hipExtLaunchKernelGGL(kern, dim3(nblocks), dim3(nthreads), 0, s, ev->w2_start, nullptr, 0, a.sl,
                                          g.slot_stride, a.grp, stride_t, (const uint16_t*)act, g.K, g.I, g.H,
                                          g.off_w2, (void*)a.y, cb);
                else
                    hipLaunchKernelGGL(kern, dim3(nblocks), dim3(nthreads), 0, s, a.sl, g.slot_stride, a.grp,
                                       stride_t, (const uint16_t*)act, g.K, g.I, g.H, g.off_w2, (void*)a.y, cb);
            }
        };
        if (wide) {
            // column blocks per tile (exact); the grid covers the bound on (tile, block) pairs
            const int cb13 = g.I / 128, cb2 = g.H / 256;
            go(k_gg<true, 2, 2, 2, 4>, true, 512, (unsigned)((tiles * cb13 + 7) / 8 * 8), cb13);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            go(k_gg<false, 2, 2, 2, 4>, false, 512, (unsigned)((tiles * cb2 + 7) / 8 * 8), cb2);
        } else {
            constexpr int W = 2;
            const int gcb13 = ((g.I + 32 * W - 1) / (32 * W) + 7) / 8 * 8, gcb2 = ((g.H + 64 * W - 1) / (64 * W) + 7) / 8 * 8;
            if (AT == A_BF16) {
                go(k_gg<true, W, W, 2, 2>, true, 256, (unsigned)(tiles * gcb13), gcb13);
            } else {
                const int ncb13 = ((g.I + kGBN - 1) / kGBN + 7) / 8 * 8;
                const dim3 g13((unsigned)(tiles * ncb13));
                if (ev && ev->w13_start)
                    hipExtLaunchKernelGGL((k_grouped_w13<AT, 4>), g13, dim3(256), 0, s, ev->w13_start, ev->w13_stop,
                                          0, a.sl, g.slot_stride, a.grp, stride_t, a.x, g.K, g.H, g.I, g.off_w13, act,
                                          ncb13);
                else
                    hipLaunchKernelGGL((k_grouped_w13<AT, 4>), g13, dim3(256), 0, s, a.sl, g.slot_stride, a.grp,
                                       stride_t, a.x, g.K, g.H, g.I, g.off_w13, act, ncb13);
            }
            if ((e = hipGetLastError()) != hipSuccess) return e;
            go(k_gg<false, W, W, 2, 2>, false, 256, (unsigned)(tiles * gcb2), gcb2);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
        return launch_grouped_combine<AT>(g, a, ev, s);
    }
    const int ncb13 = ((g.I + kGBN - 1) / kGBN + 7) / 8 * 8, ncb2 = ((g.H + kGBN - 1) / kGBN + 7) / 8 * 8;
    const dim3 g13((unsigned)(tiles * ncb13)), g2((unsigned)(tiles * ncb2));
    if (ev && ev->w13_start)
        hipExtLaunchKernelGGL((k_grouped_w13<AT, MT>), g13, dim3(256), 0, s, ev->w13_start, ev->w13_stop, 0, a.sl,
                              g.slot_stride, a.grp, stride_t, a.x, g.K, g.H, g.I, g.off_w13, act, ncb13);
    else
        hipLaunchKernelGGL((k_grouped_w13<AT, MT>), g13, dim3(256), 0, s, a.sl, g.slot_stride, a.grp, stride_t, a.x,
                           g.K, g.H, g.I, g.off_w13, act, ncb13);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev && ev->w2_start)
        hipExtLaunchKernelGGL((k_grouped_w2<MT>), g2, dim3(256), 0, s, ev->w2_start, nullptr, 0, a.sl, g.slot_stride,
                              a.grp, stride_t, act, g.H, g.I, g.off_w2, a.y, ncb2);
    else
        hipLaunchKernelGGL((k_grouped_w2<MT>), g2, dim3(256), 0, s, a.sl, g.slot_stride, a.grp, stride_t, act, g.H,
                           g.I, g.off_w2, a.y, ncb2);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_grouped_combine<AT>(g, a, ev, s);
}

template <int AT>
hipError_t run_grouped(const Geom& g, const ForwardArgs& a, const StageEvents* ev, hipStream_t s) {
    switch (grouped_mt(a.T * g.K, g.E)) {
        case 4: return run_grouped_mt<AT, 4>(g, a, ev, s);
        case 2: return run_grouped_mt<AT, 2>(g, a, ev, s);   // only when forced at build time
        default: return run_grouped_mt<AT, 1>(g, a, ev, s);
    }
}

}  // namespace

hipError_t launch_step_decode(const Geom& g, const PolicyArgs& pol, const ForwardArgs& fw, int n_copy,
                              const StageEvents* ev, hipStream_t s) {
    if (fw.T != 1 || pol.n != g.K || fw.slot_ids != pol.out || n_copy < 1 || pol.eb % 16 ||
        pol.evict < EVICT_LRU || pol.evict > EVICT_SLRU || (!pol.resident && pol.per_piece < 1))
        return hipErrorInvalidValue;
    switch (g.wtype * 2 + g.atype) {
        case W_F32 * 2 + A_F32: return run_step<W_F32, A_F32>(g, pol, fw, n_copy, ev, s);
        case W_F32 * 2 + A_BF16: return run_step<W_F32, A_BF16>(g, pol, fw, n_copy, ev, s);
        case W_BF16 * 2 + A_F32: return run_step<W_BF16, A_F32>(g, pol, fw, n_copy, ev, s);
        case W_BF16 * 2 + A_BF16: return run_step<W_BF16, A_BF16>(g, pol, fw, n_copy, ev, s);
        case W_INT4 * 2 + A_BF16: return run_step<W_INT4, A_BF16>(g, pol, fw, n_copy, ev, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_forward(const Geom& g, const ForwardArgs& a, const StageEvents* ev, hipStream_t stream) {
    if (a.T <= 0) return hipSuccess;
    if (a.T > kDecodeMaxTokens && grouped_shape(g.wtype, g.H, g.I))
        return g.atype == A_F32 ? run_grouped<A_F32>(g, a, ev, stream) : run_grouped<A_BF16>(g, a, ev, stream);
    if (a.T > 65535) return hipErrorInvalidValue;   // grid.z of the w13 kernel, grid.y of the w2 kernel
    switch (g.wtype * 2 + g.atype) {
        case W_F32 * 2 + A_F32: return run_decode<W_F32, A_F32>(g, a, ev, stream);
        case W_F32 * 2 + A_BF16: return run_decode<W_F32, A_BF16>(g, a, ev, stream);
        case W_BF16 * 2 + A_F32: return run_decode<W_BF16, A_F32>(g, a, ev, stream);
        case W_BF16 * 2 + A_BF16: return run_decode<W_BF16, A_BF16>(g, a, ev, stream);
        case W_INT4 * 2 + A_BF16: return run_decode<W_INT4, A_BF16>(g, a, ev, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace moe
