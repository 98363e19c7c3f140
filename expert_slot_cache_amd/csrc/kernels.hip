// gfx950 kernels of the expert slot cache: distinct ids, remap, and the
// slot-indexed fused MoE for decode (GEMV) shapes.
//
// Wave size is 64 throughout (CDNA).  All floating point accumulates in fp32, and
// every reduction has a fixed order, so a result depends only on the values it
// reads -- never on which slot an expert sits in.  That is what makes a pooled
// layer bit-identical to the same layer with every expert resident.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

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
// ---------------------------------------------------------------------------
constexpr int kDistinctThreads = 1024;

__global__ __launch_bounds__(kDistinctThreads) void k_distinct(const int32_t* __restrict__ ids, int n,
                                                               int E, int32_t* __restrict__ rb,
                                                               int32_t* __restrict__ rank) {
    __shared__ uint32_t bits[kMaxExperts / 32];
    __shared__ int32_t wave_cnt[kDistinctThreads / 64];
    __shared__ int32_t bad;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nwords = (E + 31) >> 5;
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
            rb[2 + pos] = e;
            rank[e] = pos;
        }
        base += total;
        __syncthreads();
    }
    if (tid == 0) {
        rb[0] = base;
        rb[1] = bad;
    }
}

hipError_t launch_distinct(const int32_t* ids, int n, int E, int32_t* rb, int32_t* rank,
                           hipStream_t stream) {
    hipLaunchKernelGGL(k_distinct, dim3(1), dim3(kDistinctThreads), 0, stream, ids, n, E, rb, rank);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// K-remap: slot_ids[i] = table[ids[i]]  [vLLM-cache: remap topk_ids through the
// persistent mapping; llama-pool: get_rows(table, ids)].  Out-of-range ids give -1,
// which the forward kernels never dereference.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_remap(const int32_t* __restrict__ ids, int n, int E,
                                               const int32_t* __restrict__ table,
                                               int32_t* __restrict__ out) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) {
        const int e = ids[i];
        out[i] = ((unsigned)e < (unsigned)E) ? table[e] : -1;
    }
}

hipError_t launch_remap(const int32_t* ids, int n, int E, const int32_t* table, int32_t* out,
                        hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_remap, dim3((n + 255) / 256), dim3(256), 0, stream, ids, n, E, table, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode GEMV kernels.
//
// A weight row is read as 16-byte chunks; lane l takes chunks l, l+64, ... of
// the row, so a wave's load instruction covers 1 KiB of contiguous row bytes.
// The activation vector sits in LDS as fp32 in a chunk-transposed layout: the
// q-th float4 of chunk c is at float4 index q * n_chunks + c, so the 64 lanes of
// a wave read 64 consecutive float4s (no bank conflicts).
//   f32  : 4 elements per chunk (1 float4)
//   bf16 : 8 elements per chunk (2 float4s)
//   int4 : 32 elements per chunk (8 float4s), one bf16 scale per 4 chunks
// ---------------------------------------------------------------------------
template <int WT>
struct WTraits;
template <>
struct WTraits<W_F32> {
    static constexpr int EPC = 4;   // elements per 16-byte chunk
};
template <>
struct WTraits<W_BF16> {
    static constexpr int EPC = 8;
};
template <>
struct WTraits<W_INT4> {
    static constexpr int EPC = 32;
};

// Partial dot of one chunk with its activations (xs = float4 base of the vector,
// c = chunk index, nc = chunks per row).
template <int WT>
__device__ __forceinline__ float chunk_dot(const uint4 w, const float4* __restrict__ xs, int c, int nc);

template <>
__device__ __forceinline__ float chunk_dot<W_F32>(const uint4 w, const float4* __restrict__ xs, int c,
                                                  int nc) {
    const float4 a = xs[c];
    float acc = __uint_as_float(w.x) * a.x;
    acc = fmaf(__uint_as_float(w.y), a.y, acc);
    acc = fmaf(__uint_as_float(w.z), a.z, acc);
    acc = fmaf(__uint_as_float(w.w), a.w, acc);
    return acc;
}

template <>
__device__ __forceinline__ float chunk_dot<W_BF16>(const uint4 w, const float4* __restrict__ xs, int c,
                                                   int nc) {
    const float4 a = xs[c];
    const float4 b = xs[nc + c];
    float acc = bf16_lo(w.x) * a.x;
    acc = fmaf(bf16_hi(w.x), a.y, acc);
    acc = fmaf(bf16_lo(w.y), a.z, acc);
    acc = fmaf(bf16_hi(w.y), a.w, acc);
    acc = fmaf(bf16_lo(w.z), b.x, acc);
    acc = fmaf(bf16_hi(w.z), b.y, acc);
    acc = fmaf(bf16_lo(w.w), b.z, acc);
    acc = fmaf(bf16_hi(w.w), b.w, acc);
    return acc;
}

// sum_{j<8} (q_j - 8) * x_j for the eight codes of one word
__device__ __forceinline__ float word_dot(uint32_t u, const float4 a, const float4 b) {
    float acc = ((float)(int)(u & 15u) - 8.0f) * a.x;
    acc = fmaf((float)(int)((u >> 4) & 15u) - 8.0f, a.y, acc);
    acc = fmaf((float)(int)((u >> 8) & 15u) - 8.0f, a.z, acc);
    acc = fmaf((float)(int)((u >> 12) & 15u) - 8.0f, a.w, acc);
    acc = fmaf((float)(int)((u >> 16) & 15u) - 8.0f, b.x, acc);
    acc = fmaf((float)(int)((u >> 20) & 15u) - 8.0f, b.y, acc);
    acc = fmaf((float)(int)((u >> 24) & 15u) - 8.0f, b.z, acc);
    acc = fmaf((float)(int)((u >> 28) & 15u) - 8.0f, b.w, acc);
    return acc;
}

template <>
__device__ __forceinline__ float chunk_dot<W_INT4>(const uint4 w, const float4* __restrict__ xs, int c,
                                                   int nc) {
    float acc = word_dot(w.x, xs[0 * nc + c], xs[1 * nc + c]);
    acc += word_dot(w.y, xs[2 * nc + c], xs[3 * nc + c]);
    acc += word_dot(w.z, xs[4 * nc + c], xs[5 * nc + c]);
    acc += word_dot(w.w, xs[6 * nc + c], xs[7 * nc + c]);
    return acc;
}

// Load element `i` (of n) of an activation row as fp32.
template <int AT>
__device__ __forceinline__ float load_act(const void* __restrict__ p, size_t i);
template <>
__device__ __forceinline__ float load_act<A_F32>(const void* __restrict__ p, size_t i) {
    return static_cast<const float*>(p)[i];
}
template <>
__device__ __forceinline__ float load_act<A_BF16>(const void* __restrict__ p, size_t i) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

// Position (in floats) of element e of a vector of nc chunks in the
// chunk-transposed LDS layout.
template <int WT>
__device__ __forceinline__ int lds_pos(int e, int nc) {
    constexpr int EPC = WTraits<WT>::EPC;
    const int c = e / EPC;
    const int r = e - c * EPC;
    return ((r >> 2) * nc + c) * 4 + (r & 3);
}

// Stage n fp32-convertible values into the chunk-transposed LDS layout.
template <int WT, int AT>
__device__ __forceinline__ void stage_vector(float* __restrict__ dst, const void* __restrict__ src,
                                             size_t src_off, int n, int nc) {
    for (int e = threadIdx.x; e < n; e += blockDim.x) dst[lds_pos<WT>(e, nc)] = load_act<AT>(src, src_off + e);
}
template <int WT>
__device__ __forceinline__ void stage_vector_f32(float* __restrict__ dst, const float* __restrict__ src,
                                                 int n, int nc) {
    for (int e = threadIdx.x; e < n; e += blockDim.x) dst[lds_pos<WT>(e, nc)] = src[e];
}

__device__ __forceinline__ uint4 load16(const char* p) { return *reinterpret_cast<const uint4*>(p); }

// Scale of chunk c of a row (int4 only): one bf16 per 128 elements = 4 chunks.
__device__ __forceinline__ float chunk_scale(const uint16_t* __restrict__ srow, int c) {
    return bf16_to_f32(srow[c >> 2]);
}

// ---- w13 + SwiGLU ------------------------------------------------------------
// grid.x: blocks of 4 waves x PPW gate/up row pairs; grid.y: (t, k) pairs.
// act[pair][i] = silu(W13[s][i] . x[t]) * (W13[s][I + i] . x[t]).
template <int WT, int AT, int CPL, int PPW>
__global__ __launch_bounds__(256) void k_w13_gemv(const char* __restrict__ wbase, size_t stride,
                                                  int nslots, const int32_t* __restrict__ slot_ids,
                                                  const void* __restrict__ x, int K, int H, int I,
                                                  size_t off_w, size_t off_s, float* __restrict__ act) {
    extern __shared__ float4 xs4[];
    float* xs = reinterpret_cast<float*>(xs4);
    constexpr int EPC = WTraits<WT>::EPC;
    const int pair = blockIdx.y;
    const int t = pair / K;
    const int nc = H / EPC;                       // chunks per row
    stage_vector<WT, AT>(xs, x, (size_t)t * H, H, nc);
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int i0 = (blockIdx.x * 4 + wave) * PPW;
    if (i0 >= I) return;
    const int slot = slot_ids[pair];
    float* arow = act + (size_t)pair * I;
    if (slot < 0 || slot >= nslots) {
        if (lane < PPW && i0 + lane < I) arow[i0 + lane] = 0.0f;
        return;
    }
    const char* ex = wbase + (size_t)slot * stride;
    const size_t row_bytes = (size_t)nc * 16;
    const char* wrows = ex + off_w;
    const uint16_t* srows = reinterpret_cast<const uint16_t*>(ex + off_s);
    const int spr = H / 128;                      // scales per row (int4)

    uint4 wg[PPW][CPL], wu[PPW][CPL];
#pragma unroll
    for (int p = 0; p < PPW; ++p) {
        const int i = min(i0 + p, I - 1);
        const char* g = wrows + (size_t)i * row_bytes;
        const char* u = wrows + (size_t)(I + i) * row_bytes;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = lane + 64 * j;
            if (c < nc) {
                wg[p][j] = load16(g + (size_t)c * 16);
                wu[p][j] = load16(u + (size_t)c * 16);
            }
        }
    }
#pragma unroll
    for (int p = 0; p < PPW; ++p) {
        const int i = min(i0 + p, I - 1);
        float pg = 0.0f, pu = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = lane + 64 * j;
            if (c < nc) {
                float dg = chunk_dot<WT>(wg[p][j], xs4, c, nc);
                float du = chunk_dot<WT>(wu[p][j], xs4, c, nc);
                if (WT == W_INT4) {
                    dg *= chunk_scale(srows + (size_t)i * spr, c);
                    du *= chunk_scale(srows + (size_t)(I + i) * spr, c);
                }
                pg += dg;
                pu += du;
            }
        }
        pg = wave_sum(pg);
        pu = wave_sum(pu);
        if (lane == 0 && i0 + p < I) arow[i0 + p] = silu(pg) * pu;
    }
}

// ---- w2 + ordered top-k combine ----------------------------------------------
// grid.x: blocks of 4 waves x RPW output rows; grid.y: tokens.
// out[t][r] = resid[t][r] + sum_k w[t][k] * (W2[s_k][r] . act[t*K+k]).
// Each lane weights its partial dot by w[t][k] (k in order), then one wave sum.
template <int WT, int AT, int CPL, int RPW>
__global__ __launch_bounds__(256) void k_w2_combine(const char* __restrict__ wbase, size_t stride,
                                                    int nslots, const int32_t* __restrict__ slot_ids,
                                                    const float* __restrict__ topk_w,
                                                    const float* __restrict__ act,
                                                    const void* __restrict__ resid, void* __restrict__ out,
                                                    int K, int H, int I, size_t off_w, size_t off_s) {
    extern __shared__ float4 as4[];
    float* as = reinterpret_cast<float*>(as4);
    __shared__ int32_t s_slot[kMaxTopK];
    __shared__ float s_w[kMaxTopK];
    constexpr int EPC = WTraits<WT>::EPC;
    const int t = blockIdx.y;
    const int nc = I / EPC;
    const int vec = nc * EPC;                     // = I
    for (int k = 0; k < K; ++k) stage_vector_f32<WT>(as + (size_t)k * vec, act + ((size_t)t * K + k) * I, I, nc);
    if (threadIdx.x < K) {
        const int s = slot_ids[t * K + threadIdx.x];
        s_slot[threadIdx.x] = (s >= 0 && s < nslots) ? s : -1;
        s_w[threadIdx.x] = topk_w[t * K + threadIdx.x];
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r0 = (blockIdx.x * 4 + wave) * RPW;
    if (r0 >= H) return;
    const size_t row_bytes = (size_t)nc * 16;
    const int spr = I / 128;

    float accl[RPW];
#pragma unroll
    for (int p = 0; p < RPW; ++p) accl[p] = 0.0f;

    for (int k = 0; k < K; ++k) {
        const int s = s_slot[k];
        if (s < 0) continue;
        const char* ex = wbase + (size_t)s * stride;
        const char* wrows = ex + off_w;
        const uint16_t* srows = reinterpret_cast<const uint16_t*>(ex + off_s);
        const float4* a4 = as4 + (size_t)k * (vec / 4);
        const float wk = s_w[k];
        uint4 wr[RPW][CPL];
#pragma unroll
        for (int p = 0; p < RPW; ++p) {
            const int r = min(r0 + p, H - 1);
            const char* row = wrows + (size_t)r * row_bytes;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = lane + 64 * j;
                if (c < nc) wr[p][j] = load16(row + (size_t)c * 16);
            }
        }
#pragma unroll
        for (int p = 0; p < RPW; ++p) {
            const int r = min(r0 + p, H - 1);
            float part = 0.0f;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = lane + 64 * j;
                if (c < nc) {
                    float d = chunk_dot<WT>(wr[p][j], a4, c, nc);
                    if (WT == W_INT4) d *= chunk_scale(srows + (size_t)r * spr, c);
                    part += d;
                }
            }
            accl[p] = fmaf(wk, part, accl[p]);
        }
    }
#pragma unroll
    for (int p = 0; p < RPW; ++p) {
        const float acc = wave_sum(accl[p]);
        const int r = r0 + p;
        if (lane == 0 && r < H) {
            const size_t o = (size_t)t * H + r;
            float v = acc;
            if (resid) v += load_act<AT>(resid, o);
            if (AT == A_F32)
                static_cast<float*>(out)[o] = v;
            else
                static_cast<uint16_t*>(out)[o] = f32_to_bf16_rne(v);
        }
    }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
namespace {

constexpr int kPPW = 2;   // gate/up row pairs per wave in k_w13_gemv
constexpr int kRPW = 2;   // output rows per wave in k_w2_combine

int elem_bytes_x2(int wtype) { return wtype == W_F32 ? 8 : (wtype == W_BF16 ? 4 : 1); }

// chunks per row for a row of `n` elements
int chunks(int wtype, int n) { return n * elem_bytes_x2(wtype) / 2 / 16; }

template <int WT, int AT, int CPL13, int CPL2>
hipError_t run_decode(const Geom& g, const ForwardArgs& a, const StageEvents* ev, hipStream_t stream) {
    const int T = a.T, K = g.K;
    const int rows13 = 4 * kPPW, rows2 = 4 * kRPW;
    const size_t lds13 = (size_t)g.H * sizeof(float);
    const size_t lds2 = (size_t)K * g.I * sizeof(float);
    hipError_t e = hipSuccess;
    if (ev && ev->w13_start && (e = hipEventRecord(ev->w13_start, stream)) != hipSuccess) return e;
    hipLaunchKernelGGL((k_w13_gemv<WT, AT, CPL13, kPPW>), dim3((g.I + rows13 - 1) / rows13, T * K), dim3(256),
                       lds13, stream, a.wbase, g.slot_stride, a.nslots, a.slot_ids, a.x, K, g.H, g.I,
                       g.off_w13, g.off_s13, a.act);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev && ev->w13_stop && (e = hipEventRecord(ev->w13_stop, stream)) != hipSuccess) return e;
    if (ev && ev->w2_start && (e = hipEventRecord(ev->w2_start, stream)) != hipSuccess) return e;
    hipLaunchKernelGGL((k_w2_combine<WT, AT, CPL2, kRPW>), dim3((g.H + rows2 - 1) / rows2, T), dim3(256), lds2,
                       stream, a.wbase, g.slot_stride, a.nslots, a.slot_ids, a.topk_w, a.act, a.resid, a.out, K,
                       g.H, g.I, g.off_w2, g.off_s2);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev && ev->w2_stop && (e = hipEventRecord(ev->w2_stop, stream)) != hipSuccess) return e;
    return hipSuccess;
}

int cpl_bucket(int nc) {
    const int c = (nc + 63) / 64;
    if (c <= 1) return 1;
    if (c <= 2) return 2;
    if (c <= 4) return 4;
    if (c <= 8) return 8;
    if (c <= 16) return 16;
    return -1;
}

template <int WT, int AT, int CPL13>
hipError_t pick_cpl2(const Geom& g, const ForwardArgs& a, const StageEvents* ev, hipStream_t s) {
    switch (cpl_bucket(chunks(WT, g.I))) {
        case 1: return run_decode<WT, AT, CPL13, 1>(g, a, ev, s);
        case 2: return run_decode<WT, AT, CPL13, 2>(g, a, ev, s);
        case 4: return run_decode<WT, AT, CPL13, 4>(g, a, ev, s);
        case 8: return run_decode<WT, AT, CPL13, 8>(g, a, ev, s);
        case 16: return run_decode<WT, AT, CPL13, 16>(g, a, ev, s);
    }
    return hipErrorInvalidValue;
}

template <int WT, int AT>
hipError_t pick_cpl13(const Geom& g, const ForwardArgs& a, const StageEvents* ev, hipStream_t s) {
    switch (cpl_bucket(chunks(WT, g.H))) {
        case 1: return pick_cpl2<WT, AT, 1>(g, a, ev, s);
        case 2: return pick_cpl2<WT, AT, 2>(g, a, ev, s);
        case 4: return pick_cpl2<WT, AT, 4>(g, a, ev, s);
        case 8: return pick_cpl2<WT, AT, 8>(g, a, ev, s);
        case 16: return pick_cpl2<WT, AT, 16>(g, a, ev, s);
    }
    return hipErrorInvalidValue;
}

template <int WT>
hipError_t pick_at(const Geom& g, const ForwardArgs& a, const StageEvents* ev, hipStream_t s) {
    return g.atype == A_F32 ? pick_cpl13<WT, A_F32>(g, a, ev, s) : pick_cpl13<WT, A_BF16>(g, a, ev, s);
}

}  // namespace

size_t grouped_index_bytes(int max_tokens, int K, int nslots) {
    (void)max_tokens;
    (void)K;
    (void)nslots;
    return 0;
}

hipError_t launch_forward(const Geom& g, const ForwardArgs& a, const StageEvents* ev, hipStream_t stream) {
    if (a.T <= 0) return hipSuccess;
    if ((long)a.T * g.K > 65535) return hipErrorInvalidValue;   // grid.y of the w13 kernel
    switch (g.wtype) {
        case W_F32: return pick_at<W_F32>(g, a, ev, stream);
        case W_BF16: return pick_at<W_BF16>(g, a, ev, stream);
        case W_INT4: return pick_at<W_INT4>(g, a, ev, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace moe
