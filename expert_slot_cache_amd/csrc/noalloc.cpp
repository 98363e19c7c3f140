// moe_forward_slots: the slot-indexed fused MoE over caller-owned slots, with its
// scratch (the SwiGLU outputs, the grouped path's per-pair w2 outputs and index
// lists) in one file-scope device array instead of memory the library allocates.
// It is meant for callers that cannot allocate device memory: code under graph
// capture, tight serving loops, harnesses that forbid hipMalloc.
//
// Each GPU the library runs on holds its own copy of `scratch` (kStaticScratch bytes,
// until the process ends).  Host code never uses the array's name as an address: the
// first call on a device (with that device current) asks HIP for the array's device
// address and keeps it per device.  Every call on a device shares that device's
// array: calls that overlap on one GPU (other streams, other threads) race.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "kernels.hpp"
#include "layout.hpp"
#include "moe_pool.h"

namespace moe {
void set_last_error(const char* msg);   // moe_pool.cpp
}

namespace {

constexpr size_t kStaticScratch = (size_t)64 << 20;   // bytes per device
constexpr int kMaxDevices = 64;

// The forward's scratch.
__device__ __align__(256) char scratch[kStaticScratch];
// The path word the forward kernels read: always the pool path (the slot ids index
// the caller's slots).  Initialised in the code object; nothing writes it.
__device__ int32_t pool_path_word = moe::PATH_POOL;

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
void* g_path[kMaxDevices] = {};

moe_status_t fail(moe_status_t code, const char* fmt, ...) {
    char msg[256];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(msg, sizeof(msg), fmt, ap);
    va_end(ap);
    moe::set_last_error(msg);
    return code;
}

// The current device's addresses of `scratch` and of the path word (looked up on the
// device's first call).
moe_status_t device_scratch(char** out, int32_t** path) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MOE_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EINVAL, "device %d outside [0,%d)", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        void* w = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return fail(MOE_EHIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
        e = hipGetSymbolAddress(&w, HIP_SYMBOL(pool_path_word));
        if (e != hipSuccess || !w)
            return fail(MOE_EHIP, "hipGetSymbolAddress(pool_path_word) failed: %s", hipGetErrorString(e));
        g_ptr[dev] = p;
        g_path[dev] = w;
    }
    *out = static_cast<char*>(g_ptr[dev]);
    *path = static_cast<int32_t*>(g_path[dev]);
    return MOE_OK;
}

size_t up256(size_t n) { return (n + 255) / 256 * 256; }

}  // namespace

extern "C" {

moe_status_t moe_forward_slots(int32_t wtype, int32_t atype, int32_t hidden, int32_t inter, int32_t top_k,
                               const void* slots_dev, int32_t n_slots, const int32_t* slot_ids_dev,
                               const void* x_dev, const float* topk_w_dev, const void* resid_dev,
                               int32_t n_tokens, void* out_dev, void* stream) {
    moe::Layout lay;
    if (!moe::make_layout(wtype, hidden, inter, &lay))
        return fail(MOE_EINVAL, "unsupported shape/format (wtype %d, H %d, I %d)", wtype, hidden, inter);
    if (atype != MOE_A_F32 && atype != MOE_A_BF16) return fail(MOE_EINVAL, "atype %d invalid", atype);
    if (!moe::decode_shape_supported(wtype, atype, hidden, inter))
        return fail(MOE_EINVAL, "shape not supported by the kernels (wtype %d, atype %d, H %d, I %d)", wtype, atype,
                    hidden, inter);
    if (top_k < 1 || top_k > moe::kMaxTopK) return fail(MOE_EINVAL, "top_k %d invalid", top_k);
    if (n_slots < 1 || n_slots > moe::kMaxExperts) return fail(MOE_EINVAL, "n_slots %d invalid", n_slots);
    if (n_tokens < 0) return fail(MOE_EINVAL, "n_tokens %d < 0", n_tokens);
    if (n_tokens == 0) return MOE_OK;
    if (!slots_dev || !slot_ids_dev || !x_dev || !topk_w_dev || !out_dev) return fail(MOE_EINVAL, "null buffer");
    const size_t pairs = (size_t)n_tokens * top_k;
    const bool grouped = n_tokens > moe::kDecodeMaxTokens && moe::grouped_shape(wtype, hidden, inter);
    if (!grouped && n_tokens > 65535) return fail(MOE_EINVAL, "n_tokens %d too large for the decode kernels", n_tokens);
    if (pairs > ((size_t)1 << 24)) return fail(MOE_EINVAL, "n_tokens * top_k too large");
    // the scratch this call needs: act, then (grouped path) y and the index lists
    const size_t act_b = up256(pairs * moe::act_bytes_per_pair(wtype, inter));
    const size_t y_b = grouped ? up256(pairs * (size_t)hidden * sizeof(float)) : 0;
    const size_t grp_b = grouped ? up256(moe::grouped_index_bytes(n_tokens, top_k, n_slots)) : 0;
    const size_t need = act_b + y_b + grp_b;
    if (need > kStaticScratch)
        return fail(MOE_EINVAL, "this forward needs %zu bytes of scratch; the static scratch holds %zu (fewer tokens "
                    "per call, or moe_pool_forward)", need, kStaticScratch);
    char* base = nullptr;
    int32_t* path = nullptr;
    const moe_status_t st = device_scratch(&base, &path);
    if (st) return st;

    moe::Geom g{};
    g.H = hidden;
    g.I = inter;
    g.K = top_k;
    g.E = n_slots;
    g.wtype = wtype;
    g.atype = atype;
    g.slot_stride = lay.total;
    g.off_w13 = lay.off_w13;
    g.off_w2 = lay.off_w2;
    g.off_s13 = lay.off_s13;
    g.off_s2 = lay.off_s2;
    moe::ForwardArgs a{};
    a.sl = moe::Slots{static_cast<const char*>(slots_dev), nullptr, n_slots, 0, 0, path};
    a.slot_ids = slot_ids_dev;
    a.x = x_dev;
    a.topk_w = topk_w_dev;
    a.resid = resid_dev;
    a.out = out_dev;
    a.T = n_tokens;
    a.act = base;
    a.y = grouped ? reinterpret_cast<float*>(base + act_b) : nullptr;
    a.grp = grouped ? reinterpret_cast<int32_t*>(base + act_b + y_b) : nullptr;
    a.nslots_alloc = n_slots;
    a.max_pairs = (int)pairs;
    const hipError_t e = moe::launch_forward(g, a, nullptr, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MOE_EHIP, "forward launch failed: %s", hipGetErrorString(e));
    return MOE_OK;
}

}  // extern "C"
