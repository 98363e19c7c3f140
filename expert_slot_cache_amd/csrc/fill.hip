// The copy kernel of the miss path (copy_engine = MOE_COPY_KERNEL): copies whole
// experts from the pinned host store, read through its device mapping over the
// host link, into HBM slots or staging entries.
//
// The pages copy a missed expert host -> GPU with a DMA copy on a copy stream
// ([vLLM-cache] "How it works", "async H2D"; [prefetch] copy stream and event
// join).  On this machine a kernel of 64-128 workgroups reading pinned memory moves
// a 12 MiB expert as fast as the DMA engine and a 2.4 MiB INT4 expert about 15 %
// faster, so the library can use either; the bytes and their destination are the
// same.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace moe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kFillThreads = 256;
constexpr size_t kFillUnit = (size_t)64 << 10;   // bytes one workgroup copies per pass

// Work unit u of the launch: job u / units_per_job, bytes [chunk * 64 KiB, +64 KiB)
// of it.  Each lane moves 16-byte words, four loads in flight before their stores.
__global__ __launch_bounds__(kFillThreads) void k_fill(FillBatch b) {
    const size_t upj = (b.bytes + kFillUnit - 1) / kFillUnit;
    const size_t total = upj * (size_t)b.n;
    for (size_t u = blockIdx.x; u < total; u += gridDim.x) {
        const int j = (int)(u / upj);
        const size_t off = (u - (size_t)j * upj) * kFillUnit;
        const size_t nvec = (b.bytes - off < kFillUnit ? b.bytes - off : kFillUnit) / 16;
        const u32x4* __restrict__ src = reinterpret_cast<const u32x4*>(b.job[j].src + off);
        u32x4* __restrict__ dst = reinterpret_cast<u32x4*>(b.job[j].dst + off);
        for (size_t i0 = threadIdx.x; i0 < nvec; i0 += 4 * kFillThreads) {
            u32x4 v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const size_t i = i0 + (size_t)q * kFillThreads;
                if (i < nvec) v[q] = src[i];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const size_t i = i0 + (size_t)q * kFillThreads;
                if (i < nvec) __builtin_nontemporal_store(v[q], dst + i);
            }
        }
    }
}

hipError_t launch_fill(const FillBatch& b, hipStream_t s) {
    if (b.n <= 0 || b.n > kFillMaxJobs || b.bytes % 16) return hipErrorInvalidValue;
    const size_t units = (b.bytes + kFillUnit - 1) / kFillUnit * (size_t)b.n;
    const int grid = (int)(units < (size_t)(b.n > 1 ? 128 : 64) ? units : (b.n > 1 ? 128 : 64));
    hipLaunchKernelGGL(k_fill, dim3(grid), dim3(kFillThreads), 0, s, b);
    return hipGetLastError();
}

}  // namespace moe
