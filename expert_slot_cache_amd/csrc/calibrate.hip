// Calibration kernel for benchmarks (not part of the slot-cache path).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace moe {

// A plain streaming read, each wave reading 4 KiB contiguous (four 16-byte loads
// per lane), xor-folded so the loads stay live.  It measures what one launch of a
// given size can read on this GPU, the ceiling a GEMV launch of the same size is
// compared with.
__global__ __launch_bounds__(256) void k_read_probe(const uint4* __restrict__ p, size_t nvec, unsigned* sink) {
    const size_t base = ((size_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 256 + (threadIdx.x & 63);
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const size_t i = base + (size_t)j * 64;
        v[j] = i < nvec ? p[i] : make_uint4(0, 0, 0, 0);
    }
    unsigned a = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) a ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    if (a == 0x9E3779B9u) sink[threadIdx.x] = a;   // practically never; keeps the loads
}

hipError_t launch_read_probe(const void* p, size_t bytes, unsigned* sink, hipEvent_t start, hipEvent_t stop,
                             hipStream_t s) {
    const size_t nvec = bytes / 16;
    const size_t blocks = (nvec + 1023) / 1024;
    if (blocks == 0 || blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipExtLaunchKernelGGL(k_read_probe, dim3((unsigned)blocks), dim3(256), 0, s, start, stop, 0,
                          static_cast<const uint4*>(p), nvec, sink);
    return hipGetLastError();
}

}  // namespace moe
