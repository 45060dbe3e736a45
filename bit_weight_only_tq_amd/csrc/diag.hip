// Measurement kernel: a plain streaming read of device memory, the best a
// single launch of given size can do against HBM under the same launch
// regime as the GEMV kernels (used for the measured bandwidth ceiling that
// the decode figures are compared with).

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;  // 16-byte loads in flight per thread

// Workgroup b reads chunks [b * per, min((b + 1) * per, chunks)) of 16
// bytes, kReadUnroll loads issued before any is consumed, and folds them
// with XOR.  Nothing is stored unless the fold equals an improbable value,
// so the write traffic is nil while the loads cannot be elided.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4* src, int64_t chunks, int64_t per,
                                                                    uint32_t* sink) {
    const int64_t b0 = (int64_t)blockIdx.x * per;
    const int64_t b1 = b0 + per < chunks ? b0 + per : chunks;
    uint32_t acc = 0;
    for (int64_t c = b0 + threadIdx.x; c < b1; c += (int64_t)kReadThreads * kReadUnroll) {
        uint4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) {
            const int64_t i = c + (int64_t)u * kReadThreads;
            v[u] = i < b1 ? src[i] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == (0x9E3779B9u ^ (uint32_t)blockIdx.x ^ ((uint32_t)threadIdx.x << 20))) sink[blockIdx.x] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int64_t blocks, hipStream_t s) {
    const int64_t chunks = (int64_t)(bytes / 16);
    if (chunks <= 0 || blocks <= 0 || blocks > chunks || blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int64_t per = (chunks + blocks - 1) / blocks;
    const int64_t grid = (chunks + per - 1) / per;  // every workgroup has work, grid <= blocks
    stream_read_kernel<<<dim3((unsigned)grid), dim3(kReadThreads), 0, s>>>(static_cast<const uint4*>(src), chunks, per,
                                                                         sink);
    return hipGetLastError();
}

}  // namespace tq
