// Measurement aid: the rate at which this device streams a buffer from HBM
// once, with the verify kernels' load shape (16-byte loads, every load of a
// thread issued before any is used).  Used as context for the verify
// kernels' achieved bandwidth; no part of the verify step.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specv_internal.hpp"

namespace specv {
namespace {

constexpr int kReadBlock = 256;
constexpr int kReadUnroll = 8;      // 16-byte loads in flight per thread (32 KB per workgroup)

__global__ __launch_bounds__(kReadBlock) void k_read_ceiling(const uint4* buf, long long n16,
                                                             unsigned* sink) {
    const long long per_round = (long long)gridDim.x * kReadBlock * kReadUnroll;
    unsigned acc = 0;
    for (long long base = (long long)blockIdx.x * kReadBlock * kReadUnroll; base < n16;
         base += per_round) {
        uint4 q[kReadUnroll];
#pragma unroll
        for (int j = 0; j < kReadUnroll; ++j) {
            const long long i = base + (long long)j * kReadBlock + threadIdx.x;
            q[j] = i < n16 ? buf[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < kReadUnroll; ++j) acc ^= q[j].x ^ q[j].y ^ q[j].z ^ q[j].w;
    }
    __shared__ unsigned red[kReadBlock];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int s = kReadBlock / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

}  // namespace

hipError_t launch_read_ceiling(const void* buf, long long n16, int grid, unsigned* sink,
                               hipStream_t stream) {
    hipLaunchKernelGGL(k_read_ceiling, dim3((unsigned)grid), dim3(kReadBlock), 0, stream,
                       static_cast<const uint4*>(buf), n16, sink);
    return hipGetLastError();
}

}  // namespace specv
