// Plain streaming read: the bandwidth a read with nothing else to do reaches on the device
// (with the readers' nontemporal load policy), set beside the readers' rates.  Not part of
// the attention path.
#include "launch.h"

namespace qkv {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;  // 16-byte loads per lane in flight together

// Workgroup g reads tiles g, g + G, g + 2G, ... of 256 x 8 16-byte words (lane-contiguous
// within each of the 8 rows of a tile) and stores the XOR of every 32-bit word it read.
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                                     uint32_t* __restrict__ sink) {
    constexpr size_t kTile = (size_t)kStreamThreads * kStreamUnroll;
    uint32_t acc = 0;
    for (size_t t0 = (size_t)blockIdx.x * kTile; t0 < n16; t0 += (size_t)gridDim.x * kTile) {
        uint4 v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            const size_t i = t0 + (size_t)u * kStreamThreads + threadIdx.x;
            v[u] = i < n16 ? ld_stream_u4(src + i) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    __shared__ uint32_t red[kStreamThreads];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int s = kStreamThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

int launch_stream_read(const void* src, size_t n_bytes, uint32_t* sink, hipStream_t st) {
    stream_read_kernel<<<QKV_STREAM_READ_GROUPS, kStreamThreads, 0, st>>>(static_cast<const uint4*>(src), n_bytes / 16,
                                                                          sink);
    return hipGetLastError() == hipSuccess ? QKV_OK : QKV_ELAUNCH;
}

}  // namespace qkv
