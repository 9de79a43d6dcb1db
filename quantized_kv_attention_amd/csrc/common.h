// Shared device-side definitions of the gfx950 kernels (layout, bf16, wave reductions).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qkv_attn.h"

namespace qkv {

constexpr int kGroup = QKV_GROUP;        // tokens per key group / channels per value group
constexpr int kTail = QKV_TAIL_SLOTS;    // BF16 tail ring slots
constexpr int kWave = 64;

// One 64-slot block of a plane, head dimension D (bytes).
template <int D>
struct Block {
    static constexpr int kRowBytes = D / 2;             // packed codes of one slot
    static constexpr int kKc = 0;                       // K codes [64][D/2]
    static constexpr int kVc = 64 * D / 2;              // V codes [64][D/2]
    static constexpr int kKm = 64 * D;                  // K s[D], z[D]
    static constexpr int kVm = 64 * D + D * 8;          // V [64][D/64] x (s, z)
    static constexpr int kBytes = kVm + 64 * (D / 64) * 8;
    static constexpr int kVGroups = D / 64;
    // lanes per row when each lane owns 32 channels (16 code bytes)
    static constexpr int kLpr = D / 32;
    static constexpr int kRpi = kWave / kLpr;           // rows covered by one wave load
};

// Per-plane view passed by value in kernel arguments.
struct PlaneArg {
    const uint8_t* data;
    const int32_t* rowmap;
    const int32_t* rowpos;
    const int32_t* rowstart;
    int32_t n_blocks;
    int32_t dense;
};

struct CacheArg {
    int32_t B, H, cap_ctx, n_ctx, n_body;
    int32_t nplanes;
    PlaneArg p[QKV_MAX_LOOPS];
    const uint16_t* tail_k[QKV_MAX_LOOPS];
    const uint16_t* tail_v[QKV_MAX_LOOPS];
};

__device__ __forceinline__ float bf16_to_f32(uint32_t u16) { return __uint_as_float(u16 << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <int D>
__device__ __forceinline__ const uint8_t* block_ptr(const PlaneArg& P, int H, int b, int h, int blk) {
    return P.data + ((size_t)((size_t)b * H + h) * P.n_blocks + blk) * Block<D>::kBytes;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Unpacks 32 codes of one lane (16 bytes; channel 2i low nibble, 2i+1 high nibble)
// and returns sum_c q[c] * code[c].
__device__ __forceinline__ float dot32_codes(const uint4 w, const float* q) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t lo = ws[k] & 0x0F0F0F0Fu;
        const uint32_t hi = (ws[k] >> 4) & 0x0F0F0F0Fu;
        a0 = fmaf((float)(lo & 0xFFu), q[8 * k + 0], a0);
        a1 = fmaf((float)(hi & 0xFFu), q[8 * k + 1], a1);
        a0 = fmaf((float)((lo >> 8) & 0xFFu), q[8 * k + 2], a0);
        a1 = fmaf((float)((hi >> 8) & 0xFFu), q[8 * k + 3], a1);
        a0 = fmaf((float)((lo >> 16) & 0xFFu), q[8 * k + 4], a0);
        a1 = fmaf((float)((hi >> 16) & 0xFFu), q[8 * k + 5], a1);
        a0 = fmaf((float)(lo >> 24), q[8 * k + 6], a0);
        a1 = fmaf((float)(hi >> 24), q[8 * k + 7], a1);
    }
    return a0 + a1;
}

// acc[c] += wt * code[c] for the 32 codes of one lane.
__device__ __forceinline__ void axpy32_codes(const uint4 w, float wt, float* acc) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t lo = ws[k] & 0x0F0F0F0Fu;
        const uint32_t hi = (ws[k] >> 4) & 0x0F0F0F0Fu;
        acc[8 * k + 0] = fmaf((float)(lo & 0xFFu), wt, acc[8 * k + 0]);
        acc[8 * k + 1] = fmaf((float)(hi & 0xFFu), wt, acc[8 * k + 1]);
        acc[8 * k + 2] = fmaf((float)((lo >> 8) & 0xFFu), wt, acc[8 * k + 2]);
        acc[8 * k + 3] = fmaf((float)((hi >> 8) & 0xFFu), wt, acc[8 * k + 3]);
        acc[8 * k + 4] = fmaf((float)((lo >> 16) & 0xFFu), wt, acc[8 * k + 4]);
        acc[8 * k + 5] = fmaf((float)((hi >> 16) & 0xFFu), wt, acc[8 * k + 5]);
        acc[8 * k + 6] = fmaf((float)(lo >> 24), wt, acc[8 * k + 6]);
        acc[8 * k + 7] = fmaf((float)(hi >> 24), wt, acc[8 * k + 7]);
    }
}

// Codes of one lane as floats (channel order).
__device__ __forceinline__ void unpack32_codes(const uint4 w, float* c) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t byte = (ws[k] >> (8 * m)) & 0xFFu;
            c[8 * k + 2 * m] = (float)(byte & 0xFu);
            c[8 * k + 2 * m + 1] = (float)(byte >> 4);
        }
    }
}

}  // namespace qkv
