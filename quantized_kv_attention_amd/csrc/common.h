// Shared device-side definitions of the gfx950 kernels (layout, bf16, wave reductions).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qkv_attn.h"

namespace qkv {

constexpr int kGroup = QKV_GROUP;        // tokens per key group / channels per value group
constexpr int kTail = QKV_TAIL_SLOTS;    // BF16 tail ring slots
constexpr int kWave = 64;

// One 64-slot block of a plane, head dimension D, BITS-bit codes (4, or 2 for 2-bit
// residual planes).  Offsets in bytes.
template <int D, int BITS = 4>
struct Block {
    static_assert(BITS == 4 || BITS == 2, "4- or 2-bit codes");
    static constexpr int kRowBytes = D * BITS / 8;      // packed codes of one slot
    static constexpr int kVGroups = D / 64;
    // d = 128: K codes [64][kRowBytes] | V records [64][kRowBytes code bytes + 2 x (s, z)]
    //          | K s[D], z[D].  A slot's value codes and value meta sit together (80 bytes
    //          at 4 bits), so a gathered slot's value takes fewer 128-byte lines.
    // d = 64:  K codes [64][kRowBytes] | V codes [64][kRowBytes] | K s[D], z[D]
    //          | V meta [64] x (s, z) (a 40-byte record would break the 16-byte alignment
    //          of the code loads).
    static constexpr bool kVRec = (D == 128);
    static constexpr int kKc = 0;                                            // K codes
    static constexpr int kV = 64 * kRowBytes;                                // value region
    static constexpr int kVStride = kVRec ? kRowBytes + kVGroups * 8 : kRowBytes;
    static constexpr int kKm = kVRec ? kV + 64 * kVStride : 2 * 64 * kRowBytes;  // K s[D], z[D]
    static constexpr int kVmArr = 2 * 64 * kRowBytes + D * 8;                // d = 64: V meta array
    static constexpr int kBytes = kVRec ? kKm + D * 8 : kVmArr + 64 * kVGroups * 8;
    // offsets of slot `row`'s key codes, value codes and value meta (s, z) for group 0
    __host__ __device__ static constexpr int kc(int row) { return kKc + row * kRowBytes; }
    __host__ __device__ static constexpr int vc(int row) { return kV + row * kVStride; }
    __host__ __device__ static constexpr int vm(int row) {
        return kVRec ? kV + row * kVStride + kRowBytes : kVmArr + row * kVGroups * 8;
    }
    // lanes per row when each lane owns 32 channels (16 code bytes at 4 bits, 8 at 2)
    static constexpr int kLpr = D / 32;
    static constexpr int kRpi = kWave / kLpr;           // rows covered by one wave load
    static constexpr int kLaneBytes = 32 * BITS / 8;    // code bytes of a lane's 32 channels
};

// Code width of plane p (0-based) of a cache: the base is 4-bit; residual planes carry RB
// bits; in the full-state codec every plane is 4-bit.
__host__ __device__ constexpr int plane_bits(int p, int RB, bool FULL) { return (p == 0 || FULL) ? 4 : RB; }

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
    int32_t rbits;     // code width of residual planes (4 or 2)
    int32_t full;      // 1: full-state codec (every loop stores its own K/V)
    PlaneArg p[QKV_MAX_LOOPS];
    const uint16_t* tail_k[QKV_MAX_LOOPS];
    const uint16_t* tail_v[QKV_MAX_LOOPS];
    uint32_t* smask;   // [B][cap_ctx]: bit p set iff sparse plane p stores the position, or null
    uint32_t* eflags;  // error word (QKV_FLAG_PLANE_FULL), or null
};

__device__ __forceinline__ float bf16_to_f32(uint32_t u16) { return __uint_as_float(u16 << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <int D, int BITS = 4>
__device__ __forceinline__ const uint8_t* block_ptr(const PlaneArg& P, int H, int b, int h, int blk) {
    return P.data + ((size_t)((size_t)b * H + h) * P.n_blocks + blk) * Block<D, BITS>::kBytes;
}

// Orders one wave's LDS writes before its later LDS reads by other lanes of the same wave.
__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- cross-lane helpers without LDS traffic ----
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kQuadEven = 0xA0;         // quad_perm [0,0,2,2]: lanes 1 and 3 of a quad read lanes 0 and 2
constexpr int kRowRor4 = 0x124;         // row_ror:4
constexpr int kRowRor8 = 0x128;         // row_ror:8 (lane i of a 16-lane row reads lane i ^ 8)
constexpr int kRowMirror = 0x140;       // row_mirror: lane i of a 16-lane row reads lane 15 - i
constexpr int kRowHalfMirror = 0x141;   // row_half_mirror: lane i of an 8-lane half row reads lane 7 - i

// The values of lane l and of lane l ^ 16 (resp. l ^ 32), in some order, from gfx950's
// v_permlane16_swap / v_permlane32_swap with both operands equal: a VALU exchange across
// 16-lane rows (resp. wave halves).
__device__ __forceinline__ float2 pair_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float2 pair_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float v) { const float2 p = pair_xor16(v); return p.x + p.y; }
// Bitwise OR over the wave (the raw bits move through the same lane exchanges).
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
    v |= __float_as_uint(dpp<0xB1>(__uint_as_float(v)));   // quad_perm [1,0,3,2]
    v |= __float_as_uint(dpp<0x4E>(__uint_as_float(v)));   // quad_perm [2,3,0,1]
    v |= __float_as_uint(dpp<0x141>(__uint_as_float(v)));  // row_half_mirror
    v |= __float_as_uint(dpp<0x140>(__uint_as_float(v)));  // row_mirror
    float2 p = pair_xor16(__uint_as_float(v));
    v = __float_as_uint(p.x) | __float_as_uint(p.y);
    p = pair_xor32(__uint_as_float(v));
    return __float_as_uint(p.x) | __float_as_uint(p.y);
}
__device__ __forceinline__ float add_xor32(float v) { const float2 p = pair_xor32(v); return p.x + p.y; }

// Whole-wave reductions, the result in every lane: DPP within each 16-lane row, then the
// rows through the lane swaps.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<kQuadXor1>(v));
    v = fmaxf(v, dpp<kQuadXor2>(v));
    v = fmaxf(v, dpp<kRowHalfMirror>(v));
    v = fmaxf(v, dpp<kRowMirror>(v));
    float2 p = pair_xor16(v);
    v = fmaxf(p.x, p.y);
    p = pair_xor32(v);
    return fmaxf(p.x, p.y);
}
__device__ __forceinline__ float wave_min(float v) {
    v = fminf(v, dpp<kQuadXor1>(v));
    v = fminf(v, dpp<kQuadXor2>(v));
    v = fminf(v, dpp<kRowHalfMirror>(v));
    v = fminf(v, dpp<kRowMirror>(v));
    float2 p = pair_xor16(v);
    v = fminf(p.x, p.y);
    p = pair_xor32(v);
    return fminf(p.x, p.y);
}
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<kQuadXor1>(v);
    v += dpp<kQuadXor2>(v);
    v += dpp<kRowHalfMirror>(v);
    v += dpp<kRowMirror>(v);
    v = add_xor16(v);
    return add_xor32(v);
}

// Sets the wave's instruction issue priority (s_setprio, 0..3) from the share of its work
// still left: a wave with more left is preferred.  The arbiter otherwise prefers the oldest
// wave, so workgroups sharing a CU would run one after another.
__device__ __forceinline__ void prio_by_work_left(int left, int total) {
    int lv = total > 0 ? (4 * left) / total : 0;
    lv = __builtin_amdgcn_readfirstlane(lv > 3 ? 3 : lv);
    if (lv == 3)
        __builtin_amdgcn_s_setprio(3);
    else if (lv == 2)
        __builtin_amdgcn_s_setprio(2);
    else if (lv == 1)
        __builtin_amdgcn_s_setprio(1);
    else
        __builtin_amdgcn_s_setprio(0);
}

// Eight bf16 values (16 bytes) to floats.
__device__ __forceinline__ void bf16x8(const uint4 w, float* f) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = bf16_to_f32(ws[e] & 0xFFFFu);
        f[2 * e + 1] = bf16_to_f32(ws[e] >> 16);
    }
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

// sum over aligned groups of N = 8 or 16 lanes, in every lane of the group
template <int N>
__device__ __forceinline__ float lane_group_sum(float v) {
    static_assert(N == 8 || N == 16, "8- or 16-lane groups");
    v += dpp<kQuadXor1>(v);
    v += dpp<kQuadXor2>(v);
    v += dpp<kRowHalfMirror>(v);
    if (N == 16) v += dpp<kRowMirror>(v);
    return v;
}
// sum over the LPR consecutive lanes of a row group (LPR = 2 or 4)
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
    v += dpp<kQuadXor1>(v);
    if (LPR == 4) v += dpp<kQuadXor2>(v);
    return v;
}
// sum over the whole wave, result in every lane
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += dpp<kQuadXor1>(v);
    v += dpp<kQuadXor2>(v);
    v += dpp<kRowRor4>(v);
    v += dpp<kRowRor8>(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// ---- nibble codes to floats through the FP8 converter ----
// A byte b in [0, 15] read as OCP FP8 E4M3 (bias 7) is exactly b * 2^-9: codes 0-7 are the
// subnormals m * 2^-9, codes 8-15 the first normal binade (8 + m) * 2^-9.  Masking a code
// word to its low (or high) nibbles and converting two bytes per instruction turns 8 codes
// into floats with 7 instructions; callers fold the 2^9 into their multiplier.
constexpr float kFp8CodeScale = 512.0f;
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void codes8_fp8(uint32_t w, float* c) {
    const uint32_t lo = w & 0x0F0F0F0Fu;          // channels 0, 2, 4, 6
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // channels 1, 3, 5, 7
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
    const f32x2 e = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
    const f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
    c[0] = a.x; c[2] = a.y; c[4] = b.x; c[6] = b.y;
    c[1] = e.x; c[3] = e.y; c[5] = f.x; c[7] = f.y;
}

// sum_c q[c] * code[c] * 2^-9 over the 32 codes of 16 bytes
__device__ __forceinline__ float dot32_fp8(const uint4 w, const float* q) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float c[8];
        codes8_fp8(ws[k], c);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            a0 = fmaf(c[e], q[8 * k + e], a0);
            a1 = fmaf(c[e + 1], q[8 * k + e + 1], a1);
        }
    }
    return a0 + a1;
}

// acc[c] += wt * code[c] * 2^-9 for the 32 codes of 16 bytes
__device__ __forceinline__ void axpy32_fp8(const uint4 w, float wt, float* acc) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float c[8];
        codes8_fp8(ws[k], c);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[8 * k + e] = fmaf(c[e], wt, acc[8 * k + e]);
    }
}

// ---- 2-bit codes (channel 4i + m in bits 2m, 2m + 1 of byte i) through the FP8 converter:
// a byte b in [0, 3] read as E4M3 is the subnormal b * 2^-9, as for the 4-bit codes ----
// 16 codes of one 32-bit word, times 2^-9, in channel order
__device__ __forceinline__ void codes16_fp8_2b(uint32_t w, float* c) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t x = (w >> (2 * m)) & 0x03030303u;   // channels m, 4 + m, 8 + m, 12 + m
        const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(x, false);
        const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(x, true);
        c[m] = a.x; c[4 + m] = a.y; c[8 + m] = b.x; c[12 + m] = b.y;
    }
}

// sum_c q[c] * code[c] * 2^-9 over the 32 codes of 8 bytes (w.x, w.y)
__device__ __forceinline__ float dot32_fp8_2b(const uint4 w, const float* q) {
    float a0 = 0.f, a1 = 0.f;
    float c[16];
    codes16_fp8_2b(w.x, c);
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
        a0 = fmaf(c[e], q[e], a0);
        a1 = fmaf(c[e + 1], q[e + 1], a1);
    }
    codes16_fp8_2b(w.y, c);
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
        a0 = fmaf(c[e], q[16 + e], a0);
        a1 = fmaf(c[e + 1], q[16 + e + 1], a1);
    }
    return a0 + a1;
}

// acc[c] += wt * code[c] * 2^-9 for the 32 codes of 8 bytes (w.x, w.y)
__device__ __forceinline__ void axpy32_fp8_2b(const uint4 w, float wt, float* acc) {
    float c[16];
    codes16_fp8_2b(w.x, c);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = fmaf(c[e], wt, acc[e]);
    codes16_fp8_2b(w.y, c);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[16 + e] = fmaf(c[e], wt, acc[16 + e]);
}

// 32 channels of one lane at BITS bits: dot with q / axpy into acc (codes times 2^-9)
template <int BITS>
__device__ __forceinline__ float dot32_bits(const uint4 w, const float* q) {
    if constexpr (BITS == 4) return dot32_fp8(w, q);
    else return dot32_fp8_2b(w, q);
}
template <int BITS>
__device__ __forceinline__ void axpy32_bits(const uint4 w, float wt, float* acc) {
    if constexpr (BITS == 4) axpy32_fp8(w, wt, acc);
    else axpy32_fp8_2b(w, wt, acc);
}

// Merge of split-softmax partials of one (sequence, head), laid out as n records of
// `stride` floats: [max, sum, a[0..D), (b[0..D) if HAS_B)], by NW waves.
// Every wave forms the global max M and L = sum_s sum_s * exp(max_s - M) itself: lanes
// over records, then fixed-order wave reductions, so all waves hold the same M and L and
// need no barrier for them.  Wave w then adds up records w, w + NW, w + 2 NW, ... in record
// order (a rescaled by exp(max_s - M), b plain), U records in flight, and leaves its sums in
// red[w * RS + c] (a) and red[w * RS + D + c] (b), RS = (HAS_B ? 2 : 1) * D.  The caller
// adds the NW wave sums in wave order after a barrier.
template <int D, int NW, int U, bool HAS_B>
__device__ __forceinline__ void merge_records(const float* pp, int n, int stride, float* red, float* gmax,
                                              float* gsum) {
    constexpr float kNeg = -__builtin_huge_valf();
    constexpr int CPL = D / 64;  // channels per lane
    constexpr int RS = (HAS_B ? 2 : 1) * D;
    static_assert(CPL == 1 || CPL == 2, "head_dim 64 or 128");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float m0 = lane < n ? pp[(size_t)lane * stride] : kNeg;
    const float l0 = lane < n ? pp[(size_t)lane * stride + 1] : 0.f;
    const float m1 = lane + 64 < n ? pp[(size_t)(lane + 64) * stride] : kNeg;
    const float l1 = lane + 64 < n ? pp[(size_t)(lane + 64) * stride + 1] : 0.f;
    float m = fmaxf(m0, m1);
    for (int s = lane + 128; s < n; s += 64) m = fmaxf(m, pp[(size_t)s * stride]);
    const float M = wave_max(m);
    float l = 0.f;
    if (m0 != kNeg) l = l0 * __expf(m0 - M);
    if (m1 != kNeg) l = fmaf(l1, __expf(m1 - M), l);
    for (int s = lane + 128; s < n; s += 64) {
        const float ms = pp[(size_t)s * stride];
        if (ms != kNeg) l = fmaf(pp[(size_t)s * stride + 1], __expf(ms - M), l);
    }
    *gmax = M;
    *gsum = wave_sum(l);

    float a[CPL], b[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) a[i] = b[i] = 0.f;
    for (int s0 = wave; s0 < n; s0 += U * NW) {
        float ms[U], av[U][CPL], bv[U][CPL];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = s0 + u * NW;
            const float* r = pp + (size_t)(s < n ? s : n - 1) * stride;  // in range; weighted 0 if s >= n
            ms[u] = s < n ? r[0] : kNeg;
            if (CPL == 2) {
                const float2 x = *reinterpret_cast<const float2*>(r + 2 + 2 * lane);
                av[u][0] = x.x;
                av[u][CPL - 1] = x.y;
                if (HAS_B) {
                    const float2 y = *reinterpret_cast<const float2*>(r + 2 + D + 2 * lane);
                    bv[u][0] = y.x;
                    bv[u][CPL - 1] = y.y;
                }
            } else {
                av[u][0] = r[2 + lane];
                if (HAS_B) bv[u][0] = r[2 + D + lane];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float w = ms[u] == kNeg ? 0.f : __expf(ms[u] - M);
#pragma unroll
            for (int i = 0; i < CPL; ++i) a[i] = fmaf(av[u][i], w, a[i]);
            if (HAS_B && s0 + u * NW < n) {
#pragma unroll
                for (int i = 0; i < CPL; ++i) b[i] += bv[u][i];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        red[wave * RS + CPL * lane + i] = a[i];
        if (HAS_B) red[wave * RS + D + CPL * lane + i] = b[i];
    }
}

// Loads of data a kernel reads once (plane codes and metadata streamed by the readers, the
// gathered rows of the sparse splice, source rows of the encoder): the nontemporal cache
// policy.  Measured at 32K context, it took ~1.2 us off each dense call and ~2.3 us off
// each sparse call against the default policy.
__device__ __forceinline__ uint32_t ld_stream_u32(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ float ld_stream_f32(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const float*>(p));
}
__device__ __forceinline__ float2 ld_stream_f2(const void* p) {
    typedef float v2 __attribute__((ext_vector_type(2)));
    const v2 v = __builtin_nontemporal_load(reinterpret_cast<const v2*>(p));
    return make_float2(v.x, v.y);
}
__device__ __forceinline__ uint4 ld_stream_u4(const void* p) {
    typedef unsigned v4 __attribute__((ext_vector_type(4)));
    const v4 v = __builtin_nontemporal_load(reinterpret_cast<const v4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_stream_u2(const void* p) {
    typedef unsigned v2 __attribute__((ext_vector_type(2)));
    const v2 v = __builtin_nontemporal_load(reinterpret_cast<const v2*>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t ld_stream_u16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
}
// A lane's 32 channels of codes at BITS bits (16 bytes, or 8 in .x, .y)
template <int BITS>
__device__ __forceinline__ uint4 ld_codes32(const uint8_t* p) {
    if constexpr (BITS == 4) return ld_stream_u4(p);
    else {
        const uint2 v = ld_stream_u2(p);
        return make_uint4(v.x, v.y, 0u, 0u);
    }
}
// A lane's 8 channels of codes at BITS bits (4 bytes, or 2), as the low bits of a word
template <int BITS>
__device__ __forceinline__ uint32_t ld_codes8(const uint8_t* p) {
    if constexpr (BITS == 4) return ld_stream_u32(p);
    else return ld_stream_u16(p);
}
// 8 codes of a word (4-bit: channel 2i low / 2i + 1 high nibble of byte i; 2-bit: channel
// 4i + m in bits 2m of byte i) as floats
template <int BITS>
__device__ __forceinline__ void codes8_bits(uint32_t w, float* c) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if constexpr (BITS == 4)
            c[i] = (float)((w >> (4 * i)) & 15u);
        else
            c[i] = (float)((w >> (2 * i)) & 3u);
    }
}

}  // namespace qkv
