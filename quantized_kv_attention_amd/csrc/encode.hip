// Residual-quantize encoder and BF16 tail append (gfx950).
//
// Loop 1's K/V become the INT4 base; loop r >= 2 stores Q(X^(r) - Xhat^(r-1)) for its
// active tokens, where Xhat^(r-1) is rebuilt exactly from planes 1..r-1 (project page,
// The Method, STEP 01 and STEP 03; flozi.net explainer section 3: keys per channel over
// 64 tokens, values per token over 64 channels, asymmetric, group 64).
//
// Exactness: every codec step is a single IEEE fp32 operation, as the oracle does it
// (correctly rounded division, rint half-to-even, fmaf dequant, no contraction).
#include "launch.h"

#pragma clang fp contract(off)

namespace qkv {

// Loop-`np` reconstruction Xhat (np >= 1 planes) of channel c of position pos.
template <int D>
__device__ float chain_value(const CacheArg& ca, int kind, int b, int h, int pos, int c, int np) {
    float acc = 0.f;
    const int cap = ca.cap_ctx;
    for (int p = 0; p < np; ++p) {
        const PlaneArg& Q = ca.p[p];
        const int slot = Q.dense ? pos : Q.rowmap[(size_t)b * cap + pos];
        if (slot < 0 || slot >= Q.n_blocks * 64) continue;  // not stored in loop p+1: keeps loop p's value
        const uint8_t* blk = block_ptr<D>(Q, ca.H, b, h, slot >> 6);
        const int row = slot & 63;
        const uint8_t byte = blk[(kind ? Block<D>::kVc : Block<D>::kKc) + row * (D / 2) + (c >> 1)];
        const float code = (float)((c & 1) ? (byte >> 4) : (byte & 15));
        float s, z;
        if (kind == 0) {
            const float* m = reinterpret_cast<const float*>(blk + Block<D>::kKm);
            s = m[c];
            z = m[D + c];
        } else {
            const float* m = reinterpret_cast<const float*>(blk + Block<D>::kVm);
            s = m[(row * (D / 64) + (c >> 6)) * 2];
            z = m[(row * (D / 64) + (c >> 6)) * 2 + 1];
        }
        const float deq = __builtin_fmaf(code, s, z);
        acc = (p == 0) ? deq : acc + deq;
    }
    return acc;
}

__device__ __forceinline__ uint8_t quant_code(float x, float s, float z) {
    if (s == 0.f) return 0;
    float t = x - z;
    float u = t / s;
    float r = __builtin_rintf(u);
    r = r < 0.f ? 0.f : r;
    r = r > 15.f ? 15.f : r;
    return (uint8_t)r;
}

template <int D>
__global__ __launch_bounds__(256) void encode_group_kernel(CacheArg ca, int loop, int pos0, int n_pos,
                                                           const int32_t* __restrict__ act_pos,
                                                           const int32_t* __restrict__ n_act, int ld_act,
                                                           const uint16_t* __restrict__ ksrc,
                                                           const uint16_t* __restrict__ vsrc, int ld_src,
                                                           int32_t* __restrict__ rowpos) {
    const int g = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const PlaneArg& P = ca.p[loop - 1];
    const bool dense = P.dense != 0;
    const int na = dense ? n_pos : min(n_act[b], n_pos);
    const int r0 = g * 64;
    if (r0 >= na) return;
    const int nr = min(64, na - r0);
    const int nstart = ca.cap_ctx / 64 + 1;
    const int base = dense ? pos0 : P.rowstart[(size_t)b * nstart + pos0 / 64];
    const int blk_idx = (base + r0) >> 6;
    if (blk_idx >= P.n_blocks) return;  // sparse plane full: rows beyond its capacity are not stored
    uint8_t* blk = const_cast<uint8_t*>(block_ptr<D>(P, ca.H, b, h, blk_idx));
    const bool from_tail = (ksrc == nullptr);

    __shared__ float X[64][D + 1];
    __shared__ uint8_t codes[64][D];
    __shared__ int spos[64];
    __shared__ float red_mn[256 / D][D], red_mx[256 / D][D];
    __shared__ float ks[D], kz[D];
    __shared__ float vs[64][D / 64], vz[64][D / 64];

    if (tid < 64) {
        int p = -1;
        if (tid < nr) p = dense ? (pos0 + r0 + tid) : act_pos[(size_t)b * ld_act + r0 + tid];
        spos[tid] = (p >= pos0 && p < pos0 + n_pos) ? p : -1;  // positions outside the call are not stored
    }
    __syncthreads();

    for (int kind = 0; kind < 2; ++kind) {
        const uint16_t* src = kind ? vsrc : ksrc;
        const uint16_t* tail = kind ? ca.tail_v[loop - 1] : ca.tail_k[loop - 1];
        for (int e = tid; e < 64 * D; e += 256) {
            const int row = e / D, c = e % D;
            float x = 0.f;
            if (row < nr && spos[row] >= 0) {
                const int pos = spos[row];
                uint32_t bits;
                if (from_tail)
                    bits = tail[((size_t)((size_t)b * ca.H + h) * kTail + (pos % kTail)) * D + c];
                else
                    bits = src[((size_t)((size_t)b * ca.H + h) * ld_src + r0 + row) * D + c];
                x = bf16_to_f32(bits);
                if (loop > 1) x = x - chain_value<D>(ca, kind, b, h, pos, c, loop - 1);
            }
            X[row][c] = x;
        }
        __syncthreads();

        if (kind == 0) {
            // keys: per channel over the group's stored rows
            constexpr int kSplit = 256 / D;
            constexpr int kRows = 64 / kSplit;
            const int c = tid % D, part = tid / D;
            float mn = 0.f, mx = 0.f;
            bool any = false;
            for (int r = part * kRows; r < (part + 1) * kRows; ++r) {
                if (r >= nr) break;
                const float v = X[r][c];
                if (!any) { mn = v; mx = v; any = true; }
                else { mn = v < mn ? v : mn; mx = v > mx ? v : mx; }
            }
            red_mn[part][c] = any ? mn : __builtin_huge_valf();
            red_mx[part][c] = any ? mx : -__builtin_huge_valf();
            __syncthreads();
            if (tid < D) {
                float a = red_mn[0][tid], bmx = red_mx[0][tid];
#pragma unroll
                for (int q = 1; q < kSplit; ++q) {
                    a = red_mn[q][tid] < a ? red_mn[q][tid] : a;
                    bmx = red_mx[q][tid] > bmx ? red_mx[q][tid] : bmx;
                }
                float range = bmx - a;
                float s = range / 15.0f;
                s = s + 0.0f;
                ks[tid] = s;
                kz[tid] = a + 0.0f;
            }
            __syncthreads();
            for (int r = part * kRows; r < (part + 1) * kRows; ++r)
                codes[r][c] = (r < nr) ? quant_code(X[r][c], ks[c], kz[c]) : (uint8_t)0;
        } else {
            // values: per row over each 64-channel group
            constexpr int kG = D / 64;
            if (tid < 64 * kG) {
                const int r = tid / kG, gg = tid % kG;
                if (r < nr) {
                    float mn = X[r][gg * 64], mx = mn;
                    for (int c = 1; c < 64; ++c) {
                        const float v = X[r][gg * 64 + c];
                        mn = v < mn ? v : mn;
                        mx = v > mx ? v : mx;
                    }
                    float range = mx - mn;
                    float s = range / 15.0f;
                    s = s + 0.0f;
                    const float z = mn + 0.0f;
                    vs[r][gg] = s;
                    vz[r][gg] = z;
                    for (int c = 0; c < 64; ++c) codes[r][gg * 64 + c] = quant_code(X[r][gg * 64 + c], s, z);
                } else {
                    vs[r][gg] = 0.f;
                    vz[r][gg] = 0.f;
                    for (int c = 0; c < 64; ++c) codes[r][gg * 64 + c] = 0;
                }
            }
        }
        __syncthreads();

        // pack two channels per byte and store the block
        uint8_t* dst = blk + (kind ? Block<D>::kVc : Block<D>::kKc);
        for (int e = tid; e < 2 * D; e += 256) {
            const int row = e / (D / 32), byte0 = (e % (D / 32)) * 16;
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t v = 0;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int by = byte0 + 4 * q + m;
                    const uint32_t lo = codes[row][2 * by], hi = codes[row][2 * by + 1];
                    v |= (lo | (hi << 4)) << (8 * m);
                }
                w[q] = v;
            }
            *reinterpret_cast<uint4*>(dst + row * (D / 2) + byte0) = make_uint4(w[0], w[1], w[2], w[3]);
        }
        if (kind == 0) {
            float* m = reinterpret_cast<float*>(blk + Block<D>::kKm);
            for (int c = tid; c < D; c += 256) {
                m[c] = ks[c];
                m[D + c] = kz[c];
            }
        } else {
            float* m = reinterpret_cast<float*>(blk + Block<D>::kVm);
            for (int e = tid; e < 64 * (D / 64); e += 256) {
                m[2 * e] = vs[e / (D / 64)][e % (D / 64)];
                m[2 * e + 1] = vz[e / (D / 64)][e % (D / 64)];
            }
        }
        __syncthreads();
    }

    if (!dense && h == 0 && tid < 64)
        rowpos[(size_t)b * P.n_blocks * 64 + base + r0 + tid] = spos[tid];
}

// position -> slot map and block starts of a sparse plane for [pos0, pos0 + n_pos)
__global__ __launch_bounds__(256) void encode_maps_kernel(int cap_ctx, int pos0, int n_pos,
                                                          const int32_t* __restrict__ act_pos,
                                                          const int32_t* __restrict__ n_act, int ld_act,
                                                          int32_t* __restrict__ rowmap,
                                                          int32_t* __restrict__ rowstart) {
    const int b = blockIdx.y;
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int nstart = cap_ctx / 64 + 1;
    const int na = min(n_act[b], n_pos);
    const int base = rowstart[(size_t)b * nstart + pos0 / 64];
    const int32_t* a = act_pos + (size_t)b * ld_act;
    if (i < n_pos) {
        const int p = pos0 + i;
        int lo = 0, hi = na;  // first index with a[idx] >= p
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (a[mid] < p) lo = mid + 1; else hi = mid;
        }
        rowmap[(size_t)b * cap_ctx + p] = (lo < na && a[lo] == p) ? base + lo : -1;
        if ((i & 63) == 0 && i > 0) rowstart[(size_t)b * nstart + p / 64] = base + lo;
    }
    if (i == 0) rowstart[(size_t)b * nstart + (pos0 + n_pos) / 64] = base + ((na + 63) / 64) * 64;
}

__global__ __launch_bounds__(64) void append_tail_kernel(int H, int D, int pos0, int n_rows,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         uint16_t* __restrict__ tk, uint16_t* __restrict__ tv) {
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const size_t src = ((size_t)((size_t)b * H + h) * n_rows + i) * D;
    const size_t dst = ((size_t)((size_t)b * H + h) * kTail + ((pos0 + i) % kTail)) * D;
    for (int c = threadIdx.x; c < D; c += 64) {
        tk[dst + c] = k[src + c];
        tv[dst + c] = v[src + c];
    }
}

// every loop at once: k, v [loops][B][H][n_rows][D]; grid.z = B * loops
__global__ __launch_bounds__(64) void append_tail_all_kernel(CacheArg ca, int D, int pos0, int n_rows,
                                                             const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v) {
    const int i = blockIdx.x, h = blockIdx.y;
    const int b = blockIdx.z % ca.B, r = blockIdx.z / ca.B;
    const size_t src = ((((size_t)r * ca.B + b) * ca.H + h) * n_rows + i) * D;
    const size_t dst = ((size_t)((size_t)b * ca.H + h) * kTail + ((pos0 + i) % kTail)) * D;
    uint16_t* tk = const_cast<uint16_t*>(ca.tail_k[r]);
    uint16_t* tv = const_cast<uint16_t*>(ca.tail_v[r]);
    for (int c = threadIdx.x; c < D; c += 64) {
        tk[dst + c] = k[src + c];
        tv[dst + c] = v[src + c];
    }
}

int launch_append_all(const CacheArg& ca, int D, int pos0, int n_rows, const uint16_t* k, const uint16_t* v,
                      hipStream_t st) {
    dim3 grid(n_rows, ca.H, ca.B * ca.nplanes);
    append_tail_all_kernel<<<grid, 64, 0, st>>>(ca, D, pos0, n_rows, k, v);
    return hipGetLastError() == hipSuccess ? QKV_OK : QKV_ELAUNCH;
}

int launch_encode(const CacheArg& ca, int D, int loop, int pos0, int n_pos, const int32_t* act_pos,
                  const int32_t* n_act, int ld_act, const uint16_t* ksrc, const uint16_t* vsrc, int ld_src,
                  hipStream_t st) {
    const PlaneArg& P = ca.p[loop - 1];
    const int ngroups = (n_pos + 63) / 64;
    dim3 grid(ngroups, ca.H, ca.B);
    int32_t* rowpos = const_cast<int32_t*>(P.rowpos);
    if (D == 128)
        encode_group_kernel<128><<<grid, 256, 0, st>>>(ca, loop, pos0, n_pos, act_pos, n_act, ld_act, ksrc, vsrc,
                                                       ld_src, rowpos);
    else
        encode_group_kernel<64><<<grid, 256, 0, st>>>(ca, loop, pos0, n_pos, act_pos, n_act, ld_act, ksrc, vsrc,
                                                      ld_src, rowpos);
    if (hipGetLastError() != hipSuccess) return QKV_ELAUNCH;
    if (!P.dense) {
        dim3 g2((n_pos + 255) / 256, ca.B);
        encode_maps_kernel<<<g2, 256, 0, st>>>(ca.cap_ctx, pos0, n_pos, act_pos, n_act, ld_act,
                                               const_cast<int32_t*>(P.rowmap), const_cast<int32_t*>(P.rowstart));
        if (hipGetLastError() != hipSuccess) return QKV_ELAUNCH;
    }
    return QKV_OK;
}

int launch_append(int B, int H, int D, int pos0, int n_rows, const uint16_t* k, const uint16_t* v, uint16_t* tk,
                  uint16_t* tv, hipStream_t st) {
    dim3 grid(n_rows, H, B);
    append_tail_kernel<<<grid, 64, 0, st>>>(H, D, pos0, n_rows, k, v, tk, tv);
    return hipGetLastError() == hipSuccess ? QKV_OK : QKV_ELAUNCH;
}

}  // namespace qkv
