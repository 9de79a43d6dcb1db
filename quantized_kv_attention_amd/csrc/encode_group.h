// Device functions of the residual-quantize encoder, shared by the encoder's kernels and by
// the attention kernels that encode the 64-row tail flush in extra workgroups (project page,
// The Method, after STEP 03: cache updates and quantization fused into the attention kernel).
//
// Exactness: every codec step is a single IEEE fp32 operation, as the oracle does it
// (correctly rounded division, rint half-to-even, fmaf dequant, no contraction: each
// function body turns contraction off).
#pragma once

#include "launch.h"

namespace qkv {

// code = clamp(rint((x - z) / s), 0, top), code 0 when s == 0, with the IEEE quotient
// (top = 15 for 4-bit codes, 3 for 2-bit codes).
// rs is an approximation of 1/s: the product t * rs is within 6e-6 of the quotient for the
// quotients that occur here (|t / s| <= 16), so rint of it agrees with rint of the exact,
// correctly rounded quotient unless that lies within 1.5e-5 of a half-integer; only then is
// the division carried out.
template <int BITS>
__device__ __forceinline__ uint32_t quant_code(float x, float s, float z, float rs) {
#pragma clang fp contract(off)
    constexpr float top = (float)((1 << BITS) - 1);
    if (s == 0.f) return 0u;
    const float t = x - z;
    const float q = t * rs;
    const float fq = q - floorf(q);
    float r;
    if (fabsf(fq - 0.5f) < 1.5e-5f || !(fabsf(q) < 16.f))
        r = __builtin_rintf(t / s);
    else
        r = __builtin_rintf(q);
    r = r < 0.f ? 0.f : r;
    r = r > top ? top : r;
    return (uint32_t)r;
}

// One workgroup encodes one group of up to 64 stored rows of one (sequence, head).  Thread
// items are 8 channels of one row (one 16-byte load of bf16); for loop r >= 2 each item
// rebuilds the 8 channels of Xhat^(r-1) through planes 1..r-1 (one code word and its scales
// per plane; the rows' slots are looked up once per group) and subtracts it.  A workgroup
// encodes one kind, with the residuals in registers: keys are quantised per channel over the
// rows (each thread's rows, then shuffles between the lanes that hold the same channels, then
// the four waves through LDS), values per row over each 64-channel group (shuffles among the
// group's 8 lanes), and each thread stores its own code words and metadata into the block.
// Four workgroups per CU (at most 128 VGPRs).
// OUTB: code width of the plane written (4, or 2 for 2-bit residual planes); RB: code width
// of the residual planes read back through the chain (plane 0 is 4-bit); nch: planes of the
// chain (loop - 1; 0 for loop 1 and for the full-state codec, which quantizes X^(loop) itself).
// (g, kind, h, b): the group, the kind (0 keys, 1 values), head and sequence this workgroup
// encodes; sslot: nch * 64 ints of LDS.  The body runs in the encoder's own kernel and, for
// the 64-row tail flush, in extra workgroups of the attention kernels.
template <int D, int OUTB, int RB>
__device__ __forceinline__ void encode_group(const CacheArg& ca, int loop, int nch, int pos0, int n_pos,
                                             const int32_t* __restrict__ act_pos, const int32_t* __restrict__ n_act,
                                             int ld_act, const uint16_t* __restrict__ ksrc,
                                             const uint16_t* __restrict__ vsrc, int ld_src,
                                             int32_t* __restrict__ rowpos, int g, int kind, int h, int b,
                                             int* sslot) {
#pragma clang fp contract(off)
    using Bo = Block<D, OUTB>;
    constexpr float kTop = (float)((1 << OUTB) - 1);
    constexpr int CH = 8;                // channels per item
    constexpr int IPR = D / CH;          // items per row
    constexpr int NIT = 64 * IPR / 256;  // items per thread
    constexpr int IB = NIT >= 2 ? 2 : 1;  // items whose chain loads go out together
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
    if (blk_idx >= P.n_blocks) {  // sparse plane full: the rows are not stored, and the caller is told
        if (tid == 0 && ca.eflags) atomicOr(ca.eflags, QKV_FLAG_PLANE_FULL);
        return;
    }
    uint8_t* blk = const_cast<uint8_t*>(block_ptr<D, OUTB>(P, ca.H, b, h, blk_idx));
    const bool from_tail = (ksrc == nullptr);
    const size_t bh = (size_t)b * ca.H + h;

    __shared__ int spos[64];
    __shared__ __align__(16) float red_mn[4][D], red_mx[4][D];  // per-wave key-channel minima, maxima

    if (tid < 64) {
        int p = -1;
        if (tid < nr) p = dense ? (pos0 + r0 + tid) : act_pos[(size_t)b * ld_act + r0 + tid];
        spos[tid] = (p >= pos0 && p < pos0 + n_pos) ? p : -1;  // positions outside the call are not stored
    }
    __syncthreads();
    for (int e = tid; e < nch * 64; e += 256) {
        const int p = e >> 6, row = e & 63;
        const int pos = spos[row];
        int slot = -1;
        if (pos >= 0) {
            const PlaneArg& Q = ca.p[p];
            slot = Q.dense ? pos : Q.rowmap[(size_t)b * ca.cap_ctx + pos];
            if (slot >= Q.n_blocks * 64) slot = -1;
        }
        sslot[p * 64 + row] = slot;
    }
    __syncthreads();

    // ---- per kind: this thread's items (8 channels of a row) in registers: residual,
    //      quantisation and the block's bytes, stored directly ----
    int ipos[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int row = (tid + 256 * it) / IPR;
        ipos[it] = row < nr ? spos[row] : -1;
    }
    const int lane = tid & 63, wave = tid >> 6;
    const int c0 = (tid % IPR) * CH;  // every item of this thread covers these channels
    {
        const uint16_t* src = kind ? vsrc : ksrc;
        const uint16_t* tail = kind ? ca.tail_v[loop - 1] : ca.tail_k[loop - 1];
        float x[NIT][CH];
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int row = (tid + 256 * it) / IPR;
#pragma unroll
            for (int c = 0; c < CH; ++c) x[it][c] = 0.f;
            if (ipos[it] >= 0) {
                const uint16_t* rp = from_tail ? tail + (bh * kTail + (ipos[it] % kTail)) * D + c0
                                               : src + (bh * ld_src + r0 + row) * D + c0;
                bf16x8(ld_stream_u4(rp), x[it]);
            }
        }
        if (nch > 0) {
            float acc[NIT][CH];
#pragma unroll
            for (int it = 0; it < NIT; ++it)
#pragma unroll
                for (int c = 0; c < CH; ++c) acc[it][c] = 0.f;
            for (int p = 0; p < nch; ++p) {
                const PlaneArg& Q = ca.p[p];
                // IB items at a time: their code words and scales of this plane in flight
                // together, then the dequantised sums
#pragma unroll
                for (int i0 = 0; i0 < NIT; i0 += IB) {
                    uint32_t cw[IB];
                    float s8[IB][CH], z8[IB][CH];
#pragma unroll
                    for (int u = 0; u < IB; ++u) {
                        const int row = (tid + 256 * (i0 + u)) / IPR;
                        const int slot = ipos[i0 + u] >= 0 ? sslot[p * 64 + row] : -1;
                        cw[u] = 0;
                        if (slot >= 0) {
                            // plane p's code width: 4 bits for the base, RB after it
                            const bool b4 = (p == 0 || RB == 4);
                            const uint8_t* bq = b4 ? block_ptr<D, 4>(Q, ca.H, b, h, slot >> 6)
                                                   : block_ptr<D, RB>(Q, ca.H, b, h, slot >> 6);
                            const int rw = slot & 63;
                            if (b4)
                                cw[u] = *reinterpret_cast<const uint32_t*>(
                                    bq + (kind ? Block<D, 4>::vc(rw) : Block<D, 4>::kc(rw)) + c0 / 2);
                            else
                                cw[u] = *reinterpret_cast<const uint16_t*>(
                                    bq + (kind ? Block<D, RB>::vc(rw) : Block<D, RB>::kc(rw)) + c0 * RB / 8);
                            const int kkm = b4 ? Block<D, 4>::kKm : Block<D, RB>::kKm;
                            const int vmo = b4 ? Block<D, 4>::vm(rw) : Block<D, RB>::vm(rw);
                            if (kind == 0) {
                                const float* m = reinterpret_cast<const float*>(bq + kkm) + c0;
                                const float4 sa = *reinterpret_cast<const float4*>(m);
                                const float4 sb = *reinterpret_cast<const float4*>(m + 4);
                                const float4 za = *reinterpret_cast<const float4*>(m + D);
                                const float4 zb = *reinterpret_cast<const float4*>(m + D + 4);
                                s8[u][0] = sa.x; s8[u][1] = sa.y; s8[u][2] = sa.z; s8[u][3] = sa.w;
                                s8[u][4] = sb.x; s8[u][5] = sb.y; s8[u][6] = sb.z; s8[u][7] = sb.w;
                                z8[u][0] = za.x; z8[u][1] = za.y; z8[u][2] = za.z; z8[u][3] = za.w;
                                z8[u][4] = zb.x; z8[u][5] = zb.y; z8[u][6] = zb.z; z8[u][7] = zb.w;
                            } else {
                                const float2 vm = *reinterpret_cast<const float2*>(bq + vmo + (c0 >> 6) * 8);
#pragma unroll
                                for (int c = 0; c < CH; ++c) {
                                    s8[u][c] = vm.x;
                                    z8[u][c] = vm.y;
                                }
                            }
                        }
                    }
#pragma unroll
                    for (int u = 0; u < IB; ++u) {
                        const int it = i0 + u;
                        const int row = (tid + 256 * it) / IPR;
                        if (ipos[it] < 0 || sslot[p * 64 + row] < 0) continue;  // not stored in loop p+1: keeps loop p's value
                        const bool b4 = (p == 0 || RB == 4);
#pragma unroll
                        for (int c = 0; c < CH; ++c) {
                            const float code = (float)(b4 ? ((cw[u] >> (4 * c)) & 15u) : ((cw[u] >> (2 * c)) & 3u));
                            const float deq = __builtin_fmaf(code, s8[u][c], z8[u][c]);
                            acc[it][c] = (p == 0) ? deq : acc[it][c] + deq;
                        }
                    }
                }
            }
#pragma unroll
            for (int it = 0; it < NIT; ++it)
                if (ipos[it] >= 0)
#pragma unroll
                    for (int c = 0; c < CH; ++c) x[it][c] = x[it][c] - acc[it][c];
        }

        if (kind == 0) {
            // keys: per channel over the group's stored rows (rows >= nr are padding).  This
            // thread's rows, then the lanes with the same channels (xor IPR, 2 IPR, ...), then
            // the waves through LDS.
            float mn[CH], mx[CH];
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                mn[c] = __builtin_huge_valf();
                mx[c] = -__builtin_huge_valf();
            }
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                if ((tid + 256 * it) / IPR >= nr) continue;
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    mn[c] = x[it][c] < mn[c] ? x[it][c] : mn[c];
                    mx[c] = x[it][c] > mx[c] ? x[it][c] : mx[c];
                }
            }
#pragma unroll
            for (int m = IPR; m < 64; m <<= 1)
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    mn[c] = fminf(mn[c], __shfl_xor(mn[c], m, 64));
                    mx[c] = fmaxf(mx[c], __shfl_xor(mx[c], m, 64));
                }
            if (lane < IPR) {
                *reinterpret_cast<float4*>(&red_mn[wave][c0]) = make_float4(mn[0], mn[1], mn[2], mn[3]);
                *reinterpret_cast<float4*>(&red_mn[wave][c0 + 4]) = make_float4(mn[4], mn[5], mn[6], mn[7]);
                *reinterpret_cast<float4*>(&red_mx[wave][c0]) = make_float4(mx[0], mx[1], mx[2], mx[3]);
                *reinterpret_cast<float4*>(&red_mx[wave][c0 + 4]) = make_float4(mx[4], mx[5], mx[6], mx[7]);
            }
            __syncthreads();
            float s[CH], z[CH], rs[CH];
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                float a = red_mn[0][c0 + c], bmx = red_mx[0][c0 + c];
#pragma unroll
                for (int q = 1; q < 4; ++q) {
                    a = red_mn[q][c0 + c] < a ? red_mn[q][c0 + c] : a;
                    bmx = red_mx[q][c0 + c] > bmx ? red_mx[q][c0 + c] : bmx;
                }
                float range = bmx - a;
                float sc = range / kTop;
                sc = sc + 0.0f;
                s[c] = sc;
                z[c] = a + 0.0f;
                rs[c] = __builtin_amdgcn_rcpf(sc);
            }
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                const int row = (tid + 256 * it) / IPR;
                uint32_t w = 0;
                if (row < nr) {
#pragma unroll
                    for (int e = 0; e < CH; ++e) w |= quant_code<OUTB>(x[it][e], s[e], z[e], rs[e]) << (OUTB * e);
                }
                if (OUTB == 4)
                    *reinterpret_cast<uint32_t*>(blk + Bo::kc(row) + c0 / 2) = w;
                else
                    *reinterpret_cast<uint16_t*>(blk + Bo::kc(row) + c0 * OUTB / 8) = (uint16_t)w;
            }
            if (tid < IPR) {
                float* m = reinterpret_cast<float*>(blk + Bo::kKm) + c0;
                *reinterpret_cast<float4*>(m) = make_float4(s[0], s[1], s[2], s[3]);
                *reinterpret_cast<float4*>(m + 4) = make_float4(s[4], s[5], s[6], s[7]);
                *reinterpret_cast<float4*>(m + D) = make_float4(z[0], z[1], z[2], z[3]);
                *reinterpret_cast<float4*>(m + D + 4) = make_float4(z[4], z[5], z[6], z[7]);
            }
        } else {
            // values: per row over each 64-channel group, i.e. the 8 lanes (xor 1, 2, 4) whose
            // items make up the group
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                const int row = (tid + 256 * it) / IPR;
                float mn = x[it][0], mx = x[it][0];
#pragma unroll
                for (int e = 1; e < CH; ++e) {
                    mn = x[it][e] < mn ? x[it][e] : mn;
                    mx = x[it][e] > mx ? x[it][e] : mx;
                }
#pragma unroll
                for (int m = 1; m < 8; m <<= 1) {
                    mn = fminf(mn, __shfl_xor(mn, m, 64));
                    mx = fmaxf(mx, __shfl_xor(mx, m, 64));
                }
                float range = mx - mn;
                float sc = range / kTop;
                sc = sc + 0.0f;
                const float zc = mn + 0.0f;
                uint32_t w = 0;
                if (row < nr) {
                    const float rs = __builtin_amdgcn_rcpf(sc);
#pragma unroll
                    for (int e = 0; e < CH; ++e) w |= quant_code<OUTB>(x[it][e], sc, zc, rs) << (OUTB * e);
                }
                if (OUTB == 4)
                    *reinterpret_cast<uint32_t*>(blk + Bo::vc(row) + c0 / 2) = w;
                else
                    *reinterpret_cast<uint16_t*>(blk + Bo::vc(row) + c0 * OUTB / 8) = (uint16_t)w;
                if ((tid & 7) == 0)
                    *reinterpret_cast<float2*>(blk + Bo::vm(row) + (c0 >> 6) * 8) =
                        make_float2(row < nr ? sc : 0.f, row < nr ? zc : 0.f);
            }
        }
    }

    if (!dense && h == 0 && kind == 0 && tid < 64)
        rowpos[(size_t)b * P.n_blocks * 64 + base + r0 + tid] = spos[tid];
}

// position -> slot map and block starts of a sparse plane for position pos0 + i of [pos0,
// pos0 + n_pos), sequence b
__device__ __forceinline__ void encode_maps(int cap_ctx, int pos0, int n_pos, const int32_t* __restrict__ act_pos,
                                            const int32_t* __restrict__ n_act, int ld_act,
                                            int32_t* __restrict__ rowmap, int32_t* __restrict__ rowstart,
                                            uint32_t* __restrict__ smask, uint32_t bit, int b, int i) {
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
        const bool stored = lo < na && a[lo] == p;
        rowmap[(size_t)b * cap_ctx + p] = stored ? base + lo : -1;
        if (smask) {
            uint32_t& m = smask[(size_t)b * cap_ctx + p];
            m = stored ? (m | bit) : (m & ~bit);
        }
        if ((i & 63) == 0 && i > 0) rowstart[(size_t)b * nstart + p / 64] = base + lo;
    }
    if (i == 0) rowstart[(size_t)b * nstart + (pos0 + n_pos) / 64] = base + ((na + 63) / 64) * 64;
}

// The tail-flush role of an attention kernel's extra workgroup e for (head h, sequence b):
// e = 0 encodes the group's keys, e = 1 its values, e = 2 (sparse planes, head 0 only) writes
// the plane's maps.  RB: code width of residual planes; the encoded plane is 4-bit for
// loop 1.  Needs f.nch * 64 ints of dynamic LDS.
template <int D, int RB>
__device__ __forceinline__ void flush_role(const CacheArg& ca, const FlushArg& f, int e, int h, int b) {
    extern __shared__ int flush_sslot[];
    const PlaneArg& P = ca.p[f.loop - 1];
    if (e < 2) {
        if (f.loop == 1 || RB == 4)
            encode_group<D, 4, RB>(ca, f.loop, f.nch, f.pos0, 64, f.act_pos, f.n_act, f.ld_act, nullptr, nullptr, 0,
                                   const_cast<int32_t*>(P.rowpos), 0, e, h, b, flush_sslot);
        else
            encode_group<D, RB, RB>(ca, f.loop, f.nch, f.pos0, 64, f.act_pos, f.n_act, f.ld_act, nullptr, nullptr, 0,
                                    const_cast<int32_t*>(P.rowpos), 0, e, h, b, flush_sslot);
    } else if (h == 0 && threadIdx.x < 64) {
        encode_maps(ca.cap_ctx, f.pos0, 64, f.act_pos, f.n_act, f.ld_act, const_cast<int32_t*>(P.rowmap),
                    const_cast<int32_t*>(P.rowstart), f.smask, f.bit, b, threadIdx.x);
    }
}

}  // namespace qkv
