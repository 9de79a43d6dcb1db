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

// code = clamp(rint((x - z) / s), 0, 15), code 0 when s == 0, with the IEEE quotient.
// rs is an approximation of 1/s: the product t * rs is within 6e-6 of the quotient for the
// quotients that occur here (|t / s| <= 16), so rint of it agrees with rint of the exact,
// correctly rounded quotient unless that lies within 1.5e-5 of a half-integer; only then is
// the division carried out.
__device__ __forceinline__ uint32_t quant_code(float x, float s, float z, float rs) {
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
    r = r > 15.f ? 15.f : r;
    return (uint32_t)r;
}

// One workgroup encodes one group of up to 64 stored rows of one (sequence, head).  Thread
// items are 8 channels of one row (one 16-byte load of bf16); for loop r >= 2 each item
// rebuilds the 8 channels of Xhat^(r-1) through planes 1..r-1 (one code word and its scales
// per plane; the rows' slots are looked up once per group) and subtracts it.  Keys are
// quantised per channel over the rows (a thread per channel pair and 16 rows), values per
// row over each 64-channel group (8 lanes of 8 channels each); codes are packed into bytes
// in LDS as they are made and the block is written with 16-byte stores.
template <int D>
__global__ __launch_bounds__(256) void encode_group_kernel(CacheArg ca, int loop, int pos0, int n_pos,
                                                           const int32_t* __restrict__ act_pos,
                                                           const int32_t* __restrict__ n_act, int ld_act,
                                                           const uint16_t* __restrict__ ksrc,
                                                           const uint16_t* __restrict__ vsrc, int ld_src,
                                                           int32_t* __restrict__ rowpos) {
    constexpr int CH = 8;                // channels per item
    constexpr int IPR = D / CH;          // items per row
    constexpr int NIT = 64 * IPR / 256;  // items per thread
    constexpr int XS = D + 4;            // LDS row stride of X in floats (keeps 16-byte alignment)
    constexpr int NCP = D / 2;           // channel pairs (code bytes per row)
    constexpr int KPARTS = 256 / NCP;    // row parts of the key pass
    constexpr int KROWS = 64 / KPARTS;
    constexpr int VG = D / 64;           // value groups per row
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
    const int nch = loop - 1;           // planes of the chain Xhat^(r-1)
    const size_t bh = (size_t)b * ca.H + h;

    __shared__ __align__(16) float Xk[64 * D];        // key residuals (read along rows)
    __shared__ __align__(16) float Xv[64 * XS];       // value residuals (padded rows: read across rows)
    // packed codes [kind][row][channel pair]; before any code is written the same bytes
    // hold the per-part channel minima and maxima of the key pass
    __shared__ __align__(16) uint8_t pkbuf[2 * 64 * NCP];
    static_assert(2 * 64 * NCP >= 2 * KPARTS * D * (int)sizeof(float), "key-pass scratch");
    uint8_t (*pk)[64][NCP] = reinterpret_cast<uint8_t (*)[64][NCP]>(pkbuf);
    float (*red_mn)[D] = reinterpret_cast<float (*)[D]>(pkbuf);
    float (*red_mx)[D] = reinterpret_cast<float (*)[D]>(pkbuf) + KPARTS;
    __shared__ int spos[64];
    extern __shared__ int sslot[];                  // [nch][64], sized at launch
    __shared__ float ks[D], kz[D];
    __shared__ float vs[64][VG], vz[64][VG];

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

    // ---- residuals of both kinds into LDS ----
    int ipos[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int row = (tid + 256 * it) / IPR;
        ipos[it] = row < nr ? spos[row] : -1;
    }
    for (int kind = 0; kind < 2; ++kind) {
        const uint16_t* src = kind ? vsrc : ksrc;
        const uint16_t* tail = kind ? ca.tail_v[loop - 1] : ca.tail_k[loop - 1];
        float x[NIT][CH];
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int item = tid + 256 * it;
            const int row = item / IPR, c0 = (item % IPR) * CH;
#pragma unroll
            for (int c = 0; c < CH; ++c) x[it][c] = 0.f;
            if (ipos[it] >= 0) {
                const uint16_t* rp = from_tail ? tail + (bh * kTail + (ipos[it] % kTail)) * D + c0
                                               : src + (bh * ld_src + r0 + row) * D + c0;
                bf16x8(*reinterpret_cast<const uint4*>(rp), x[it]);
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
                // every item's code word and scales of this plane, then the dequantised sums
                uint32_t cw[NIT];
                float s8[NIT][CH], z8[NIT][CH];
#pragma unroll
                for (int it = 0; it < NIT; ++it) {
                    const int item = tid + 256 * it;
                    const int row = item / IPR, c0 = (item % IPR) * CH;
                    const int slot = ipos[it] >= 0 ? sslot[p * 64 + row] : -1;
                    cw[it] = 0;
                    if (slot >= 0) {
                        const uint8_t* bq = block_ptr<D>(Q, ca.H, b, h, slot >> 6);
                        const int rw = slot & 63;
                        cw[it] = *reinterpret_cast<const uint32_t*>(
                            bq + (kind ? Block<D>::vc(rw) : Block<D>::kKc + rw * (D / 2)) + c0 / 2);
                        if (kind == 0) {
                            const float* m = reinterpret_cast<const float*>(bq + Block<D>::kKm) + c0;
                            const float4 sa = *reinterpret_cast<const float4*>(m);
                            const float4 sb = *reinterpret_cast<const float4*>(m + 4);
                            const float4 za = *reinterpret_cast<const float4*>(m + D);
                            const float4 zb = *reinterpret_cast<const float4*>(m + D + 4);
                            s8[it][0] = sa.x; s8[it][1] = sa.y; s8[it][2] = sa.z; s8[it][3] = sa.w;
                            s8[it][4] = sb.x; s8[it][5] = sb.y; s8[it][6] = sb.z; s8[it][7] = sb.w;
                            z8[it][0] = za.x; z8[it][1] = za.y; z8[it][2] = za.z; z8[it][3] = za.w;
                            z8[it][4] = zb.x; z8[it][5] = zb.y; z8[it][6] = zb.z; z8[it][7] = zb.w;
                        } else {
                            const float2 vm = *reinterpret_cast<const float2*>(bq + Block<D>::vm(rw) + (c0 >> 6) * 8);
#pragma unroll
                            for (int c = 0; c < CH; ++c) {
                                s8[it][c] = vm.x;
                                z8[it][c] = vm.y;
                            }
                        }
                    }
                }
#pragma unroll
                for (int it = 0; it < NIT; ++it) {
                    const int item = tid + 256 * it;
                    const int row = item / IPR;
                    if (ipos[it] < 0 || sslot[p * 64 + row] < 0) continue;  // not stored in loop p+1: keeps loop p's value
#pragma unroll
                    for (int c = 0; c < CH; ++c) {
                        const uint32_t byte = (cw[it] >> (8 * (c >> 1))) & 0xFFu;
                        const float code = (float)((c & 1) ? (byte >> 4) : (byte & 15u));
                        const float deq = __builtin_fmaf(code, s8[it][c], z8[it][c]);
                        acc[it][c] = (p == 0) ? deq : acc[it][c] + deq;
                    }
                }
            }
#pragma unroll
            for (int it = 0; it < NIT; ++it)
                if (ipos[it] >= 0)
#pragma unroll
                    for (int c = 0; c < CH; ++c) x[it][c] = x[it][c] - acc[it][c];
        }
        float* Xd = kind ? Xv : Xk;
        const int xs = kind ? XS : D;
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int item = tid + 256 * it;
            const int row = item / IPR, c0 = (item % IPR) * CH;
            *reinterpret_cast<float4*>(&Xd[row * xs + c0]) = make_float4(x[it][0], x[it][1], x[it][2], x[it][3]);
            *reinterpret_cast<float4*>(&Xd[row * xs + c0 + 4]) = make_float4(x[it][4], x[it][5], x[it][6], x[it][7]);
        }
    }
    __syncthreads();

    // ---- keys: per channel over the group's stored rows; thread = channel pair x row part ----
    {
        const int cp = tid % NCP, part = tid / NCP;
        const int ca0 = 2 * cp;
        float mn0 = __builtin_huge_valf(), mx0 = -__builtin_huge_valf(), mn1 = mn0, mx1 = mx0;
        for (int r = part * KROWS; r < (part + 1) * KROWS && r < nr; ++r) {
            const float2 v = *reinterpret_cast<const float2*>(&Xk[r * D + ca0]);
            mn0 = v.x < mn0 ? v.x : mn0;
            mx0 = v.x > mx0 ? v.x : mx0;
            mn1 = v.y < mn1 ? v.y : mn1;
            mx1 = v.y > mx1 ? v.y : mx1;
        }
        red_mn[part][ca0] = mn0;
        red_mn[part][ca0 + 1] = mn1;
        red_mx[part][ca0] = mx0;
        red_mx[part][ca0 + 1] = mx1;
        __syncthreads();
        if (tid < D) {
            float a = red_mn[0][tid], bmx = red_mx[0][tid];
#pragma unroll
            for (int q = 1; q < KPARTS; ++q) {
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
        const float s0 = ks[ca0], z0 = kz[ca0], s1 = ks[ca0 + 1], z1 = kz[ca0 + 1];
        const float rs0 = __builtin_amdgcn_rcpf(s0), rs1 = __builtin_amdgcn_rcpf(s1);
        for (int r = part * KROWS; r < (part + 1) * KROWS; ++r) {
            uint32_t byte = 0;
            if (r < nr) {
                const float2 v = *reinterpret_cast<const float2*>(&Xk[r * D + ca0]);
                byte = quant_code(v.x, s0, z0, rs0) | (quant_code(v.y, s1, z1, rs1) << 4);
            }
            pk[0][r][cp] = (uint8_t)byte;
        }
    }
    // ---- values: per row over each 64-channel group; 8 lanes of 8 channels per (row, group) ----
    {
        for (int t = tid; t < 64 * VG * 8; t += 256) {
            const int sub = t & 7, rg = t >> 3;
            const int r = rg / VG, gg = rg % VG;
            const int c0 = gg * 64 + sub * 8;
            const float4 a = *reinterpret_cast<const float4*>(&Xv[r * XS + c0]);
            const float4 c = *reinterpret_cast<const float4*>(&Xv[r * XS + c0 + 4]);
            const float v8[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
            float mn = v8[0], mx = v8[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) {
                mn = v8[e] < mn ? v8[e] : mn;
                mx = v8[e] > mx ? v8[e] : mx;
            }
#pragma unroll
            for (int m = 1; m < 8; m <<= 1) {  // the 8 lanes of this (row, group)
                mn = fminf(mn, __shfl_xor(mn, m, 64));
                mx = fmaxf(mx, __shfl_xor(mx, m, 64));
            }
            float range = mx - mn;
            float s = range / 15.0f;
            s = s + 0.0f;
            const float z = mn + 0.0f;
            uint32_t w = 0;
            if (r < nr) {
                const float rs = __builtin_amdgcn_rcpf(s);
#pragma unroll
                for (int e = 0; e < 8; e += 2)
                    w |= (quant_code(v8[e], s, z, rs) | (quant_code(v8[e + 1], s, z, rs) << 4)) << (4 * e);
            }
            if (sub == 0) {
                vs[r][gg] = r < nr ? s : 0.f;
                vz[r][gg] = r < nr ? z : 0.f;
            }
            *reinterpret_cast<uint32_t*>(&pk[1][r][c0 / 2]) = w;
        }
    }
    __syncthreads();

    // ---- the block: codes of both kinds, key scales/zeros, value meta ----
    for (int e = tid; e < 2 * 64 * NCP / 16; e += 256) {
        const int kind = e / (64 * NCP / 16), rest = e % (64 * NCP / 16);
        const int row = rest / (NCP / 16), byte0 = (rest % (NCP / 16)) * 16;
        const uint4 w = *reinterpret_cast<const uint4*>(&pk[kind][row][byte0]);
        *reinterpret_cast<uint4*>(blk + (kind ? Block<D>::vc(row) : Block<D>::kKc + row * (D / 2)) + byte0) = w;
    }
    {
        float* m = reinterpret_cast<float*>(blk + Block<D>::kKm);
        for (int c = tid; c < D; c += 256) {
            m[c] = ks[c];
            m[D + c] = kz[c];
        }
        for (int e = tid; e < 64 * VG; e += 256) {
            float* mv = reinterpret_cast<float*>(blk + Block<D>::vm(e / VG)) + 2 * (e % VG);
            mv[0] = vs[e / VG][e % VG];
            mv[1] = vz[e / VG][e % VG];
        }
    }

    if (!dense && h == 0 && tid < 64)
        rowpos[(size_t)b * P.n_blocks * 64 + base + r0 + tid] = spos[tid];
}

// position -> slot map and block starts of a sparse plane for [pos0, pos0 + n_pos)
__global__ __launch_bounds__(256) void encode_maps_kernel(int cap_ctx, int pos0, int n_pos,
                                                          const int32_t* __restrict__ act_pos,
                                                          const int32_t* __restrict__ n_act, int ld_act,
                                                          int32_t* __restrict__ rowmap,
                                                          int32_t* __restrict__ rowstart,
                                                          uint32_t* __restrict__ smask, uint32_t bit) {
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
    const size_t dyn = (size_t)(loop - 1) * 64 * sizeof(int);  // chain slots of the stored rows
    if (D == 128)
        encode_group_kernel<128><<<grid, 256, dyn, st>>>(ca, loop, pos0, n_pos, act_pos, n_act, ld_act, ksrc, vsrc,
                                                         ld_src, rowpos);
    else
        encode_group_kernel<64><<<grid, 256, dyn, st>>>(ca, loop, pos0, n_pos, act_pos, n_act, ld_act, ksrc, vsrc,
                                                        ld_src, rowpos);
    if (hipGetLastError() != hipSuccess) return QKV_ELAUNCH;
    if (!P.dense) {
        dim3 g2((n_pos + 255) / 256, ca.B);
        encode_maps_kernel<<<g2, 256, 0, st>>>(ca.cap_ctx, pos0, n_pos, act_pos, n_act, ld_act,
                                               const_cast<int32_t*>(P.rowmap), const_cast<int32_t*>(P.rowstart),
                                               ca.smask, 1u << (loop - 1));
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
