// Dense decode attention over the quantized cross-loop chain: split-KV reader + combine.
//
// Column j's key in loop r is the base plus every residual plane p <= r storing j
// (project page STEP 01/03; explainer section 3).  By linearity the logit is a sum of
// per-plane partial logits, and per plane and key group (64 slots x channel c with
// scale s_c, zero z_c):  q . khat = sum_c (q_c s_c) code_c + sum_c q_c z_c,
// so each lane folds the group's scales into the query once and streams nibbles.
// Values are per-slot groups: p_j vhat_j = (p_j s_j) code + p_j z_j.
//
// Each workgroup (4 waves) owns a contiguous range of 64-position blocks: pass 1 streams
// the K codes of every plane into LDS logits, then a local softmax, pass 2 streams the V
// codes; partial (max, sum, o) go to the workspace and a second kernel merges the splits
// in a fixed order.  One extra workgroup per (sequence, head) reads the BF16 tail.
#include "launch.h"

namespace qkv {

constexpr int kMaxSpb = 16;  // 64-position blocks per split, at most

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
__device__ __forceinline__ float block_reduce_max(float v, float* red) {
    v = wave_max(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
template <int D>
__device__ __forceinline__ float block_reduce_sum(float v, float* red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// K pass over one 64-slot block: calls emit(row, partial_logit) on one lane per row.
template <int D, typename Emit>
__device__ __forceinline__ void kpass_block(const uint8_t* bp, const float* qsh, float* qp_lds, int lane, int prt,
                                            int rsub, Emit emit) {
    constexpr int LPR = Block<D>::kLpr, RPI = Block<D>::kRpi, NLD = 64 / RPI;
    uint4 w[NLD];
#pragma unroll
    for (int it = 0; it < NLD; ++it)
        w[it] = *reinterpret_cast<const uint4*>(bp + Block<D>::kKc + (rsub + RPI * it) * (D / 2) + prt * 16);
    const float* km = reinterpret_cast<const float*>(bp + Block<D>::kKm);
    float bias = 0.f;
#pragma unroll
    for (int c = lane; c < D; c += 64) {
        const float qc = qsh[c];
        qp_lds[c] = qc * km[c];
        bias = fmaf(qc, km[D + c], bias);
    }
    bias = wave_sum(bias);
    wave_sync_lds();
    float qp[32];
#pragma unroll
    for (int k = 0; k < 32; k += 4) {
        const float4 t = *reinterpret_cast<const float4*>(qp_lds + 32 * prt + k);
        qp[k] = t.x; qp[k + 1] = t.y; qp[k + 2] = t.z; qp[k + 3] = t.w;
    }
    wave_sync_lds();
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
        float v = dot32_codes(w[it], qp);
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1) v += __shfl_xor(v, m, 64);
        if (prt == 0) emit(rsub + RPI * it, v + bias);
    }
}

// V pass over one block: weight(row) returns the row's probability (0 to skip).
template <int D, typename Weight>
__device__ __forceinline__ void vpass_block(const uint8_t* bp, int prt, int rsub, float* acc, float& vb,
                                            Weight weight) {
    constexpr int RPI = Block<D>::kRpi, NLD = 64 / RPI;
    uint4 w[NLD];
    float2 m[NLD];
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
        const int row = rsub + RPI * it;
        w[it] = *reinterpret_cast<const uint4*>(bp + Block<D>::kVc + row * (D / 2) + prt * 16);
        m[it] = *reinterpret_cast<const float2*>(bp + Block<D>::kVm + (row * (D / 64) + (prt >> 1)) * 8);
    }
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
        const float pw = weight(rsub + RPI * it);
        vb = fmaf(pw, m[it].y, vb);
        axpy32_codes(w[it], pw * m[it].x, acc);
    }
}

// Merges the nsplit1 partials of one (sequence, head) in split order; threads < D.
template <int D>
__device__ __forceinline__ void dense_combine(const float* pp, int nsplit1, int c, uint16_t* o, float* o32,
                                              float* lse, int bh) {
    float M = -__builtin_huge_valf();
    for (int s = 0; s < nsplit1; ++s) M = fmaxf(M, pp[(size_t)s * (D + 2)]);
    float L = 0.f, a = 0.f;
    for (int s = 0; s < nsplit1; ++s) {
        const float e = __expf(pp[(size_t)s * (D + 2)] - M);
        L = fmaf(pp[(size_t)s * (D + 2) + 1], e, L);
        a = fmaf(pp[(size_t)s * (D + 2) + 2 + c], e, a);
    }
    const float oc = a / L;
    o32[(size_t)bh * D + c] = oc;
    if (o) o[(size_t)bh * D + c] = f32_to_bf16_rne(oc);
    if (c == 0) lse[bh] = M + __logf(L);
}

template <int D>
__global__ __launch_bounds__(256) void dense_split_kernel(CacheArg ca, int loop, const uint16_t* __restrict__ q,
                                                          float sm, float* __restrict__ scores, int ld,
                                                          float* __restrict__ part, unsigned* __restrict__ counters,
                                                          int nsplit, int spb, uint16_t* __restrict__ o,
                                                          float* __restrict__ o32, float* __restrict__ lse) {
    constexpr int LPR = Block<D>::kLpr, RPI = Block<D>::kRpi;
    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int prt = lane % LPR, rsub = lane / LPR;
    const int bh = b * ca.H + h;

    __shared__ float qsh[D];
    __shared__ float logit[kMaxSpb * 64];
    __shared__ float qps[4][D];
    __shared__ float red[4];
    __shared__ float ored[4][D];

    for (int c = tid; c < D; c += 256) qsh[c] = bf16_to_f32(q[(size_t)bh * D + c]) * sm;
    __syncthreads();
    float* out = part + ((size_t)bh * (nsplit + 1) + s) * (D + 2);
    float* srow = scores + (size_t)bh * ld;

    float acc[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) acc[k] = 0.f;
    float vb = 0.f;
    float mx, lsum;

    if (s == nsplit) {
        // ---- BF16 tail: positions [n_body, n_ctx) at ring slots t % 128 ----
        const int T = ca.n_ctx - ca.n_body;
        const uint16_t* tk = ca.tail_k[loop - 1] + (size_t)bh * kTail * D;
        const uint16_t* tv = ca.tail_v[loop - 1] + (size_t)bh * kTail * D;
        float qv[32];
#pragma unroll
        for (int k = 0; k < 32; ++k) qv[k] = qsh[32 * prt + k];
        for (int i0 = wave * RPI; i0 < T; i0 += 4 * RPI) {
            const int i = i0 + rsub;
            float v = 0.f;
            if (i < T) {
                const uint16_t* kr = tk + (size_t)((ca.n_body + i) % kTail) * D + 32 * prt;
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4) {
                    const uint4 w = *reinterpret_cast<const uint4*>(kr + 8 * k4);
                    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v = fmaf(qv[8 * k4 + 2 * e], bf16_to_f32(ws[e] & 0xFFFFu), v);
                        v = fmaf(qv[8 * k4 + 2 * e + 1], bf16_to_f32(ws[e] >> 16), v);
                    }
                }
            }
#pragma unroll
            for (int m = 1; m < LPR; m <<= 1) v += __shfl_xor(v, m, 64);
            if (prt == 0 && i < T) logit[i] = v;
        }
        __syncthreads();
        float lm = -__builtin_huge_valf();
        for (int i = tid; i < T; i += 256) {
            srow[ca.n_body + i] = logit[i];
            lm = fmaxf(lm, logit[i]);
        }
        mx = block_reduce_max<D>(lm, red);
        float ls = 0.f;
        for (int i = tid; i < T; i += 256) {
            const float pv = __expf(logit[i] - mx);
            logit[i] = pv;
            ls += pv;
        }
        lsum = block_reduce_sum<D>(ls, red);
        for (int i0 = wave * RPI; i0 < T; i0 += 4 * RPI) {
            const int i = i0 + rsub;
            if (i < T) {
                const float pw = logit[i];
                const uint16_t* vr = tv + (size_t)((ca.n_body + i) % kTail) * D + 32 * prt;
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4) {
                    const uint4 w = *reinterpret_cast<const uint4*>(vr + 8 * k4);
                    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[8 * k4 + 2 * e] = fmaf(pw, bf16_to_f32(ws[e] & 0xFFFFu), acc[8 * k4 + 2 * e]);
                        acc[8 * k4 + 2 * e + 1] = fmaf(pw, bf16_to_f32(ws[e] >> 16), acc[8 * k4 + 2 * e + 1]);
                    }
                }
            }
        }
    } else {
        // ---- body split: blocks [blk0, blk1) ----
        const int nblk = ca.n_body / 64;
        const int blk0 = s * spb, blk1 = min(blk0 + spb, nblk);
        const int j0 = blk0 * 64, L = (blk1 - blk0) * 64;
        const int nstart = ca.cap_ctx / 64 + 1;
        for (int i = tid; i < L; i += 256) logit[i] = 0.f;
        __syncthreads();
        for (int p = 0; p < loop; ++p) {
            const PlaneArg& P = ca.p[p];
            if (P.dense) {
                for (int blk = blk0 + wave; blk < blk1; blk += 4) {
                    const uint8_t* bp = block_ptr<D>(P, ca.H, b, h, blk);
                    float* lg = logit + (blk - blk0) * 64;
                    kpass_block<D>(bp, qsh, qps[wave], lane, prt, rsub, [&](int row, float v) { lg[row] += v; });
                }
            } else {
                const int rs0 = P.rowstart[(size_t)b * nstart + blk0];
                const int rs1 = P.rowstart[(size_t)b * nstart + blk1];
                const int32_t* rp = P.rowpos + (size_t)b * P.n_blocks * 64;
                for (int sb = (rs0 >> 6) + wave; sb * 64 < rs1 && sb < P.n_blocks; sb += 4) {
                    const uint8_t* bp = block_ptr<D>(P, ca.H, b, h, sb);
                    kpass_block<D>(bp, qsh, qps[wave], lane, prt, rsub, [&](int row, float v) {
                        const int slot = sb * 64 + row;
                        if (slot >= rs0 && slot < rs1) {
                            const int pos = rp[slot] - j0;
                            if (pos >= 0 && pos < L) logit[pos] += v;
                        }
                    });
                }
            }
            __syncthreads();
        }
        float lm = -__builtin_huge_valf();
        for (int i = tid; i < L; i += 256) {
            srow[j0 + i] = logit[i];
            lm = fmaxf(lm, logit[i]);
        }
        mx = block_reduce_max<D>(lm, red);
        float ls = 0.f;
        for (int i = tid; i < L; i += 256) {
            const float pv = __expf(logit[i] - mx);
            logit[i] = pv;
            ls += pv;
        }
        lsum = block_reduce_sum<D>(ls, red);
        for (int p = 0; p < loop; ++p) {
            const PlaneArg& P = ca.p[p];
            if (P.dense) {
                for (int blk = blk0 + wave; blk < blk1; blk += 4) {
                    const uint8_t* bp = block_ptr<D>(P, ca.H, b, h, blk);
                    const float* lg = logit + (blk - blk0) * 64;
                    vpass_block<D>(bp, prt, rsub, acc, vb, [&](int row) { return lg[row]; });
                }
            } else {
                const int rs0 = P.rowstart[(size_t)b * nstart + blk0];
                const int rs1 = P.rowstart[(size_t)b * nstart + blk1];
                const int32_t* rp = P.rowpos + (size_t)b * P.n_blocks * 64;
                for (int sb = (rs0 >> 6) + wave; sb * 64 < rs1 && sb < P.n_blocks; sb += 4) {
                    const uint8_t* bp = block_ptr<D>(P, ca.H, b, h, sb);
                    vpass_block<D>(bp, prt, rsub, acc, vb, [&](int row) {
                        const int slot = sb * 64 + row;
                        float pw = 0.f;
                        if (slot >= rs0 && slot < rs1) {
                            const int pos = rp[slot] - j0;
                            if (pos >= 0 && pos < L) pw = logit[pos];
                        }
                        return pw;
                    });
                }
            }
        }
    }

    // reduce the per-lane accumulators over the rows of the wave, then over waves
#pragma unroll
    for (int m = LPR; m < 64; m <<= 1) {
#pragma unroll
        for (int k = 0; k < 32; ++k) acc[k] += __shfl_xor(acc[k], m, 64);
        vb += __shfl_xor(vb, m, 64);
    }
    if (rsub == 0) {
#pragma unroll
        for (int k = 0; k < 32; ++k) ored[wave][32 * prt + k] = acc[k] + vb;
    }
    __syncthreads();
    for (int c = tid; c < D; c += 256) out[2 + c] = (ored[0][c] + ored[1][c]) + (ored[2][c] + ored[3][c]);
    if (tid == 0) {
        out[0] = mx;
        out[1] = lsum;
    }

    // the last workgroup of this (sequence, head) to finish merges every split
    __shared__ unsigned last;
    __threadfence();
    __syncthreads();
    if (tid == 0) last = (atomicAdd(&counters[bh], 1u) == (unsigned)nsplit) ? 1u : 0u;
    __syncthreads();
    if (!last) return;
    __threadfence();
    if (tid < D) dense_combine<D>(part + (size_t)bh * (nsplit + 1) * (D + 2), nsplit + 1, tid, o, o32, lse, bh);
    if (tid == 0) atomicExch(&counters[bh], 0u);
}

DensePlan dense_plan(int B, int H, int n_body) {
    const int nblk = n_body / 64;
    DensePlan pl;
    if (nblk == 0) {
        pl.spb = 1;
        pl.nsplit = 0;
        return pl;
    }
    // aim for about 1024 body workgroups, 4..16 blocks each
    long target = 1024;
    int spb = (int)(((long)nblk * B * H + target - 1) / target);
    spb = spb < 4 ? 4 : (spb > kMaxSpb ? kMaxSpb : spb);
    pl.spb = spb;
    pl.nsplit = (nblk + spb - 1) / spb;
    return pl;
}

// workspace: per-(sequence, head) counters first, then the split partials
size_t ws_counter_bytes(int B, int H) { return (((size_t)B * H * sizeof(unsigned)) + 255) & ~(size_t)255; }

size_t dense_ws_bytes(int B, int H, int D, int n_body) {
    const DensePlan pl = dense_plan(B, H, n_body);
    return ws_counter_bytes(B, H) + (size_t)B * H * (pl.nsplit + 1) * (D + 2) * sizeof(float);
}

int launch_dense(const CacheArg& ca, int D, int loop, const uint16_t* q, float sm, uint16_t* o, float* o32,
                 float* scores, int ld, float* lse, void* ws, hipStream_t st) {
    const DensePlan pl = dense_plan(ca.B, ca.H, ca.n_body);
    unsigned* counters = reinterpret_cast<unsigned*>(ws);
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + ws_counter_bytes(ca.B, ca.H));
    dim3 grid(pl.nsplit + 1, ca.H, ca.B);
    if (D == 128)
        dense_split_kernel<128><<<grid, 256, 0, st>>>(ca, loop, q, sm, scores, ld, part, counters, pl.nsplit, pl.spb,
                                                      o, o32, lse);
    else
        dense_split_kernel<64><<<grid, 256, 0, st>>>(ca, loop, q, sm, scores, ld, part, counters, pl.nsplit, pl.spb,
                                                     o, o32, lse);
    return hipGetLastError() == hipSuccess ? QKV_OK : QKV_ELAUNCH;
}

}  // namespace qkv
