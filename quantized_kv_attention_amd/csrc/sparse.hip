// Sparse late-loop decode attention with the mass-preserving splice (project page
// STEP 02; explainer section 3: only the top-K columns picked from the preceding loop are
// recomputed, as a rank-K correction of the preceding loop's output that keeps their
// cached mass m).
//
//   o^(r) = o^(r-1) + sum_{j in S} ( m * alpha_j * vhat^(r)_j - p_j * vhat^(r-1)_j ),
//   alpha = softmax over S of s^(r),
//   scores[j] <- lse + log m + s^(r)_j - log sum_S exp(s^(r)).
//
// One wave per chunk of 64 selected columns (4 lanes x 32 channels per column at d=128).
// Each column's key/value chain (base plus the residual planes that store it) is
// dequantised exactly in registers.  Per-chunk partials (max, sum, U = sum e_j vhat^(r)_j,
// W = sum p_j vhat^(r-1)_j) are merged by a second kernel, which also writes o and
// shifts the selected scores.
#include "launch.h"

namespace qkv {

constexpr int kChunk = 64;

// Merges the chunk partials of one (sequence, head): o = o_prev + m * U / L - W, then
// shifts the selected scores onto the previous lse scale.  nthreads >= D threads.
template <int D>
__device__ __forceinline__ void sparse_combine(const float* pp, int nchunk, float m, const float* o_prev,
                                               float lse_prev, const int32_t* id, int k, float* srow, int ld,
                                               uint16_t* o, float* o32, int bh, int tid, int nthreads) {
    float M = -__builtin_huge_valf();
    for (int s = 0; s < nchunk; ++s) M = fmaxf(M, pp[(size_t)s * (2 + 2 * D)]);
    float L = 0.f;
    for (int s = 0; s < nchunk; ++s) L = fmaf(pp[(size_t)s * (2 + 2 * D) + 1], __expf(pp[(size_t)s * (2 + 2 * D)] - M), L);
    if (tid < D) {
        const int c = tid;
        float u = 0.f, w = 0.f;
        for (int s = 0; s < nchunk; ++s) {
            const float* q = pp + (size_t)s * (2 + 2 * D);
            u = fmaf(q[2 + c], __expf(q[0] - M), u);
            w += q[2 + D + c];
        }
        const float oc = o_prev[(size_t)bh * D + c] + m * (u / L) - w;
        o32[(size_t)bh * D + c] = oc;
        if (o) o[(size_t)bh * D + c] = f32_to_bf16_rne(oc);
    }
    const float shift = lse_prev + __logf(m) - (M + __logf(L));
    for (int i = tid; i < k; i += nthreads) {
        const int j = id[i];
        if (j >= 0 && j < ld) srow[j] += shift;
    }
}

// k == 0: the output is the previous loop's output
template <int D>
__global__ __launch_bounds__(D) void sparse_copy_kernel(const float* o_prev, uint16_t* __restrict__ o, float* o32) {
    const int bh = blockIdx.x, c = threadIdx.x;
    const float v = o_prev[(size_t)bh * D + c];
    o32[(size_t)bh * D + c] = v;
    if (o) o[(size_t)bh * D + c] = f32_to_bf16_rne(v);
}

template <int D>
__global__ __launch_bounds__(64) void sparse_chunk_kernel(CacheArg ca, int loop, const uint16_t* __restrict__ q,
                                                          float sm, const int32_t* __restrict__ idx,
                                                          const float* __restrict__ p_sel, int k,
                                                          float* __restrict__ scores, int ld,
                                                          float* __restrict__ part, unsigned* __restrict__ counters,
                                                          int nchunk, const float* __restrict__ mass,
                                                          const float* o_prev, const float* __restrict__ lse,
                                                          uint16_t* __restrict__ o, float* o32) {
    constexpr int LPR = Block<D>::kLpr, RPI = Block<D>::kRpi, ROUNDS = kChunk / RPI;
    const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x, prt = lane % LPR, rsub = lane / LPR;
    const int bh = b * ca.H + h;
    const int cap = ca.cap_ctx;

    float qv[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) qv[c] = bf16_to_f32(q[(size_t)bh * D + 32 * prt + c]) * sm;

    float U[32], W[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) { U[c] = 0.f; W[c] = 0.f; }
    float mxw = -__builtin_huge_valf(), lw = 0.f;
    const int32_t* id = idx + (size_t)bh * k;
    const float* ps = p_sel + (size_t)bh * k;

    for (int round = 0; round < ROUNDS; ++round) {
        const int i = chunk * kChunk + round * RPI + rsub;
        int j = i < k ? id[i] : 0;
        const bool valid = i < k && j >= 0 && j < ca.n_ctx;
        j = valid ? j : 0;
        const float pj = valid ? ps[i] : 0.f;
        float kh[32], vh[32], vc[32];
        if (j >= ca.n_body) {
            const size_t slot = ((size_t)bh * kTail + (j % kTail)) * D + 32 * prt;
            const uint16_t* tk = ca.tail_k[loop - 1] + slot;
            const uint16_t* tv = ca.tail_v[loop - 1] + slot;
            const uint16_t* tp = ca.tail_v[loop - 2] + slot;
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                const uint4 a = *reinterpret_cast<const uint4*>(tk + 8 * c4);
                const uint4 bv = *reinterpret_cast<const uint4*>(tv + 8 * c4);
                const uint4 cp = *reinterpret_cast<const uint4*>(tp + 8 * c4);
                const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {bv.x, bv.y, bv.z, bv.w},
                               wc[4] = {cp.x, cp.y, cp.z, cp.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kh[8 * c4 + 2 * e] = bf16_to_f32(wa[e] & 0xFFFFu);
                    kh[8 * c4 + 2 * e + 1] = bf16_to_f32(wa[e] >> 16);
                    vc[8 * c4 + 2 * e] = bf16_to_f32(wb[e] & 0xFFFFu);
                    vc[8 * c4 + 2 * e + 1] = bf16_to_f32(wb[e] >> 16);
                    vh[8 * c4 + 2 * e] = bf16_to_f32(wc[e] & 0xFFFFu);
                    vh[8 * c4 + 2 * e + 1] = bf16_to_f32(wc[e] >> 16);
                }
            }
        } else {
            bool act_r = false;
            for (int p = 0; p < loop; ++p) {
                const PlaneArg& P = ca.p[p];
                const int slot = P.dense ? j : P.rowmap[(size_t)b * cap + j];
                if (slot < 0 || slot >= P.n_blocks * 64) continue;
                const uint8_t* bp = block_ptr<D>(P, ca.H, b, h, slot >> 6);
                const int row = slot & 63;
                float code[32];
                unpack32_codes(*reinterpret_cast<const uint4*>(bp + Block<D>::kKc + row * (D / 2) + prt * 16), code);
                const float* ks = reinterpret_cast<const float*>(bp + Block<D>::kKm) + 32 * prt;
                const float* kz = ks + D;
#pragma unroll
                for (int c = 0; c < 32; ++c) {
                    const float deq = fmaf(code[c], ks[c], kz[c]);
                    kh[c] = (p == 0) ? deq : kh[c] + deq;
                }
                unpack32_codes(*reinterpret_cast<const uint4*>(bp + Block<D>::kVc + row * (D / 2) + prt * 16), code);
                const float2 vm = *reinterpret_cast<const float2*>(bp + Block<D>::kVm + (row * (D / 64) + (prt >> 1)) * 8);
                if (p < loop - 1) {
#pragma unroll
                    for (int c = 0; c < 32; ++c) {
                        const float deq = fmaf(code[c], vm.x, vm.y);
                        vh[c] = (p == 0) ? deq : vh[c] + deq;
                    }
                } else {
                    act_r = true;
#pragma unroll
                    for (int c = 0; c < 32; ++c) vc[c] = vh[c] + fmaf(code[c], vm.x, vm.y);
                }
            }
            if (!act_r) {
#pragma unroll
                for (int c = 0; c < 32; ++c) vc[c] = vh[c];
            }
        }
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < 32; ++c) s = fmaf(qv[c], kh[c], s);
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1) s += __shfl_xor(s, m, 64);
        if (!valid) s = -__builtin_huge_valf();
        else if (prt == 0) scores[(size_t)bh * ld + j] = s;
        const float rm = wave_max(s);
        const float nm = fmaxf(mxw, rm);
        const float scale = (mxw == -__builtin_huge_valf()) ? 0.f : __expf(mxw - nm);
        const float e = valid ? __expf(s - nm) : 0.f;
        lw = lw * scale + ((prt == 0) ? e : 0.f);
#pragma unroll
        for (int c = 0; c < 32; ++c) {
            U[c] = fmaf(e, vc[c], U[c] * scale);
            W[c] = fmaf(pj, vh[c], W[c]);
        }
        mxw = nm;
    }

#pragma unroll
    for (int m = LPR; m < 64; m <<= 1) {
#pragma unroll
        for (int c = 0; c < 32; ++c) {
            U[c] += __shfl_xor(U[c], m, 64);
            W[c] += __shfl_xor(W[c], m, 64);
        }
    }
    lw = wave_sum(lw);
    float* out = part + ((size_t)bh * nchunk + chunk) * (2 + 2 * D);
    if (rsub == 0) {
#pragma unroll
        for (int c = 0; c < 32; ++c) {
            out[2 + 32 * prt + c] = U[c];
            out[2 + D + 32 * prt + c] = W[c];
        }
    }
    if (lane == 0) {
        out[0] = mxw;
        out[1] = lw;
    }

    // the last chunk of this (sequence, head) to finish merges every chunk
    __threadfence();
    unsigned last = 0;
    if (lane == 0) last = (atomicAdd(&counters[bh], 1u) == (unsigned)(nchunk - 1)) ? 1u : 0u;
    last = __shfl(last, 0, 64);
    if (!last) return;
    __threadfence();
    for (int t0 = 0; t0 < D; t0 += 64) {
        // each pass of 64 lanes covers 64 channels; the score shift is applied once
        sparse_combine<D>(part + (size_t)bh * nchunk * (2 + 2 * D), nchunk, mass[bh], o_prev, lse[bh], id,
                          t0 == 0 ? k : 0, scores + (size_t)bh * ld, ld, o, o32, bh, t0 + lane, 64);
    }
    if (lane == 0) atomicExch(&counters[bh], 0u);
}

size_t sparse_ws_bytes(int B, int H, int D, int k) {
    const int nchunk = (k + kChunk - 1) / kChunk;
    return ws_counter_bytes(B, H) + (size_t)B * H * nchunk * (2 + 2 * D) * sizeof(float);
}

int launch_sparse(const CacheArg& ca, int D, int loop, const uint16_t* q, float sm, const int32_t* idx,
                  const float* p_sel, const float* mass, int k, const float* o_prev, const float* lse,
                  float* scores, int ld, uint16_t* o, float* o32, void* ws, hipStream_t st) {
    const int nchunk = (k + kChunk - 1) / kChunk;
    if (nchunk == 0) {
        if (D == 128)
            sparse_copy_kernel<128><<<ca.B * ca.H, 128, 0, st>>>(o_prev, o, o32);
        else
            sparse_copy_kernel<64><<<ca.B * ca.H, 64, 0, st>>>(o_prev, o, o32);
        return hipGetLastError() == hipSuccess ? QKV_OK : QKV_ELAUNCH;
    }
    unsigned* counters = reinterpret_cast<unsigned*>(ws);
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + ws_counter_bytes(ca.B, ca.H));
    dim3 grid(nchunk, ca.H, ca.B);
    if (D == 128)
        sparse_chunk_kernel<128><<<grid, 64, 0, st>>>(ca, loop, q, sm, idx, p_sel, k, scores, ld, part, counters,
                                                      nchunk, mass, o_prev, lse, o, o32);
    else
        sparse_chunk_kernel<64><<<grid, 64, 0, st>>>(ca, loop, q, sm, idx, p_sel, k, scores, ld, part, counters,
                                                     nchunk, mass, o_prev, lse, o, o32);
    return hipGetLastError() == hipSuccess ? QKV_OK : QKV_ELAUNCH;
}

}  // namespace qkv
