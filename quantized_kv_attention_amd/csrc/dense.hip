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
// in a fixed order.  The last split of each (sequence, head) also reads the BF16 tail.
#include <type_traits>

#include "encode_group.h"
#include "launch.h"

namespace qkv {

constexpr int kMaxSpb = 16;  // 64-position blocks per split, at most

__device__ __forceinline__ float block_reduce_max(float v, float* red) {
    v = wave_max(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ __forceinline__ float block_reduce_sum(float v, float* red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// Folded query of one key block: qp[c] = 2^9 * q[c] * s[c] (LDS), returns sum_c q[c] z[c].
template <int D, int BITS>
__device__ __forceinline__ float fold_query(const uint8_t* bp, const float* qsh, float* qp, int lane) {
    const float* km = reinterpret_cast<const float*>(bp + Block<D, BITS>::kKm);
    float bias = 0.f;
#pragma unroll
    for (int c = lane; c < D; c += 64) {
        const float qc = qsh[c];
        qp[c] = qc * km[c] * kFp8CodeScale;
        bias = fmaf(qc, km[D + c], bias);
    }
    return wave_sum_dpp(bias);
}

// K pass over one 64-slot block with the folded query computed here (planes that are not
// prepared per split): calls emit(row, partial_logit) on one lane per row.
template <int D, int BITS, typename Emit>
__device__ __forceinline__ void kpass_block(const uint8_t* bp, const float* qsh, float* qp_lds, int lane, int prt,
                                            int rsub, Emit emit) {
    using Bk = Block<D, BITS>;
    constexpr int LPR = Bk::kLpr, RPI = Bk::kRpi, NLD = 64 / RPI;
    uint4 w[NLD];
#pragma unroll
    for (int it = 0; it < NLD; ++it) w[it] = ld_codes32<BITS>(bp + Bk::kc(rsub + RPI * it) + prt * Bk::kLaneBytes);
    const float bias = fold_query<D, BITS>(bp, qsh, qp_lds, lane);
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
        const float v = group_sum<LPR>(dot32_bits<BITS>(w[it], qp));
        if (prt == 0) emit(rsub + RPI * it, v + bias);
    }
}

// V pass over one block: weight(row) returns the row's probability (0 to skip).
template <int D, int BITS, typename Weight>
__device__ __forceinline__ void vpass_block(const uint8_t* bp, int prt, int rsub, float* acc, float& vb,
                                            Weight weight) {
    using Bk = Block<D, BITS>;
    constexpr int RPI = Bk::kRpi, NLD = 64 / RPI;
    uint4 w[NLD];
    float2 m[NLD];
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
        const int row = rsub + RPI * it;
        w[it] = ld_codes32<BITS>(bp + Bk::vc(row) + prt * Bk::kLaneBytes);
        m[it] = ld_stream_f2(bp + Bk::vm(row) + (prt >> 1) * 8);
    }
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
        const float pw = weight(rsub + RPI * it);
        vb = fmaf(pw, m[it].y, vb);
        axpy32_bits<BITS>(w[it], pw * m[it].x * kFp8CodeScale, acc);
    }
}

// NPRE (1 or 2): leading dense planes whose blocks are read together, with their folded
// queries prepared once per split; later planes (sparse, or dense beyond NPRE) follow one
// by one.  Three waves per SIMD (the plan's three workgroups per CU) leave up to 168 VGPRs
// per wave.  With its plane loads on the streaming policy the two-plane kernel compiles to
// 128, but four workgroups per CU made the decode step slower.
// RB: code width of the residual planes (planes >= 1).  REPLACE (the full-state codec,
// whose planes hold whole K/V states, not residuals): a column's key and value are those of
// the last plane that stores it, so later planes overwrite logits instead of adding to
// them, and in the V pass the deepest plane storing a position takes its probability (the
// host passes the planes from the last dense one on, which then stores every position).
// FLUSH: the grid carries extra workgroups past the splits that encode this loop's 64-row
// tail flush (FlushArg); the splits never read those rows in this launch.
template <int D, int NPRE, int RB, bool REPLACE, bool FLUSH>
__global__ __launch_bounds__(256, 3) void dense_split_kernel(CacheArg ca, int loop, const uint16_t* __restrict__ q,
                                                          NewRow nr, float sm, float* __restrict__ scores, int ld,
                                                          float* __restrict__ part, int nsplit, int spb,
                                                          FlushArg fa) {
    static_assert(!REPLACE || (NPRE == 1 && RB == 4), "full-state planes: one prepared plane, 4-bit codes");
    if constexpr (FLUSH) {
        if ((int)blockIdx.x >= nsplit) {
            flush_role<D, REPLACE ? 4 : RB>(ca, fa, (int)blockIdx.x - nsplit, blockIdx.y, blockIdx.z);
            return;
        }
    }
    constexpr int LPR = Block<D>::kLpr, RPI = Block<D>::kRpi, NLD = 64 / RPI;
    constexpr int RBITS = REPLACE ? 4 : RB;  // code width of the planes after the first
    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: block addresses stay scalar
    const int prt = lane % LPR, rsub = lane / LPR;
    const int bh = b * ca.H + h;

    __shared__ float qsh[D];
    __shared__ float logit[kMaxSpb * 64];
    __shared__ float qpre[NPRE][kMaxSpb][D];
    __shared__ float bpre[NPRE][kMaxSpb];
    __shared__ float qps[4][D];
    __shared__ float red[4];
    __shared__ float ored[4][D];

    // ---- body split: blocks [blk0, blk1); the last split also takes the BF16 tail ----
    const int nblk = ca.n_body / 64;
    const int blk0 = s * spb, blk1 = min(blk0 + spb, nblk);
    const int nb = max(0, blk1 - blk0);
    const int j0 = blk0 * 64, L = nb * 64;
    const bool has_tail = (s == nsplit - 1);
    const int T = has_tail ? ca.n_ctx - ca.n_body : 0;  // tail rows land in logit[L + i]
    // The newest position's row (if given) goes into the tail ring first; this workgroup
    // reads the tail only after several barriers, and no other workgroup reads it.
    if (has_tail && nr.k) {
        const size_t dst = ((size_t)(b * ca.H + h) * kTail + (ca.n_ctx - 1) % kTail) * D;
        for (int c = threadIdx.x; c < D; c += 256) {
            const_cast<uint16_t*>(ca.tail_k[loop - 1])[dst + c] = nr.k[(size_t)(b * ca.H + h) * D + c];
            const_cast<uint16_t*>(ca.tail_v[loop - 1])[dst + c] = nr.v[(size_t)(b * ca.H + h) * D + c];
        }
    }
    const int nstart = ca.cap_ctx / 64 + 1;
    const int blkA = blk0 + wave;                         // this wave's first block
    // Prefetches are unconditional (a branch around them makes the compiler wait for them at
    // the join): a wave without blocks loads a valid block it does not use.
    const int blkP = max(0, min(blkA, blk1 - 1));

    // Codes of a block of the prepared planes: K codes, V codes + per-row V meta.  Plane p's
    // code width is 4 bits for p = 0 and RBITS after it (compile-time once unrolled).
    uint4 wk[NPRE][NLD];
    auto load_k = [&](int blk) {
#pragma unroll
        for (int p = 0; p < NPRE; ++p) {
#pragma unroll
            for (int it = 0; it < NLD; ++it) {
                const int row = rsub + RPI * it;
                if (p == 0 || RBITS == 4)
                    wk[p][it] = ld_codes32<4>(block_ptr<D, 4>(ca.p[p], ca.H, b, h, blk) + Block<D, 4>::kc(row) +
                                              prt * Block<D, 4>::kLaneBytes);
                else
                    wk[p][it] = ld_codes32<RBITS>(block_ptr<D, RBITS>(ca.p[p], ca.H, b, h, blk) +
                                                  Block<D, RBITS>::kc(row) + prt * Block<D, RBITS>::kLaneBytes);
            }
        }
    };
    for (int c = tid; c < D; c += 256) qsh[c] = bf16_to_f32(q[(size_t)bh * D + c]) * sm;
    float* out = part + ((size_t)bh * nsplit + s) * (D + 2);
    float* srow = scores ? scores + (size_t)bh * ld : nullptr;  // null: raw scores not stored

    float acc[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) acc[k] = 0.f;
    float vb = 0.f;
    float mx, lsum;
    // Every plane of the chain prepared (loops 1 and 2 of the residual codec): each wave reads
    // only the logits of its own blocks and tail rows, so it keeps a softmax of its own
    // (max, sum) and the waves are merged once at the end, with no workgroup barrier between
    // the key and the value pass.
    const bool wl = loop == NPRE;

    {
        {
        // Folded queries of the prepared planes, once per split: each wave takes blocks
        // wave, wave + 4, ... of every prepared plane (the plane index stays a compile-time
        // constant, so the plane descriptors are scalar loads).  All key scales and zeros
        // are loaded before any is used.
        constexpr int npre = NPRE;
        constexpr int kFold = (kMaxSpb + 3) / 4;
        constexpr int CPL = D / 64;  // channels per lane
        float fs[NPRE][kFold][CPL], fz[NPRE][kFold][CPL];
#pragma unroll
        for (int p = 0; p < NPRE; ++p) {
#pragma unroll
            for (int u = 0; u < kFold; ++u) {
                const int bb = wave + 4 * u;
                if (bb < nb) {
                    const float* km = reinterpret_cast<const float*>(
                        (p == 0 || RBITS == 4)
                            ? block_ptr<D, 4>(ca.p[p], ca.H, b, h, blk0 + bb) + Block<D, 4>::kKm
                            : block_ptr<D, RBITS>(ca.p[p], ca.H, b, h, blk0 + bb) + Block<D, RBITS>::kKm);
#pragma unroll
                    for (int cc = 0; cc < CPL; ++cc) {
                        fs[p][u][cc] = ld_stream_f32(km + lane + 64 * cc);
                        fz[p][u][cc] = ld_stream_f32(km + D + lane + 64 * cc);
                    }
                }
            }
        }
        // the first block's key codes are in flight while the query is folded
        load_k(blkP);
        __syncthreads();  // qsh
#pragma unroll
        for (int p = 0; p < NPRE; ++p) {
#pragma unroll
            for (int u = 0; u < kFold; ++u) {
                const int bb = wave + 4 * u;
                if (bb < nb) {
                    float bias = 0.f;
#pragma unroll
                    for (int cc = 0; cc < CPL; ++cc) {
                        const float qc = qsh[lane + 64 * cc];
                        qpre[p][bb][lane + 64 * cc] = qc * fs[p][u][cc] * kFp8CodeScale;
                        bias = fmaf(qc, fz[p][u][cc], bias);
                    }
                    bias = wave_sum_dpp(bias);
                    if (lane == 0) bpre[p][bb] = bias;
                }
            }
        }
        if (wl) wave_sync_lds();  // a wave folds the blocks it reads
        else __syncthreads();

        // K pass, prepared planes: logits of every row of the block summed over the planes.
        // Each block step sets the wave's issue priority from the share of its blocks still
        // to go (both passes): co-resident workgroups then keep pace with each other, where
        // oldest-first issue would finish them one after another and leave the CU with a
        // single workgroup's loads in flight at the end.
        const int nbw = blkA < blk1 ? (blk1 - blkA + 3) >> 2 : 0;  // this wave's blocks
        for (int blk = blkA; blk < blk1; blk += 4) {
            const int bb = blk - blk0;
            prio_by_work_left(2 * nbw - ((blk - blkA) >> 2), 2 * nbw);
            if (blk != blkA) load_k(blk);
            float lg[NLD];
#pragma unroll
            for (int it = 0; it < NLD; ++it) lg[it] = 0.f;
            float bias = 0.f;
#pragma unroll
            for (int p = 0; p < NPRE; ++p) {
                float qp[32];
#pragma unroll
                for (int k = 0; k < 32; k += 4) {
                    const float4 t = *reinterpret_cast<const float4*>(&qpre[p][bb][32 * prt + k]);
                    qp[k] = t.x; qp[k + 1] = t.y; qp[k + 2] = t.z; qp[k + 3] = t.w;
                }
#pragma unroll
                for (int it = 0; it < NLD; ++it)
                    lg[it] += (p == 0 || RBITS == 4) ? dot32_bits<4>(wk[p][it], qp) : dot32_bits<RBITS>(wk[p][it], qp);
                bias += bpre[p][bb];
            }
#pragma unroll
            for (int it = 0; it < NLD; ++it) {
                const float v = group_sum<LPR>(lg[it]);
                if (prt == 0) logit[bb * 64 + rsub + RPI * it] = v + bias;
            }
        }
        if (!wl) __syncthreads();
        // K pass, remaining planes (sparse planes, or dense planes beyond the prepared ones),
        // in ascending order: their partial logits add up (or, full-state, overwrite)
        for (int p = npre; p < loop; ++p) {
            const PlaneArg& P = ca.p[p];
            if (P.dense) {
                for (int blk = blk0 + wave; blk < blk1; blk += 4) {
                    const uint8_t* bp = block_ptr<D, RBITS>(P, ca.H, b, h, blk);
                    float* lg = logit + (blk - blk0) * 64;
                    kpass_block<D, RBITS>(bp, qsh, qps[wave], lane, prt, rsub, [&](int row, float v) {
                        lg[row] = REPLACE ? v : lg[row] + v;
                    });
                }
            } else {
                const int rs0 = P.rowstart[(size_t)b * nstart + blk0];
                const int rs1 = P.rowstart[(size_t)b * nstart + blk1];
                const int32_t* rp = P.rowpos + (size_t)b * P.n_blocks * 64;
                for (int sb = (rs0 >> 6) + wave; sb * 64 < rs1 && sb < P.n_blocks; sb += 4) {
                    const uint8_t* bp = block_ptr<D, RBITS>(P, ca.H, b, h, sb);
                    kpass_block<D, RBITS>(bp, qsh, qps[wave], lane, prt, rsub, [&](int row, float v) {
                        const int slot = sb * 64 + row;
                        if (slot >= rs0 && slot < rs1) {
                            const int pos = rp[slot] - j0;
                            if (pos >= 0 && pos < L) logit[pos] = REPLACE ? v : logit[pos] + v;
                        }
                    });
                }
            }
            __syncthreads();
        }
        if (has_tail) {
            const uint16_t* tk = ca.tail_k[loop - 1] + (size_t)bh * kTail * D;
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
                v = group_sum<LPR>(v);
                if (prt == 0 && i < T) logit[L + i] = v;
            }
            if (!wl) __syncthreads();
        }
        if (wl) wave_sync_lds();
        // The first block's value codes are in flight during the softmax.
        uint4 wv[NPRE][NLD];
        float2 mv[NPRE][NLD];
        auto load_v = [&](int blk) {
#pragma unroll
            for (int p = 0; p < NPRE; ++p) {
#pragma unroll
                for (int it = 0; it < NLD; ++it) {
                    const int row = rsub + RPI * it;
                    // a row's value meta: the even lanes of its quad load it (lane 2 the second
                    // 64-channel group at d = 128), the odd lanes take it by DPP at use
                    mv[p][it] = make_float2(0.f, 0.f);
                    if (p == 0 || RBITS == 4) {
                        const uint8_t* bp = block_ptr<D, 4>(ca.p[p], ca.H, b, h, blk);
                        wv[p][it] = ld_codes32<4>(bp + Block<D, 4>::vc(row) + prt * Block<D, 4>::kLaneBytes);
                        if ((prt & 1) == 0) mv[p][it] = ld_stream_f2(bp + Block<D, 4>::vm(row) + (prt >> 1) * 8);
                    } else {
                        const uint8_t* bp = block_ptr<D, RBITS>(ca.p[p], ca.H, b, h, blk);
                        wv[p][it] = ld_codes32<RBITS>(bp + Block<D, RBITS>::vc(row) + prt * Block<D, RBITS>::kLaneBytes);
                        if ((prt & 1) == 0) mv[p][it] = ld_stream_f2(bp + Block<D, RBITS>::vm(row) + (prt >> 1) * 8);
                    }
                }
            }
        };
        load_v(blkP);
        if (wl) {
            // this wave's rows: lane l of each of its blocks, then its tail rows (RPI-row
            // groups wave, wave + 4, ... as the tail passes take them)
            float lm = -__builtin_huge_valf();
            for (int bb = wave; bb < nb; bb += 4) {
                const float x = logit[bb * 64 + lane];
                if (srow) srow[j0 + bb * 64 + lane] = x;
                lm = fmaxf(lm, x);
            }
            for (int i0 = wave * RPI; i0 < T; i0 += 4 * RPI) {
                const int i = i0 + lane;
                if (lane < RPI && i < T) {
                    const float x = logit[L + i];
                    if (srow) srow[j0 + L + i] = x;  // j0 + L == n_body
                    lm = fmaxf(lm, x);
                }
            }
            mx = wave_max(lm);
            float ls = 0.f;
            if (mx != -__builtin_huge_valf()) {
                for (int bb = wave; bb < nb; bb += 4) {
                    const float pv = __expf(logit[bb * 64 + lane] - mx);
                    logit[bb * 64 + lane] = pv;
                    ls += pv;
                }
                for (int i0 = wave * RPI; i0 < T; i0 += 4 * RPI) {
                    const int i = i0 + lane;
                    if (lane < RPI && i < T) {
                        const float pv = __expf(logit[L + i] - mx);
                        logit[L + i] = pv;
                        ls += pv;
                    }
                }
            }
            lsum = wave_sum(ls);
            wave_sync_lds();
        } else {
            float lm = -__builtin_huge_valf();
            for (int i = tid; i < L + T; i += 256) {
                if (srow) srow[j0 + i] = logit[i];  // the tail rows follow the split's body rows (j0 + L == n_body)
                lm = fmaxf(lm, logit[i]);
            }
            mx = block_reduce_max(lm, red);
            float ls = 0.f;
            for (int i = tid; i < L + T; i += 256) {
                const float pv = __expf(logit[i] - mx);
                logit[i] = pv;
                ls += pv;
            }
            lsum = block_reduce_sum(ls, red);
        }

        // V pass, remaining planes.  Residual codec: every plane adds its part of each stored
        // position's value.  Full-state codec: the deepest plane storing a position takes its
        // probability, so the planes run deepest first and each one clears the probabilities
        // it used before the next (shallower) one, and finally the prepared plane, runs.
        auto vpass_plane = [&](int p) {
            const PlaneArg& P = ca.p[p];
            if (P.dense) {
                for (int blk = blk0 + wave; blk < blk1; blk += 4) {
                    const uint8_t* bp = block_ptr<D, RBITS>(P, ca.H, b, h, blk);
                    const float* lg = logit + (blk - blk0) * 64;
                    vpass_block<D, RBITS>(bp, prt, rsub, acc, vb, [&](int row) { return lg[row]; });
                }
                if (REPLACE) {
                    __syncthreads();
                    for (int i = tid; i < L; i += 256) logit[i] = 0.f;
                }
            } else {
                const int rs0 = P.rowstart[(size_t)b * nstart + blk0];
                const int rs1 = P.rowstart[(size_t)b * nstart + blk1];
                const int32_t* rp = P.rowpos + (size_t)b * P.n_blocks * 64;
                for (int sb = (rs0 >> 6) + wave; sb * 64 < rs1 && sb < P.n_blocks; sb += 4) {
                    const uint8_t* bp = block_ptr<D, RBITS>(P, ca.H, b, h, sb);
                    vpass_block<D, RBITS>(bp, prt, rsub, acc, vb, [&](int row) {
                        const int slot = sb * 64 + row;
                        float pw = 0.f;
                        if (slot >= rs0 && slot < rs1) {
                            const int pos = rp[slot] - j0;
                            if (pos >= 0 && pos < L) pw = logit[pos];
                        }
                        return pw;
                    });
                }
                if (REPLACE) {
                    __syncthreads();  // every wave has read the probabilities of this plane's positions
                    for (int slot = rs0 + tid; slot < rs1; slot += 256) {
                        const int pos = rp[slot] - j0;
                        if (pos >= 0 && pos < L) logit[pos] = 0.f;
                    }
                }
            }
            if (REPLACE) __syncthreads();
        };
        if (REPLACE) {
            for (int p = loop - 1; p >= npre; --p) vpass_plane(p);
        }
        // V pass, prepared planes: every plane's codes of the block loaded together
        for (int blk = blkA; blk < blk1; blk += 4) {
            const int bb = blk - blk0;
            prio_by_work_left(nbw - ((blk - blkA) >> 2), 2 * nbw);
            if (blk != blkA) load_v(blk);
#pragma unroll
            for (int it = 0; it < NLD; ++it) {
                const float pw = logit[bb * 64 + rsub + RPI * it];
#pragma unroll
                for (int p = 0; p < NPRE; ++p) {
                    const float vs = dpp<kQuadEven>(mv[p][it].x), vz = dpp<kQuadEven>(mv[p][it].y);
                    vb = fmaf(pw, vz, vb);
                    if (p == 0 || RBITS == 4)
                        axpy32_bits<4>(wv[p][it], pw * vs * kFp8CodeScale, acc);
                    else
                        axpy32_bits<RBITS>(wv[p][it], pw * vs * kFp8CodeScale, acc);
                }
            }
        }
        if (!REPLACE) {
            for (int p = npre; p < loop; ++p) vpass_plane(p);
        }
        }  // general path
        if (has_tail) {
            const uint16_t* tv = ca.tail_v[loop - 1] + (size_t)bh * kTail * D;
            for (int i0 = wave * RPI; i0 < T; i0 += 4 * RPI) {
                const int i = i0 + rsub;
                if (i < T) {
                    const float pw = logit[L + i];
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
        }
    }

    // reduce the per-lane accumulators over the rows of the wave, then over waves
#pragma unroll
    for (int k = 0; k < 32; ++k) {
        float v = acc[k];
        if (LPR == 4) {
            v += dpp<kRowRor4>(v);   // lanes of a 16-lane row with the same channel part
            v += dpp<kRowRor8>(v);
        } else {
            v += dpp<kQuadXor2>(v);  // LPR 2: rows of a quad
            v += dpp<kRowRor4>(v);
            v += dpp<kRowRor8>(v);
        }
        v = add_xor32(add_xor16(v));
        acc[k] = v;
    }
    {
        float v = vb;
        if (LPR == 4) {
            v += dpp<kRowRor4>(v);
            v += dpp<kRowRor8>(v);
        } else {
            v += dpp<kQuadXor2>(v);
            v += dpp<kRowRor4>(v);
            v += dpp<kRowRor8>(v);
        }
        v = add_xor32(add_xor16(v));
        vb = v;
    }
    if (rsub == 0) {
#pragma unroll
        for (int k = 0; k < 32; ++k) ored[wave][32 * prt + k] = acc[k] + vb;
    }
    if (wl) {
        // the waves' (max, sum, o) merged on the workgroup maximum, in wave order
        __shared__ float wmx[4], wls[4];
        if (lane == 0) {
            wmx[wave] = mx;
            wls[wave] = lsum;
        }
        __syncthreads();
        const float M = fmaxf(fmaxf(wmx[0], wmx[1]), fmaxf(wmx[2], wmx[3]));
        float e[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) e[w] = wmx[w] == -__builtin_huge_valf() ? 0.f : __expf(wmx[w] - M);
        for (int c = tid; c < D; c += 256)
            out[2 + c] = fmaf(ored[0][c], e[0], ored[1][c] * e[1]) + fmaf(ored[2][c], e[2], ored[3][c] * e[3]);
        if (tid == 0) {
            out[0] = M;
            out[1] = fmaf(wls[0], e[0], wls[1] * e[1]) + fmaf(wls[2], e[2], wls[3] * e[3]);
        }
        return;
    }
    __syncthreads();
    for (int c = tid; c < D; c += 256) out[2 + c] = (ored[0][c] + ored[1][c]) + (ored[2][c] + ored[3][c]);
    if (tid == 0) {
        out[0] = mx;
        out[1] = lsum;
    }
}

// Second kernel of the reader: merges the splits of each (sequence, head) in split order.
// (A kernel boundary publishes the partials; a per-workgroup device-scope fence in the
// split kernel would write back and invalidate L2 once per workgroup.)
constexpr int kCombineWaves = 4;  // 4 / 8 / 16 waves measured on the step: 4 fastest

template <int D>
__global__ __launch_bounds__(64 * kCombineWaves) void dense_combine_kernel(const float* __restrict__ part, int nsplit,
                                                                          uint16_t* __restrict__ o,
                                                                          float* __restrict__ o32,
                                                                          float* __restrict__ lse) {
    const int bh = blockIdx.x, tid = threadIdx.x;
    __shared__ float red[kCombineWaves * D];
    float M, L;
    merge_records<D, kCombineWaves, 12, false>(part + (size_t)bh * nsplit * (D + 2), nsplit, D + 2, red, &M, &L);
    __syncthreads();
    if (tid < D) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < kCombineWaves; ++w) t += red[w * D + tid];
        const float oc = t / L;
        o32[(size_t)bh * D + tid] = oc;
        if (o) o[(size_t)bh * D + tid] = f32_to_bf16_rne(oc);
    }
    if (tid == 0) lse[bh] = M + __logf(L);
}

DensePlan dense_plan(int B, int H, int n_body) {
    const int nblk = n_body / 64;
    DensePlan pl;
    if (nblk == 0) {
        pl.spb = 1;
        pl.nsplit = 1;  // the tail alone
        return pl;
    }
    // Splits for 3 workgroups per CU (768 over 256 CUs; the split kernel's launch bounds fit 3):
    // measured at 32K context, this beats both one full round (1024) and several rounds.
    // More than kMaxSpb - 2 blocks per split would leave no LDS for the tail.
    const long slots = 768;
    long per_bh = slots / ((long)B * H);
    if (per_bh < 1) per_bh = 1;
    int spb = (int)((nblk + per_bh - 1) / per_bh);
    spb = spb < 4 ? 4 : (spb > kMaxSpb - 2 ? kMaxSpb - 2 : spb);  // leave room for 127 tail rows
    pl.spb = spb;
    pl.nsplit = (nblk + spb - 1) / spb;
    return pl;
}

// workspace: the split partials [B][H][nsplit][2 + D]
size_t dense_ws_bytes(int B, int H, int D, int n_body) {
    const DensePlan pl = dense_plan(B, H, n_body);
    return (size_t)B * H * pl.nsplit * (D + 2) * sizeof(float);
}

// The planes a full-state read of loop `loop` needs: from the last dense plane at or before
// it (which stores every position and overrides every earlier plane) to `loop`.  The
// argument's planes and tails are shifted so that plane 0 is that dense plane; *loop_out is
// the loop's index in the shifted argument.
CacheArg full_state_view(const CacheArg& ca, int loop, int* loop_out) {
    int pd = 0;
    for (int p = 0; p < loop; ++p)
        if (ca.p[p].dense) pd = p;
    CacheArg v = ca;
    for (int p = 0; p < QKV_MAX_LOOPS; ++p) {
        const int src = p + pd;
        v.p[p] = src < QKV_MAX_LOOPS ? ca.p[src] : PlaneArg{};
        v.tail_k[p] = src < QKV_MAX_LOOPS ? ca.tail_k[src] : nullptr;
        v.tail_v[p] = src < QKV_MAX_LOOPS ? ca.tail_v[src] : nullptr;
    }
    v.nplanes = ca.nplanes - pd;
    v.smask = nullptr;  // its bits name the unshifted planes
    *loop_out = loop - pd;
    return v;
}

template <int D>
static void launch_dense_d(const CacheArg& ca, int loop, const uint16_t* q, NewRow nr, float sm, uint16_t* o, float* o32,
                           float* scores, int ld, float* lse, float* part, hipStream_t st, FlushArg fl) {
    const DensePlan pl = dense_plan(ca.B, ca.H, ca.n_body);
    int lv = loop;
    const CacheArg v = ca.full ? full_state_view(ca, loop, &lv) : ca;
    if (fl.pos0 >= 0) fl.loop = lv;
    const int extra = flush_groups(fl, !ca.p[loop - 1].dense);
    dim3 grid(pl.nsplit + extra, ca.H, ca.B);
    const size_t dyn = extra ? (size_t)fl.nch * 64 * sizeof(int) : 0;
    auto go = [&](auto npre, auto rb, auto rep) {
        constexpr int NP = decltype(npre)::value, RBB = decltype(rb)::value;
        constexpr bool RP = decltype(rep)::value;
        if (extra)
            dense_split_kernel<D, NP, RBB, RP, true><<<grid, 256, dyn, st>>>(v, lv, q, nr, sm, scores, ld, part,
                                                                            pl.nsplit, pl.spb, fl);
        else
            dense_split_kernel<D, NP, RBB, RP, false><<<grid, 256, 0, st>>>(v, lv, q, nr, sm, scores, ld, part,
                                                                           pl.nsplit, pl.spb, fl);
    };
    using N1 = std::integral_constant<int, 1>;
    using N2 = std::integral_constant<int, 2>;
    using B2 = std::integral_constant<int, 2>;
    using B4 = std::integral_constant<int, 4>;
    // plane 1 (the base) is always dense; plane 2 joins it when it is dense too
    const bool two = loop >= 2 && ca.p[1].dense;
    if (ca.full) go(N1{}, B4{}, std::true_type{});
    else if (ca.rbits == 2) { if (two) go(N2{}, B2{}, std::false_type{}); else go(N1{}, B2{}, std::false_type{}); }
    else { if (two) go(N2{}, B4{}, std::false_type{}); else go(N1{}, B4{}, std::false_type{}); }
    dense_combine_kernel<D><<<ca.B * ca.H, 64 * kCombineWaves, 0, st>>>(part, pl.nsplit, o, o32, lse);
}

int launch_dense(const CacheArg& ca, int D, int loop, const uint16_t* q, NewRow nr, float sm, uint16_t* o, float* o32,
                 float* scores, int ld, float* lse, void* ws, hipStream_t st, FlushArg fl) {
    float* part = static_cast<float*>(ws);
    if (D == 128)
        launch_dense_d<128>(ca, loop, q, nr, sm, o, o32, scores, ld, lse, part, st, fl);
    else
        launch_dense_d<64>(ca, loop, q, nr, sm, o, o32, scores, ld, lse, part, st, fl);
    return hipGetLastError() == hipSuccess ? QKV_OK : QKV_ELAUNCH;
}

}  // namespace qkv
