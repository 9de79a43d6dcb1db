// Sparse late-loop decode attention with the mass-preserving splice (project page
// STEP 02; explainer section 3: only the top-K columns picked from the preceding loop are
// recomputed, as a rank-K correction of the preceding loop's output that keeps their
// cached mass m).
//
//   o^(r) = o^(r-1) + sum_{j in S} ( m * alpha_j * vhat^(r)_j - p_j * vhat^(r-1)_j ),
//   alpha = softmax over S of s^(r),
//   scores[j] <- lse + log m + s^(r)_j - log sum_S exp(s^(r)).
//
// Gather layout: a column is handled by d/8 lanes of 8 channels each, so one column's
// codes (d/2 bytes), key scales and zeros (4d bytes each) are read with coalesced loads.
// Each wave takes three rounds of 64/(d/8) columns (12 columns at d = 128), dequantises
// each column's key/value chain exactly in registers (base plus the residual planes that
// store it) and keeps an online softmax; the 4 waves of a workgroup merge into one
// partial (max, sum, U = sum e_j vhat^(r)_j, W = sum p_j vhat^(r-1)_j) per chunk.  Three
// rounds per wave keep every wave of a 32K launch resident at once (5 waves per SIMD):
// the gather is a sequence of dependent loads per round, and fewer rounds per wave with
// more waves in flight is what shortens it.
// A second kernel merges the partials of each (sequence, head), writes o and shifts the
// selected scores.
#include <type_traits>

#include "encode_group.h"
#include "launch.h"

namespace qkv {

// Column rounds per wave: three when the launch has waves enough for two or more per SIMD at
// three rounds (a 32K context over 16 heads: 4 416 waves, all resident at 5 per SIMD), two for
// smaller launches, whose waves then carry shorter chains of dependent loads (2 heads x 32K,
// one GPU's share of 16 heads over 8: 65.0 against 72.3 us per layer-step, one round 65.7).
constexpr int kWaveRounds = 3;
constexpr int kWaveRoundsSmall = 2;
constexpr int kSmallLaunchWaves = 2048;        // fewer waves than this at three rounds: two rounds
// selected columns per workgroup (4 waves): d/8 lanes per column, 64 / (d/8) per round
constexpr int kSpWaves = 4;                    // waves per workgroup
constexpr int chunk_cols(int D, int rounds = kWaveRounds) { return kSpWaves * rounds * (64 / (D / 8)); }
// A chunk's partial record: [max, sum, -, -, U[0..D), W[0..D)], 16-byte aligned.
constexpr int sp_record(int D) { return 2 * D + 4; }

// One plane's data of a gathered slot for a lane's 8 channels c0..c0+7: key and value code
// words (BITS bytes each), the key group's scales and zeros, the slot's value (s, z).
struct SlotData {
    uint32_t kw, vw;
    float4 s0, s1, z0, z1;
    float2 vm;
};
template <int D, int BITS>
__device__ __forceinline__ SlotData load_slot(const PlaneArg& P, int H, int b, int h, int slot, int prt, int c0) {
    using Bk = Block<D, BITS>;
    const uint8_t* bp = block_ptr<D, BITS>(P, H, b, h, slot >> 6);
    const int row = slot & 63;
    SlotData d;
    d.kw = ld_codes8<BITS>(bp + Bk::kc(row) + prt * BITS);
    d.vw = ld_codes8<BITS>(bp + Bk::vc(row) + prt * BITS);
    const float* km = reinterpret_cast<const float*>(bp + Bk::kKm) + c0;
    d.s0 = *reinterpret_cast<const float4*>(km);
    d.s1 = *reinterpret_cast<const float4*>(km + 4);
    d.z0 = *reinterpret_cast<const float4*>(km + D);
    d.z1 = *reinterpret_cast<const float4*>(km + D + 4);
    d.vm = ld_stream_f2(bp + Bk::vm(row) + (c0 >> 6) * 8);
    return d;
}

// Stores the newest position's row (nr, [B*H][D]) of (sequence, head) bh in tail ring slot
// `slot` of tk / tv ([B*H][kTail][D]).
template <int D>
__device__ __forceinline__ void store_new_row(NewRow nr, uint16_t* tk, uint16_t* tv, int bh, int slot) {
    if (!nr.k) return;
    const size_t dst = ((size_t)bh * kTail + slot) * D;
    for (int c = threadIdx.x; c < D; c += blockDim.x) {
        tk[dst + c] = nr.k[(size_t)bh * D + c];
        tv[dst + c] = nr.v[(size_t)bh * D + c];
    }
}

// SB: planes whose slots and data a column loads together.  SB = 1 (chains of up to four
// planes) compiles to 92 VGPRs, 5 waves per SIMD, with no occupancy hint: a hint of 5 waves
// makes the scheduler trade 64-bit moves for selects and costs about 1.5 us per call at
// 32K context.  SB = 3 (deeper chains, whose
// loads would otherwise be one memory latency per plane) issues a batch's slot lookups
// together and then every plane's data of the batch together; a plane that does not store
// the column loads its block 0 and weighs it 0, so every plane must hold a block.  It
// runs at 3 waves per SIMD (up to 168 VGPRs).
// RB: code width of the residual planes (planes >= 1).  REPLACE (full-state codec): a
// column's key and value are those of the last plane storing it, not the sum of the chain
// (the host passes the planes from the last dense one before `loop` on).
// FLUSH: extra workgroups past the chunks encode this loop's 64-row tail flush (FlushArg);
// the chunks never read those rows' plane slots in this launch.
template <int D, int SB, int RB, bool REPLACE, bool FLUSH, int ROUNDS = kWaveRounds>
__global__ __launch_bounds__(64 * kSpWaves, SB > 1 ? 3 : 1) void sparse_chunk_kernel(CacheArg ca, int loop, const uint16_t* __restrict__ q,
                                                           NewRow nr, float sm, const int32_t* __restrict__ idx,
                                                           const float* __restrict__ p_sel, int k,
                                                           float* __restrict__ cs,
                                                           float* __restrict__ part, int nchunk, FlushArg fa) {
    constexpr int RBITS = REPLACE ? 4 : RB;  // code width of the planes after the first
    if constexpr (FLUSH) {
        if ((int)blockIdx.x >= nchunk) {
            flush_role<D, RBITS>(ca, fa, (int)blockIdx.x - nchunk, blockIdx.y, blockIdx.z);
            return;
        }
    }
    constexpr int LPC = D / 8;             // lanes per column
    constexpr int CPR = 64 / LPC;          // columns per wave round
    constexpr int kWaveCols = ROUNDS * CPR;
    constexpr int kChunk = chunk_cols(D, ROUNDS);
    static_assert(kChunk == kSpWaves * kWaveCols, "a chunk is the workgroup's columns");
    const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // The newest position is the largest column, so when it is selected it is the last entry
    // of the last chunk: that workgroup stores the position's row (if given) in the tail ring
    // before any of its waves reads the tail, and no other workgroup reads that slot.
    if (nr.k && chunk == nchunk - 1) {
        store_new_row<D>(nr, const_cast<uint16_t*>(ca.tail_k[loop - 1]), const_cast<uint16_t*>(ca.tail_v[loop - 1]),
                         b * ca.H + h, (ca.n_ctx - 1) % kTail);
        __syncthreads();
    }
    const int cid = lane / LPC, prt = lane % LPC;
    const int bh = b * ca.H + h;
    const int cap = ca.cap_ctx;
    const int c0 = 8 * prt;

    float qv[8];
    {
        const uint4 w = *reinterpret_cast<const uint4*>(q + (size_t)bh * D + c0);
        bf16x8(w, qv);
#pragma unroll
        for (int c = 0; c < 8; ++c) qv[c] *= sm;
    }
    float U[8], W[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) { U[c] = 0.f; W[c] = 0.f; }
    float mxw = -__builtin_huge_valf(), lw = 0.f;
    const int32_t* id = idx + (size_t)bh * k;
    const float* ps = p_sel + (size_t)bh * k;

    // planes of the chain (bit p: plane p), and those of them that are dense
    const uint32_t chain_bits = loop >= 32 ? ~0u : ((1u << loop) - 1u);
    uint32_t dense_bits = 0;
    if constexpr (SB > 1) {
        for (int p = 0; p < loop; ++p)
            if (ca.p[p].dense) dense_bits |= 1u << p;
    }
    // Deep chains: the chunk's entries whose column the first sparse plane stores (the long
    // chains) are taken first, spread over the first round of every wave, so that a wave
    // runs at most one long round while a chunk has no more long columns than a round has
    // columns over the workgroup.  perm[s] = the entry at sorted position s.
    __shared__ int perm[SB > 1 ? kChunk : 1];
    if constexpr (SB > 1) {
        if (wave == 0) {
            int probe = -1;  // first sparse plane of the chain (uniform)
            for (int p = 1; p < loop && probe < 0; ++p)
                if (!ca.p[p].dense) probe = p;
            constexpr int NPASS = (kChunk + 63) / 64;
            const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
            uint64_t lm[NPASS], vm[NPASS];
            int nlong = 0;
#pragma unroll
            for (int t = 0; t < NPASS; ++t) {
                const int e = t * 64 + lane, i = chunk * kChunk + e;
                bool lng = false;
                if (e < kChunk && i < k && probe >= 0) {
                    const int j = id[i];
                    if (j >= 0 && j < ca.n_body)
                        lng = ca.smask ? (ca.smask[(size_t)b * cap + j] & chain_bits & ~dense_bits) != 0u
                                       : ca.p[probe].rowmap[(size_t)b * cap + j] >= 0;
                }
                lm[t] = __ballot(lng);
                vm[t] = __ballot(e < kChunk);
                nlong += __popcll(lm[t]);
            }
            int nl = 0, ns = 0;
#pragma unroll
            for (int t = 0; t < NPASS; ++t) {
                const int e = t * 64 + lane;
                const bool lng = (lm[t] >> lane) & 1ull;
                const uint64_t sm_ = ~lm[t] & vm[t];
                const int s = lng ? nl + __popcll(lm[t] & below) : nlong + ns + __popcll(sm_ & below);
                if (e < kChunk) perm[s] = e;
                nl += __popcll(lm[t]);
                ns += __popcll(sm_);
            }
        }
        __syncthreads();
    }

    for (int round = 0; round < ROUNDS; ++round) {
        const int i = chunk * kChunk + (SB > 1 ? perm[round * (kSpWaves * CPR) + wave * CPR + cid]
                                               : wave * kWaveCols + round * CPR + cid);
        int j = i < k ? id[i] : 0;
        const bool valid = i < k && j >= 0 && j < ca.n_ctx;
        j = valid ? j : 0;
        const float pj = valid ? ps[i] : 0.f;
        // deep chains: the planes some column of this wave needs (dense ones, and the sparse
        // ones that store a column), visited in ascending order
        uint32_t cm = 0u, todo = 0u;
        if constexpr (SB > 1) {
            if (ca.smask) {
                cm = j < ca.n_body ? ca.smask[(size_t)b * cap + j] : 0u;
                todo = (dense_bits | __builtin_amdgcn_readfirstlane(wave_or(cm))) & chain_bits;
            } else {
                cm = ~0u;
                todo = chain_bits;
            }
        }
        float kh[8], vh[8], vc[8];
        if (j >= ca.n_body) {
            const size_t off = ((size_t)bh * kTail + (j % kTail)) * D + c0;
            bf16x8(*reinterpret_cast<const uint4*>(ca.tail_k[loop - 1] + off), kh);
            bf16x8(*reinterpret_cast<const uint4*>(ca.tail_v[loop - 1] + off), vc);
            bf16x8(*reinterpret_cast<const uint4*>(ca.tail_v[loop - 2] + off), vh);
        } else {
            bool act_r = false;
            if constexpr (SB > 1) {
                // SB planes of the chain at a time: their slot lookups all in flight together,
                // then all their data (a plane that does not store the column loads its
                // block 0, weighted 0)
                while (todo) {
                    int pp[SB], sl[SB];
#pragma unroll
                    for (int u = 0; u < SB; ++u) {
                        pp[u] = todo ? __builtin_ctz(todo) : -1;
                        todo &= todo - 1u;
                    }
#pragma unroll
                    for (int u = 0; u < SB; ++u) {
                        sl[u] = -1;
                        if (pp[u] >= 0) {
                            const PlaneArg& P = ca.p[pp[u]];
                            if (P.dense)
                                sl[u] = j;
                            else if ((cm >> pp[u]) & 1u)
                                sl[u] = P.rowmap[(size_t)b * cap + j];
                        }
                    }
                    SlotData sd[SB];
                    bool act[SB];
#pragma unroll
                    for (int u = 0; u < SB; ++u) {
                        const int pu = pp[u] >= 0 ? pp[u] : pp[0];
                        const PlaneArg& P = ca.p[pu];
                        act[u] = pp[u] >= 0 && sl[u] >= 0 && sl[u] < P.n_blocks * 64;
                        const int slot = act[u] ? sl[u] : 0;
                        if (pu == 0 || RBITS == 4)
                            sd[u] = load_slot<D, 4>(P, ca.H, b, h, slot, prt, c0);
                        else
                            sd[u] = load_slot<D, RBITS>(P, ca.H, b, h, slot, prt, c0);
                    }
#pragma unroll
                    for (int u = 0; u < SB; ++u) {
                        const int p = pp[u];
                        if (!act[u]) continue;
                        const float ks[8] = {sd[u].s0.x, sd[u].s0.y, sd[u].s0.z, sd[u].s0.w,
                                             sd[u].s1.x, sd[u].s1.y, sd[u].s1.z, sd[u].s1.w};
                        const float kz[8] = {sd[u].z0.x, sd[u].z0.y, sd[u].z0.z, sd[u].z0.w,
                                             sd[u].z1.x, sd[u].z1.y, sd[u].z1.z, sd[u].z1.w};
                        float code[8], vcode[8];
                        if (p == 0 || RBITS == 4) {
                            codes8_bits<4>(sd[u].kw, code);
                            codes8_bits<4>(sd[u].vw, vcode);
                        } else {
                            codes8_bits<RBITS>(sd[u].kw, code);
                            codes8_bits<RBITS>(sd[u].vw, vcode);
                        }
#pragma unroll
                        for (int c = 0; c < 8; ++c) {
                            const float deq = fmaf(code[c], ks[c], kz[c]);
                            kh[c] = (p == 0 || REPLACE) ? deq : kh[c] + deq;
                        }
                        if (p < loop - 1) {
#pragma unroll
                            for (int c = 0; c < 8; ++c) {
                                const float deq = fmaf(vcode[c], sd[u].vm.x, sd[u].vm.y);
                                vh[c] = (p == 0 || REPLACE) ? deq : vh[c] + deq;
                            }
                        } else {
                            act_r = true;
#pragma unroll
                            for (int c = 0; c < 8; ++c) {
                                const float deq = fmaf(vcode[c], sd[u].vm.x, sd[u].vm.y);
                                vc[c] = REPLACE ? deq : vh[c] + deq;
                            }
                        }
                    }
                }
            } else {
                // one plane at a time: its slot, then its data
                for (int p0 = 0; p0 < loop; p0 += SB) {
                    int sl[SB];
#pragma unroll
                    for (int u = 0; u < SB; ++u) {
                        sl[u] = -1;
                        if (p0 + u < loop) {
                            const PlaneArg& P = ca.p[p0 + u];
                            sl[u] = P.dense ? j : P.rowmap[(size_t)b * cap + j];
                        }
                    }
#pragma unroll
                    for (int u = 0; u < SB; ++u) {
                        const int p = p0 + u;
                        if (p >= loop) break;
                        const PlaneArg& P = ca.p[p];
                        const int slot = sl[u];
                        if (slot < 0 || slot >= P.n_blocks * 64) continue;
                        SlotData sd;
                        float code[8], vcode[8];
                        if (p == 0 || RBITS == 4) {
                            sd = load_slot<D, 4>(P, ca.H, b, h, slot, prt, c0);
                            codes8_bits<4>(sd.kw, code);
                            codes8_bits<4>(sd.vw, vcode);
                        } else {
                            sd = load_slot<D, RBITS>(P, ca.H, b, h, slot, prt, c0);
                            codes8_bits<RBITS>(sd.kw, code);
                            codes8_bits<RBITS>(sd.vw, vcode);
                        }
                        const float ks[8] = {sd.s0.x, sd.s0.y, sd.s0.z, sd.s0.w, sd.s1.x, sd.s1.y, sd.s1.z, sd.s1.w};
                        const float kz[8] = {sd.z0.x, sd.z0.y, sd.z0.z, sd.z0.w, sd.z1.x, sd.z1.y, sd.z1.z, sd.z1.w};
#pragma unroll
                        for (int c = 0; c < 8; ++c) {
                            const float deq = fmaf(code[c], ks[c], kz[c]);
                            kh[c] = (p == 0 || REPLACE) ? deq : kh[c] + deq;
                        }
                        if (p < loop - 1) {
#pragma unroll
                            for (int c = 0; c < 8; ++c) {
                                const float deq = fmaf(vcode[c], sd.vm.x, sd.vm.y);
                                vh[c] = (p == 0 || REPLACE) ? deq : vh[c] + deq;
                            }
                        } else {
                            act_r = true;
#pragma unroll
                            for (int c = 0; c < 8; ++c) {
                                const float deq = fmaf(vcode[c], sd.vm.x, sd.vm.y);
                                vc[c] = REPLACE ? deq : vh[c] + deq;
                            }
                        }
                    }
                }
            }
            if (!act_r) {
#pragma unroll
                for (int c = 0; c < 8; ++c) vc[c] = vh[c];
            }
        }
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) s = fmaf(qv[c], kh[c], s);
        s = lane_group_sum<LPC>(s);
        if (!valid) s = -__builtin_huge_valf();
        else if (prt == 0 && cs) cs[(size_t)bh * k + i] = s;  // raw score of entry i; the combine shifts it
        const float nm = fmaxf(mxw, wave_max(s));
        const float scale = (mxw == -__builtin_huge_valf()) ? 0.f : __expf(mxw - nm);
        const float e = valid ? __expf(s - nm) : 0.f;
        lw = lw * scale + ((prt == 0) ? e : 0.f);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            U[c] = fmaf(e, vc[c], U[c] * scale);
            W[c] = fmaf(pj, vh[c], W[c]);
        }
        mxw = nm;
    }

    // wave totals: sum the columns of the wave (lanes with the same channels)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        if (LPC == 8) {   // the two column groups of a 16-lane row
            U[c] += dpp<kRowRor8>(U[c]);
            W[c] += dpp<kRowRor8>(W[c]);
        }
        U[c] = add_xor32(add_xor16(U[c]));
        W[c] = add_xor32(add_xor16(W[c]));
    }
    lw = wave_sum(lw);
    __shared__ float wU[kSpWaves][D], wW[kSpWaves][D], wm[kSpWaves], wl[kSpWaves];
    if (cid == 0) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            wU[wave][c0 + c] = U[c];
            wW[wave][c0 + c] = W[c];
        }
    }
    if (lane == 0) {
        wm[wave] = mxw;
        wl[wave] = lw;
    }
    __syncthreads();
    float M = wm[0];
#pragma unroll
    for (int w = 1; w < kSpWaves; ++w) M = fmaxf(M, wm[w]);
    float* out = part + ((size_t)bh * nchunk + chunk) * sp_record(D);
    for (int t = tid; t < 2 * D; t += 64 * kSpWaves) {
        float a = 0.f;
        if (t < D) {
#pragma unroll
            for (int w = 0; w < kSpWaves; ++w)
                if (wm[w] != -__builtin_huge_valf()) a = fmaf(wU[w][t], __expf(wm[w] - M), a);
        } else {
#pragma unroll
            for (int w = 0; w < kSpWaves; ++w) a += wW[w][t - D];
        }
        out[4 + t] = a;
    }
    if (tid == 0) {
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < kSpWaves; ++w)
            if (wm[w] != -__builtin_huge_valf()) L = fmaf(wl[w], __expf(wm[w] - M), L);
        out[0] = M;
        out[1] = L;
    }
}

// Merges the chunk partials of each (sequence, head): o = o_prev + m * U / L - W, then
// shifts the selected scores onto the previous lse scale.
constexpr int kSpCombineWaves = 16;

// Merge of the n chunk records of one (sequence, head) by NW waves.  Every wave forms the
// global max M and L = sum_s sum_s * exp(max_s - M) itself (lanes over records, fixed-order
// wave reductions).  Wave w then adds up records w, w + NW, ... in record order, U in
// flight: one 16-byte load per lane and record, lanes [0, D/4) holding U (rescaled by
// exp(max_s - M)) and lanes [D/4, D/2) holding W (plain sums).  Its sums go to
// red[w * 2D + c] (U) and red[w * 2D + D + c] (W); the caller adds the NW wave sums in wave
// order after a barrier.
template <int D, int NW, int U>
__device__ __forceinline__ void merge_chunk_records(const float* pp, int n, float* red, float* gmax, float* gsum) {
    constexpr float kNeg = -__builtin_huge_valf();
    constexpr int SR = sp_record(D);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float m0 = lane < n ? pp[(size_t)lane * SR] : kNeg;
    const float l0 = lane < n ? pp[(size_t)lane * SR + 1] : 0.f;
    const float m1 = lane + 64 < n ? pp[(size_t)(lane + 64) * SR] : kNeg;
    const float l1 = lane + 64 < n ? pp[(size_t)(lane + 64) * SR + 1] : 0.f;
    float m = fmaxf(m0, m1);
    for (int s = lane + 128; s < n; s += 64) m = fmaxf(m, pp[(size_t)s * SR]);
    const float M = wave_max(m);
    float l = 0.f;
    if (m0 != kNeg) l = l0 * __expf(m0 - M);
    if (m1 != kNeg) l = fmaf(l1, __expf(m1 - M), l);
    for (int s = lane + 128; s < n; s += 64) {
        const float ms = pp[(size_t)s * SR];
        if (ms != kNeg) l = fmaf(pp[(size_t)s * SR + 1], __expf(ms - M), l);
    }
    *gmax = M;
    *gsum = wave_sum(l);

    const bool on = lane < D / 2, is_u = lane < D / 4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = wave; s0 < n; s0 += U * NW) {
        float4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = s0 + u * NW;
            x[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (s < n && on) x[u] = reinterpret_cast<const float4*>(pp + (size_t)s * SR)[1 + lane];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = s0 + u * NW;
            if (s < n) {
                const int mb = s < 64 ? __builtin_amdgcn_readlane(__float_as_int(m0), s)
                                      : s < 128 ? __builtin_amdgcn_readlane(__float_as_int(m1), s - 64)
                                                : __float_as_int(pp[(size_t)s * SR]);
                const float msf = __int_as_float(mb);
                const float w = is_u ? (msf == kNeg ? 0.f : __expf(msf - M)) : 1.f;
                acc.x = fmaf(x[u].x, w, acc.x);
                acc.y = fmaf(x[u].y, w, acc.y);
                acc.z = fmaf(x[u].z, w, acc.z);
                acc.w = fmaf(x[u].w, w, acc.w);
            }
        }
    }
    if (on) *reinterpret_cast<float4*>(red + wave * 2 * D + 4 * lane) = acc;
}

template <int D>
__global__ __launch_bounds__(64 * kSpCombineWaves) void sparse_combine_kernel(
    const float* __restrict__ part, int nchunk, const float* __restrict__ mass, const float* o_prev,
    const float* __restrict__ lse, const int32_t* __restrict__ idx, const float* __restrict__ cs, int k,
    float* __restrict__ scores, int ld, uint16_t* __restrict__ o, float* o32) {
    constexpr int NT = 64 * kSpCombineWaves;
    const int bh = blockIdx.x, tid = threadIdx.x;
    __shared__ __align__(16) float red[kSpCombineWaves * 2 * D];
    // the selected columns and their raw scores (entry order), the mass, the previous lse
    // and output: none depends on the merge, so all go out with the partials
    // (no score buffer: the splice is not stored)
    constexpr int kPre = 4;
    const bool splice = scores != nullptr;
    float* srow = splice ? scores + (size_t)bh * ld : nullptr;
    const int32_t* id = idx + (size_t)bh * k;
    const float* cr = splice ? cs + (size_t)bh * k : nullptr;
    int jv[kPre];
    float sv[kPre];
#pragma unroll
    for (int e = 0; e < kPre; ++e) {
        const int i = tid + e * NT;
        jv[e] = splice && i < k ? id[i] : -1;
        sv[e] = splice && i < k ? cr[i] : 0.f;
    }
    const float m = mass[bh], lse_prev = lse[bh];
    const float op = tid < D ? o_prev[(size_t)bh * D + tid] : 0.f;
    float M, L;
    merge_chunk_records<D, kSpCombineWaves, 6>(part + (size_t)bh * nchunk * sp_record(D), nchunk, red, &M, &L);
    // every wave holds M and L: the spliced scores need no barrier
    const float shift = lse_prev + __logf(m) - (M + __logf(L));
#pragma unroll
    for (int e = 0; e < kPre; ++e)
        if (jv[e] >= 0 && jv[e] < ld) srow[jv[e]] = sv[e] + shift;
    for (int i = tid + kPre * NT; splice && i < k; i += NT) {
        const int j = id[i];
        if (j >= 0 && j < ld) srow[j] = cr[i] + shift;
    }
    __syncthreads();
    if (tid < D) {
        float u = 0.f, w = 0.f;
#pragma unroll
        for (int wv = 0; wv < kSpCombineWaves; ++wv) {
            u += red[wv * 2 * D + tid];
            w += red[wv * 2 * D + D + tid];
        }
        const float oc = op + m * (u / L) - w;
        o32[(size_t)bh * D + tid] = oc;
        if (o) o[(size_t)bh * D + tid] = f32_to_bf16_rne(oc);
    }
}

// k == 0: the output is the previous loop's output
template <int D>
__global__ __launch_bounds__(D) void sparse_copy_kernel(const float* o_prev, uint16_t* __restrict__ o, float* o32,
                                                        NewRow nr, uint16_t* tk, uint16_t* tv, int slot) {
    const int bh = blockIdx.x, c = threadIdx.x;
    store_new_row<D>(nr, tk, tv, bh, slot);
    const float v = o_prev[(size_t)bh * D + c];
    o32[(size_t)bh * D + c] = v;
    if (o) o[(size_t)bh * D + c] = f32_to_bf16_rne(v);
}

// workspace: chunk partials [B][H][nchunk][2 + 2D], then the raw selected scores [B][H][k]
size_t sparse_ws_bytes(int B, int H, int D, int k) {
    const int cc = chunk_cols(D, kWaveRoundsSmall);   // the smaller chunks: the most records
    const int nchunk = (k + cc - 1) / cc;
    return (size_t)B * H * nchunk * sp_record(D) * sizeof(float) + (size_t)B * H * k * sizeof(float);
}

int launch_sparse(const CacheArg& ca, int D, int loop, const uint16_t* q, NewRow nr, float sm, const int32_t* idx,
                  const float* p_sel, const float* mass, int k, const float* o_prev, const float* lse,
                  float* scores, int ld, uint16_t* o, float* o32, void* ws, hipStream_t st, FlushArg fl) {
    // full-state codec: the planes from the last dense one before `loop` on
    int lv = loop;
    const CacheArg v = ca.full ? full_state_view(ca, loop - 1, &lv) : ca;
    if (ca.full) lv += 1;  // the view was taken for loop - 1
    // deep chains: batched loads (and long chains first), which need every plane of the
    // chain to hold a block
    bool batched = lv > 4;
    for (int p = 0; batched && p < lv; ++p) batched = v.p[p].data != nullptr && v.p[p].n_blocks > 0;
    // rounds per wave: two for launches too small to fill the chip at three
    const long waves3 = (long)((k + chunk_cols(D) - 1) / chunk_cols(D)) * ca.H * ca.B * kSpWaves;
    const bool small = !batched && waves3 < kSmallLaunchWaves;
    const int ccols = small ? chunk_cols(D, kWaveRoundsSmall) : chunk_cols(D);
    const int nchunk = (k + ccols - 1) / ccols;
    uint16_t* tk = const_cast<uint16_t*>(ca.tail_k[loop - 1]);
    uint16_t* tv = const_cast<uint16_t*>(ca.tail_v[loop - 1]);
    const int slot = (ca.n_ctx - 1) % kTail;
    if (nchunk == 0) {
        if (D == 128)
            sparse_copy_kernel<128><<<ca.B * ca.H, 128, 0, st>>>(o_prev, o, o32, nr, tk, tv, slot);
        else
            sparse_copy_kernel<64><<<ca.B * ca.H, 64, 0, st>>>(o_prev, o, o32, nr, tk, tv, slot);
        if (hipGetLastError() != hipSuccess) return QKV_ELAUNCH;
        // no chunk kernel to carry the tail flush: the encoder's own launch
        if (fl.pos0 >= 0)
            return launch_encode(ca, D, loop, fl.pos0, 64, fl.act_pos, fl.n_act, fl.ld_act, nullptr, nullptr, 0, st);
        return QKV_OK;
    }
    float* part = static_cast<float*>(ws);
    float* cs = scores ? part + (size_t)ca.B * ca.H * nchunk * sp_record(D) : nullptr;  // raw scores for the splice
    dim3 grid(nchunk, ca.H, ca.B);
    if (fl.pos0 >= 0) fl.loop = lv;
    const int extra = flush_groups(fl, !ca.p[loop - 1].dense);
    grid.x += extra;
    const size_t dyn = extra ? (size_t)fl.nch * 64 * sizeof(int) : 0;
    auto chunks = [&](auto dc, auto rbc, auto fullc) {
        constexpr int DD = decltype(dc)::value, RBB = decltype(rbc)::value;
        constexpr bool FF = decltype(fullc)::value;
        if (!batched) {
            auto go = [&](auto rc) {
                constexpr int RR = decltype(rc)::value;
                if (extra)
                    sparse_chunk_kernel<DD, 1, RBB, FF, true, RR><<<grid, 64 * kSpWaves, dyn, st>>>(
                        v, lv, q, nr, sm, idx, p_sel, k, cs, part, nchunk, fl);
                else
                    sparse_chunk_kernel<DD, 1, RBB, FF, false, RR><<<grid, 64 * kSpWaves, 0, st>>>(
                        v, lv, q, nr, sm, idx, p_sel, k, cs, part, nchunk, fl);
            };
            if (small) go(std::integral_constant<int, kWaveRoundsSmall>{});
            else go(std::integral_constant<int, kWaveRounds>{});
        } else {
            if (extra)
                sparse_chunk_kernel<DD, 3, RBB, FF, true><<<grid, 64 * kSpWaves, dyn, st>>>(v, lv, q, nr, sm, idx, p_sel,
                                                                                        k, cs, part, nchunk, fl);
            else
                sparse_chunk_kernel<DD, 3, RBB, FF, false><<<grid, 64 * kSpWaves, 0, st>>>(v, lv, q, nr, sm, idx, p_sel,
                                                                                       k, cs, part, nchunk, fl);
        }
        sparse_combine_kernel<DD><<<ca.B * ca.H, 64 * kSpCombineWaves, 0, st>>>(part, nchunk, mass, o_prev, lse, idx, cs,
                                                                              k, scores, ld, o, o32);
    };
    using I64 = std::integral_constant<int, 64>;
    using I128 = std::integral_constant<int, 128>;
    using B2 = std::integral_constant<int, 2>;
    using B4 = std::integral_constant<int, 4>;
    using T = std::true_type;
    using F = std::false_type;
    if (D == 128) {
        if (ca.full) chunks(I128{}, B4{}, T{});
        else if (ca.rbits == 2) chunks(I128{}, B2{}, F{});
        else chunks(I128{}, B4{}, F{});
    } else {
        if (ca.full) chunks(I64{}, B4{}, T{});
        else if (ca.rbits == 2) chunks(I64{}, B2{}, F{});
        else chunks(I64{}, B4{}, F{});
    }
    return hipGetLastError() == hipSuccess ? QKV_OK : QKV_ELAUNCH;
}

}  // namespace qkv
