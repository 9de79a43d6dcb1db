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
// planes a lane group of the deep-chain kernel loads together for a long column (two keep it
// within the registers of 3 waves per SIMD beside the short rounds' two columns per group)
constexpr int kDeepBatch = 2;
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
// The slot's block bp and row in it.
template <int D, int BITS>
__device__ __forceinline__ SlotData load_slot_bp(const uint8_t* bp, int row, int prt, int c0) {
    using Bk = Block<D, BITS>;
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
// From a plane given by its data and blocks per (sequence, head); bh = b * H + h.
template <int D, int BITS>
__device__ __forceinline__ SlotData load_slot_at(const uint8_t* data, int n_blocks, int bh, int slot, int prt,
                                                 int c0) {
    return load_slot_bp<D, BITS>(data + ((size_t)bh * n_blocks + (slot >> 6)) * Block<D, BITS>::kBytes, slot & 63,
                                 prt, c0);
}
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

// The chunk's partial record from the waves' online-softmax states: each wave sums U and W
// over its column groups (lanes holding the same channels), then the waves are merged on
// the workgroup maximum, in wave order.
template <int D>
__device__ __forceinline__ void write_chunk_record(float (&U)[8], float (&W)[8], float mxw, float lw, float* out) {
    constexpr int LPC = D / 8;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cid = lane / LPC, c0 = 8 * (lane % LPC);
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

// Chains of up to four planes.  A column's planes are read one after another (its slot in a
// sparse plane, then the plane's data); the kernel compiles to 94 VGPRs, 5 waves per SIMD,
// with no occupancy hint: a hint of 5 waves makes the scheduler trade 64-bit moves for
// selects and costs about 1.5 us per call at 32K context.
// RB: code width of the residual planes (planes >= 1).  REPLACE (full-state codec): a
// column's key and value are those of the last plane storing it, not the sum of the chain
// (the host passes the planes from the last dense one before `loop` on).
// FLUSH: extra workgroups past the chunks encode this loop's 64-row tail flush (FlushArg);
// the chunks never read those rows' plane slots in this launch.
template <int D, int RB, bool REPLACE, bool FLUSH, int ROUNDS = kWaveRounds>
__global__ __launch_bounds__(64 * kSpWaves, 1) void sparse_chunk_kernel(CacheArg ca, int loop, const uint16_t* __restrict__ q,
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

    for (int round = 0; round < ROUNDS; ++round) {
        const int i = chunk * kChunk + wave * kWaveCols + round * CPR + cid;
        int j = i < k ? id[i] : 0;
        const bool valid = i < k && j >= 0 && j < ca.n_ctx;
        j = valid ? j : 0;
        const float pj = valid ? ps[i] : 0.f;
        float kh[8], vh[8], vc[8];
        if (j >= ca.n_body) {
            const size_t off = ((size_t)bh * kTail + (j % kTail)) * D + c0;
            bf16x8(*reinterpret_cast<const uint4*>(ca.tail_k[loop - 1] + off), kh);
            bf16x8(*reinterpret_cast<const uint4*>(ca.tail_v[loop - 1] + off), vc);
            bf16x8(*reinterpret_cast<const uint4*>(ca.tail_v[loop - 2] + off), vh);
        } else if constexpr (ROUNDS == kWaveRoundsSmall) {
            // Launches too small to fill the chip wait on memory latency, not on bandwidth:
            // every load that depends on no other plane's is issued together (the sparse
            // planes' slot lookups with the dense planes' data), so a round waits on three
            // memory round trips (its entry, those, then the sparse planes' data) instead of
            // one or two per plane.  Registers are not short at this wave count.
            constexpr int NPM = 4;  // this kernel's chains have at most four planes
            int sl[NPM];
#pragma unroll
            for (int p = 0; p < NPM; ++p) {
                const PlaneArg& P = ca.p[p < loop ? p : 0];
                sl[p] = p >= loop ? -1 : (P.dense ? j : P.rowmap[(size_t)b * cap + j]);
            }
            SlotData sd[NPM];
            bool ok[NPM];
#pragma unroll
            for (int p = 0; p < NPM; ++p) {
                const PlaneArg& P = ca.p[p < loop ? p : 0];
                ok[p] = sl[p] >= 0 && sl[p] < P.n_blocks * 64;
                const int slot = ok[p] ? sl[p] : 0;  // a plane not read loads a valid slot
                if (p == 0 || RBITS == 4)
                    sd[p] = load_slot<D, 4>(P, ca.H, b, h, slot, prt, c0);
                else
                    sd[p] = load_slot<D, RBITS>(P, ca.H, b, h, slot, prt, c0);
            }
            bool act_r = false;
#pragma unroll
            for (int p = 0; p < NPM; ++p) {
                if (!ok[p]) continue;
                float code[8], vcode[8];
                if (p == 0 || RBITS == 4) {
                    codes8_bits<4>(sd[p].kw, code);
                    codes8_bits<4>(sd[p].vw, vcode);
                } else {
                    codes8_bits<RBITS>(sd[p].kw, code);
                    codes8_bits<RBITS>(sd[p].vw, vcode);
                }
                const float ks[8] = {sd[p].s0.x, sd[p].s0.y, sd[p].s0.z, sd[p].s0.w,
                                     sd[p].s1.x, sd[p].s1.y, sd[p].s1.z, sd[p].s1.w};
                const float kz[8] = {sd[p].z0.x, sd[p].z0.y, sd[p].z0.z, sd[p].z0.w,
                                     sd[p].z1.x, sd[p].z1.y, sd[p].z1.z, sd[p].z1.w};
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const float deq = fmaf(code[c], ks[c], kz[c]);
                    kh[c] = (p == 0 || REPLACE) ? deq : kh[c] + deq;
                }
                if (p < loop - 1) {
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        const float deq = fmaf(vcode[c], sd[p].vm.x, sd[p].vm.y);
                        vh[c] = (p == 0 || REPLACE) ? deq : vh[c] + deq;
                    }
                } else {
                    act_r = true;
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        const float deq = fmaf(vcode[c], sd[p].vm.x, sd[p].vm.y);
                        vc[c] = REPLACE ? deq : vh[c] + deq;
                    }
                }
            }
            if (!act_r) {
#pragma unroll
                for (int c = 0; c < 8; ++c) vc[c] = vh[c];
            }
        } else {
            bool act_r = false;
            // one plane at a time: its slot, then its data
            constexpr int SB = 1;
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

// Sum (max) of a value over the wave's CPR lane groups of 64 / CPR lanes, the same in every
// lane: the groups are added pairwise by lane exchanges, so every lane forms the same sums.
template <int CPR>
__device__ __forceinline__ float xgroup_sum(float v) {
    if (CPR == 8) v += dpp<kRowRor8>(v);
    return add_xor32(add_xor16(v));
}
template <int CPR>
__device__ __forceinline__ int xgroup_max(int v) {
    if (CPR == 8) v = max(v, __float_as_int(dpp<kRowRor8>(__int_as_float(v))));
    float2 p = pair_xor16(__int_as_float(v));
    v = max(__float_as_int(p.x), __float_as_int(p.y));
    p = pair_xor32(__int_as_float(v));
    return max(__float_as_int(p.x), __float_as_int(p.y));
}
// planes p with p % CPR == g
template <int CPR>
__device__ __forceinline__ uint32_t group_planes(int g) {
    return (CPR == 4 ? 0x11111111u : 0x01010101u) << g;
}

// Deep chains (more than four planes, as in a 32-loop recurrence).  A column that a sparse
// plane of its chain stores ("long") has up to one plane per loop to read, each behind a
// row-map lookup; the other columns ("short": dense planes only, whose slot is the position,
// or tail rows) have few.
//  * Prologue: the first wave reads the chunk's entries (column, selection probability,
//    stored-loops word) once and sorts them long first into LDS; then the workgroup looks up
//    every long column's slot in every plane of its chain, all in one memory round trip.
//  * A long column is taken by a whole wave: its CPR lane groups walk the planes p = g,
//    g + CPR, g + 2 CPR, ... of the chain, SB at a time, each keeping its part of the score
//    and of the value sums, which are then added across the wave.
//  * A short round takes 2 CPR columns, two per lane group, with both columns' loads of a
//    plane in flight together.  A column's key enters only through its score, so each column
//    keeps its part of the score over the lane's channels rather than the key itself.
//  The rounds, long ones first, are dealt to the waves in turn.  Without the stored-loops
// words the first wave looks every entry up in each sparse plane of the chain instead (the
// same split, at one dependent lookup per plane).  Plane p of `ca` is bit p + sshift of a
// stored-loops word (a full-state view starts at a later plane).
// dense_bits: bit p set iff plane p of `ca` is dense (from the host: reading the flags from the
// kernel arguments in a loop costs one scalar round trip per plane).
// Every plane of the chain must hold a block: a lane group without a plane in a batch loads
// the block 0 of plane 0 and weighs it 0.
// At 40 heads x 128, 8K context and 32 loops this took the layer-step from 1758 to 1123 us,
// against the batched form of the shallow kernel (three planes of four columns per wave at a
// time, each batch behind its own row-map lookups).
template <int D, int RB, bool REPLACE, bool FLUSH, int SB>
__global__ __launch_bounds__(64 * kSpWaves, 3) void deep_chunk_kernel(CacheArg ca, int loop, const uint16_t* __restrict__ q,
                                                                     NewRow nr, float sm, const int32_t* __restrict__ idx,
                                                                     const float* __restrict__ p_sel, int k,
                                                                     float* __restrict__ cs, float* __restrict__ part,
                                                                     int nchunk, FlushArg fa, int sshift,
                                                                     uint32_t dense_bits) {
    constexpr int RBITS = REPLACE ? 4 : RB;
    const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    if constexpr (FLUSH) {
        if (chunk >= nchunk) {
            flush_role<D, RBITS>(ca, fa, chunk - nchunk, h, b);
            return;
        }
    }
    constexpr int LPC = D / 8;             // lanes per column (8 channels each)
    constexpr int CPR = 64 / LPC;          // columns of a short round; plane groups of a long one
    constexpr int kChunk = chunk_cols(D);
    constexpr int NPASS = (kChunk + 63) / 64;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (nr.k && chunk == nchunk - 1) {
        store_new_row<D>(nr, const_cast<uint16_t*>(ca.tail_k[loop - 1]), const_cast<uint16_t*>(ca.tail_v[loop - 1]),
                         b * ca.H + h, (ca.n_ctx - 1) % kTail);
        __syncthreads();
    }
    const int cid = lane / LPC, prt = lane % LPC;
    const int bh = b * ca.H + h;
    const int cap = ca.cap_ctx;
    const int c0 = 8 * prt;
    const uint32_t chain_bits = loop >= 32 ? ~0u : ((1u << loop) - 1u);

    // the chain's planes, for lanes that each read another plane
    __shared__ const uint8_t* t_data[QKV_MAX_LOOPS];
    __shared__ const int32_t* t_map[QKV_MAX_LOOPS];
    __shared__ int t_nb[QKV_MAX_LOOPS];
    // the chunk's entries, long columns first: entry index, column, p_sel, stored-loops word
    __shared__ int e_i[kChunk], e_j[kChunk];
    __shared__ float e_p[kChunk];
    __shared__ uint32_t e_cm[kChunk];
    __shared__ int e_slot[kChunk][QKV_MAX_LOOPS];   // long entries: the column's slot in each plane
    __shared__ int s_n[2];
    if (wave == 1 && lane < QKV_MAX_LOOPS) {
        const bool in = lane < loop;
        t_data[lane] = in ? ca.p[lane].data : nullptr;
        t_map[lane] = in ? ca.p[lane].rowmap : nullptr;
        t_nb[lane] = in ? ca.p[lane].n_blocks : 0;
    }
    if (wave == 0) {
        const int32_t* id = idx + (size_t)bh * k;
        const float* ps = p_sel + (size_t)bh * k;
        const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
        int col[NPASS];
        float pr[NPASS];
        uint32_t cmv[NPASS];
        uint64_t lm[NPASS], sm_[NPASS];
        int nlong = 0, nshort = 0;
#pragma unroll
        for (int t = 0; t < NPASS; ++t) {
            const int e = t * 64 + lane, i = chunk * kChunk + e;
            int j = -1;
            float pj = 0.f;
            if (e < kChunk && i < k) {
                j = id[i];
                pj = ps[i];
                if (j < 0 || j >= ca.n_ctx) j = -1;   // an unused entry: no weight, no score
            }
            uint32_t cm = 0u;
            bool lng = false;
            if (j >= 0 && j < ca.n_body) {
                if (ca.smask) {
                    cm = ca.smask[(size_t)b * cap + j] >> sshift;
                    lng = (cm & chain_bits & ~dense_bits) != 0u;
                } else {
                    cm = ~0u;
                    for (int p = 1; p < loop; ++p)
                        if (!((dense_bits >> p) & 1u)) lng |= ca.p[p].rowmap[(size_t)b * cap + j] >= 0;
                }
            }
            col[t] = j;
            pr[t] = pj;
            cmv[t] = cm;
            lm[t] = __ballot(lng);
            sm_[t] = __ballot(j >= 0 && !lng);
            nlong += __popcll(lm[t]);
            nshort += __popcll(sm_[t]);
        }
        int nl = 0, ns = 0;
#pragma unroll
        for (int t = 0; t < NPASS; ++t) {
            const int e = t * 64 + lane;
            const bool lng = (lm[t] >> lane) & 1ull, sht = (sm_[t] >> lane) & 1ull;
            const int s = lng ? nl + __popcll(lm[t] & below) : nlong + ns + __popcll(sm_[t] & below);
            if (lng || sht) {
                e_i[s] = chunk * kChunk + e;
                e_j[s] = col[t];
                e_p[s] = pr[t];
                e_cm[s] = cmv[t];
            }
            nl += __popcll(lm[t]);
            ns += __popcll(sm_[t]);
        }
        if (lane == 0) {
            s_n[0] = nlong;
            s_n[1] = nshort;
        }
    }

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
    __syncthreads();
    const int nlong = s_n[0], nshort = s_n[1];
    const int nrounds = nlong + (nshort + 2 * CPR - 1) / (2 * CPR);   // short rounds take 2 CPR columns
    // every long column's slot in every plane of its chain, in one memory round trip
    for (int x = tid; x < nlong * QKV_MAX_LOOPS; x += 64 * kSpWaves) {
        const int e = x / QKV_MAX_LOOPS, p = x % QKV_MAX_LOOPS;
        const int j = e_j[e];
        int slot = -1;
        if (((dense_bits | e_cm[e]) & chain_bits) >> p & 1u)
            slot = ((dense_bits >> p) & 1u) ? j : t_map[p][(size_t)b * cap + j];
        e_slot[e][p] = slot;
    }
    if (nlong) __syncthreads();

    // The online-softmax update of the wave with the columns of one round: NC columns per
    // lane group, the column's score s (all lanes of a group hold it, -inf if unused), its
    // weight in U (e = exp(s - max); 0 for groups that do not count the column), p_sel, and
    // its values.
    auto update = [&](auto ncc, const float* sv, const bool* cnt, const float* pw, const float (*vcv)[8],
                      const float (*vhv)[8]) __attribute__((always_inline)) {
        constexpr int NC = decltype(ncc)::value;
        float m = sv[0];
#pragma unroll
        for (int u = 1; u < NC; ++u) m = fmaxf(m, sv[u]);
        const float nm = fmaxf(mxw, wave_max(m));
        const float scale = (mxw == -__builtin_huge_valf()) ? 0.f : __expf(mxw - nm);
        float e[NC], esum = 0.f;
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            e[u] = cnt[u] ? __expf(sv[u] - nm) : 0.f;
            esum += e[u];
        }
        lw = lw * scale + ((prt == 0) ? esum : 0.f);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float a = U[c] * scale, w = W[c];
#pragma unroll
            for (int u = 0; u < NC; ++u) {
                a = fmaf(e[u], vcv[u][c], a);
                w = fmaf(pw[u], vhv[u][c], w);
            }
            U[c] = a;
            W[c] = w;
        }
        mxw = nm;
    };
    const uint32_t dchain = dense_bits & chain_bits;

    for (int t = wave; t < nrounds; t += kSpWaves) {
        if (t < nlong) {
            // one long column over the whole wave
            const int i = e_i[t];
            const float pj = e_p[t];
            const uint32_t set = (dense_bits | e_cm[t]) & chain_bits;
            uint32_t gset = set & group_planes<CPR>(cid);
            float vh[1][8], vc[1][8], vr[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) { vh[0][c] = 0.f; vr[c] = 0.f; }
            float sq = 0.f;         // the group's planes' part of the score over the lane's channels
            int pk = -1, pv = -1;   // full-state codec: the last planes seen for keys and values
            bool ar = false;
            while (__ballot(gset != 0u)) {
                int pp[SB], sl[SB];
#pragma unroll
                for (int u = 0; u < SB; ++u) {
                    pp[u] = gset ? __builtin_ctz(gset) : -1;
                    gset &= gset - 1u;
                }
#pragma unroll
                for (int u = 0; u < SB; ++u) sl[u] = pp[u] < 0 ? -1 : e_slot[t][pp[u]];
                SlotData sd[SB];
                bool act[SB];
#pragma unroll
                for (int u = 0; u < SB; ++u) {
                    const int pu = pp[u] < 0 ? 0 : pp[u];
                    const int nb = t_nb[pu];
                    act[u] = pp[u] >= 0 && sl[u] >= 0 && sl[u] < nb * 64;
                    const int slot = act[u] ? sl[u] : 0;
                    if (pu == 0 || RBITS == 4)
                        sd[u] = load_slot_at<D, 4>(t_data[pu], nb, bh, slot, prt, c0);
                    else
                        sd[u] = load_slot_at<D, RBITS>(t_data[pu], nb, bh, slot, prt, c0);
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
                    float sp = 0.f;
#pragma unroll
                    for (int c = 0; c < 8; ++c) sp = fmaf(qv[c], fmaf(code[c], ks[c], kz[c]), sp);
                    sq = REPLACE ? sp : sq + sp;
                    if (REPLACE) pk = p;
                    if (p < loop - 1) {
#pragma unroll
                        for (int c = 0; c < 8; ++c) {
                            const float deq = fmaf(vcode[c], sd[u].vm.x, sd[u].vm.y);
                            vh[0][c] = REPLACE ? deq : vh[0][c] + deq;
                        }
                        if (REPLACE) pv = p;
                    } else {
                        ar = true;
#pragma unroll
                        for (int c = 0; c < 8; ++c) vr[c] = fmaf(vcode[c], sd[u].vm.x, sd[u].vm.y);
                    }
                }
            }
            if constexpr (REPLACE) {
                // only the group holding the last plane keeps its key (value) term
                const int PK = xgroup_max<CPR>(pk), PV = xgroup_max<CPR>(pv);
                sq = pk == PK ? sq : 0.f;
#pragma unroll
                for (int c = 0; c < 8; ++c) vh[0][c] = pv == PV ? vh[0][c] : 0.f;
            }
            const bool act_r = __ballot(ar) != 0ull;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                vh[0][c] = xgroup_sum<CPR>(vh[0][c]);
                vr[c] = xgroup_sum<CPR>(vr[c]);
                vc[0][c] = act_r ? (REPLACE ? vr[c] : vh[0][c] + vr[c]) : vh[0][c];
            }
            const float s = lane_group_sum<LPC>(xgroup_sum<CPR>(sq));
            const bool own = cid == 0;   // every group holds the column: the first one counts it
            if (own && prt == 0 && cs) cs[(size_t)bh * k + i] = s;
            const float sv[1] = {s}, pw[1] = {own ? pj : 0.f};
            const bool cnt[1] = {own};
            update(std::integral_constant<int, 1>{}, sv, cnt, pw, vc, vh);
        } else {
            // 2 CPR short columns: lane group cid takes entries base + cid and base + CPR + cid,
            // the dense planes of both in flight together (slot = position); a column's key
            // enters only through its score, so each keeps its part of the score (sq) over the
            // lane's channels, plane by plane
            constexpr int NC = 2;
            const int base = nlong + (t - nlong) * NC * CPR + cid;
            bool valid[NC], act_r[NC];
            int i[NC], j[NC];
            float pj[NC], sq[NC], vh[NC][8], vr[NC][8];
#pragma unroll
            for (int u = 0; u < NC; ++u) {
                const int sp = base + u * CPR;
                valid[u] = sp < nlong + nshort;
                i[u] = valid[u] ? e_i[sp] : 0;
                j[u] = valid[u] ? e_j[sp] : 0;
                pj[u] = valid[u] ? e_p[sp] : 0.f;
                sq[u] = 0.f;
                act_r[u] = false;
                if (j[u] >= ca.n_body) {
                    const size_t off = ((size_t)bh * kTail + (j[u] % kTail)) * D + c0;
                    float kt[8];
                    bf16x8(*reinterpret_cast<const uint4*>(ca.tail_k[loop - 1] + off), kt);
                    bf16x8(*reinterpret_cast<const uint4*>(ca.tail_v[loop - 1] + off), vr[u]);
                    bf16x8(*reinterpret_cast<const uint4*>(ca.tail_v[loop - 2] + off), vh[u]);
#pragma unroll
                    for (int c = 0; c < 8; ++c) sq[u] = fmaf(qv[c], kt[c], sq[u]);
                    act_r[u] = true;   // the tail holds this loop's value itself
                }
            }
            uint32_t todo = dchain;
            while (todo) {
                const int p = __builtin_ctz(todo);
                todo &= todo - 1u;
                const PlaneArg& P = ca.p[p];
                SlotData sd[NC];
                bool act[NC];
#pragma unroll
                for (int u = 0; u < NC; ++u) {
                    act[u] = j[u] < ca.n_body && j[u] < P.n_blocks * 64;
                    const int slot = act[u] ? j[u] : 0;
                    if (p == 0 || RBITS == 4)
                        sd[u] = load_slot<D, 4>(P, ca.H, b, h, slot, prt, c0);
                    else
                        sd[u] = load_slot<D, RBITS>(P, ca.H, b, h, slot, prt, c0);
                }
#pragma unroll
                for (int u = 0; u < NC; ++u) {
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
                    float spp = 0.f;
#pragma unroll
                    for (int c = 0; c < 8; ++c) spp = fmaf(qv[c], fmaf(code[c], ks[c], kz[c]), spp);
                    sq[u] = (p == 0 || REPLACE) ? spp : sq[u] + spp;
                    if (p < loop - 1) {
#pragma unroll
                        for (int c = 0; c < 8; ++c) {
                            const float deq = fmaf(vcode[c], sd[u].vm.x, sd[u].vm.y);
                            vh[u][c] = (p == 0 || REPLACE) ? deq : vh[u][c] + deq;
                        }
                    } else {
                        act_r[u] = true;
#pragma unroll
                        for (int c = 0; c < 8; ++c) vr[u][c] = fmaf(vcode[c], sd[u].vm.x, sd[u].vm.y);
                    }
                }
            }
            float sv[NC], vc[NC][8];
#pragma unroll
            for (int u = 0; u < NC; ++u) {
                const bool tail = j[u] >= ca.n_body;
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    vc[u][c] = !act_r[u] ? vh[u][c] : (REPLACE || tail) ? vr[u][c] : vh[u][c] + vr[u][c];
                float s = lane_group_sum<LPC>(sq[u]);
                if (!valid[u]) s = -__builtin_huge_valf();
                else if (prt == 0 && cs) cs[(size_t)bh * k + i[u]] = s;
                sv[u] = s;
            }
            update(std::integral_constant<int, NC>{}, sv, valid, pj, vc, vh);
        }
    }
    write_chunk_record<D>(U, W, mxw, lw, part + ((size_t)bh * nchunk + chunk) * sp_record(D));
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
    CacheArg v = ca.full ? full_state_view(ca, loop - 1, &lv) : ca;
    if (ca.full) lv += 1;  // the view was taken for loop - 1
    // the view's plane p is the cache's plane p + sshift: the deep-chain kernel reads the
    // stored-loops words shifted by as much
    const int sshift = loop - lv;
    if (ca.full) v.smask = ca.smask;
    uint32_t dbits = 0;   // the dense planes of the chain
    for (int p = 0; p < lv && p < QKV_MAX_LOOPS; ++p)
        if (v.p[p].dense) dbits |= 1u << p;
    // deep chains: the kernel that spreads a long column's planes over a wave, which needs
    // every plane of the chain to hold a block
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
                    sparse_chunk_kernel<DD, RBB, FF, true, RR><<<grid, 64 * kSpWaves, dyn, st>>>(
                        v, lv, q, nr, sm, idx, p_sel, k, cs, part, nchunk, fl);
                else
                    sparse_chunk_kernel<DD, RBB, FF, false, RR><<<grid, 64 * kSpWaves, 0, st>>>(
                        v, lv, q, nr, sm, idx, p_sel, k, cs, part, nchunk, fl);
            };
            if (small) go(std::integral_constant<int, kWaveRoundsSmall>{});
            else go(std::integral_constant<int, kWaveRounds>{});
        } else {
            if (extra)
                deep_chunk_kernel<DD, RBB, FF, true, kDeepBatch><<<grid, 64 * kSpWaves, dyn, st>>>(
                    v, lv, q, nr, sm, idx, p_sel, k, cs, part, nchunk, fl, sshift, dbits);
            else
                deep_chunk_kernel<DD, RBB, FF, false, kDeepBatch><<<grid, 64 * kSpWaves, 0, st>>>(
                    v, lv, q, nr, sm, idx, p_sel, k, cs, part, nchunk, fl, sshift, dbits);
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
