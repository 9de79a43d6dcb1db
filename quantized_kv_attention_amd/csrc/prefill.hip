// Prefill-side sparse loop over compact buffers (project page, The Method, after STEP 03:
// the selected tokens and keys are gathered into compact, compute-friendly buffers so that
// the work stays regular GEMMs; STEP 02 and explainer section 3: the rank-K correction of
// the preceding loop's output that keeps the cached mass).
//
// For each active query row i (position qpos[i]) and the selected columns j at or before
// it (positions cpos[j], ascending):
//   p_ij = exp(sm q0_i . K0_j - lse0_i),  m_i = sum_j p_ij,
//   alpha_ij = softmax_j(sm q_i . K_j),   o_i = o0_i + sum_j (m_i alpha_ij V_j - p_ij V0_j).
//
// kv_gather_rows builds the compact buffers: query rows and key rows as they are, value
// rows transposed ([channel][column]), so that both products read their operands with the
// contraction index contiguous.  The attention kernel runs on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16: lane l holds A[l % 16][8 (l / 16) + e], B[8 (l / 16) + e][l % 16],
// and D[4 (l / 16) + r][l % 16]).  It forms S^T = K Q^T, so that a lane's accumulator values
// belong to query row l % 16 and to columns 4 (l / 16) + r of each 16-column block, and
// O^T = V^T P^T with the same k order on both operands: the transposed probabilities are
// then already in the B layout, and the softmax statistics, the rescaling and the output
// rows all live on the lanes of their row, with no LDS round trip.
#include "launch.h"

namespace qkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 w) { return __builtin_bit_cast(bf16x8_t, w); }

__device__ __forceinline__ uint4 ld_u4(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ld_u2(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats to bf16 (round to nearest even), a in the low half: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

constexpr float kLog2e = 1.4426950408889634f;

// Max and sum over the four lanes of a wave that hold the same row (lanes l, l ^ 16, l ^ 32, l ^ 48).
__device__ __forceinline__ float row_max4(float v) {
    float2 p = pair_xor16(v);
    v = fmaxf(p.x, p.y);
    p = pair_xor32(v);
    return fmaxf(p.x, p.y);
}
__device__ __forceinline__ float row_sum4(float v) { return add_xor32(add_xor16(v)); }

constexpr int kPfWaves = 8;                 // waves per workgroup
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfRows = 16 * kPfWaves;      // query rows per workgroup (16 per wave): every
                                            // step's key and value tiles serve all of them
constexpr int kPfCols = 32;                 // columns per step (two 16-column blocks)

// LDS tiles of one step, shared by the workgroup's waves: key rows of both loops
// ([column][channel], rows padded by 16 bytes so that the 16 lanes reading 16 columns at one
// channel offset fall into distinct banks) and transposed values of both loops ([channel]
// [column], rows of 32 columns padded to 72 bytes for the same reason).
template <int D>
struct PfTile {
    static constexpr int kKRow = D * 2 + 16;
    static constexpr int kVRow = kPfCols * 2 + 8;
    static constexpr int kK = kPfCols * kKRow;       // one key tile
    static constexpr int kV = D * kVRow;             // one value tile
    static constexpr int kPos = 2 * kK + 2 * kV;     // the step's column positions (int32)
    static constexpr int kBytes = kPos + kPfCols * 4;  // k1 | k0 | v1t | v0t | positions
    static constexpr int kKChunks = kPfCols * D / 8;  // 16-byte pieces of a key tile
    static constexpr int kVChunks = D * 4;            // 16-byte pieces of a value tile (64 bytes per channel)
    static constexpr int kPer = (kKChunks + kPfThreads - 1) / kPfThreads;  // pieces of each tile per thread
};

template <int D>
__global__ __launch_bounds__(kPfThreads, 1) void prefill_sparse_kernel(
    const uint16_t* __restrict__ q1, const uint16_t* __restrict__ q0, const int32_t* __restrict__ qpos, int n_q,
    const float* __restrict__ lse0, const float* __restrict__ o0, const uint16_t* __restrict__ k1,
    const uint16_t* __restrict__ k0, const uint16_t* __restrict__ v1t, const uint16_t* __restrict__ v0t, int ldt,
    const int32_t* __restrict__ cpos, int n_c, int H, float sm, float* __restrict__ o32, uint16_t* __restrict__ o16,
    float* __restrict__ mass) {
    using T = PfTile<D>;
    static_assert(T::kKChunks == T::kVChunks, "one staging pattern for key and value tiles");
    constexpr int KS = D / 32;   // k-steps of the score products
    constexpr int CB = D / 16;   // 16-channel blocks of the output
    constexpr int PER = T::kPer;
    __shared__ __align__(16) uint8_t lds[2][T::kBytes];
    // heads vary fastest and row blocks run last to first: the blocks that see the most
    // columns start first, and the short ones fill the tail
    const int h = blockIdx.x, b = blockIdx.z;
    const int rb = gridDim.y - 1 - blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, rl = lane & 15;
    const size_t bh = (size_t)b * H + h;
    const int row = rb * kPfRows + wave * 16 + rl;
    const bool rvalid = row < n_q;
    const int rowc = rvalid ? row : n_q - 1;
    const int my_pos = rvalid ? qpos[(size_t)b * n_q + row] : -1;
    // exponentials as 2^x: the scale and the row's lse carry the factor log2(e)
    const float sm2 = sm * kLog2e;
    const float my_lse2 = lse0[bh * n_q + rowc] * kLog2e;

    // B operands of S^T = K Q^T: this lane's row, channels 32 ks + 8 g .. + 7
    bf16x8_t bq1[KS], bq0[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        bq1[ks] = as_bf16x8(ld_u4(q1 + (bh * n_q + rowc) * D + 32 * ks + 8 * g));
        bq0[ks] = as_bf16x8(ld_u4(q0 + (bh * n_q + rowc) * D + 32 * ks + 8 * g));
    }
    // the columns some row of this workgroup sees: cpos ascending, so a prefix
    const int last = qpos[(size_t)b * n_q + min(n_q, (rb + 1) * kPfRows) - 1];
    const int first_pos = qpos[(size_t)b * n_q + rb * kPfRows];   // the workgroup's first row
    const int32_t* cp = cpos + bh * n_c;
    int lo = 0, hi = n_c;  // first column with cpos > last
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (cp[mid] <= last) lo = mid + 1; else hi = mid;
    }
    const int ntiles = (lo + kPfCols - 1) / kPfCols;

    // staging of a step's tiles: PER 16-byte pieces of each of the four tiles per thread, and
    // one column position per thread of the first kPfCols (so that the visibility test reads
    // LDS: waiting on a global load would also wait on the next step's loads issued before it)
    uint4 st[4][PER];
    int stpos = 0;
    auto gload = [&](int c0) {
        if (tid < kPfCols) stpos = c0 + tid < n_c ? cp[c0 + tid] : 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = tid + kPfThreads * i;
            if (e < T::kKChunks) {
                const int col = c0 + e / (D / 8), ch = (e % (D / 8)) * 8;
                const int colc = col < n_c ? col : n_c - 1;
                st[0][i] = ld_u4(k1 + (bh * n_c + colc) * D + ch);
                st[1][i] = ld_u4(k0 + (bh * n_c + colc) * D + ch);
                const int vc = e >> 2, part = (e & 3) * 8;  // channel, 8 columns of it
                st[2][i] = ld_u4(v1t + (bh * D + vc) * (size_t)ldt + c0 + part);
                st[3][i] = ld_u4(v0t + (bh * D + vc) * (size_t)ldt + c0 + part);
            }
        }
    };
    auto sstore = [&](int buf) {
        uint8_t* base = lds[buf];
        if (tid < kPfCols) reinterpret_cast<int*>(base + T::kPos)[tid] = stpos;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = tid + kPfThreads * i;
            if (e < T::kKChunks) {
                const int kofs = (e / (D / 8)) * T::kKRow + (e % (D / 8)) * 16;
                *reinterpret_cast<uint4*>(base + kofs) = st[0][i];
                *reinterpret_cast<uint4*>(base + T::kK + kofs) = st[1][i];
                const int vofs = (e >> 2) * T::kVRow + (e & 3) * 16;
                // a 72-byte row keeps 8-byte alignment only: two 8-byte stores
                *reinterpret_cast<uint2*>(base + 2 * T::kK + vofs) = make_uint2(st[2][i].x, st[2][i].y);
                *reinterpret_cast<uint2*>(base + 2 * T::kK + vofs + 8) = make_uint2(st[2][i].z, st[2][i].w);
                *reinterpret_cast<uint2*>(base + 2 * T::kK + T::kV + vofs) = make_uint2(st[3][i].x, st[3][i].y);
                *reinterpret_cast<uint2*>(base + 2 * T::kK + T::kV + vofs + 8) = make_uint2(st[3][i].z, st[3][i].w);
            }
        }
    };

    f32x4_t U[CB], W[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        U[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        W[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    float M = -__builtin_huge_valf(), Lp = 0.f, mp = 0.f;  // row max; lane-partial sums

    if (ntiles > 0) {
        gload(0);
        sstore(0);
    }
    __syncthreads();
    // every load issued so far (the query operands above all) has landed: without this wait
    // the compiler's counter tracking, merging the paths into the loop, would make the first
    // use of those operands in each step wait for the next step's tiles as well
    __builtin_amdgcn_s_waitcnt(0);
    for (int t = 0; t < ntiles; ++t) {
        const int c0 = t * kPfCols;
        const uint8_t* base = lds[t & 1];
        if (t + 1 < ntiles) gload(c0 + kPfCols);   // the next step's tiles, in flight meanwhile
        f32x4_t s1[2], s0[2];
        int cposv[2][4];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            // A operands: key rows of columns c0 + 16 blk + rl
            const uint8_t* kr = base + (16 * blk + rl) * T::kKRow + 16 * g;
            s1[blk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            s0[blk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8_t a1 = as_bf16x8(*reinterpret_cast<const uint4*>(kr + 64 * ks));
                const bf16x8_t a0 = as_bf16x8(*reinterpret_cast<const uint4*>(kr + T::kK + 64 * ks));
                s1[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bq1[ks], s1[blk], 0, 0, 0);
                s0[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bq0[ks], s0[blk], 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)   // this lane's column of value r (past n_c: never visible)
                cposv[blk][r] = reinterpret_cast<const int*>(base + T::kPos)[16 * blk + 4 * g + r];
        }
        // probabilities of the preceding loop, and the new logits' running max per row (the
        // logits in log2 units).  A step whose last column precedes the workgroup's first row
        // is visible to every row: no masks (all but a workgroup's last few steps).
        const bool full = reinterpret_cast<const int*>(base + T::kPos)[kPfCols - 1] <= first_pos;
        float e1[8], p0[8];
        float tmax = -__builtin_huge_valf();
        if (full) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    e1[4 * blk + r] = sm2 * s1[blk][r];
                    p0[4 * blk + r] = __builtin_amdgcn_exp2f(fmaf(sm2, s0[blk][r], -my_lse2));
                    tmax = fmaxf(tmax, e1[4 * blk + r]);
                }
            }
        } else {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool vis = cposv[blk][r] <= my_pos;
                    e1[4 * blk + r] = vis ? sm2 * s1[blk][r] : -__builtin_huge_valf();
                    p0[4 * blk + r] = vis ? __builtin_amdgcn_exp2f(fmaf(sm2, s0[blk][r], -my_lse2)) : 0.f;
                    tmax = fmaxf(tmax, e1[4 * blk + r]);
                }
            }
        }
        tmax = row_max4(tmax);
        const float Mn = fmaxf(M, tmax);
        const float scale = (M == -__builtin_huge_valf()) ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
        M = Mn;
        float x[8];
        if (full) {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = __builtin_amdgcn_exp2f(e1[e] - Mn);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                x[e] = e1[e] == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(e1[e] - Mn);
        }
        uint32_t w1[4], w0[4];
        float lsum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            w1[e / 2] = pack_bf16(x[e], x[e + 1]);
            w0[e / 2] = pack_bf16(p0[e], p0[e + 1]);
            // the normalisation sums the weights the product uses (bf16)
            lsum += bf16_to_f32(w1[e / 2] & 0xFFFFu) + bf16_to_f32(w1[e / 2] >> 16);
            mp += p0[e] + p0[e + 1];
        }
        Lp = Lp * scale + lsum;
        // B operands of O^T = V^T P^T: element e is column 4 g + e (e < 4) or 16 + 4 g + (e - 4)
        const bf16x8_t pb1 = as_bf16x8(make_uint4(w1[0], w1[1], w1[2], w1[3]));
        const bf16x8_t pb0 = as_bf16x8(make_uint4(w0[0], w0[1], w0[2], w0[3]));
        // the running sums need rescaling only where some row's max moved
        if (__ballot(scale != 1.f)) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) U[cb] *= scale;
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            // A operands: channel 16 cb + rl of the transposed values, the same eight columns
            const uint8_t* vr = base + 2 * T::kK + (16 * cb + rl) * T::kVRow + 8 * g;
            const uint2 a1lo = *reinterpret_cast<const uint2*>(vr), a1hi = *reinterpret_cast<const uint2*>(vr + 32);
            const uint2 a0lo = *reinterpret_cast<const uint2*>(vr + T::kV);
            const uint2 a0hi = *reinterpret_cast<const uint2*>(vr + T::kV + 32);
            U[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(make_uint4(a1lo.x, a1lo.y, a1hi.x, a1hi.y)), pb1,
                                                            U[cb], 0, 0, 0);
            W[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(make_uint4(a0lo.x, a0lo.y, a0hi.x, a0hi.y)), pb0,
                                                            W[cb], 0, 0, 0);
        }
        if (t + 1 < ntiles) sstore((t + 1) & 1);   // the other buffer: every wave left it a step ago
        __syncthreads();
    }
    const float L = row_sum4(Lp);
    const float m = row_sum4(mp);
    if (!rvalid) return;
    // lane holds O^T[channel 16 cb + 4 g + r][row]: four consecutive channels per block
    const float* o0r = o0 + (bh * n_q + row) * D;
    float* o32r = o32 + (bh * n_q + row) * D;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int c = 16 * cb + 4 * g;
        const float4 prev = *reinterpret_cast<const float4*>(o0r + c);
        float4 out = prev;
        if (L > 0.f) {
            const float f = m / L;
            out.x = prev.x + f * U[cb][0] - W[cb][0];
            out.y = prev.y + f * U[cb][1] - W[cb][1];
            out.z = prev.z + f * U[cb][2] - W[cb][2];
            out.w = prev.w + f * U[cb][3] - W[cb][3];
        }
        *reinterpret_cast<float4*>(o32r + c) = out;
        if (o16) {
            uint16_t* o16r = o16 + (bh * n_q + row) * D + c;
            *reinterpret_cast<uint2*>(o16r) = make_uint2(pack_bf16(out.x, out.y), pack_bf16(out.z, out.w));
        }
    }
    if (mass && g == 0) mass[bh * n_q + row] = m;
}

// Compact rows: dst[b][h][i] = src[b][h][idx[b][(h)][i]] (zeros for an index outside
// [0, ld_src)); transposed: dst[b][h][c][i], columns past n up to ldt zero-filled.
// One thread per 8 channels of a row.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ src, int H, int ld_src, int D,
                                                          const int32_t* __restrict__ idx, int n, int per_head,
                                                          int transpose, int ldt, uint16_t* __restrict__ dst) {
    const int h = blockIdx.y, b = blockIdx.z;
    const int cpr = D / 8;
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    const int rows = transpose ? ldt : n;
    if (e >= (long)rows * cpr) return;
    const int i = (int)(e / cpr), c = (int)(e % cpr) * 8;
    const size_t bh = (size_t)b * H + h;
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (i < n) {
        const int j = idx[(per_head ? bh : (size_t)b) * n + i];
        if (j >= 0 && j < ld_src) w = *reinterpret_cast<const uint4*>(src + (bh * ld_src + j) * D + c);
    }
    if (!transpose) {
        *reinterpret_cast<uint4*>(dst + (bh * n + i) * D + c) = w;
    } else {
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int t = 0; t < 8; ++t)
            dst[(bh * D + c + t) * (size_t)ldt + i] = (uint16_t)((ws[t >> 1] >> (16 * (t & 1))) & 0xFFFFu);
    }
}

int launch_gather_rows(const uint16_t* src, int B, int H, int ld_src, int D, const int32_t* idx, int n, int per_head,
                       int transpose, uint16_t* dst, hipStream_t st) {
    const int ldt = transpose ? ((n + 31) / 32) * 32 : n;
    const long work = (long)(transpose ? ldt : n) * (D / 8);
    dim3 grid((unsigned)((work + 255) / 256), H, B);
    gather_rows_kernel<<<grid, 256, 0, st>>>(src, H, ld_src, D, idx, n, per_head, transpose, ldt, dst);
    return hipGetLastError() == hipSuccess ? QKV_OK : QKV_ELAUNCH;
}

int launch_prefill_sparse(int B, int H, int D, const uint16_t* q1, const uint16_t* q0, const int32_t* qpos, int n_q,
                          const float* lse0, const float* o0, const uint16_t* k1, const uint16_t* k0,
                          const uint16_t* v1t, const uint16_t* v0t, const int32_t* cpos, int n_c, float sm,
                          float* o32, uint16_t* o16, float* mass, hipStream_t st) {
    const int ldt = ((n_c + 31) / 32) * 32;
    dim3 grid(H, (n_q + kPfRows - 1) / kPfRows, B);
    if (D == 128)
        prefill_sparse_kernel<128><<<grid, kPfThreads, 0, st>>>(q1, q0, qpos, n_q, lse0, o0, k1, k0, v1t, v0t, ldt, cpos,
                                                         n_c, H, sm, o32, o16, mass);
    else
        prefill_sparse_kernel<64><<<grid, kPfThreads, 0, st>>>(q1, q0, qpos, n_q, lse0, o0, k1, k0, v1t, v0t, ldt, cpos,
                                                        n_c, H, sm, o32, o16, mass);
    return hipGetLastError() == hipSuccess ? QKV_OK : QKV_ELAUNCH;
}

}  // namespace qkv
