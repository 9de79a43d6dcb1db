// Exact top-k column selection with the cached probability mass (project page STEP 02;
// explainer section 3: top-K key columns chosen from the preceding loop's statistics,
// their total probability under the preceding full distribution cached as m).
//
// Order: fp32 score descending, ties to the lower index; +0 and -0 compare equal.
// One 1024-thread workgroup per (sequence, head).  Thread t keeps columns t, t+1024, ...
// (up to PT of them: 10, 20 or 40, the fewest that hold the row) in registers.  A histogram
// over 2048 equal-width value bins between the smallest and largest score finds the bin
// holding the k-th column (bins are a monotone function of the score, so every bin above it
// is taken whole; a bin of more than 256 columns is split again by a second histogram over its
// own [min, max]); the few columns of that bin are ranked exactly as 64-bit (key, index)
// words, which gives the threshold word (x_t, j_t).  A column is taken iff its score is above
// x_t, or equal to it at an index up to j_t: ties across the threshold are decided here too.
// One scan over per-(row, wave) counts places the selected columns in ascending index order.
//
// The fast path is kept small (its unrolled loops carry no mode branches); -inf scores
// (masked columns) stay on it as long as k scores are finite.  Everything else (k >= n,
// all scores equal, +inf or NaN, fewer than k finite scores, a crowded threshold bin,
// contexts beyond 40960 columns) goes to plain loops over memory: a 3-pass radix threshold
// on an order-preserving integer key and a row-by-row compaction.
#include <type_traits>

#include "launch.h"

namespace qkv {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelPerThread = 40;      // register-resident scores per thread at most (n <= 40960)
constexpr int kBins = 2048;
constexpr int kCandCap = 2048;         // threshold-bin columns ranked exactly
constexpr int kRefine = 256;           // threshold bins above this size get a second histogram
constexpr int kStage = 4096;           // selections staged in LDS for coalesced stores
constexpr uint32_t kNoBin = 0xFFFFFFFFu;  // no threshold bin found

__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;  // -0 == +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// inverse of order_key (the key of -0 gives +0)
__device__ __forceinline__ float key_float(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// (key, index) as one word whose unsigned order is the selection order: larger first
__device__ __forceinline__ uint64_t sort_word(float x, int j) {
    return ((uint64_t)order_key(x) << 32) | (uint64_t)(~(uint32_t)j);
}

// Bin of a score x >= lo in [0, kBins); -inf (a column past n) gets bin -1.  The difference
// x - lo of two fp32 values x >= lo rounds to a value >= +0, so every finite score lands in
// [0, kBins) however far the scores sit from zero (a bias folded into one FMA, -lo * scale,
// is itself rounded and sent scores near lo to bin -1 once |lo| / (hi - lo) reached ~8192).
// Rounding is monotone, so the bin is monotone in x, which is all the selection needs of it.
__device__ __forceinline__ int value_bin(float x, float lo, float scale) {
    return (int)__builtin_amdgcn_fmed3f((x - lo) * scale, -1.f, (float)(kBins - 1));
}

// Bin of a score x >= lo from its order key (monotone: the key is, and so are the unsigned
// difference, its rounding to fp32 and the product); -inf gets bin -1.
__device__ __forceinline__ int key_bin(float x, uint32_t klo, float scale) {
    if (x == -__builtin_huge_valf()) return -1;
    return (int)__builtin_amdgcn_fmed3f((float)(order_key(x) - klo) * scale, -1.f, (float)(kBins - 1));
}

__device__ __forceinline__ uint64_t lanes_below() {
    const int lane = threadIdx.x & 63;
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Inclusive prefix sum over the wave: row shifts by 1, 2, 4 and 8 (a lane whose source is
// outside its 16-lane row adds 0), then each row's last lane carried into the rows after it.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
    return x;
}

// Exclusive prefix sum over the workgroup (one barrier); *total = sum over all threads.
// sh (kSelWaves words) may be reused after the caller's next barrier.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t x = wave_incl_scan(v);
    if (lane == 63) sh[wave] = x;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        const uint32_t t = sh[w];
        before += (w < wave) ? t : 0u;
        all += t;
    }
    *total = all;
    return before + x - v;
}

// Threshold by radix passes over the order key (any n, scores read from memory).  Returns
// the threshold key; *need_eq = how many columns equal to it are taken (lowest indices).
__device__ __noinline__ uint32_t radix_threshold(const float* sc, int n, uint32_t need, uint32_t* hist,
                                                 uint32_t* scan_sh, uint32_t* bcast, uint32_t* need_eq) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, pmask = 0;
    for (int pass = 0; pass < 3; ++pass) {
        const int sh = pass == 0 ? 21 : pass == 1 ? 10 : 0;
        const uint32_t nb = pass == 2 ? 1024u : 2048u;
        for (uint32_t i = tid; i < nb; i += kSelThreads) hist[i] = 0;
        __syncthreads();
        for (int j = tid; j < n; j += kSelThreads) {
            const uint32_t key = order_key(sc[j]);
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & (nb - 1)], 1u);
        }
        __syncthreads();
        // bins from the top: thread t holds bins nb-1-per*t .. nb-per-per*t
        const uint32_t per = nb / kSelThreads;
        uint32_t cnt[2] = {0, 0}, bins[2] = {0, 0}, local = 0;
        for (uint32_t e = 0; e < per; ++e) {
            bins[e] = nb - 1 - (tid * per + e);
            cnt[e] = hist[bins[e]];
            local += cnt[e];
        }
        uint32_t tot;
        uint32_t above = block_excl_scan(local, scan_sh, &tot);
        for (uint32_t e = 0; e < per; ++e) {
            if (above < need && need <= above + cnt[e]) {
                bcast[0] = bins[e];
                bcast[1] = above;
            }
            above += cnt[e];
        }
        __syncthreads();
        prefix |= bcast[0] << sh;
        pmask |= (nb - 1) << sh;
        need -= bcast[1];
        __syncthreads();
    }
    *need_eq = need;
    return prefix;
}

// Compaction from memory for the slow paths, one row of 1024 columns at a time: a column
// is taken if its key exceeds T, or equals T and is among the first need_eq such columns
// (every column when take_all).  Returns this thread's share of the mass.
__device__ __noinline__ float compact_memory(const float* sc, int n, bool take_all, uint32_t T, uint32_t need_eq,
                                             float l, int32_t* id, float* ps, uint32_t* row_cnt,
                                             uint32_t* scan_sh) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t below = lanes_below();
    float psum = 0.f;
    uint32_t base = 0, eq_seen = 0;
    for (int j0 = 0; j0 < n; j0 += kSelThreads) {
        const int j = j0 + tid;
        const float x = j < n ? sc[j] : 0.f;
        const uint32_t key = order_key(x);
        const bool eq = !take_all && j < n && key == T;
        uint32_t tot;
        const uint32_t eq_rank = eq_seen + block_excl_scan(eq ? 1u : 0u, scan_sh, &tot);
        eq_seen += tot;
        const bool f = j < n && (take_all || key > T || (eq && eq_rank < need_eq));
        const uint64_t bal = __ballot(f);
        if (lane == 0) row_cnt[wave] = (uint32_t)__popcll(bal);
        __syncthreads();
        uint32_t before = 0, all = 0;
        for (int w = 0; w < kSelWaves; ++w) {
            const uint32_t t = row_cnt[w];
            before += (w < wave) ? t : 0u;
            all += t;
        }
        if (f) {
            const uint32_t pos = base + before + (uint32_t)__popcll(bal & below);
            const float p = __expf(x - l);
            id[pos] = j;
            ps[pos] = p;
            psum += p;
        }
        base += all;
        __syncthreads();
    }
    return psum;
}

template <int PT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ scores, int ld,
                                                             const float* __restrict__ lse, int n, int k,
                                                             int32_t* __restrict__ idx, float* __restrict__ p_sel,
                                                             float* __restrict__ mass) {
    const int bh = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* sc = scores + (size_t)bh * ld;
    int32_t* id = idx + (size_t)bh * k;
    float* ps = p_sel + (size_t)bh * k;
    __shared__ uint32_t hist[kBins];
    __shared__ uint32_t scan_sh[kSelWaves];
    __shared__ float fmin_sh[kSelWaves], fmax_sh[kSelWaves];
    __shared__ uint32_t bcast[6];
    __shared__ uint64_t cand[kCandCap];
    __shared__ uint64_t thr_sh;
    __shared__ uint32_t thr_found;
    __shared__ uint32_t row_off[PT * kSelWaves];  // [row][wave]: counts, then offsets
    __shared__ int32_t st_idx[kStage];
    __shared__ float st_p[kStage];
    __shared__ float msum[kSelWaves];

    if (k <= 0) {
        if (tid == 0) mass[bh] = 0.f;
        return;
    }
    const float l = lse[bh];
    const int E = (n + kSelThreads - 1) / kSelThreads;  // rows of 1024 columns
    float psum = 0.f;
    bool done = false;  // uniform

    if (k < n && E <= PT) {
        // ---- fast path: column j = e * 1024 + tid in v[e]; the slots past n first hold
        //      copies of column n - 1 (no change to the extremes), then -inf, which no bin
        //      counts and no threshold takes ----
        const float kNegInf = -__builtin_huge_valf();
        float v[PT];
#pragma unroll
        for (int e = 0; e < PT; ++e) v[e] = sc[min(e * kSelThreads + tid, n - 1)];
        for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0;
        for (int i = tid; i < kCandCap; i += kSelThreads) cand[i] = 0;  // padding ranks below everything
        // -inf scores (masked columns) take no bin and are never taken here; the k-th score
        // must be finite, which the histogram below checks (fewer than k finite scores: the
        // memory paths decide)
        float mn = __builtin_huge_valf(), mx = kNegInf;
        float vsum = 0.f;  // NaN iff some score is NaN (or +inf and -inf meet: not finite either)
#pragma unroll
        for (int e = 0; e < PT; ++e) {
            mn = fminf(mn, v[e] == kNegInf ? __builtin_huge_valf() : v[e]);
            mx = fmaxf(mx, v[e]);
            vsum += v[e];
        }
        if (__ballot(__builtin_isnan(vsum))) mx = __builtin_huge_valf();  // the memory paths decide
        mn = wave_min(mn);
        mx = wave_max(mx);
        if (lane == 0) {
            fmin_sh[wave] = mn;
            fmax_sh[wave] = mx;
        }
        if (tid == 0) {
            bcast[0] = kNoBin;  // stays so only if the histogram misses the k-th column
            bcast[2] = 0;       // candidate count
            thr_found = 0u;     // 1: the threshold column found, its score unique; 2: found, shared
        }
#pragma unroll
        for (int e = 0; e < PT; ++e) v[e] = e * kSelThreads + tid < n ? v[e] : kNegInf;
        __syncthreads();
        float lo = fmin_sh[0], hi = fmax_sh[0];
#pragma unroll
        for (int w = 1; w < kSelWaves; ++w) {
            lo = fminf(lo, fmin_sh[w]);
            hi = fmaxf(hi, fmax_sh[w]);
        }
        const float range = hi - lo;
        // First-level bins: of the score over [lo, hi], or (kmode), for rows whose finite scores
        // are all >= 0 and span more than a factor of 64, of its order key over [key(lo),
        // key(hi)], which is close to log2 of the score: heavy-tailed rows (token-change ratios)
        // then spread over the bins instead of piling into the lowest few.  The mode is uniform,
        // so each loop that bins comes in two forms rather than testing it per column.
        const bool kmode = lo >= 0.f && hi > 64.f * lo;
        const uint32_t klo = order_key(lo);
        const float scale = kmode ? (float)kBins / (float)(order_key(hi) - klo) : (float)kBins / range;
        if (range > 0.f && __builtin_isfinite(range) && __builtin_isfinite(scale)) {
            if (kmode) {
#pragma unroll
                for (int e = 0; e < PT; ++e)
                    if (v[e] > kNegInf) atomicAdd(&hist[key_bin(v[e], klo, scale)], 1u);
            } else {
#pragma unroll
                for (int e = 0; e < PT; ++e)
                    if (v[e] > kNegInf) atomicAdd(&hist[value_bin(v[e], lo, scale)], 1u);
            }
            __syncthreads();
            // bin of the k-th largest, counting from the top bin (thread t: bins 2047-2t, 2046-2t)
            const int b0 = kBins - 1 - 2 * tid, b1 = b0 - 1;
            const uint32_t c0 = hist[b0], c1 = hist[b1];
            uint32_t tot;
            const uint32_t above = block_excl_scan(c0 + c1, scan_sh, &tot);
            if (above < (uint32_t)k && (uint32_t)k <= above + c0) {
                bcast[0] = (uint32_t)b0;
                bcast[1] = above;
            } else if (above + c0 < (uint32_t)k && (uint32_t)k <= above + c0 + c1) {
                bcast[0] = (uint32_t)b1;
                bcast[1] = above + c0;
            }
            __syncthreads();
            const int bstar = (int)bcast[0];
            uint32_t need_in = (uint32_t)k - bcast[1];  // columns taken inside the threshold bin
            // every column of the fast path is finite and binned, so the k-th is always found;
            // should it not be, the memory paths decide
            bool ok = bcast[0] != kNoBin;
            const uint32_t cb = ok ? hist[bstar] : 0u;
            // A crowded threshold bin (heavy-tailed scores put most columns in the lowest bins
            // of [min, max]) is split once more, by a second histogram over the bin's own
            // [min, max]; the bin of the k-th column there holds the candidates.  Without it
            // the exact ranking costs (bin size)^2 comparisons.
            int sb = -1;
            float lo2 = 0.f, scale2 = 0.f;
            if (ok && cb > (uint32_t)kRefine) {
                float mn2 = __builtin_huge_valf(), mx2 = kNegInf;
                if (kmode) {
#pragma unroll
                    for (int e = 0; e < PT; ++e) {
                        if (key_bin(v[e], klo, scale) == bstar) {
                            mn2 = fminf(mn2, v[e]);
                            mx2 = fmaxf(mx2, v[e]);
                        }
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < PT; ++e) {
                        if (value_bin(v[e], lo, scale) == bstar) {
                            mn2 = fminf(mn2, v[e]);
                            mx2 = fmaxf(mx2, v[e]);
                        }
                    }
                }
                mn2 = wave_min(mn2);
                mx2 = wave_max(mx2);
                __syncthreads();  // every thread has read the first level's extremes and counts
                if (lane == 0) {
                    fmin_sh[wave] = mn2;
                    fmax_sh[wave] = mx2;
                }
                for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0;
                if (tid == 0) bcast[3] = kNoBin;
                __syncthreads();
                lo2 = fmin_sh[0];
                float hi2 = fmax_sh[0];
#pragma unroll
                for (int w = 1; w < kSelWaves; ++w) {
                    lo2 = fminf(lo2, fmin_sh[w]);
                    hi2 = fmaxf(hi2, fmax_sh[w]);
                }
                const float range2 = hi2 - lo2;
                scale2 = (float)kBins / range2;
                if (range2 > 0.f && __builtin_isfinite(scale2)) {
                    if (kmode) {
#pragma unroll
                        for (int e = 0; e < PT; ++e)
                            if (key_bin(v[e], klo, scale) == bstar) atomicAdd(&hist[value_bin(v[e], lo2, scale2)], 1u);
                    } else {
#pragma unroll
                        for (int e = 0; e < PT; ++e)
                            if (value_bin(v[e], lo, scale) == bstar) atomicAdd(&hist[value_bin(v[e], lo2, scale2)], 1u);
                    }
                    __syncthreads();
                    const int s0 = kBins - 1 - 2 * tid, s1 = s0 - 1;
                    const uint32_t d0 = hist[s0], d1 = hist[s1];
                    uint32_t tot2;
                    const uint32_t above2 = block_excl_scan(d0 + d1, scan_sh, &tot2);
                    if (above2 < need_in && need_in <= above2 + d0) {
                        bcast[3] = (uint32_t)s0;
                        bcast[4] = above2;
                    } else if (above2 + d0 < need_in && need_in <= above2 + d0 + d1) {
                        bcast[3] = (uint32_t)s1;
                        bcast[4] = above2 + d0;
                    }
                    __syncthreads();
                    ok = bcast[3] != kNoBin;
                    if (ok) {
                        sb = (int)bcast[3];
                        need_in -= bcast[4];
                        ok = hist[sb] <= (uint32_t)kCandCap;
                    }
                } else {
                    ok = cb <= (uint32_t)kCandCap;  // one score throughout the bin: all tie
                }
            } else {
                ok = ok && cb <= (uint32_t)kCandCap;
            }
            if (ok) {
                // the threshold (sub)bin's columns as (key, index) sort words
                // (never for -inf: bin -1)
                if (kmode) {
#pragma unroll
                    for (int e = 0; e < PT; ++e) {
                        if (key_bin(v[e], klo, scale) == bstar && (sb < 0 || value_bin(v[e], lo2, scale2) == sb)) {
                            const uint32_t slot = atomicAdd(&bcast[2], 1u);
                            cand[slot] = sort_word(v[e], e * kSelThreads + tid);
                        }
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < PT; ++e) {
                        if (value_bin(v[e], lo, scale) == bstar && (sb < 0 || value_bin(v[e], lo2, scale2) == sb)) {
                            const uint32_t slot = atomicAdd(&bcast[2], 1u);
                            cand[slot] = sort_word(v[e], e * kSelThreads + tid);
                        }
                    }
                }
                __syncthreads();
                // the candidate of rank need_in - 1 (bins are monotone in the score, so every
                // column of a higher bin precedes it and every column of a lower bin follows)
                const uint32_t c = bcast[2];
                const uint32_t cpad = (c + 7u) & ~7u;
                for (uint32_t t = tid; t < c; t += kSelThreads) {
                    const uint64_t rt = cand[t];
                    const uint32_t kt = (uint32_t)(rt >> 32);
                    uint32_t rank = 0, same = 0;
                    for (uint32_t u = 0; u < cpad; u += 8) {
#pragma unroll
                        for (int w = 0; w < 8; ++w) {
                            const uint64_t cu = cand[u + w];
                            rank += cu > rt ? 1u : 0u;
                            same += (uint32_t)(cu >> 32) == kt ? 1u : 0u;
                        }
                    }
                    if (rank == need_in - 1) {
                        thr_sh = rt;
                        thr_found = same == 1u ? 1u : 2u;
                    }
                }
                __syncthreads();
                // the threshold word (tx, jt): a column is taken iff its word is at least that,
                // i.e. its score is above tx, or equal to it (+0 and -0 alike) at an index up
                // to jt; when no other column has the score tx (TIE false) that is just a
                // score of at least tx (columns past n hold -inf).  Per-(row, wave) counts
                // (lane e of cnts: row e), one scan, then each column's position.
                auto compact = [&](auto tiec) {
                    constexpr bool TIE = decltype(tiec)::value;
                    const float tx = key_float((uint32_t)(thr_sh >> 32));
                    const int jt = (int)~(uint32_t)thr_sh;
                    uint32_t cnts = 0;
#pragma unroll
                    for (int e = 0; e < PT; ++e) {
                        const bool f = TIE ? v[e] > tx || (v[e] == tx && e * kSelThreads + tid <= jt) : v[e] >= tx;
                        const uint32_t cnt = (uint32_t)__popcll(__ballot(f));
                        cnts = lane == e ? cnt : cnts;
                    }
                    if (lane < E) row_off[lane * kSelWaves + wave] = cnts;
                    __syncthreads();
                    const int nrw = E * kSelWaves;
                    uint32_t tot2;
                    const uint32_t x = tid < nrw ? row_off[tid] : 0u;
                    const uint32_t ex = block_excl_scan(x, scan_sh, &tot2);
                    __syncthreads();  // every count has been read
                    if (tid < nrw) row_off[tid] = ex;
                    __syncthreads();
                    const uint32_t offs = lane < E ? row_off[lane * kSelWaves + wave] : 0u;
                    const bool stage = k <= kStage;
                    // the comparisons are made again below rather than kept across the scan
                    // (40 lane masks would not fit in scalar registers)
                    float txp = tx;
                    asm volatile("" : "+v"(txp));
#pragma unroll
                    for (int e = 0; e < PT; ++e) {
                        const bool f = TIE ? v[e] > txp || (v[e] == txp && e * kSelThreads + tid <= jt) : v[e] >= txp;
                        const uint64_t bal = __ballot(f);
                        const uint32_t base = __builtin_amdgcn_readlane(offs, e);
                        if (f) {
                            const uint32_t pos =
                                base + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
                            const int j = e * kSelThreads + tid;
                            if (stage) {  // the score; its probability is formed once, below
                                st_idx[pos] = j;
                                st_p[pos] = v[e];
                            } else {
                                const float p = __expf(v[e] - l);
                                psum += p;
                                id[pos] = j;
                                ps[pos] = p;
                            }
                        }
                    }
                    if (stage) {
                        __syncthreads();
                        for (int i = tid; i < k; i += kSelThreads) {
                            const float p = __expf(st_p[i] - l);
                            psum += p;
                            id[i] = st_idx[i];
                            ps[i] = p;
                        }
                    }
                    done = true;
                };
                if (thr_found == 1u) compact(std::false_type{});
                else if (thr_found == 2u) compact(std::true_type{});
            }
        }
        __syncthreads();
    }
    if (!done) {
        // ---- slow paths, from memory ----
        uint32_t T = 0, need_eq = 0;
        const bool take_all = k >= n;
        if (!take_all) T = radix_threshold(sc, n, (uint32_t)k, hist, scan_sh, bcast, &need_eq);
        psum = compact_memory(sc, n, take_all, T, need_eq, l, id, ps, row_off, scan_sh);
    }
    // mass: fixed-order reduction (waves in order)
    psum = wave_sum(psum);
    if (lane == 0) msum[wave] = psum;
    __syncthreads();
    if (tid == 0) {
        float m = 0.f;
        for (int w = 0; w < kSelWaves; ++w) m += msum[w];
        mass[bh] = m;
    }
}

size_t select_ws_bytes(int, int, int) { return 0; }

int launch_select(const float* scores, int ld, const float* lse, int B, int H, int n, int k, int32_t* idx,
                  float* p_sel, float* mass, void*, hipStream_t st) {
    // the fewest register-resident scores per thread that hold the row (longer rows take the
    // memory paths from the largest)
    const int E = (n + kSelThreads - 1) / kSelThreads;
    if (E <= 10)
        select_kernel<10><<<B * H, kSelThreads, 0, st>>>(scores, ld, lse, n, k, idx, p_sel, mass);
    else if (E <= 20)
        select_kernel<20><<<B * H, kSelThreads, 0, st>>>(scores, ld, lse, n, k, idx, p_sel, mass);
    else
        select_kernel<kSelPerThread><<<B * H, kSelThreads, 0, st>>>(scores, ld, lse, n, k, idx, p_sel, mass);
    return hipGetLastError() == hipSuccess ? QKV_OK : QKV_ELAUNCH;
}

}  // namespace qkv
