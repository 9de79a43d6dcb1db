// Exact top-k column selection with the cached probability mass (project page STEP 02;
// explainer section 3: top-K key columns chosen from the preceding loop's statistics,
// their total probability under the preceding full distribution cached as m).
//
// Order: fp32 score descending, ties to the lower index; +0 and -0 compare equal.
// One 1024-thread workgroup per (sequence, head).  Thread t keeps columns t, t+1024, ...
// (up to 40 of them) in registers.  A histogram over 2048 equal-width value bins between the
// smallest and largest score (bins are a monotone function of the score, so every bin
// above the threshold bin is taken whole) finds the bin holding the k-th column; the few
// columns of that bin are ranked exactly to give the threshold (score, index); a last
// pass compacts the selection in ascending index order.  Degenerate inputs (equal
// scores, a crowded threshold bin, contexts beyond 40960 columns) take a 3-pass radix path
// over an order-preserving integer key.
#include "launch.h"

namespace qkv {

constexpr int kSelThreads = 1024;
constexpr int kSelPerThread = 40;      // register-resident scores per thread (n <= 40960)
constexpr int kBins = 2048;
constexpr int kCandCap = 2048;         // threshold-bin columns ranked exactly

__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;  // -0 == +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// exclusive prefix sum over the 1024 threads; returns the block total in *total
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(x, o, 64);
        if (lane >= o) x += t;
    }
    __syncthreads();
    if (lane == 63) sh[wave] = x;
    __syncthreads();
    if (tid == 0) {
        uint32_t run = 0;
        for (int w = 0; w < kSelThreads / 64; ++w) {
            const uint32_t t = sh[w];
            sh[w] = run;
            run += t;
        }
        sh[kSelThreads / 64] = run;
    }
    __syncthreads();
    *total = sh[kSelThreads / 64];
    return sh[wave] + x - v;
}

__device__ __forceinline__ float block_min(float v, float* sh) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fminf(v, __shfl_xor(v, m, 64));
    __syncthreads();
    if (lane == 0) sh[wave] = v;
    __syncthreads();
    float r = sh[0];
    for (int w = 1; w < kSelThreads / 64; ++w) r = fminf(r, sh[w]);
    return r;
}
__device__ __forceinline__ float block_max(float v, float* sh) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    __syncthreads();
    if (lane == 0) sh[wave] = v;
    __syncthreads();
    float r = sh[0];
    for (int w = 1; w < kSelThreads / 64; ++w) r = fmaxf(r, sh[w]);
    return r;
}

// Threshold by radix passes over the order key (any n, reads scores from memory).
// Returns the threshold key; *need_eq = number of columns equal to it that are taken.
__device__ uint32_t radix_threshold(const float* sc, int n, uint32_t need, uint32_t* hist, uint32_t* scan_sh,
                                    uint32_t* sel_bin, uint32_t* sel_above, uint32_t* need_eq) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, pmask = 0;
    const int shifts[3] = {21, 10, 0};
    const int nbits[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
        const int sh = shifts[pass];
        const uint32_t nb = 1u << nbits[pass];
        for (uint32_t i = tid; i < nb; i += kSelThreads) hist[i] = 0;
        __syncthreads();
        for (int j = tid; j < n; j += kSelThreads) {
            const uint32_t key = order_key(sc[j]);
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & (nb - 1)], 1u);
        }
        __syncthreads();
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
                *sel_bin = bins[e];
                *sel_above = above;
            }
            above += cnt[e];
        }
        __syncthreads();
        prefix |= *sel_bin << sh;
        pmask |= (nb - 1) << sh;
        need -= *sel_above;
        __syncthreads();
    }
    *need_eq = need;
    return prefix;
}

__device__ __forceinline__ uint32_t value_bin(float x, float lo, float scale) {
    float f = (x - lo) * scale;
    f = fminf(fmaxf(f, 0.f), (float)(kBins - 1));
    return (uint32_t)(int)f;
}

// Writes the selected columns in ascending index order, 64 rows of 1024 columns per batch:
// per-wave ballots rank each lane inside its 64 columns, a scan over (row, wave) gives the
// offsets.  In mode 2 a first scan ranks the columns equal to the threshold key.  Rows are
// read again from memory (coalesced; the scores are cache resident).
__device__ __forceinline__ float compact_rows(const float* sc, int n, int E,
                                              int mode, float lo, float scale, uint32_t bstar, uint32_t tk,
                                              int32_t ti, uint32_t T, uint32_t need_eq, float l, int32_t* id,
                                              float* ps, uint32_t* row_off, uint32_t* scan_sh) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    constexpr int kRows = 64;
    float psum = 0.f;
    uint32_t base = 0, eq_base = 0;
    for (int r0 = 0; r0 < E; r0 += 64) {
        const int nr = min(64, E - r0);
        uint64_t eqbits = 0;  // bit rr: this thread's column of row r0+rr equals T and is taken
        if (mode == 2) {
#pragma unroll
            for (int rr = 0; rr < kRows; ++rr) {
                if (rr >= nr) break;
                const int j = (r0 + rr) * kSelThreads + tid;
                const bool f = j < n && order_key(sc[j]) == T;
                const uint64_t bal = __ballot(f);
                if (lane == 0) row_off[rr * 16 + wave] = (uint32_t)__popcll(bal);
            }
            __syncthreads();
            uint32_t tot;
            const uint32_t x = tid < nr * 16 ? row_off[tid] : 0u;
            const uint32_t ex = block_excl_scan(x, scan_sh, &tot);
            if (tid < nr * 16) row_off[tid] = eq_base + ex;
            __syncthreads();
#pragma unroll
            for (int rr = 0; rr < kRows; ++rr) {
                if (rr >= nr) break;
                const int j = (r0 + rr) * kSelThreads + tid;
                const bool f = j < n && order_key(sc[j]) == T;
                const uint64_t bal = __ballot(f);
                const uint32_t rank = row_off[rr * 16 + wave] + (uint32_t)__popcll(bal & below);
                if (f && rank < need_eq) eqbits |= 1ull << rr;
            }
            eq_base += tot;
            __syncthreads();
        }
        uint64_t takebits = 0;
#pragma unroll
        for (int rr = 0; rr < kRows; ++rr) {
            if (rr >= nr) break;
            const int j = (r0 + rr) * kSelThreads + tid;
            bool f = false;
            if (j < n) {
                if (mode == 0) {
                    f = true;
                } else if (mode == 1) {
                    const float x = sc[j];
                    const uint32_t bn = value_bin(x, lo, scale);
                    const uint32_t key = order_key(x);
                    f = bn > bstar || (bn == bstar && (key > tk || (key == tk && j <= ti)));
                } else {
                    f = order_key(sc[j]) > T || ((eqbits >> rr) & 1ull);
                }
            }
            if (f) takebits |= 1ull << rr;
            const uint64_t bal = __ballot(f);
            if (lane == 0) row_off[rr * 16 + wave] = (uint32_t)__popcll(bal);
        }
        __syncthreads();
        uint32_t tot;
        const uint32_t x = tid < nr * 16 ? row_off[tid] : 0u;
        const uint32_t ex = block_excl_scan(x, scan_sh, &tot);
        if (tid < nr * 16) row_off[tid] = base + ex;
        __syncthreads();
#pragma unroll
        for (int rr = 0; rr < kRows; ++rr) {
            if (rr >= nr) break;
            const bool f = (takebits >> rr) & 1ull;
            const uint64_t bal = __ballot(f);
            if (f) {
                const int j = (r0 + rr) * kSelThreads + tid;
                const float x = sc[j];
                const uint32_t pos = row_off[rr * 16 + wave] + (uint32_t)__popcll(bal & below);
                const float p = __expf(x - l);
                id[pos] = j;
                ps[pos] = p;
                psum += p;
            }
        }
        base += tot;
        __syncthreads();
    }
    return psum;
}

// Register-resident variant of compact_rows for E <= kSelPerThread (one batch; rows are
// unrolled so that v[] stays in registers).
__device__ __forceinline__ float compact_regs(const float (&v)[kSelPerThread], int n, int E, int mode, float lo,
                                              float scale, uint32_t bstar, uint32_t tk, int32_t ti, uint32_t T,
                                              uint32_t need_eq, float l, int32_t* id, float* ps, uint32_t* row_off,
                                              uint32_t* scan_sh) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint64_t eqbits = 0;
    uint32_t tot;
    if (mode == 2) {
#pragma unroll
        for (int rr = 0; rr < kSelPerThread; ++rr) {
            if (rr < E) {
                const int j = rr * kSelThreads + tid;
                const bool f = j < n && order_key(v[rr]) == T;
                const uint64_t bal = __ballot(f);
                if (lane == 0) row_off[rr * 16 + wave] = (uint32_t)__popcll(bal);
            }
        }
        __syncthreads();
        const uint32_t x = tid < E * 16 ? row_off[tid] : 0u;
        const uint32_t ex = block_excl_scan(x, scan_sh, &tot);
        if (tid < E * 16) row_off[tid] = ex;
        __syncthreads();
#pragma unroll
        for (int rr = 0; rr < kSelPerThread; ++rr) {
            if (rr < E) {
                const int j = rr * kSelThreads + tid;
                const bool f = j < n && order_key(v[rr]) == T;
                const uint64_t bal = __ballot(f);
                const uint32_t rank = row_off[rr * 16 + wave] + (uint32_t)__popcll(bal & below);
                if (f && rank < need_eq) eqbits |= 1ull << rr;
            }
        }
        __syncthreads();
    }
    uint64_t takebits = 0;
#pragma unroll
    for (int rr = 0; rr < kSelPerThread; ++rr) {
        if (rr < E) {
            const int j = rr * kSelThreads + tid;
            bool f = false;
            if (j < n) {
                if (mode == 0) {
                    f = true;
                } else if (mode == 1) {
                    const uint32_t bn = value_bin(v[rr], lo, scale);
                    const uint32_t key = order_key(v[rr]);
                    f = bn > bstar || (bn == bstar && (key > tk || (key == tk && j <= ti)));
                } else {
                    f = order_key(v[rr]) > T || ((eqbits >> rr) & 1ull);
                }
            }
            if (f) takebits |= 1ull << rr;
            const uint64_t bal = __ballot(f);
            if (lane == 0) row_off[rr * 16 + wave] = (uint32_t)__popcll(bal);
        }
    }
    __syncthreads();
    const uint32_t x = tid < E * 16 ? row_off[tid] : 0u;
    const uint32_t ex = block_excl_scan(x, scan_sh, &tot);
    if (tid < E * 16) row_off[tid] = ex;
    __syncthreads();
    float psum = 0.f;
#pragma unroll
    for (int rr = 0; rr < kSelPerThread; ++rr) {
        if (rr < E) {
            const bool f = (takebits >> rr) & 1ull;
            const uint64_t bal = __ballot(f);
            if (f) {
                const uint32_t pos = row_off[rr * 16 + wave] + (uint32_t)__popcll(bal & below);
                const float p = __expf(v[rr] - l);
                id[pos] = rr * kSelThreads + tid;
                ps[pos] = p;
                psum += p;
            }
        }
    }
    return psum;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ scores, int ld,
                                                             const float* __restrict__ lse, int n, int k,
                                                             int32_t* __restrict__ idx, float* __restrict__ p_sel,
                                                             float* __restrict__ mass) {
    const int bh = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* sc = scores + (size_t)bh * ld;
    __shared__ uint32_t hist[kBins];
    __shared__ uint32_t scan_sh[kSelThreads / 64 + 1];
    __shared__ float red_sh[kSelThreads / 64];
    __shared__ uint32_t sel_bin, sel_above, cand_n, fast_ok;
    __shared__ uint32_t cand_key[kCandCap];
    __shared__ int32_t cand_idx[kCandCap];
    __shared__ uint32_t thr_key;
    __shared__ int32_t thr_idx;
    __shared__ uint32_t row_off[kSelThreads];  // [row in batch][wave] output offsets
    __shared__ float msum[kSelThreads / 64];

    if (k <= 0) {
        if (tid == 0) mass[bh] = 0.f;
        return;
    }
    // element e of this thread is column j = e * 1024 + tid (coalesced rows of 1024 columns)
    const int E = (n + kSelThreads - 1) / kSelThreads;
    const bool take_all = (k >= n);
    const bool in_regs = E <= kSelPerThread;
    // mode 0: every column; mode 1: value bins; mode 2: radix threshold on the order key
    int mode = take_all ? 0 : 1;
    float lo = 0.f, scale = 0.f;
    uint32_t bstar = 0, need_eq = 0, T = 0;

    float v[kSelPerThread];
    if (in_regs) {
#pragma unroll
        for (int e = 0; e < kSelPerThread; ++e) {
            const int j = e * kSelThreads + tid;
            v[e] = (e < E && j < n) ? sc[j] : 0.f;
        }
    }

    if (!take_all && in_regs) {
        float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
#pragma unroll
        for (int e = 0; e < kSelPerThread; ++e)
            if (e < E && e * kSelThreads + tid < n) {
                mn = fminf(mn, v[e]);
                mx = fmaxf(mx, v[e]);
            }
        lo = block_min(mn, red_sh);
        const float hi = block_max(mx, red_sh);
        const float range = hi - lo;
        scale = (float)kBins / range;
        if (tid == 0) fast_ok = (range > 0.f && __builtin_isfinite(range) && __builtin_isfinite(scale)) ? 1u : 0u;
        for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0;
        if (tid == 0) cand_n = 0;
        __syncthreads();
        if (fast_ok) {
#pragma unroll
            for (int e = 0; e < kSelPerThread; ++e)
                if (e < E && e * kSelThreads + tid < n) atomicAdd(&hist[value_bin(v[e], lo, scale)], 1u);
            __syncthreads();
            // bin of the k-th largest, scanning from the top bin
            uint32_t cnt[2], bins[2], local = 0;
            for (int e = 0; e < 2; ++e) {
                bins[e] = kBins - 1 - (tid * 2 + e);
                cnt[e] = hist[bins[e]];
                local += cnt[e];
            }
            uint32_t tot;
            uint32_t above = block_excl_scan(local, scan_sh, &tot);
            for (int e = 0; e < 2; ++e) {
                if (above < (uint32_t)k && (uint32_t)k <= above + cnt[e]) {
                    sel_bin = bins[e];
                    sel_above = above;
                }
                above += cnt[e];
            }
            __syncthreads();
            bstar = sel_bin;
            const uint32_t need_in = (uint32_t)k - sel_above;  // columns taken inside the threshold bin
            if (hist[bstar] > (uint32_t)kCandCap) {
                if (tid == 0) fast_ok = 0;
            } else {
#pragma unroll
                for (int e = 0; e < kSelPerThread; ++e) {
                    const int j = e * kSelThreads + tid;
                    if (e < E && j < n && value_bin(v[e], lo, scale) == bstar) {
                        const uint32_t slot = atomicAdd(&cand_n, 1u);
                        cand_key[slot] = order_key(v[e]);
                        cand_idx[slot] = j;
                    }
                }
                __syncthreads();
                const uint32_t c = cand_n;
                // exact rank of each candidate under (key descending, index ascending)
                for (uint32_t t = tid; t < c; t += kSelThreads) {
                    const uint32_t kt = cand_key[t];
                    const int32_t it = cand_idx[t];
                    uint32_t rank = 0;
                    for (uint32_t u = 0; u < c; ++u) {
                        const uint32_t ku = cand_key[u];
                        rank += (ku > kt || (ku == kt && cand_idx[u] < it)) ? 1u : 0u;
                    }
                    if (rank == need_in - 1) {
                        thr_key = kt;
                        thr_idx = it;
                    }
                }
            }
            __syncthreads();
        }
        if (!fast_ok) mode = 2;
    } else if (!take_all) {
        mode = 2;
    }
    __syncthreads();
    if (mode == 2) T = radix_threshold(sc, n, (uint32_t)k, hist, scan_sh, &sel_bin, &sel_above, &need_eq);
    const uint32_t tk = thr_key;
    const int32_t ti = thr_idx;

    // compaction in ascending index order (see compact_rows)
    const float l = lse[bh];
    float psum;
    if (in_regs)
        psum = compact_regs(v, n, E, mode, lo, scale, bstar, tk, ti, T, need_eq, l, idx + (size_t)bh * k,
                            p_sel + (size_t)bh * k, row_off, scan_sh);
    else
        psum = compact_rows(sc, n, E, mode, lo, scale, bstar, tk, ti, T, need_eq, l, idx + (size_t)bh * k,
                            p_sel + (size_t)bh * k, row_off, scan_sh);
    // mass: fixed-order reduction (waves in order)
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) psum += __shfl_xor(psum, m, 64);
    if (lane == 0) msum[wave] = psum;
    __syncthreads();
    if (tid == 0) {
        float m = 0.f;
        for (int w = 0; w < kSelThreads / 64; ++w) m += msum[w];
        mass[bh] = m;
    }
}

size_t select_ws_bytes(int, int, int) { return 0; }

int launch_select(const float* scores, int ld, const float* lse, int B, int H, int n, int k, int32_t* idx,
                  float* p_sel, float* mass, void*, hipStream_t st) {
    select_kernel<<<B * H, kSelThreads, 0, st>>>(scores, ld, lse, n, k, idx, p_sel, mass);
    return hipGetLastError() == hipSuccess ? QKV_OK : QKV_ELAUNCH;
}

}  // namespace qkv
