// Exact top-k column selection with the cached probability mass (project page STEP 02;
// explainer section 3: top-K key columns chosen from the preceding loop's statistics,
// their total probability under the preceding full distribution cached as m).
//
// Order: fp32 score descending, ties to the lower index; +0 and -0 compare equal.
// One 1024-thread workgroup per (sequence, head): three radix passes (11/11/10 bits of
// an order-preserving key) find the k-th largest key T and how many columns equal to
// T are taken; a final pass compacts the selected columns in ascending index order.
#include "launch.h"

namespace qkv {

constexpr int kSelThreads = 1024;

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

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ scores, int ld,
                                                             const float* __restrict__ lse, int n, int k,
                                                             int32_t* __restrict__ idx, float* __restrict__ p_sel,
                                                             float* __restrict__ mass) {
    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    const float* sc = scores + (size_t)bh * ld;
    const int kk = k < n ? k : n;
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t scan_sh[kSelThreads / 64 + 1];
    __shared__ uint32_t sel_bin, sel_above;
    __shared__ float msum[kSelThreads / 64];

    if (kk <= 0) {
        if (tid == 0) mass[bh] = 0.f;
        return;
    }

    uint32_t prefix = 0, pmask = 0;
    uint32_t need = (uint32_t)kk;
    const bool take_all = (kk >= n);
    if (!take_all) {
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
            // suffix counts from the top bin: thread t owns bins (nb-1-2t) and (nb-2-2t)
            const uint32_t per = nb / kSelThreads;  // 2 or 1
            uint32_t cnt[2] = {0, 0};
            uint32_t bins[2] = {0, 0};
            uint32_t local = 0;
            for (uint32_t e = 0; e < per; ++e) {
                bins[e] = nb - 1 - (tid * per + e);
                cnt[e] = hist[bins[e]];
                local += cnt[e];
            }
            uint32_t tot;
            uint32_t above = block_excl_scan(local, scan_sh, &tot);
            for (uint32_t e = 0; e < per; ++e) {
                if (above < need && need <= above + cnt[e]) {
                    sel_bin = bins[e];
                    sel_above = above;
                }
                above += cnt[e];
            }
            __syncthreads();
            prefix |= sel_bin << sh;
            pmask |= (nb - 1) << sh;
            need -= sel_above;
            __syncthreads();
        }
    }
    // prefix is now the threshold key T; `need` columns equal to T are taken (lowest first)
    const uint32_t T = prefix;
    const int C = (n + kSelThreads - 1) / kSelThreads;
    const int j0 = tid * C, j1 = min(n, j0 + C);
    uint32_t gt = 0, eq = 0;
    for (int j = j0; j < j1; ++j) {
        const uint32_t key = order_key(sc[j]);
        if (take_all || key > T) ++gt;
        else if (key == T) ++eq;
    }
    uint32_t tot;
    const uint32_t eq_before = block_excl_scan(eq, scan_sh, &tot);
    uint32_t take_eq = 0;
    if (!take_all) {
        take_eq = eq_before >= need ? 0u : (need - eq_before < eq ? need - eq_before : eq);
    }
    uint32_t out = block_excl_scan(gt + take_eq, scan_sh, &tot);
    const float l = lse[bh];
    float psum = 0.f;
    uint32_t eq_seen = 0;
    int32_t* id = idx + (size_t)bh * kk;
    float* ps = p_sel + (size_t)bh * kk;
    for (int j = j0; j < j1; ++j) {
        const float v = sc[j];
        const uint32_t key = order_key(v);
        bool take = take_all || key > T;
        if (!take && key == T) {
            take = eq_seen < take_eq;
            ++eq_seen;
        }
        if (take) {
            const float p = __expf(v - l);
            id[out] = j;
            ps[out] = p;
            psum += p;
            ++out;
        }
    }
    // mass: fixed-order reduction (waves in order)
    psum = wave_sum(psum);
    if ((tid & 63) == 0) msum[tid >> 6] = psum;
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
