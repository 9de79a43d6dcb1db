// Online token selection (explainer section 3, cross-loop token-sparse updates: after the
// dense loops each loop ranks the tokens updated in the preceding loop by their normalized
// hidden-state change and keeps a top-k subset, so the active sets nest; project page
// STEP 01: only active tokens write new K/V).  The result is the next loop's active list,
// in the form kv_encode_loop takes it.
//
// score[t] = ||H_cur[t] - H_prev[t]|| / ||H_prev[t]|| for t in the preceding active set
// (-inf elsewhere; a zero previous state gives +inf for a nonzero change, 0 otherwise),
// then the top k of the scores (ties to the lower index) by the column selector's kernel,
// then the entries that fell outside the preceding set (k above its size) are dropped.
#include "launch.h"

namespace qkv {

constexpr int kTokWaves = 4;

// score[b][t] = -inf for every token; the zero lse the selector is given (only needed when
// the preceding set is a list: with every token scored, the score kernel writes the lse)
__global__ __launch_bounds__(256) void token_fill_kernel(float* __restrict__ score, int n, float* __restrict__ zlse) {
    const int b = blockIdx.y;
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t < n) score[(size_t)b * n + t] = -__builtin_huge_valf();
    if (blockIdx.x == 0 && threadIdx.x == 0) zlse[b] = 0.f;
}

// One wave per scored token: the squared change and the squared previous state summed over
// dm channels (16-byte loads, 8 channels per lane per step), in a fixed order.
__global__ __launch_bounds__(64 * kTokWaves) void token_score_kernel(const uint16_t* __restrict__ hc,
                                                                     const uint16_t* __restrict__ hp, int ld_tok,
                                                                     int n, int dm, const int32_t* __restrict__ act,
                                                                     const int32_t* __restrict__ n_act, int ld_act,
                                                                     float* __restrict__ score, float* __restrict__ zlse) {
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    if (zlse && blockIdx.x == 0 && threadIdx.x == 0) zlse[b] = 0.f;
    const int i = blockIdx.x * kTokWaves + (threadIdx.x >> 6);
    int t;
    if (act) {
        if (i >= n_act[b]) return;
        t = act[(size_t)b * ld_act + i];
        if (t < 0 || t >= n) return;
    } else {
        if (i >= n) return;
        t = i;
    }
    const uint16_t* rc = hc + ((size_t)b * ld_tok + t) * dm;
    const uint16_t* rp = hp + ((size_t)b * ld_tok + t) * dm;
    float dd = 0.f, pp = 0.f;
    for (int c = lane * 8; c < dm; c += 64 * 8) {
        float a[8], p[8];
        bf16x8(ld_stream_u4(rc + c), a);
        bf16x8(ld_stream_u4(rp + c), p);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float dlt = a[e] - p[e];
            dd = fmaf(dlt, dlt, dd);
            pp = fmaf(p[e], p[e], pp);
        }
    }
    dd = wave_sum(dd);
    pp = wave_sum(pp);
    if (lane == 0)
        score[(size_t)b * n + t] = pp > 0.f ? sqrtf(dd) / sqrtf(pp) : (dd > 0.f ? __builtin_huge_valf() : 0.f);
}

// Drops the selected entries whose score is -inf (tokens outside the preceding set, picked
// only when k exceeds its size), in place and in order; writes the count and the count of
// positions below `split`.  One workgroup of kCompactWaves waves per sequence; each pass
// reads kCompactPer chunks of entries and their scores with all loads in flight, then
// places the chunks one after another.
constexpr int kCompactWaves = 16;
constexpr int kCompactThreads = 64 * kCompactWaves;
constexpr int kCompactPer = 8;

__global__ __launch_bounds__(kCompactThreads) void token_compact_kernel(const float* __restrict__ score, int n, int k,
                                                                        int32_t* __restrict__ act_out,
                                                                        int32_t* __restrict__ n_out,
                                                                        int32_t* __restrict__ n_before, int split) {
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int32_t* a = act_out + (size_t)b * k;
    __shared__ uint32_t wcnt[kCompactWaves], wlow[kCompactWaves];
    uint32_t base = 0, below = 0;
    const uint64_t lower = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    for (int p0 = 0; p0 < k; p0 += kCompactThreads * kCompactPer) {
        int t[kCompactPer];
        bool keep[kCompactPer];
#pragma unroll
        for (int e = 0; e < kCompactPer; ++e) {
            const int i = p0 + e * kCompactThreads + tid;
            t[e] = i < k ? a[i] : -1;
        }
        // (every entry read here is complete before the first barrier below: its score load,
        // issued before it, needs the entry as its address)
#pragma unroll
        for (int e = 0; e < kCompactPer; ++e)
            keep[e] = t[e] >= 0 && t[e] < n && score[(size_t)b * n + t[e]] > -__builtin_huge_valf();
#pragma unroll
        for (int e = 0; e < kCompactPer; ++e) {
            if (p0 + e * kCompactThreads >= k) break;   // uniform
            const uint64_t bal = __ballot(keep[e]);
            // positions below the split: the kept entries are ascending
            const uint64_t bs = __ballot(keep[e] && t[e] < split);
            if (lane == 0) {
                wcnt[wave] = (uint32_t)__popcll(bal);
                wlow[wave] = (uint32_t)__popcll(bs);
            }
            // every entry of this pass has been read (chunk 0), the counts are written
            __syncthreads();
            uint32_t before = 0, all = 0, low = 0;
#pragma unroll
            for (int w = 0; w < kCompactWaves; ++w) {
                before += w < wave ? wcnt[w] : 0u;
                all += wcnt[w];
                low += wlow[w];
            }
            if (keep[e]) a[base + before + (uint32_t)__popcll(bal & lower)] = t[e];  // never past its entry
            below += low;
            base += all;
            __syncthreads();  // the counts are read before the next chunk writes them
        }
    }
    if (tid == 0) {
        n_out[b] = (int32_t)base;
        if (n_before) n_before[b] = (int32_t)below;
    }
}

size_t token_ws_bytes(int B, int k) { return (size_t)(2 * B + (size_t)B * k) * sizeof(float); }

int launch_select_tokens(const uint16_t* hc, const uint16_t* hp, int ld_tok, int B, int n, int dm,
                         const int32_t* act, const int32_t* n_act, int ld_act, int k, int split, float* score,
                         int32_t* act_out, int32_t* n_out, int32_t* n_before, void* ws, hipStream_t st) {
    float* zlse = static_cast<float*>(ws);
    float* mass = zlse + B;
    float* p_sel = mass + B;
    // with every token scored, every score is written: no fill
    if (act) token_fill_kernel<<<dim3((n + 255) / 256, B), 256, 0, st>>>(score, n, zlse);
    const int rows = act ? ld_act : n;
    token_score_kernel<<<dim3((rows + kTokWaves - 1) / kTokWaves, B), 64 * kTokWaves, 0, st>>>(
        hc, hp, ld_tok, n, dm, act, n_act, ld_act, score, act ? nullptr : zlse);
    if (hipGetLastError() != hipSuccess) return QKV_ELAUNCH;
    const int rc = launch_select(score, n, zlse, B, 1, n, k, act_out, p_sel, mass, nullptr, st);
    if (rc != QKV_OK) return rc;
    token_compact_kernel<<<B, kCompactThreads, 0, st>>>(score, n, k, act_out, n_out, n_before, split);
    return hipGetLastError() == hipSuccess ? QKV_OK : QKV_ELAUNCH;
}

}  // namespace qkv
