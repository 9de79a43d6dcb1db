// Residual-quantize encoder kernels and BF16 tail append (gfx950); the encoder's device
// functions are in encode_group.h.
//
// Loop 1's K/V become the INT4 base; loop r >= 2 stores Q(X^(r) - Xhat^(r-1)) for its
// active tokens, where Xhat^(r-1) is rebuilt exactly from planes 1..r-1 (project page,
// The Method, STEP 01 and STEP 03; flozi.net explainer section 3: keys per channel over
// 64 tokens, values per token over 64 channels, asymmetric, group 64).
//
// Exactness: every codec step is a single IEEE fp32 operation, as the oracle does it
// (correctly rounded division, rint half-to-even, fmaf dequant, no contraction).
#include <type_traits>

#include "encode_group.h"
#include "launch.h"

#pragma clang fp contract(off)

namespace qkv {

// keys and values of a group are encoded by two workgroups (they write disjoint parts of the block)
template <int D, int OUTB, int RB>
__global__ __launch_bounds__(256, 4) void encode_group_kernel(CacheArg ca, int loop, int nch, int pos0, int n_pos,
                                                           const int32_t* __restrict__ act_pos,
                                                           const int32_t* __restrict__ n_act, int ld_act,
                                                           const uint16_t* __restrict__ ksrc,
                                                           const uint16_t* __restrict__ vsrc, int ld_src,
                                                           int32_t* __restrict__ rowpos) {
    extern __shared__ int sslot[];  // [nch][64], sized at launch
    encode_group<D, OUTB, RB>(ca, loop, nch, pos0, n_pos, act_pos, n_act, ld_act, ksrc, vsrc, ld_src, rowpos,
                              blockIdx.x >> 1, blockIdx.x & 1, blockIdx.y, blockIdx.z, sslot);
}

__global__ __launch_bounds__(256) void encode_maps_kernel(int cap_ctx, int pos0, int n_pos,
                                                          const int32_t* __restrict__ act_pos,
                                                          const int32_t* __restrict__ n_act, int ld_act,
                                                          int32_t* __restrict__ rowmap,
                                                          int32_t* __restrict__ rowstart,
                                                          uint32_t* __restrict__ smask, uint32_t bit) {
    encode_maps(cap_ctx, pos0, n_pos, act_pos, n_act, ld_act, rowmap, rowstart, smask, bit, blockIdx.y,
                blockIdx.x * 256 + threadIdx.x);
}

__global__ __launch_bounds__(64) void append_tail_kernel(int H, int D, int pos0, int n_rows,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         uint16_t* __restrict__ tk, uint16_t* __restrict__ tv) {
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const size_t src = ((size_t)((size_t)b * H + h) * n_rows + i) * D;
    const size_t dst = ((size_t)((size_t)b * H + h) * kTail + ((pos0 + i) % kTail)) * D;
    for (int c = threadIdx.x; c < D; c += 64) {
        tk[dst + c] = k[src + c];
        tv[dst + c] = v[src + c];
    }
}

// every loop at once: k, v [loops][B][H][n_rows][D]; grid.z = B * loops
__global__ __launch_bounds__(64) void append_tail_all_kernel(CacheArg ca, int D, int pos0, int n_rows,
                                                             const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v) {
    const int i = blockIdx.x, h = blockIdx.y;
    const int b = blockIdx.z % ca.B, r = blockIdx.z / ca.B;
    const size_t src = ((((size_t)r * ca.B + b) * ca.H + h) * n_rows + i) * D;
    const size_t dst = ((size_t)((size_t)b * ca.H + h) * kTail + ((pos0 + i) % kTail)) * D;
    uint16_t* tk = const_cast<uint16_t*>(ca.tail_k[r]);
    uint16_t* tv = const_cast<uint16_t*>(ca.tail_v[r]);
    for (int c = threadIdx.x; c < D; c += 64) {
        tk[dst + c] = k[src + c];
        tv[dst + c] = v[src + c];
    }
}

int launch_append_all(const CacheArg& ca, int D, int pos0, int n_rows, const uint16_t* k, const uint16_t* v,
                      hipStream_t st) {
    dim3 grid(n_rows, ca.H, ca.B * ca.nplanes);
    append_tail_all_kernel<<<grid, 64, 0, st>>>(ca, D, pos0, n_rows, k, v);
    return hipGetLastError() == hipSuccess ? QKV_OK : QKV_ELAUNCH;
}

int launch_encode(const CacheArg& ca, int D, int loop, int pos0, int n_pos, const int32_t* act_pos,
                  const int32_t* n_act, int ld_act, const uint16_t* ksrc, const uint16_t* vsrc, int ld_src,
                  hipStream_t st) {
    const PlaneArg& P = ca.p[loop - 1];
    const int ngroups = (n_pos + 63) / 64;
    dim3 grid(2 * ngroups, ca.H, ca.B);  // a key and a value workgroup per group
    int32_t* rowpos = const_cast<int32_t*>(P.rowpos);
    // the chain Xhat^(loop-1) is rebuilt for residual planes only
    const int nch = ca.full ? 0 : loop - 1;
    const int outb = (loop == 1 || ca.full) ? 4 : ca.rbits;
    const size_t dyn = (size_t)nch * 64 * sizeof(int);  // chain slots of the stored rows
    auto go = [&](auto dc, auto oc, auto rc) {
        constexpr int DD = decltype(dc)::value, OB = decltype(oc)::value, RBB = decltype(rc)::value;
        encode_group_kernel<DD, OB, RBB><<<grid, 256, dyn, st>>>(ca, loop, nch, pos0, n_pos, act_pos, n_act, ld_act,
                                                                ksrc, vsrc, ld_src, rowpos);
    };
    using I64 = std::integral_constant<int, 64>;
    using I128 = std::integral_constant<int, 128>;
    using B2 = std::integral_constant<int, 2>;
    using B4 = std::integral_constant<int, 4>;
    if (D == 128) {
        if (ca.rbits == 2 && !ca.full) {
            if (outb == 2) go(I128{}, B2{}, B2{}); else go(I128{}, B4{}, B2{});
        } else {
            go(I128{}, B4{}, B4{});
        }
    } else {
        if (ca.rbits == 2 && !ca.full) {
            if (outb == 2) go(I64{}, B2{}, B2{}); else go(I64{}, B4{}, B2{});
        } else {
            go(I64{}, B4{}, B4{});
        }
    }
    if (hipGetLastError() != hipSuccess) return QKV_ELAUNCH;
    if (!P.dense) {
        dim3 g2((n_pos + 255) / 256, ca.B);
        encode_maps_kernel<<<g2, 256, 0, st>>>(ca.cap_ctx, pos0, n_pos, act_pos, n_act, ld_act,
                                               const_cast<int32_t*>(P.rowmap), const_cast<int32_t*>(P.rowstart),
                                               ca.smask, 1u << (loop - 1));
        if (hipGetLastError() != hipSuccess) return QKV_ELAUNCH;
    }
    return QKV_OK;
}

int launch_append(int B, int H, int D, int pos0, int n_rows, const uint16_t* k, const uint16_t* v, uint16_t* tk,
                  uint16_t* tv, hipStream_t st) {
    dim3 grid(n_rows, H, B);
    append_tail_kernel<<<grid, 64, 0, st>>>(H, D, pos0, n_rows, k, v, tk, tv);
    return hipGetLastError() == hipSuccess ? QKV_OK : QKV_ELAUNCH;
}

}  // namespace qkv
