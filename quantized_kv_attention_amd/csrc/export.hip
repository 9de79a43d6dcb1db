// qkv_export_plane: one (sequence, head)'s stored slots of one loop's plane unpacked into
// plain arrays (one code per byte, fp32 metadata), so that tests compare logical content
// and never decode the packed block layout themselves.
#include <type_traits>

#include "launch.h"

namespace qkv {

// One thread per (slot, channel) of slots [0, n_slots): both codes; a key group's metadata
// by its block's first slot, a value group's by the group's first channel.
template <int D, int BITS>
__global__ __launch_bounds__(256) void export_plane_kernel(PlaneArg P, int H, int b, int h, int n_slots,
                                                           uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                                           float* __restrict__ ks, float* __restrict__ kz,
                                                           float* __restrict__ vs, float* __restrict__ vz) {
    using Bk = Block<D, BITS>;
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    if (e >= (long)n_slots * D) return;
    const int slot = (int)(e / D), c = (int)(e % D);
    const uint8_t* bp = block_ptr<D, BITS>(P, H, b, h, slot >> 6);
    const int row = slot & 63;
    constexpr int per_byte = 8 / BITS;
    const int byte = c / per_byte, sh = (c % per_byte) * BITS;
    constexpr uint32_t mask = (1u << BITS) - 1u;
    kc[e] = (uint8_t)((bp[Bk::kc(row) + byte] >> sh) & mask);
    vc[e] = (uint8_t)((bp[Bk::vc(row) + byte] >> sh) & mask);
    const float* km = reinterpret_cast<const float*>(bp + Bk::kKm);
    if (row == 0) {
        ks[(size_t)(slot >> 6) * D + c] = km[c];
        kz[(size_t)(slot >> 6) * D + c] = km[D + c];
    }
    if ((c & 63) == 0) {
        const float* vm = reinterpret_cast<const float*>(bp + Bk::vm(row) + (c >> 6) * 8);
        vs[(size_t)slot * (D / 64) + (c >> 6)] = vm[0];
        vz[(size_t)slot * (D / 64) + (c >> 6)] = vm[1];
    }
}

int launch_export_plane(const CacheArg& ca, int D, int loop, int b, int h, int n_slots, uint8_t* kc, uint8_t* vc,
                        float* ks, float* kz, float* vs, float* vz, hipStream_t st) {
    const PlaneArg& P = ca.p[loop - 1];
    const int bits = plane_bits(loop - 1, ca.rbits, ca.full != 0);
    const long n = (long)n_slots * D;
    const int grid = (int)((n + 255) / 256);
    auto go = [&](auto dc, auto bc) {
        constexpr int DD = decltype(dc)::value, BB = decltype(bc)::value;
        export_plane_kernel<DD, BB><<<grid, 256, 0, st>>>(P, ca.H, b, h, n_slots, kc, vc, ks, kz, vs, vz);
    };
    using I64 = std::integral_constant<int, 64>;
    using I128 = std::integral_constant<int, 128>;
    using B2 = std::integral_constant<int, 2>;
    using B4 = std::integral_constant<int, 4>;
    if (D == 128) {
        if (bits == 2) go(I128{}, B2{}); else go(I128{}, B4{});
    } else {
        if (bits == 2) go(I64{}, B2{}); else go(I64{}, B4{});
    }
    return hipGetLastError() == hipSuccess ? QKV_OK : QKV_ELAUNCH;
}

}  // namespace qkv
