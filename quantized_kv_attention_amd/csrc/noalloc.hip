// attn_decode_dense_noalloc: the dense reader with its split partials in a fixed device
// array instead of a caller-supplied workspace, for callers that cannot allocate (code
// under HIP graph capture, tight serving loops, harnesses that forbid allocation).
//
// `scratch` below is a file-scope device array.  In host code its name is only a host-side
// stand-in: its device address on the current GPU comes from hipGetSymbolAddress, taken
// once per device on the first call there, and only that address is ever handed to a
// kernel.  Every call on one GPU shares that GPU's copy; the reader writes every partial it
// later reads, so nothing needs clearing between calls, but calls that overlap in time on
// one GPU race on it.
#include <mutex>

#include "launch.h"

namespace qkv {
namespace {

constexpr size_t kScratchBytes = QKV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per device).
int scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return QKV_ELAUNCH;
    if (dev < 0 || dev >= kMaxDevices) return QKV_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QKV_ELAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return QKV_OK;
}

}  // namespace

int launch_dense_noalloc(const CacheArg& ca, int D, int loop, const uint16_t* q, NewRow nr, float sm, uint16_t* o,
                         float* o32, float* scores, int ld, float* lse, hipStream_t st) {
    if (dense_ws_bytes(ca.B, ca.H, D, ca.n_body) > kScratchBytes) return QKV_EWORKSPACE;
    void* ws = nullptr;
    const int rc = scratch_on_current_device(&ws);
    if (rc != QKV_OK) return rc;
    return launch_dense(ca, D, loop, q, nr, sm, o, o32, scores, ld, lse, ws, st);
}

}  // namespace qkv
