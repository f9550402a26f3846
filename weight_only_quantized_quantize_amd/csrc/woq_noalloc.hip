// The split-K INT4O product for callers that cannot allocate device memory.
//
// woq_qgemm_int4o_splitk takes its partial-sum workspace from the caller;
// woq_qgemm_int4o_splitk_noalloc runs the same launches on a workspace that
// lives in the library's code object instead: each device holds its own copy
// from the module's load until the process ends, and a call allocates
// nothing.  Host code never passes the array's name to a kernel (on the host
// it only stands in for the symbol); it passes the device address that
// hipGetSymbolAddress gives, looked up once per device with that device
// current, on the first call there.
#include <hip/hip_runtime.h>

#include <mutex>

#include "woq_internal.h"

namespace {

static __device__ __align__(256) float scratch[WOQ_SPLITK_NOALLOC_BYTES / sizeof(float)];

// Device address of this device's copy of `scratch` (cached per device).
int scratch_address(float** out) {
    static std::mutex mu;
    static float* addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= 64) {
        woq::set_hip_error((int)e);
        return WOQ_EHIP;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            woq::set_hip_error((int)e);
            return WOQ_EHIP;
        }
        addr[dev] = static_cast<float*>(p);
    }
    *out = addr[dev];
    return WOQ_OK;
}

}  // namespace

extern "C" int woq_qgemm_int4o_splitk_noalloc(const woq_int4o_w* w, const uint16_t* xp, int64_t b, uint16_t* y,
                                              int64_t ldy, int32_t splits, void* stream) {
    if (!w || b < 0 || splits < 1 || splits > 16) return WOQ_EINVAL;
    if (b == 0 || w->N <= 0) return woq_qgemm_int4o_splitk(w, xp, b, y, ldy, splits, nullptr, 0, stream);
    const int64_t need = woq_qgemm_int4o_splitk_workspace(w->N, b, splits);
    if (need < 0) return WOQ_EINVAL;
    if (need > WOQ_SPLITK_NOALLOC_BYTES) return WOQ_EUNSUPPORTED;
    float* ws = nullptr;
    const int rc = scratch_address(&ws);
    if (rc) return rc;
    // every split writes all of its b x N partial sums before the reduction
    // reads them, so nothing left by an earlier call needs clearing
    return woq_qgemm_int4o_splitk(w, xp, b, y, ldy, splits, ws, need, stream);
}
