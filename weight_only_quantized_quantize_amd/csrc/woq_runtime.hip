// Decode-stack runner: drives a sequence of quantised linears on one stream.
//
// A decode step walks the layers in order; within a layer, linears that read
// the same activation (q|k|v, gate|up) are stacked along N into one launch.
// Each INT4O step first gathers its input through the input space's global
// permutation into the runner's workspace, then launches the product.
#include <hip/hip_runtime.h>

#include <new>
#include <vector>

#include "woq_internal.h"

struct woq_stack {
    std::vector<woq_stack_step> steps;
    int64_t max_b = 0;
    int64_t xp_elems = 0;      // per workspace row
    uint16_t* xp = nullptr;    // [max_b][xp_elems]
    int device = 0;
};

extern "C" {

int woq_stack_create(const woq_stack_step* steps, int32_t n_steps, int64_t max_b, woq_stack** out) {
    if (!out || n_steps < 0 || (n_steps > 0 && !steps) || max_b < 1 || max_b > 64) return WOQ_EINVAL;
    *out = nullptr;
    int64_t xp_elems = 8;
    int max_slot = 0;
    for (int i = 0; i < n_steps; ++i) {
        const woq_stack_step& s = steps[i];
        if (s.in_slot < 0 || s.out_slot < 0) return WOQ_EINVAL;
        max_slot = std::max(max_slot, std::max(s.in_slot, s.out_slot));
        if (s.fmt == WOQ_FMT_INT4O) {
            if (!woq::int4o_geom_valid(&s.w4.geom) || !s.perm) return WOQ_EINVAL;
            xp_elems = std::max(xp_elems, s.w4.geom.xp_len);
        } else if (s.fmt == WOQ_FMT_INT8) {
            if (max_b > 8) return WOQ_EUNSUPPORTED;
        } else {
            return WOQ_EINVAL;
        }
    }
    woq_stack* st = new (std::nothrow) woq_stack;
    if (!st) return WOQ_ENOMEM;
    st->steps.assign(steps, steps + n_steps);
    st->max_b = max_b;
    st->xp_elems = xp_elems;
    hipError_t e = hipGetDevice(&st->device);
    if (e == hipSuccess) e = hipMalloc((void**)&st->xp, (size_t)(max_b * xp_elems * 2));
    if (e != hipSuccess) {
        woq::set_hip_error((int)e);
        delete st;
        return e == hipErrorOutOfMemory ? WOQ_ENOMEM : WOQ_EHIP;
    }
    *out = st;
    return WOQ_OK;
}

namespace {

// One pass over the steps; ev (2 per step) brackets each product launch.
int run_pass(woq_stack* st, const uint16_t* const* inputs, uint16_t* const* outputs, int64_t b, void* stream,
             hipEvent_t* ev) {
    hipStream_t hs = (hipStream_t)stream;
    for (size_t i = 0; i < st->steps.size(); ++i) {
        const woq_stack_step& s = st->steps[i];
        const uint16_t* x = inputs[s.in_slot];
        uint16_t* y = outputs[s.out_slot];
        int rc;
        if (s.fmt == WOQ_FMT_INT4O) {
            rc = woq_permute_x(x, s.w4.geom.K, s.perm, b, &s.w4.geom, st->xp, stream);
            if (rc) return rc;
            if (ev) hipEventRecord(ev[2 * i], hs);
            rc = woq_qgemv_int4o(&s.w4, st->xp, b, y, s.w4.N, stream);
        } else {
            if (ev) hipEventRecord(ev[2 * i], hs);
            rc = woq_qgemv_int8(&s.w8, x, s.w8.K, b, y, s.w8.N, stream);
        }
        if (ev) hipEventRecord(ev[2 * i + 1], hs);
        if (rc) return rc;
    }
    return WOQ_OK;
}

}  // namespace

int woq_stack_run(woq_stack* st, const uint16_t* const* inputs, uint16_t* const* outputs, int64_t b, void* stream) {
    if (!st || !inputs || !outputs || b < 1 || b > st->max_b) return WOQ_EINVAL;
    return run_pass(st, inputs, outputs, b, stream, nullptr);
}

int woq_stack_time(woq_stack* st, const uint16_t* const* inputs, uint16_t* const* outputs, int64_t b, void* stream,
                   int32_t iters, float* step_ms, float* pass_ms) {
    if (!st || !inputs || !outputs || b < 1 || b > st->max_b || iters < 1 || !pass_ms ||
        (!step_ms && !st->steps.empty()))
        return WOQ_EINVAL;
    const size_t n = st->steps.size();
    const size_t per_iter = 2 * n + 2;
    std::vector<hipEvent_t> ev(per_iter * (size_t)iters, nullptr);
    hipError_t e = hipSuccess;
    for (auto& x : ev)
        if (e == hipSuccess) e = hipEventCreate(&x);
    int rc = WOQ_OK;
    hipStream_t hs = (hipStream_t)stream;
    for (int it = 0; it < iters && e == hipSuccess && rc == WOQ_OK; ++it) {
        hipEvent_t* base = ev.data() + per_iter * it;
        e = hipEventRecord(base[2 * n], hs);
        if (e == hipSuccess) rc = run_pass(st, inputs, outputs, b, stream, base);
        if (e == hipSuccess && rc == WOQ_OK) e = hipEventRecord(base[2 * n + 1], hs);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(hs);
    if (e == hipSuccess && rc == WOQ_OK) {
        for (size_t i = 0; i < n; ++i) step_ms[i] = 0.0f;
        double total = 0.0;
        for (int it = 0; it < iters && e == hipSuccess; ++it) {
            hipEvent_t* base = ev.data() + per_iter * it;
            for (size_t i = 0; i < n && e == hipSuccess; ++i) {
                float ms = 0.0f;
                e = hipEventElapsedTime(&ms, base[2 * i], base[2 * i + 1]);
                step_ms[i] += ms / iters;
            }
            float ms = 0.0f;
            if (e == hipSuccess) e = hipEventElapsedTime(&ms, base[2 * n], base[2 * n + 1]);
            total += ms;
        }
        *pass_ms = (float)(total / iters);
    }
    for (auto& x : ev)
        if (x) hipEventDestroy(x);
    if (rc) return rc;
    if (e != hipSuccess) {
        woq::set_hip_error((int)e);
        return WOQ_EHIP;
    }
    return WOQ_OK;
}

int woq_stack_destroy(woq_stack* st) {
    if (!st) return WOQ_OK;
    hipError_t e = hipSuccess;
    if (st->xp) e = hipFree(st->xp);
    delete st;
    if (e != hipSuccess) {
        woq::set_hip_error((int)e);
        return WOQ_EHIP;
    }
    return WOQ_OK;
}

}  // extern "C"
