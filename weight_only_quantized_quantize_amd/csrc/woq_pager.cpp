// Streamed decode over INT8 layers held in pinned host memory.
//
// Two device slots alternate between layers: while the products of layer l
// run on the compute stream out of slot l mod 2, the copy stream fills slot
// (l + 1) mod 2 with layer l + 1.  Events order the two streams both ways:
//   copied[s]    copy of the layer now in slot s has landed  -> products may start
//   released[s]  products of the layer in slot s are done     -> slot may be refilled
#include <hip/hip_runtime.h>

#include <algorithm>
#include <new>
#include <vector>

#include "woq_internal.h"

struct woq_pager {
    const uint8_t* pool = nullptr;
    std::vector<int64_t> off, bytes;
    std::vector<woq_pager_step> steps;
    int32_t L = 0, S = 0;
    int64_t max_b = 0;
    int64_t slot_bytes = 0;
    uint8_t* slot[2] = {nullptr, nullptr};
    hipEvent_t copied[2] = {nullptr, nullptr};
    hipEvent_t released[2] = {nullptr, nullptr};
};

namespace {

int hip_status(hipError_t e) {
    if (e == hipSuccess) return WOQ_OK;
    woq::set_hip_error((int)e);
    return e == hipErrorOutOfMemory ? WOQ_ENOMEM : WOQ_EHIP;
}

void release(woq_pager* p) {
    for (int s = 0; s < 2; ++s) {
        if (p->slot[s]) (void)hipFree(p->slot[s]);
        if (p->copied[s]) (void)hipEventDestroy(p->copied[s]);
        if (p->released[s]) (void)hipEventDestroy(p->released[s]);
    }
    delete p;
}

}  // namespace

extern "C" {

int woq_pager_create(const void* pinned_pool, const int64_t* layer_off, const int64_t* layer_bytes,
                     int32_t n_layers, const woq_pager_step* steps, int32_t steps_per_layer, int64_t max_b,
                     woq_pager** out) {
    if (!out) return WOQ_EINVAL;
    *out = nullptr;
    if (!pinned_pool || !layer_off || !layer_bytes || n_layers < 1 || !steps || steps_per_layer < 1 || max_b < 1 ||
        max_b > 8)
        return WOQ_EINVAL;
    int64_t slot_bytes = 0;
    for (int l = 0; l < n_layers; ++l) {
        if (layer_off[l] < 0 || layer_bytes[l] < 1) return WOQ_EINVAL;
        slot_bytes = std::max(slot_bytes, layer_bytes[l]);
        for (int s = 0; s < steps_per_layer; ++s) {
            const woq_pager_step& st = steps[(size_t)l * steps_per_layer + s];
            const woq_int8_w& w = st.w;
            if (w.N < 1 || w.K < 1 || w.nseg < 1 || w.nseg > WOQ_MAX_SEGMENTS || w.seg_end[w.nseg - 1] != w.N)
                return WOQ_EINVAL;
            if (st.code_offset < 0 || (st.code_offset & 15) ||
                st.code_offset + woq_int8_dev_bytes(w.N, w.K) > layer_bytes[l])
                return WOQ_EINVAL;
        }
    }
    woq_pager* p = new (std::nothrow) woq_pager;
    if (!p) return WOQ_ENOMEM;
    p->pool = (const uint8_t*)pinned_pool;
    p->off.assign(layer_off, layer_off + n_layers);
    p->bytes.assign(layer_bytes, layer_bytes + n_layers);
    p->steps.assign(steps, steps + (size_t)n_layers * steps_per_layer);
    p->L = n_layers;
    p->S = steps_per_layer;
    p->max_b = max_b;
    p->slot_bytes = slot_bytes;
    hipError_t e = hipSuccess;
    for (int s = 0; s < 2 && e == hipSuccess; ++s) {
        e = hipMalloc((void**)&p->slot[s], (size_t)slot_bytes);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&p->copied[s], hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&p->released[s], hipEventDisableTiming);
    }
    if (e != hipSuccess) {
        int rc = hip_status(e);
        release(p);
        return rc;
    }
    *out = p;
    return WOQ_OK;
}

int woq_pager_run(woq_pager* p, const uint16_t* const* inputs, uint16_t* const* outputs, int64_t b,
                  void* compute_stream, void* copy_stream) {
    if (!p || !inputs || !outputs || b < 1 || b > p->max_b || compute_stream == copy_stream) return WOQ_EINVAL;
    hipStream_t cs = (hipStream_t)compute_stream, xs = (hipStream_t)copy_stream;
    // A slot may still be read by the previous pass: the copy stream starts
    // after everything already queued on the compute stream.
    hipEvent_t start = p->released[0];
    hipError_t e = hipEventRecord(start, cs);
    if (e == hipSuccess) e = hipStreamWaitEvent(xs, start, 0);
    if (e != hipSuccess) return hip_status(e);
    auto issue_copy = [&](int l) -> hipError_t {
        const int s = l & 1;
        hipError_t r = hipSuccess;
        if (l >= 2) r = hipStreamWaitEvent(xs, p->released[s], 0);
        if (r == hipSuccess)
            r = hipMemcpyAsync(p->slot[s], p->pool + p->off[l], (size_t)p->bytes[l], hipMemcpyHostToDevice, xs);
        if (r == hipSuccess) r = hipEventRecord(p->copied[s], xs);
        return r;
    };
    e = issue_copy(0);
    if (e == hipSuccess && p->L > 1) e = issue_copy(1);
    if (e != hipSuccess) return hip_status(e);
    for (int l = 0; l < p->L; ++l) {
        const int s = l & 1;
        e = hipStreamWaitEvent(cs, p->copied[s], 0);
        if (e != hipSuccess) return hip_status(e);
        for (int k = 0; k < p->S; ++k) {
            const size_t i = (size_t)l * p->S + k;
            woq_int8_w w = p->steps[i].w;
            w.codes = p->slot[s] + p->steps[i].code_offset;
            int rc = woq_qgemv_int8(&w, inputs[i], w.K, b, outputs[i], w.N, compute_stream);
            if (rc) return rc;
        }
        e = hipEventRecord(p->released[s], cs);
        // slot s is refilled with layer l + 2 once these products are done
        if (e == hipSuccess && l + 2 < p->L) e = issue_copy(l + 2);
        if (e != hipSuccess) return hip_status(e);
    }
    return WOQ_OK;
}

int woq_pager_destroy(woq_pager* p) {
    if (p) release(p);
    return WOQ_OK;
}

}  // extern "C"
