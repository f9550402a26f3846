// Tiered decode pass: resident layers (tier A) run out of device memory,
// streamed layers (tier B) out of two device slots that a copy stream fills
// from pinned host memory.
//
// Streamed layer j (the j-th streamed layer in layer order) uses slot j mod 2.
// While the products of streamed layer j run on the compute stream, the copy
// stream fills the other slot with streamed layer j + 1; the resident layers in
// between run meanwhile.  Events order the two streams both ways:
//   copied[s]    copy of the layer now in slot s has landed  -> products may start
//   released[s]  products of the layer in slot s are done     -> slot may be refilled
// The products themselves are launched through the stack runner (the same
// kernels, permutation folding and workspace as woq_stack_run).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <new>
#include <vector>

#include "woq_internal.h"

struct woq_pager {
    const uint8_t* pool = nullptr;
    std::vector<int64_t> off, bytes;          // bytes[l] == 0: layer l is resident
    std::vector<woq_stack_step> steps;        // steps_per_layer per layer, as given
    std::vector<int32_t> streamed;            // indices of the streamed layers, in order
    int32_t L = 0, S = 0;
    int64_t max_b = 0;
    int64_t slot_bytes = 0;
    woq_stack* stack = nullptr;               // launches the products; owns the workspace
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
    if (p->stack) (void)woq_stack_destroy(p->stack);
    delete p;
}

// [off, off + len) inside a block of `bytes`, 16-byte aligned.
bool in_block(int64_t off, int64_t len, int64_t bytes) {
    return off >= 0 && (off & 15) == 0 && len >= 0 && off <= bytes && len <= bytes - off;
}

// A streamed step's weight pointers hold byte offsets into its layer's block.
bool streamed_step_fits(const woq_stack_step& s, int64_t bytes) {
    if (s.fmt == WOQ_FMT_INT8)
        return in_block((int64_t)(uintptr_t)s.w8.codes, woq_int8_dev_bytes(s.w8.N, s.w8.K), bytes);
    if (s.fmt != WOQ_FMT_INT4O) return false;
    int64_t cb = 0, sb = 0, wb = 0;
    if (woq_int4o_dev_sizes(s.w4.N, &s.w4.geom, &cb, &sb, &wb) != WOQ_OK) return false;
    return in_block((int64_t)(uintptr_t)s.w4.codes, cb, bytes) && in_block((int64_t)(uintptr_t)s.w4.scales, sb, bytes) &&
           (wb == 0 || in_block((int64_t)(uintptr_t)s.w4.w_out, wb, bytes));
}

woq_stack_step in_slot(const woq_stack_step& s, const uint8_t* base) {
    woq_stack_step t = s;
    if (s.fmt == WOQ_FMT_INT8) {
        t.w8.codes = base + (uintptr_t)s.w8.codes;
    } else {
        t.w4.codes = base + (uintptr_t)s.w4.codes;
        t.w4.scales = base + (uintptr_t)s.w4.scales;
        t.w4.w_out = base + (uintptr_t)s.w4.w_out;   // not read when the space has no outliers
    }
    return t;
}

}  // namespace

extern "C" {

int woq_plan_tiers(const int64_t* layer_bytes, int32_t n_layers, int64_t budget_bytes, int32_t* resident,
                   int64_t* device_bytes) {
    if (!layer_bytes || n_layers < 0 || !resident || budget_bytes < 0) return WOQ_EINVAL;
    for (int l = 0; l < n_layers; ++l)
        if (layer_bytes[l] < 1) return WOQ_EINVAL;
    // suffix maxima: the slot size if layers n.. stream
    std::vector<int64_t> smax((size_t)n_layers + 1, 0);
    for (int l = n_layers - 1; l >= 0; --l) smax[l] = std::max(smax[l + 1], layer_bytes[l]);
    int64_t prefix = 0;
    int best = -1;
    int64_t best_bytes = 0;
    for (int n = 0; n <= n_layers; ++n) {
        if (n > 0) prefix += layer_bytes[n - 1];
        const int64_t need = prefix + (n < n_layers ? 2 * smax[n] : 0);
        if (need <= budget_bytes) {
            best = n;
            best_bytes = need;
        }
    }
    if (best < 0) return WOQ_ENOMEM;
    for (int l = 0; l < n_layers; ++l) resident[l] = l < best ? 1 : 0;
    if (device_bytes) *device_bytes = best_bytes;
    return WOQ_OK;
}

int woq_tiered_create(const void* pinned_pool, const int64_t* layer_off, const int64_t* layer_bytes,
                      int32_t n_layers, const woq_stack_step* steps, int32_t steps_per_layer, int64_t max_b,
                      woq_pager** out) {
    if (!out) return WOQ_EINVAL;
    *out = nullptr;
    if (!layer_off || !layer_bytes || n_layers < 1 || !steps || steps_per_layer < 1 || max_b < 1) return WOQ_EINVAL;
    int64_t slot_bytes = 0;
    bool any_streamed = false;
    for (int l = 0; l < n_layers; ++l) {
        if (layer_bytes[l] < 0) return WOQ_EINVAL;
        if (layer_bytes[l] == 0) continue;
        any_streamed = true;
        if (layer_off[l] < 0) return WOQ_EINVAL;
        slot_bytes = std::max(slot_bytes, layer_bytes[l]);
        for (int s = 0; s < steps_per_layer; ++s)
            if (!streamed_step_fits(steps[(size_t)l * steps_per_layer + s], layer_bytes[l])) return WOQ_EINVAL;
    }
    if (any_streamed && !pinned_pool) return WOQ_EINVAL;
    woq_pager* p = new (std::nothrow) woq_pager;
    if (!p) return WOQ_ENOMEM;
    p->pool = (const uint8_t*)pinned_pool;
    p->off.assign(layer_off, layer_off + n_layers);
    p->bytes.assign(layer_bytes, layer_bytes + n_layers);
    p->steps.assign(steps, steps + (size_t)n_layers * steps_per_layer);
    for (int l = 0; l < n_layers; ++l)
        if (layer_bytes[l] > 0) p->streamed.push_back(l);
    p->L = n_layers;
    p->S = steps_per_layer;
    p->max_b = max_b;
    p->slot_bytes = slot_bytes;
    // the stack validates the steps, builds the channel-position tables and
    // the permutation workspace; its weight pointers are never dereferenced
    // for streamed layers (each launch gets a copy pointing into a slot)
    int rc = woq_stack_create(p->steps.data(), (int32_t)p->steps.size(), max_b, &p->stack);
    if (rc != WOQ_OK) {
        p->stack = nullptr;
        release(p);
        return rc;
    }
    hipError_t e = hipSuccess;
    for (int s = 0; s < 2 && e == hipSuccess && any_streamed; ++s) {
        e = hipMalloc((void**)&p->slot[s], (size_t)slot_bytes);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&p->copied[s], hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&p->released[s], hipEventDisableTiming);
    }
    if (e != hipSuccess) {
        rc = hip_status(e);
        release(p);
        return rc;
    }
    *out = p;
    return WOQ_OK;
}

int woq_pager_create(const void* pinned_pool, const int64_t* layer_off, const int64_t* layer_bytes,
                     int32_t n_layers, const woq_pager_step* steps, int32_t steps_per_layer, int64_t max_b,
                     woq_pager** out) {
    if (!out) return WOQ_EINVAL;
    *out = nullptr;
    if (!pinned_pool || !layer_off || !layer_bytes || n_layers < 1 || !steps || steps_per_layer < 1 || max_b < 1 ||
        max_b > 8)
        return WOQ_EINVAL;
    std::vector<woq_stack_step> st((size_t)n_layers * steps_per_layer);
    for (int l = 0; l < n_layers; ++l) {
        if (layer_bytes[l] < 1) return WOQ_EINVAL;
        for (int s = 0; s < steps_per_layer; ++s) {
            const size_t i = (size_t)l * steps_per_layer + s;
            const woq_int8_w& w = steps[i].w;
            if (w.N < 1 || w.K < 1 || w.nseg < 1 || w.nseg > WOQ_MAX_SEGMENTS || w.seg_end[w.nseg - 1] != w.N ||
                steps[i].code_offset < 0)
                return WOQ_EINVAL;
            woq_stack_step& t = st[i];
            t = woq_stack_step{};
            t.fmt = WOQ_FMT_INT8;
            t.in_slot = t.out_slot = (int32_t)i;
            t.w8 = w;
            t.w8.codes = (const void*)(uintptr_t)steps[i].code_offset;
        }
    }
    return woq_tiered_create(pinned_pool, layer_off, layer_bytes, n_layers, st.data(), steps_per_layer, max_b, out);
}

}  // extern "C"

namespace {

// One pass; with cev (3 events per streamed layer) the copy stream records,
// for streamed layer j, cev[3j] before its wait for the slot, cev[3j + 1]
// when that wait is over (the copy starts) and cev[3j + 2] when the copy has
// landed.
int pager_pass(woq_pager* p, const uint16_t* const* inputs, uint16_t* const* outputs, int64_t b,
               void* compute_stream, void* copy_stream, hipEvent_t* cev) {
    if (!p || !inputs || !outputs || b < 1 || b > p->max_b) return WOQ_EINVAL;
    const int nB = (int)p->streamed.size();
    if (nB > 0 && compute_stream == copy_stream) return WOQ_EINVAL;
    hipStream_t cs = (hipStream_t)compute_stream, xs = (hipStream_t)copy_stream;
    hipError_t e = hipSuccess;
    auto issue_copy = [&](int j) -> hipError_t {
        const int s = j & 1, l = p->streamed[j];
        hipError_t r = hipSuccess;
        if (cev) r = hipEventRecord(cev[3 * j], xs);
        if (r == hipSuccess && j >= 2) r = hipStreamWaitEvent(xs, p->released[s], 0);
        if (r == hipSuccess && cev) r = hipEventRecord(cev[3 * j + 1], xs);
        if (r == hipSuccess)
            r = hipMemcpyAsync(p->slot[s], p->pool + p->off[l], (size_t)p->bytes[l], hipMemcpyHostToDevice, xs);
        if (r == hipSuccess) r = hipEventRecord(p->copied[s], xs);
        if (r == hipSuccess && cev) r = hipEventRecord(cev[3 * j + 2], xs);
        return r;
    };
    if (nB > 0) {
        // A slot may still be read by the previous pass: the copy stream starts
        // after everything already queued on the compute stream.
        e = hipEventRecord(p->released[0], cs);
        if (e == hipSuccess) e = hipStreamWaitEvent(xs, p->released[0], 0);
        if (e == hipSuccess) e = issue_copy(0);
        if (e == hipSuccess && nB > 1) e = issue_copy(1);
        if (e != hipSuccess) return hip_status(e);
    }
    int j = 0;   // streamed layers seen so far
    for (int l = 0; l < p->L; ++l) {
        const bool streamed = p->bytes[l] > 0;
        const int s = j & 1;
        if (streamed) {
            e = hipStreamWaitEvent(cs, p->copied[s], 0);
            if (e != hipSuccess) return hip_status(e);
        }
        for (int k = 0; k < p->S; ++k) {
            const int64_t i = (int64_t)l * p->S + k;
            const woq_stack_step& st = p->steps[(size_t)i];
            woq_stack_step t = streamed ? in_slot(st, p->slot[s]) : st;
            int rc = woq::stack_run_step(p->stack, i, &t, inputs[st.in_slot], outputs[st.out_slot], b,
                                         compute_stream);
            if (rc) return rc;
        }
        if (streamed) {
            e = hipEventRecord(p->released[s], cs);
            // slot s is refilled with streamed layer j + 2 once these products are done
            if (e == hipSuccess && j + 2 < nB) e = issue_copy(j + 2);
            if (e != hipSuccess) return hip_status(e);
            ++j;
        }
    }
    return WOQ_OK;
}

}  // namespace

extern "C" {

int woq_pager_run(woq_pager* p, const uint16_t* const* inputs, uint16_t* const* outputs, int64_t b,
                  void* compute_stream, void* copy_stream) {
    return pager_pass(p, inputs, outputs, b, compute_stream, copy_stream, nullptr);
}

int woq_pager_streamed_layers(const woq_pager* p, int32_t* n) {
    if (!p || !n) return WOQ_EINVAL;
    *n = (int32_t)p->streamed.size();
    return WOQ_OK;
}

int woq_pager_time(woq_pager* p, const uint16_t* const* inputs, uint16_t* const* outputs, int64_t b,
                   void* compute_stream, void* copy_stream, float* wait_ms, float* copy_ms, float* end_ms,
                   float* pass_ms) {
    if (!p || !pass_ms) return WOQ_EINVAL;
    const int nB = (int)p->streamed.size();
    if (nB > 0 && (!wait_ms || !copy_ms || !end_ms)) return WOQ_EINVAL;
    hipStream_t cs = (hipStream_t)compute_stream;
    std::vector<hipEvent_t> ev(3 * (size_t)nB + 2, nullptr);
    hipError_t e = hipSuccess;
    for (auto& x : ev)
        if (e == hipSuccess) e = hipEventCreate(&x);
    hipEvent_t* pass = ev.data() + 3 * (size_t)nB;
    int rc = WOQ_OK;
    // the pass's start on the compute stream: the copy stream starts behind it
    if (e == hipSuccess) e = hipEventRecord(pass[0], cs);
    if (e == hipSuccess) rc = pager_pass(p, inputs, outputs, b, compute_stream, copy_stream, ev.data());
    if (e == hipSuccess && rc == WOQ_OK) e = hipEventRecord(pass[1], cs);
    if (e == hipSuccess && rc == WOQ_OK) e = hipStreamSynchronize(cs);
    if (e == hipSuccess && rc == WOQ_OK && nB > 0) e = hipStreamSynchronize((hipStream_t)copy_stream);
    for (int j = 0; j < nB && e == hipSuccess && rc == WOQ_OK; ++j) {
        e = hipEventElapsedTime(&wait_ms[j], pass[0], ev[3 * j]);
        if (e == hipSuccess) e = hipEventElapsedTime(&copy_ms[j], pass[0], ev[3 * j + 1]);
        if (e == hipSuccess) e = hipEventElapsedTime(&end_ms[j], pass[0], ev[3 * j + 2]);
    }
    if (e == hipSuccess && rc == WOQ_OK) e = hipEventElapsedTime(pass_ms, pass[0], pass[1]);
    for (auto& x : ev)
        if (x) (void)hipEventDestroy(x);
    if (rc) return rc;
    return hip_status(e);
}

int woq_pager_destroy(woq_pager* p) {
    if (p) release(p);
    return WOQ_OK;
}

}  // extern "C"
