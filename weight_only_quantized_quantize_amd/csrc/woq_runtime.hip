// Decode-stack runner: drives a sequence of quantised linears on one stream.
//
// A decode step walks the layers in order; within a layer, linears that read
// the same activation (q|k|v, gate|up) are stacked along N into one product.
//
// A pass (woq_stack_run) is one launch per product, stream-ordered: each
// product starts after the previous one has finished, as a real decode chain
// (every product reads the output of the one before) requires.  An INT4O
// product folds its input permutation into the launch where the vector kernel
// serves it; otherwise a permutation launch precedes it (and a reduction
// launch follows a split-K product).
#include <hip/hip_runtime.h>

#include <new>
#include <vector>

#include "woq_internal.h"

struct woq_stack {
    std::vector<woq_stack_step> steps;
    int64_t max_b = 0;
    int64_t xp_elems = 0;      // per workspace row
    uint16_t* xp = nullptr;    // [max_b][xp_elems]
    float* part = nullptr;     // split-K partial sums of the long-row INT4O products
    int64_t part_bytes = 0;
    int device = 0;
    // INT4O: device channel-position table of each step's permutation (null
    // where the row is too long for 16-bit positions); one table per distinct
    // permutation, owned here
    std::vector<const uint16_t*> pos;
    std::vector<uint16_t*> pos_owned;
};

namespace {

int hip_status(hipError_t e) {
    if (e == hipSuccess) return WOQ_OK;
    woq::set_hip_error((int)e);
    return e == hipErrorOutOfMemory ? WOQ_ENOMEM : WOQ_EHIP;
}

// Every device buffer the runner owns, released in one place (the failure
// path of woq_stack_create and woq_stack_destroy).  Returns the first HIP
// error, if any; the runner is deleted either way.
hipError_t free_stack(woq_stack* st) {
    hipError_t first = hipSuccess;
    auto release = [&](void* p) {
        if (!p) return;
        hipError_t e = hipFree(p);
        if (first == hipSuccess) first = e;
    };
    release(st->xp);
    release(st->part);
    for (uint16_t* p : st->pos_owned) release(p);
    delete st;
    return first;
}

// Channel-position tables of the INT4O steps' permutations (read back from
// the device once; an invalid permutation is rejected here).
int make_positions(woq_stack* st) {
    st->pos.assign(st->steps.size(), nullptr);
    for (size_t i = 0; i < st->steps.size(); ++i) {
        const woq_stack_step& s = st->steps[i];
        if (s.fmt != WOQ_FMT_INT4O || s.w4.geom.xp_len > 65535) continue;
        for (size_t j = 0; j < i && !st->pos[i]; ++j) {
            const woq_stack_step& t = st->steps[j];
            if (st->pos[j] && t.perm == s.perm && t.w4.geom.K == s.w4.geom.K && t.w4.geom.n_out == s.w4.geom.n_out)
                st->pos[i] = st->pos[j];
        }
        if (st->pos[i]) continue;
        const int64_t K = s.w4.geom.K, K8 = woq::round_up(K, 8);
        std::vector<int32_t> perm((size_t)K);
        std::vector<uint16_t> pos((size_t)K8);
        hipError_t e = hipMemcpy(perm.data(), s.perm, sizeof(int32_t) * K, hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_status(e);
        int rc = woq_perm_positions(perm.data(), &s.w4.geom, pos.data());
        if (rc) return rc;
        uint16_t* d = nullptr;
        e = hipMalloc((void**)&d, sizeof(uint16_t) * K8);
        if (e != hipSuccess) return hip_status(e);
        st->pos_owned.push_back(d);
        e = hipMemcpy(d, pos.data(), sizeof(uint16_t) * K8, hipMemcpyHostToDevice);
        if (e != hipSuccess) return hip_status(e);
        st->pos[i] = d;
    }
    return WOQ_OK;
}

// Every step that runs the vector kernel folds the permutation into the
// product (one launch instead of two): each workgroup gathers the whole
// activation row into LDS while its first weights are in flight.  Measured on
// MI355X over the 70B-shaped layer, folding every product, the 57344-row
// gate|up and the 28672-channel down included, against folding only rows of
// up to 16384 x 8704 channels (the earlier rule): 109-112 -> 102 us per layer
// at b = 1 and 138-142 -> 131 us at b = 2 with a timing event around each
// launch; the whole 80-layer step without events went from 7.20 to 7.17 ms.
//
// Where the matrix-core kernel serves the batch (b <= 8), rows of 64 groups
// or more whose permuted row fits on chip fold it the same way
// (woq_qgemm_int4o_x: each workgroup gathers the row of its 8 staged columns
// instead of staging the permuted copy chunk by chunk).
// 0: a permutation launch before the product; 1: folded into the vector
// kernel; 2: folded into the matrix-core kernel.
int fold_permutation(const woq_stack_step& s, int64_t b) {
    const woq_int4o_geom& g = s.w4.geom;
    if ((g.K & 7) != 0) return 0;
    if (woq::int4o_use_valu(s.w4.N, g, b)) return woq_qgemv_int4o_x_supported(&g, b) ? 1 : 0;
    if (woq::int4o_splitk(s.w4.N, g, b)) return 0;
    return woq_qgemm_int4o_x_supported(&g, s.w4.N, b) ? 2 : 0;
}

// One step (the step table's entry i, or a copy of it whose weight pointers
// were moved, e.g. into a pager slot); ev (2 entries, or null) brackets every
// launch of the step: the first launch records ev[0] at its start, the last
// records ev[1] at its end.
int run_step(woq_stack* st, size_t i, const woq_stack_step& s, const uint16_t* x, uint16_t* y, int64_t b,
             void* stream, hipEvent_t* ev) {
    struct Bracket {
        explicit Bracket(hipEvent_t* e) : on(e != nullptr) {
            if (on) woq::set_launch_events(e[0], e[1]);
        }
        ~Bracket() {
            if (on) woq::set_launch_events(nullptr, nullptr);
        }
        bool on;
    } bracket(ev);
    if (s.fmt == WOQ_FMT_INT4O && st->pos[i] && woq::aligned16(x)) {
        // permutation folded into the product: one launch
        const int fold = fold_permutation(s, b);
        if (fold == 1) return woq_qgemv_int4o_x(&s.w4, x, s.w4.geom.K, st->pos[i], b, y, s.w4.N, stream);
        if (fold == 2) return woq_qgemm_int4o_x(&s.w4, x, s.w4.geom.K, st->pos[i], b, y, s.w4.N, stream);
    }
    if (s.fmt == WOQ_FMT_INT8) return woq_qgemv_int8(&s.w8, x, s.w8.K, b, y, s.w8.N, stream);
    int rc = woq_permute_x(x, s.w4.geom.K, s.perm, b, &s.w4.geom, st->xp, stream);
    if (rc) return rc;
    const int splits = woq::int4o_splitk(s.w4.N, s.w4.geom, b);
    if (splits) return woq_qgemm_int4o_splitk(&s.w4, st->xp, b, y, s.w4.N, splits, st->part, st->part_bytes, stream);
    return woq_qgemv_int4o(&s.w4, st->xp, b, y, s.w4.N, stream);
}

// One pass over the steps; ev (2 per step) brackets each step's launches.
int run_pass(woq_stack* st, const uint16_t* const* inputs, uint16_t* const* outputs, int64_t b, void* stream,
             hipEvent_t* ev) {
    for (size_t i = 0; i < st->steps.size(); ++i) {
        const woq_stack_step& s = st->steps[i];
        int rc = run_step(st, i, s, inputs[s.in_slot], outputs[s.out_slot], b, stream, ev ? ev + 2 * i : nullptr);
        if (rc) return rc;
    }
    return WOQ_OK;
}

// A kernel that does nothing: its duration between the dispatch-boundary
// events is the time any launch costs before and after its own work.
__global__ void empty_kernel() {}

}  // namespace

namespace woq {

int stack_run_step(woq_stack* st, int64_t i, const woq_stack_step* s, const uint16_t* x, uint16_t* y, int64_t b,
                   void* stream) {
    if (!st || !s || i < 0 || i >= (int64_t)st->steps.size() || b < 1 || b > st->max_b) return WOQ_EINVAL;
    return run_step(st, (size_t)i, *s, x, y, b, stream, nullptr);
}

}  // namespace woq

extern "C" {

int woq_stack_create(const woq_stack_step* steps, int32_t n_steps, int64_t max_b, woq_stack** out) {
    if (!out || n_steps < 0 || (n_steps > 0 && !steps) || max_b < 1 || max_b > 64) return WOQ_EINVAL;
    *out = nullptr;
    int64_t xp_elems = 8;
    for (int i = 0; i < n_steps; ++i) {
        const woq_stack_step& s = steps[i];
        if (s.in_slot < 0 || s.out_slot < 0) return WOQ_EINVAL;
        if (s.fmt == WOQ_FMT_INT4O) {
            if (!woq::int4o_geom_valid(&s.w4.geom) || !s.perm) return WOQ_EINVAL;
            xp_elems = std::max(xp_elems, s.w4.geom.xp_len);
        } else if (s.fmt == WOQ_FMT_INT8) {
            if (max_b > 8) return WOQ_EUNSUPPORTED;
            if (s.w8.nseg < 1 || s.w8.nseg > WOQ_MAX_SEGMENTS || s.w8.K < 1) return WOQ_EINVAL;
        } else {
            return WOQ_EINVAL;
        }
    }
    woq_stack* st = new (std::nothrow) woq_stack;
    if (!st) return WOQ_ENOMEM;
    st->steps.assign(steps, steps + n_steps);
    st->max_b = max_b;
    st->xp_elems = xp_elems;
    for (int i = 0; i < n_steps; ++i) {
        const woq_stack_step& s = steps[i];
        if (s.fmt != WOQ_FMT_INT4O) continue;
        for (int64_t bb = 1; bb <= max_b; ++bb) {
            const int sp = woq::int4o_splitk(s.w4.N, s.w4.geom, bb);
            if (sp) st->part_bytes = std::max(st->part_bytes, woq_qgemm_int4o_splitk_workspace(s.w4.N, bb, sp));
        }
    }
    hipError_t e = hipGetDevice(&st->device);
    if (e == hipSuccess) e = hipMalloc((void**)&st->xp, (size_t)(max_b * xp_elems * 2));
    if (e == hipSuccess && st->part_bytes > 0) e = hipMalloc((void**)&st->part, (size_t)st->part_bytes);
    int rc = hip_status(e);
    if (rc == WOQ_OK) rc = make_positions(st);
    if (rc != WOQ_OK) {
        (void)free_stack(st);
        return rc;
    }
    *out = st;
    return WOQ_OK;
}

int woq_stack_launches(const woq_stack* st, int64_t b, int32_t* launches) {
    if (!st || !launches || b < 1 || b > st->max_b) return WOQ_EINVAL;
    int32_t n = 0;
    for (size_t i = 0; i < st->steps.size(); ++i) {
        const woq_stack_step& s = st->steps[i];
        n += (s.fmt == WOQ_FMT_INT4O && !(st->pos[i] && fold_permutation(s, b) != 0)) ? 2 : 1;
        if (s.fmt == WOQ_FMT_INT4O && woq::int4o_splitk(s.w4.N, s.w4.geom, b)) n += 1;   // the reduction
    }
    *launches = n;
    return WOQ_OK;
}

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
        if (x) (void)hipEventDestroy(x);
    if (rc) return rc;
    return hip_status(e);
}

int woq_dispatch_floor(int32_t blocks, int32_t threads, int32_t iters, void* stream, float* span_us,
                       float* interval_us) {
    if (blocks < 1 || threads < 1 || threads > 1024 || iters < 1 || iters > 100000 || !span_us || !interval_us)
        return WOQ_EINVAL;
    std::vector<hipEvent_t> ev(2 * (size_t)iters + 2, nullptr);
    hipError_t e = hipSuccess;
    for (auto& x : ev)
        if (e == hipSuccess) e = hipEventCreate(&x);
    hipStream_t hs = (hipStream_t)stream;
    const dim3 grid((unsigned)blocks), block((unsigned)threads);
    // each launch between its own dispatch-boundary events
    for (int it = 0; it < iters && e == hipSuccess; ++it)
        e = hipExtLaunchKernel((const void*)&empty_kernel, grid, block, nullptr, 0, hs, ev[2 * it], ev[2 * it + 1], 0);
    // the same launches back to back, one pair of events around all of them
    hipEvent_t* outer = ev.data() + 2 * (size_t)iters;
    if (e == hipSuccess) e = hipEventRecord(outer[0], hs);
    for (int it = 0; it < iters && e == hipSuccess; ++it)
        e = hipLaunchKernel((const void*)&empty_kernel, grid, block, nullptr, 0, hs);
    if (e == hipSuccess) e = hipEventRecord(outer[1], hs);
    if (e == hipSuccess) e = hipStreamSynchronize(hs);
    double total = 0.0;
    for (int it = 0; it < iters && e == hipSuccess; ++it) {
        float ms = 0.0f;
        e = hipEventElapsedTime(&ms, ev[2 * it], ev[2 * it + 1]);
        total += ms;
    }
    float all_ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&all_ms, outer[0], outer[1]);
    if (e == hipSuccess) {
        *span_us = (float)(1e3 * total / iters);
        *interval_us = (float)(1e3 * all_ms / iters);
    }
    for (auto& x : ev)
        if (x) (void)hipEventDestroy(x);
    return hip_status(e);
}

int woq_stack_destroy(woq_stack* st) {
    if (!st) return WOQ_OK;
    return hip_status(free_stack(st));
}

}  // extern "C"
