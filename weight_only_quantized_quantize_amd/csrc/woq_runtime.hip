// Decode-stack runner: drives a sequence of quantised linears on one stream.
//
// A decode step walks the layers in order; within a layer, linears that read
// the same activation (q|k|v, gate|up) are stacked along N into one product.
//
// Two ways to run a pass:
//  * woq_stack_run: one launch per permutation and per product, stream-ordered.
//  * woq_stack_run_fused (INT8 stacks): one persistent launch for the whole
//    pass.  On this hardware a dependent launch costs several microseconds,
//    comparable to the time it takes to stream one decode linear, so the fused
//    pass keeps every workgroup resident and separates steps with a
//    device-side barrier.
#include <hip/hip_runtime.h>

#include <cstring>
#include <new>
#include <vector>

#include "woq_gemv.cuh"
#include "woq_internal.h"

namespace {

using namespace woqk;

// An INT8 step as the persistent kernel sees it (device memory, read-only).
struct DevStep {
    const uint4* codes;
    const uint16_t* x;
    uint16_t* y;
    int N, CPR, nchunks, xlen, K, ldx, ldy, nseg;
    int seg_end[WOQ_MAX_SEGMENTS];
    float seg_scale[WOQ_MAX_SEGMENTS];
};

// Barrier state: one 128-byte line per counter.
constexpr int SYNC_LINE = 16;                 // uint64 per line
constexpr int SYNC_GROUPS = 16;
constexpr int SYNC_GROUP0 = 1, SYNC_DEPART = 1 + SYNC_GROUPS, SYNC_ERR = 2 + SYNC_GROUPS;   // line 0 unused
constexpr int SYNC_WORDS = (3 + SYNC_GROUPS) * SYNC_LINE;
constexpr int FUSED_THREADS = 512;
// polls of s_sleep(2) before a barrier is declared stuck (far above any step)
constexpr unsigned SPIN_LIMIT = 1u << 24;

typedef unsigned long long u64;

__device__ __forceinline__ u64 ld_relaxed(u64* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_relaxed(u64* p, u64 v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ u64 add_relaxed(u64* p, u64 v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// register window of weight items per wave (narrower for wide batches, which
// need the registers for activations and accumulators)
template <int B>
constexpr int prefetch_items_for() { return B <= 4 ? 4 : 2; }
// Items per wave issued before a step boundary.  The barrier's own atomics
// queue behind outstanding loads in the memory system, so only about what
// drains within one barrier latency is issued early (about 1 item per wave,
// 4 KB: ~7 MB over the chip); the rest of the window follows the barrier.
constexpr int EARLY_ITEMS = 1;
constexpr int PREFETCH_SRC = 18;    // staged activation sources per thread resolved before a barrier

__device__ __forceinline__ QuadTask make_task(const DevStep& st, int gw, int NW) {
    QuadTask t;
    t.codes = st.codes;
    t.CPR = st.CPR;
    t.nchunks = st.nchunks;
    t.IT = (t.nchunks + 63) >> 6;
    const int quads = (st.N + 3) >> 2;
    t.q0 = gw;
    t.qstride = NW;
    t.nq = gw < quads ? (quads - 1 - gw) / NW + 1 : 0;
    return t;
}

// Source index in the activation row of staged element k (-1: zero padding).
__device__ __forceinline__ int stage_src(const DevStep& st, int k) { return k < st.K ? k : -1; }

template <int B, int U>
__device__ __forceinline__ void fused_step(const DevStep& st, const QuadTask& task, Slots<U>& slots,
                                           const int (&src)[PREFETCH_SRC], uint16_t* xs, int tid, int lane) {
    const int xlen = st.xlen;
    // Stage activations.  The loads are unconditional (padding reads element 0
    // and is replaced by zero afterwards), so they are all in flight at once and
    // the step waits for one memory round trip.
    uint16_t v[PREFETCH_SRC][B];
#pragma unroll
    for (int i = 0; i < PREFETCH_SRC; ++i)
#pragma unroll
        for (int b = 0; b < B; ++b) v[i][b] = *gptr(st.x + (int64_t)b * st.ldx + (src[i] >= 0 ? src[i] : 0));
#pragma unroll
    for (int i = 0; i < PREFETCH_SRC; ++i) {
        const int k = tid + i * FUSED_THREADS;
        if (k < xlen)
#pragma unroll
            for (int b = 0; b < B; ++b) xs[b * xlen + k] = src[i] >= 0 ? v[i][b] : (uint16_t)0;
    }
    for (int k = tid + PREFETCH_SRC * FUSED_THREADS; k < xlen; k += FUSED_THREADS) {
        const int sk = stage_src(st, k);
        for (int b = 0; b < B; ++b) xs[b * xlen + k] = sk >= 0 ? *gptr(st.x + (int64_t)b * st.ldx + sk) : (uint16_t)0;
    }
    lds_barrier();
    stream_task<B, U>(task, slots, (lx_ptr)xs, xlen, lane, EARLY_ITEMS, [&](int q, float out) {
        if (lane < 4 * B) {
            const int r = lane / B, b = lane % B, n = 4 * q + r;
            if (n < st.N) {
                float scale = st.seg_scale[st.nseg - 1];
                for (int i = st.nseg - 1; i >= 0; --i)
                    if (n < st.seg_end[i]) scale = st.seg_scale[i];
                *gptr(st.y + (int64_t)b * st.ldy + n) = f_to_h(out * scale);
            }
        }
    });
}

template <int U>
__device__ __forceinline__ void prefetch_step(const DevStep& st, const QuadTask& task, Slots<U>& slots,
                                              int (&src)[PREFETCH_SRC], int tid, int lane) {
    prefetch_items<U>(task, lane, slots, 0, EARLY_ITEMS);
#pragma unroll
    for (int i = 0; i < PREFETCH_SRC; ++i) {
        const int k = tid + i * FUSED_THREADS;
        src[i] = k < st.xlen ? stage_src(st, k) : -1;
    }
}

template <int B>
__global__ __launch_bounds__(FUSED_THREADS) void stack_fused(const DevStep* __restrict__ steps, int nsteps, u64* sync) {
    extern __shared__ __align__(16) uint16_t xs[];   // [B][xlen] staged activations
    __shared__ int stuck_flag;
    constexpr int U = prefetch_items_for<B>();
    const int tid = threadIdx.x, lane = tid & 63;
    // consecutive quads go to different workgroups first, so a small step
    // spreads over every compute unit
    const int gw = (tid >> 6) * gridDim.x + blockIdx.x;
    const int NW = gridDim.x * (FUSED_THREADS / 64);
    const unsigned P = gridDim.x;
    const unsigned ng = P < (unsigned)SYNC_GROUPS ? P : (unsigned)SYNC_GROUPS;
    const unsigned g = blockIdx.x % ng;
    u64* grp = sync + (SYNC_GROUP0 + g) * SYNC_LINE;
    u64* err = sync + SYNC_ERR * SYNC_LINE;

    Slots<U> slots;
    int src[PREFETCH_SRC];
    QuadTask task = make_task(steps[0], gw, NW);
    prefetch_step<U>(steps[0], task, slots, src, tid, lane);
    bool ok = true;
    for (int si = 0; si < nsteps && ok; ++si) {
        fused_step<B, U>(steps[si], task, slots, src, xs, tid, lane);
        // every wave of this workgroup has finished the step's products and its
        // LDS reads (its output stores may still be in flight: nothing reads them)
        lds_barrier();
        if (si + 1 < nsteps) {
            // The last wave arrives and waits; the other waves issue the next
            // step's weight and index loads first, so those travel while the
            // workgroups finish.  (The polling wave issues its own loads after
            // the wait: vector loads return in order, and an earlier prefetch
            // would hold back every poll.)  Steps only order computation (no step
            // reads another step's outputs), so the counters are relaxed atomics
            // without fences.
            const u64 j = (u64)(si + 1);
            constexpr int POLLER = FUSED_THREADS - 64;
            task = make_task(steps[si + 1], gw, NW);
            int stuck = 0;
            if (tid < POLLER) {
                prefetch_step<U>(steps[si + 1], task, slots, src, tid, lane);
            } else {
                // Arrive with a fire-and-forget add to this workgroup's group
                // counter; lane g then watches group counter g, so the release is
                // seen one memory round trip after the last arrival.
                if (tid == POLLER) add_relaxed(grp, 1ull);
                const unsigned lg = (unsigned)lane;
                const u64 want = lg < ng ? j * (P / ng + (lg < P % ng ? 1 : 0)) : 0;
                u64* mine = sync + (SYNC_GROUP0 + (lg < ng ? lg : 0)) * SYNC_LINE;
                unsigned n = 0;
                for (;;) {
                    const u64 have = lg < ng ? ld_relaxed(mine) : 0;
                    if (__ballot(have < want) == 0) break;
                    if (ld_relaxed(err)) {
                        stuck = 1;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                    if (++n > SPIN_LIMIT) {
                        if (tid == POLLER) st_relaxed(err, 1ull);
                        stuck = 1;
                        break;
                    }
                }
                prefetch_step<U>(steps[si + 1], task, slots, src, tid, lane);
            }
            // Control barrier only: the poller's LDS flag is complete before it
            // reaches s_barrier, and no wave waits for its outstanding vector
            // loads (a __syncthreads fence would wait for the whole prefetch).
            if (tid == POLLER) stuck_flag = stuck;
            lds_barrier();
            ok = stuck_flag == 0;
            lds_barrier();                    // the flag is read before anyone rewrites it
        }
    }
    // The last workgroup to leave resets the counters for the next run; by
    // then every workgroup has passed its last barrier poll.
    if (tid == 0) {
        u64* depart = sync + SYNC_DEPART * SYNC_LINE;
        if (add_relaxed(depart, 1ull) + 1 == P) {
            for (int gi = 0; gi < SYNC_GROUPS; ++gi) st_relaxed(sync + (SYNC_GROUP0 + gi) * SYNC_LINE, 0ull);
            st_relaxed(depart, 0ull);
        }
    }
}

}  // namespace

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
    // fused pass
    DevStep* dsteps = nullptr;             // device step table
    std::vector<DevStep> hsteps;           // host copy (pointers of the last bound inputs/outputs)
    u64* sync = nullptr;
    int max_xlen = 0;
    int grid = 0;
    bool fused_ok = true;                  // every step supported by the fused kernel (INT8 only)
};

namespace {

int hip_status(hipError_t e) {
    if (e == hipSuccess) return WOQ_OK;
    woq::set_hip_error((int)e);
    return e == hipErrorOutOfMemory ? WOQ_ENOMEM : WOQ_EHIP;
}

void free_stack(woq_stack* st) {
    if (st->xp) (void)hipFree(st->xp);
    if (st->part) (void)hipFree(st->part);
    if (st->dsteps) (void)hipFree(st->dsteps);
    if (st->sync) (void)hipFree(st->sync);
    for (uint16_t* p : st->pos_owned) (void)hipFree(p);
    delete st;
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
bool fold_permutation(const woq_stack_step& s, int64_t b) {
    const woq_int4o_geom& g = s.w4.geom;
    return woq::int4o_use_valu(s.w4.N, g, b) && woq_qgemv_int4o_x_supported(&g, b) && (g.K & 7) == 0;
}

// One step (the step table's entry i, or a copy of it whose weight pointers
// were moved, e.g. into a pager slot); ev (2 entries, or null) brackets the
// product launch.
int run_step(woq_stack* st, size_t i, const woq_stack_step& s, const uint16_t* x, uint16_t* y, int64_t b,
             void* stream, hipEvent_t* ev) {
    int rc;
    if (s.fmt == WOQ_FMT_INT4O && st->pos[i] && fold_permutation(s, b) && woq::aligned16(x)) {
        // permutation folded into the product: one launch
        if (ev) woq::set_launch_events(ev[0], ev[1]);
        rc = woq_qgemv_int4o_x(&s.w4, x, s.w4.geom.K, st->pos[i], b, y, s.w4.N, stream);
        if (ev) woq::set_launch_events(nullptr, nullptr);
        return rc;
    }
    if (s.fmt == WOQ_FMT_INT4O) {
        rc = woq_permute_x(x, s.w4.geom.K, s.perm, b, &s.w4.geom, st->xp, stream);
        if (rc) return rc;
    }
    // with events, the product launch records them at its own dispatch boundaries
    if (ev) woq::set_launch_events(ev[0], ev[1]);
    const int splits = s.fmt == WOQ_FMT_INT4O ? woq::int4o_splitk(s.w4.N, s.w4.geom, b) : 0;
    if (splits)
        rc = woq_qgemm_int4o_splitk(&s.w4, st->xp, b, y, s.w4.N, splits, st->part, st->part_bytes, stream);
    else if (s.fmt == WOQ_FMT_INT4O) rc = woq_qgemv_int4o(&s.w4, st->xp, b, y, s.w4.N, stream);
    else rc = woq_qgemv_int8(&s.w8, x, s.w8.K, b, y, s.w8.N, stream);
    if (ev) woq::set_launch_events(nullptr, nullptr);
    return rc;
}

// One pass over the steps; ev (2 per step) brackets each product launch.
int run_pass(woq_stack* st, const uint16_t* const* inputs, uint16_t* const* outputs, int64_t b, void* stream,
             hipEvent_t* ev) {
    for (size_t i = 0; i < st->steps.size(); ++i) {
        const woq_stack_step& s = st->steps[i];
        int rc = run_step(st, i, s, inputs[s.in_slot], outputs[s.out_slot], b, stream, ev ? ev + 2 * i : nullptr);
        if (rc) return rc;
    }
    return WOQ_OK;
}

template <int B>
const void* fused_kernel() {
    return reinterpret_cast<const void*>(&stack_fused<B>);
}

const void* fused_kernel_for(int64_t b) {
    switch (b) {
        case 1: return fused_kernel<1>();
        case 2: return fused_kernel<2>();
        case 3: return fused_kernel<3>();
        case 4: return fused_kernel<4>();
        case 5: return fused_kernel<5>();
        case 6: return fused_kernel<6>();
        case 7: return fused_kernel<7>();
        default: return fused_kernel<8>();
    }
}

// Upload the step table if the bound inputs/outputs changed.
int bind_fused(woq_stack* st, const uint16_t* const* inputs, uint16_t* const* outputs, void* stream) {
    bool changed = false;
    for (size_t i = 0; i < st->steps.size(); ++i) {
        const woq_stack_step& s = st->steps[i];
        DevStep& d = st->hsteps[i];
        if (d.x != inputs[s.in_slot] || d.y != outputs[s.out_slot]) {
            d.x = inputs[s.in_slot];
            d.y = outputs[s.out_slot];
            changed = true;
        }
    }
    if (!changed) return WOQ_OK;
    // the previous table may still be in use by queued runs on this stream
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e == hipSuccess)
        e = hipMemcpy(st->dsteps, st->hsteps.data(), sizeof(DevStep) * st->hsteps.size(), hipMemcpyHostToDevice);
    return hip_status(e);
}

int launch_fused(woq_stack* st, int64_t b, void* stream) {
    const int nsteps = (int)st->steps.size();
    size_t lds = (size_t)b * st->max_xlen * 2;
    void* args[] = {&st->dsteps, (void*)&nsteps, &st->sync};
    hipError_t e = hipLaunchCooperativeKernel(fused_kernel_for(b), dim3(st->grid), dim3(FUSED_THREADS), args,
                                              (unsigned)lds, (hipStream_t)stream);
    return hip_status(e);
}

int prepare_fused(woq_stack* st, int64_t b) {
    if (!st->fused_ok || b > 8) return WOQ_EUNSUPPORTED;   // the persistent pass streams INT8 quads, b <= 8
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, st->device);
    if (e != hipSuccess) return hip_status(e);
    const size_t lds = (size_t)b * st->max_xlen * 2;
    if (lds > prop.sharedMemPerBlock) return WOQ_EUNSUPPORTED;
    const void* k = fused_kernel_for(b);
    if (lds > 64 * 1024) {
        e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return hip_status(e);
    }
    int per_cu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, FUSED_THREADS, lds);
    if (e != hipSuccess) return hip_status(e);
    if (per_cu < 1) return WOQ_EUNSUPPORTED;
    st->grid = prop.multiProcessorCount;   // one resident workgroup per compute unit
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
    // host step table of the fused pass
    st->hsteps.resize(n_steps);
    for (int i = 0; i < n_steps; ++i) {
        const woq_stack_step& s = steps[i];
        DevStep d;
        std::memset(&d, 0, sizeof d);
        if (s.fmt == WOQ_FMT_INT4O) {
            // the persistent pass streams INT8 quads only
            st->fused_ok = false;
            continue;
        } else {
            d.codes = (const uint4*)s.w8.codes;
            d.N = (int)s.w8.N;
            d.K = (int)s.w8.K;
            d.CPR = (int)(woq::round_up(s.w8.K, 64) / 16);
            d.nchunks = (int)woq::ceil_div(s.w8.K, 16);
            d.xlen = 16 * d.nchunks;
            d.ldx = (int)s.w8.K;
            d.ldy = (int)s.w8.N;
            d.nseg = s.w8.nseg;
            for (int j = 0; j < WOQ_MAX_SEGMENTS; ++j) {
                d.seg_end[j] = j < s.w8.nseg ? (int)s.w8.seg_end[j] : (int)s.w8.N;
                d.seg_scale[j] = j < s.w8.nseg ? s.w8.seg_scale[j] : 0.0f;
            }
            if (!woq::aligned16(s.w8.codes)) st->fused_ok = false;
        }
        st->max_xlen = std::max(st->max_xlen, d.xlen);
        st->hsteps[i] = d;
    }
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
    if (e == hipSuccess && n_steps > 0) e = hipMalloc((void**)&st->dsteps, sizeof(DevStep) * n_steps);
    if (e == hipSuccess) e = hipMalloc((void**)&st->sync, sizeof(u64) * SYNC_WORDS);
    if (e == hipSuccess) e = hipMemset(st->sync, 0, sizeof(u64) * SYNC_WORDS);
    if (e == hipSuccess && n_steps > 0)
        e = hipMemcpy(st->dsteps, st->hsteps.data(), sizeof(DevStep) * n_steps, hipMemcpyHostToDevice);
    int rc = hip_status(e);
    if (rc == WOQ_OK) rc = make_positions(st);
    if (rc != WOQ_OK) {
        free_stack(st);
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
        n += (s.fmt == WOQ_FMT_INT4O && !(st->pos[i] && fold_permutation(s, b))) ? 2 : 1;
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

int woq_dispatch_floor(int32_t blocks, int32_t threads, int32_t iters, void* stream, float* mean_us) {
    if (blocks < 1 || threads < 1 || threads > 1024 || iters < 1 || iters > 100000 || !mean_us) return WOQ_EINVAL;
    std::vector<hipEvent_t> ev(2 * (size_t)iters, nullptr);
    hipError_t e = hipSuccess;
    for (auto& x : ev)
        if (e == hipSuccess) e = hipEventCreate(&x);
    hipStream_t hs = (hipStream_t)stream;
    for (int it = 0; it < iters && e == hipSuccess; ++it)
        e = hipExtLaunchKernel((const void*)&empty_kernel, dim3((unsigned)blocks), dim3((unsigned)threads), nullptr,
                               0, hs, ev[2 * it], ev[2 * it + 1], 0);
    if (e == hipSuccess) e = hipStreamSynchronize(hs);
    double total = 0.0;
    for (int it = 0; it < iters && e == hipSuccess; ++it) {
        float ms = 0.0f;
        e = hipEventElapsedTime(&ms, ev[2 * it], ev[2 * it + 1]);
        total += ms;
    }
    if (e == hipSuccess) *mean_us = (float)(1e3 * total / iters);
    for (auto& x : ev)
        if (x) (void)hipEventDestroy(x);
    return hip_status(e);
}

int woq_stack_run_fused(woq_stack* st, const uint16_t* const* inputs, uint16_t* const* outputs, int64_t b,
                        void* stream) {
    if (!st || !inputs || !outputs || b < 1 || b > st->max_b) return WOQ_EINVAL;
    if (st->steps.empty()) return WOQ_OK;
    int rc = prepare_fused(st, b);
    if (rc) return rc;
    rc = bind_fused(st, inputs, outputs, stream);
    if (rc) return rc;
    return launch_fused(st, b, stream);
}

int woq_stack_check(woq_stack* st, void* stream) {
    if (!st) return WOQ_EINVAL;
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e);
    u64 err = 0;
    e = hipMemcpy(&err, st->sync + SYNC_ERR * SYNC_LINE, sizeof err, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_status(e);
    if (err) {
        // a run gave up: clear every counter (no kernel of this runner is in flight now)
        e = hipMemset(st->sync, 0, sizeof(u64) * SYNC_WORDS);
        if (e != hipSuccess) return hip_status(e);
        return WOQ_ETIMEOUT;
    }
    return WOQ_OK;
}

int woq_stack_time_fused(woq_stack* st, const uint16_t* const* inputs, uint16_t* const* outputs, int64_t b,
                         void* stream, int32_t iters, float* pass_ms) {
    if (!st || !inputs || !outputs || b < 1 || b > st->max_b || iters < 1 || !pass_ms) return WOQ_EINVAL;
    int rc = prepare_fused(st, b);
    if (rc) return rc;
    rc = bind_fused(st, inputs, outputs, stream);
    if (rc) return rc;
    hipStream_t hs = (hipStream_t)stream;
    std::vector<hipEvent_t> ev(2 * (size_t)iters, nullptr);
    hipError_t e = hipSuccess;
    for (auto& x : ev)
        if (e == hipSuccess) e = hipEventCreate(&x);
    for (int it = 0; it < iters && e == hipSuccess && rc == WOQ_OK; ++it) {
        e = hipEventRecord(ev[2 * it], hs);
        if (e == hipSuccess) rc = launch_fused(st, b, stream);
        if (e == hipSuccess && rc == WOQ_OK) e = hipEventRecord(ev[2 * it + 1], hs);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(hs);
    double total = 0.0;
    for (int it = 0; it < iters && e == hipSuccess && rc == WOQ_OK; ++it) {
        float ms = 0.0f;
        e = hipEventElapsedTime(&ms, ev[2 * it], ev[2 * it + 1]);
        total += ms;
    }
    for (auto& x : ev)
        if (x) (void)hipEventDestroy(x);
    if (rc) return rc;
    if (e != hipSuccess) return hip_status(e);
    *pass_ms = (float)(total / iters);
    return woq_stack_check(st, stream);
}

int woq_stack_destroy(woq_stack* st) {
    if (!st) return WOQ_OK;
    hipError_t e = hipSuccess;
    auto release = [&](void* p) {
        if (!p) return;
        hipError_t e2 = hipFree(p);
        if (e == hipSuccess) e = e2;
    };
    release(st->xp);
    release(st->dsteps);
    release(st->sync);
    for (uint16_t* p : st->pos_owned) release(p);
    delete st;
    return hip_status(e);
}

}  // extern "C"
