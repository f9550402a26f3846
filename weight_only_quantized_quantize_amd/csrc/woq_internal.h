// Internal helpers shared by the host and device translation units of libwoq.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <thread>
#include <vector>

#include "woq.h"

namespace woq {

// hipError_t of the last failing HIP call on this thread.
void set_hip_error(int code);

// Events (hipEvent_t, or null) that the next product launch on this thread
// records at its own dispatch boundaries (the timestamps a kernel trace
// reports); set by the runner's timing pass around one launch.
void set_launch_events(void* start, void* stop);

// Launch step i of a stack with the given step contents (the entry itself or
// a copy whose weight pointers were moved); argument checks as woq_stack_run.
int stack_run_step(woq_stack* st, int64_t i, const woq_stack_step* s, const uint16_t* x, uint16_t* y, int64_t b,
                   void* stream);

inline int64_t round_up(int64_t a, int64_t m) { return (a + m - 1) / m * m; }
inline int64_t ceil_div(int64_t a, int64_t m) { return (a + m - 1) / m; }

// Geometry of an outlier split (validated); mirrors woq_int4o_geometry.
int int4o_geom(int64_t K, int64_t n_out, woq_int4o_geom* g);
// True if *g is what woq_int4o_geometry gives for its own K and n_out.
bool int4o_geom_valid(const woq_int4o_geom* g);

inline int num_threads() {
    static int n = [] {
        int hw = (int)std::thread::hardware_concurrency();
        if (hw <= 0) hw = 1;
        int want = std::min(hw, 16);
        if (const char* e = std::getenv("WOQ_NUM_THREADS")) {
            int v = std::atoi(e);
            if (v > 0) want = v;
        }
        return want;
    }();
    return n;
}

// Run f(lo, hi) over [0, n) split into contiguous ranges, one per worker.
// The split only decides which thread does which range; every caller makes
// each element's result independent of the split, so results do not depend on
// the thread count.
template <class F>
void parallel_for(int64_t n, F&& f, int64_t min_per_thread = 1) {
    if (n <= 0) return;
    int64_t nt = std::min<int64_t>(num_threads(), std::max<int64_t>(1, n / std::max<int64_t>(1, min_per_thread)));
    if (nt <= 1) {
        f((int64_t)0, n);
        return;
    }
    std::vector<std::thread> th;
    th.reserve(nt - 1);
    int64_t chunk = ceil_div(n, nt);
    for (int64_t t = 1; t < nt; ++t) {
        int64_t lo = t * chunk, hi = std::min(n, lo + chunk);
        if (lo >= hi) break;
        th.emplace_back([&f, lo, hi] { f(lo, hi); });
    }
    f((int64_t)0, std::min(n, chunk));
    for (auto& t : th) t.join();
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// LDS of the INT4O vector kernel: the staged activation rows (b * xp_len
// fp16) and the bias correction of every 32-channel background chunk
// (b * 4 * G4 floats).
constexpr int64_t INT4O_VALU_LDS_BYTES = 62 * 1024;
inline int64_t int4o_valu_lds_bytes(int64_t xp_len, int64_t chunks, int64_t b) {
    return b * (xp_len * 2 + chunks * 4);
}

// Which INT4O kernel serves a product of N rows at batch b: the vector kernel
// for b <= 2, and for b <= 4 on narrow products (fewer than 384 tiles of 16
// rows), where it is the faster of the two on MI355X; the matrix-core kernel
// otherwise, and whenever the staged activation rows would not fit in LDS.
inline bool int4o_use_valu(int64_t N, const woq_int4o_geom& g, int64_t b) {
    if (b < 1 || b > 4 || int4o_valu_lds_bytes(g.xp_len, 4 * g.G4, b) > INT4O_VALU_LDS_BYTES) return false;
    return b <= 2 || ceil_div(N, 16) < 384;
}

// K splits the stack runner gives a matrix-core INT4O product (0: none).
// Rows of 128 groups or more (the 70B-shaped down product, 224 groups) at
// 9 <= b <= 32 are split in 8: every workgroup then covers 128 rows and one
// eighth of K, which cuts the activation staging per weight byte (70B down at
// b = 32: 62 -> 46 us, the reduction launch included); shorter rows gained
// nothing.  At b <= 8, where eight staged columns keep the staging small, the
// unsplit two-tile plan of sixteen waves is as fast or faster and saves the
// reduction launch (measured on MI355X, 70B down: 32.7 -> 31.0 us at b = 4,
// 33.7 -> 33.3 us at b = 8).
constexpr int INT4O_SPLITS = 8;
inline int int4o_splitk(int64_t N, const woq_int4o_geom& g, int64_t b) {
    if (int4o_use_valu(N, g, b) || g.G4 < 128 || b <= 8 || b > 32) return 0;
    return INT4O_SPLITS;
}

}  // namespace woq
