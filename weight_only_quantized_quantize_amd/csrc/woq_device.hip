// Device kernels of libwoq for gfx950 (CDNA4), and their C-ABI launchers.
//
// Decode linears are bound by HBM bandwidth: every packed weight byte is read
// once per call and never reused, while the activations are a few kilobytes
// shared by every row.  The kernels therefore
//   * stream the codes with 16-byte non-temporal vector loads (each lane owns
//     one 16-byte chunk of each of four consecutive rows, so a wave's load of
//     one row is a contiguous kilobyte),
//   * turn codes into exact fp16 values in registers with the exponent-bias
//     trick (an offset-binary code u in the low mantissa bits of 0x6400 is the
//     fp16 number 1024 + u; subtracting 1024 + offset leaves the signed code),
//   * multiply with v_dot2_f32_f16 (two fp16 products summed into an fp32
//     accumulator, so the products are exact and the accumulation is fp32),
//   * apply the per-group (INT4O) or per-tensor (INT8) scale in fp32 and
//     reduce the 64 lanes of a wave with cross-lane shuffles,
//   * for batch >= 8 (INT4O), feed the same in-register fp16 codes to the
//     16x16x32 fp16 matrix-core instruction, where the work becomes a real
//     contraction over the batch.
//
// Formats: "Open Origin - ELG Stream Layer" (INT8 per-tensor scale, the
// reconstruction code * scale, fused here into the product) and "On-The-Fly
// Weight Synthesizer (OTF-LLM Engine)" (outlier-aware INT4: permuted input,
// FP16 outlier columns plus INT4 background with per-128-channel scales, both
// partial products added into one FP16 output).
#include <hip/hip_runtime.h>

#include "woq_gemv.cuh"
#include "woq_internal.h"

#include <hip/hip_ext.h>

namespace woq {
static thread_local int g_last_hip_error = 0;
void set_hip_error(int code) { g_last_hip_error = code; }
static thread_local hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;
void set_launch_events(void* start, void* stop) {
    g_ev_start = (hipEvent_t)start;
    g_ev_stop = (hipEvent_t)stop;
}
}  // namespace woq

extern "C" int woq_last_hip_error(void) { return woq::g_last_hip_error; }

namespace {

using namespace woqk;

// ------------------------------------------------------------ permute/split

__global__ void permute_x_kernel(const uint16_t* __restrict__ x, int64_t ldx, const int32_t* __restrict__ perm,
                                 int K, int K_bg, int n_out, int bg_len, int xp_len, uint16_t* __restrict__ xp) {
    const int64_t r = blockIdx.y;
    const uint16_t* xr = x + r * ldx;
    for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < xp_len; k += gridDim.x * blockDim.x) {
        int src = -1;
        if (k < K_bg) src = *gptr(perm + k);
        else if (k >= bg_len && k - bg_len < n_out) src = *gptr(perm + K_bg + (k - bg_len));
        // an index outside [0, K) cannot come from a valid permutation; read 0
        uint16_t v = ((unsigned)src < (unsigned)K) ? *gptr(xr + src) : (uint16_t)0;
        *gptr(xp + r * xp_len + k) = v;
    }
}

// ------------------------------------------------------- INT4O, batch <= 7

struct Int4oArgs {
    const uint4* codes;     // [N4][4*G4] chunks of 16 bytes
    const uint2* scales;    // [N4/4][G4] x 4 fp16
    const uint4* wout;      // [N4][n_out8/8] chunks of 8 fp16
    const uint16_t* xp;     // [b][xp_len]
    uint16_t* y;            // [b][ldy]
    int N, G4, no8, xp_len, ldy;
};

// One wave per quad of four output rows; lanes stride over the rows' 16-byte
// chunks (a chunk = 32 background channels of one group).
template <int B>
__global__ __launch_bounds__(64) void qgemv_int4o_valu(Int4oArgs a) {
    constexpr int U = B <= 4 ? 4 : 2;
    const int lane = threadIdx.x;
    QuadTask t;
    t.codes = a.codes;
    t.scales = a.scales;
    t.wout = a.wout;
    t.CPR = 4 * a.G4;
    t.no8 = a.no8;
    t.nchunks = t.CPR + t.no8;
    t.IT = (t.nchunks + 63) >> 6;
    t.q0 = blockIdx.x;
    t.qstride = 1;
    t.nq = 1;
    Slots<U> slots;
    prefetch_items<true, U>(t, lane, slots);
    stream_task<true, B, U>(t, slots, (gx_ptr)a.xp, a.xp_len, 128 * a.G4, lane, U, [&](int q, float out) {
        if (lane < 4 * B) {
            const int r = lane / B, b = lane % B, n = 4 * q + r;
            if (n < a.N) *gptr(a.y + (int64_t)b * a.ldy + n) = f_to_h(out);
        }
    });
}

// ------------------------------- INT4O, batch <= 7, permutation in the kernel

// The activation permutation and split folded into the product: a workgroup
// of GX_WAVES waves reads the activations in their natural channel order
// (coalesced 16-byte loads of 8 channels, together with the 8 channels'
// positions in the permuted row) and scatters them into LDS, where they form
// the permuted, zero-padded row that the waves' quads then read.  The weight
// loads of every wave are issued right after the activation loads, so the
// staging costs no extra memory round trip.
constexpr int GX_WAVES = 4;
constexpr int GX_THREADS = 64 * GX_WAVES;
constexpr int GX_LDS_BYTES = 64 * 1024;

struct Int4oGxArgs {
    Int4oArgs p;             // p.xp unused
    const uint16_t* x;       // [b][ldx], natural channel order
    const uint16_t* pos;     // [round_up(K, 8)] position of each channel in the permuted row (0xFFFF: none)
    int K, K_bg, n_out, ldx, qpw;   // qpw: quads per wave
};

// Write 8 channels (one 16-byte chunk per batch row) to their positions in
// the staged row; positions outside the row (table padding) are skipped.
template <int B>
__device__ __forceinline__ void gx_scatter(uint16_t* xs, int xp_len, const uint4 (&xv)[B], uint4 pv) {
    const uint32_t pw[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int p = (int)((pw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
        if (p < xp_len) {
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const uint32_t xw[4] = {xv[b].x, xv[b].y, xv[b].z, xv[b].w};
                xs[b * xp_len + p] = (uint16_t)(xw[j >> 1] >> (16 * (j & 1)));
            }
        }
    }
}

template <int B>
__global__ __launch_bounds__(GX_THREADS) void qgemv_int4o_gx(Int4oGxArgs a) {
    extern __shared__ __align__(16) uint16_t xs[];   // [B][xp_len]
    constexpr int U = B <= 4 ? 4 : 2;
    constexpr int SC = B == 1 ? 4 : B == 2 ? 2 : 1;   // activation chunks per thread per pass
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int xp_len = a.p.xp_len, bg_len = 128 * a.p.G4;
    const int quads = (a.p.N + 3) >> 2;
    // quads base + wave, base + wave + GX_WAVES, ... (qpw of them, within N)
    const int base = blockIdx.x * GX_WAVES * a.qpw;
    const int q0 = base + wave;
    const int last = min(quads, base + GX_WAVES * a.qpw);
    QuadTask t;
    t.codes = a.p.codes;
    t.scales = a.p.scales;
    t.wout = a.p.wout;
    t.CPR = 4 * a.p.G4;
    t.no8 = a.p.no8;
    t.nchunks = t.CPR + t.no8;
    t.IT = (t.nchunks + 63) >> 6;
    t.q0 = q0 < last ? q0 : 0;              // a wave without quads streams quad 0's first item and ignores it
    t.qstride = GX_WAVES;
    t.nq = q0 < last ? (last - 1 - q0) / GX_WAVES + 1 : 0;

    const int nc = (a.K + 7) >> 3;          // 8-channel activation chunks
    const g_u32x4* xg = (const g_u32x4*)a.x;
    const g_u32x4* pg = (const g_u32x4*)a.pos;
    const int ldx16 = a.ldx >> 3;
    // first pass of activation loads (unconditional; out-of-range chunks reload chunk 0)
    uint4 xv[SC][B], pv[SC];
#pragma unroll
    for (int i = 0; i < SC; ++i) {
        const int c = tid + i * GX_THREADS;
        const int cc = c < nc ? c : 0;
        pv[i] = as_uint4(pg[cc]);
#pragma unroll
        for (int b = 0; b < B; ++b) xv[i][b] = as_uint4(xg[b * ldx16 + cc]);
    }
    Slots<U> slots;
    prefetch_items_fixed<true, U>(t, lane, slots);
    // padding of the permuted row: [K_bg, bg_len) and [bg_len + n_out, xp_len)
    for (int k = a.K_bg + tid; k < bg_len; k += GX_THREADS)
#pragma unroll
        for (int b = 0; b < B; ++b) xs[b * xp_len + k] = 0;
    for (int k = bg_len + a.n_out + tid; k < xp_len; k += GX_THREADS)
#pragma unroll
        for (int b = 0; b < B; ++b) xs[b * xp_len + k] = 0;
#pragma unroll
    for (int i = 0; i < SC; ++i)
        if (tid + i * GX_THREADS < nc) gx_scatter<B>(xs, xp_len, xv[i], pv[i]);
    for (int c = tid + SC * GX_THREADS; c < nc; c += GX_THREADS) {
        uint4 xv1[B];
        const uint4 pv1 = as_uint4(pg[c]);
#pragma unroll
        for (int b = 0; b < B; ++b) xv1[b] = as_uint4(xg[b * ldx16 + c]);
        gx_scatter<B>(xs, xp_len, xv1, pv1);
    }
    lds_barrier();
    stream_task<true, B, U>(t, slots, (lx_ptr)xs, xp_len, bg_len, lane, U, [&](int q, float out) {
        if (lane < 4 * B) {
            const int r = lane / B, b = lane % B, n = 4 * q + r;
            if (n < a.p.N) *gptr(a.p.y + (int64_t)b * a.p.ldy + n) = f_to_h(out);
        }
    });
}

// --------------------------------------------------------- INT8, batch <= 8

struct Int8Args {
    const uint4* codes;     // [N4][Kd/16] chunks of 16 bytes
    const uint16_t* x;      // [b][ldx]
    uint16_t* y;            // [b][ldy]
    int N, K, CPR, ldx, ldy, nseg;
    int seg_end[WOQ_MAX_SEGMENTS];
    float seg_scale[WOQ_MAX_SEGMENTS];
};

template <int B>
__global__ __launch_bounds__(64) void qgemv_int8_valu(Int8Args a) {
    const int lane = threadIdx.x;
    const int quad = blockIdx.x;
    const uint4* w0 = a.codes + (int64_t)quad * 4 * a.CPR;
    const int nchunks = (a.K + 15) >> 4;   // chunks that hold real columns
    float acc[4][B];
    zero_acc(acc);
#pragma unroll 2
    for (int cc = lane; cc < nchunks; cc += 64) {
        uint4 w[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = gload_nt(w0 + r * a.CPR + cc);
        uint4 xv[B][2];
        const int k0 = 16 * cc;
        if (k0 + 16 <= a.K) {
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const gx_ptr xs = (gx_ptr)(a.x + (int64_t)b * a.ldx + k0);
                xv[b][0] = load_x16(xs);
                xv[b][1] = load_x16(xs + 8);
            }
        } else {
#pragma unroll
            for (int b = 0; b < B; ++b) {
                uint32_t t[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int k = k0 + 2 * j;
                    const uint32_t lo = (k < a.K) ? *gptr(a.x + (int64_t)b * a.ldx + k) : 0u;
                    const uint32_t hi = (k + 1 < a.K) ? *gptr(a.x + (int64_t)b * a.ldx + k + 1) : 0u;
                    t[j] = lo | (hi << 16);
                }
                xv[b][0] = make_uint4(t[0], t[1], t[2], t[3]);
                xv[b][1] = make_uint4(t[4], t[5], t[6], t[7]);
            }
        }
        int8_chunk<B>(w, xv, acc);
    }
    const float out = quad_reduce<B>(acc, lane);
    if (lane < 4 * B) {
        const int r = lane / B, b = lane % B;
        const int n = quad * 4 + r;
        if (n < a.N) {
            float s = a.seg_scale[a.nseg - 1];
            for (int i = a.nseg - 1; i >= 0; --i)
                if (n < a.seg_end[i]) s = a.seg_scale[i];
            *gptr(a.y + (int64_t)b * a.ldy + n) = f_to_h(out * s);
        }
    }
}

// ------------------------------------------------ INT4O, matrix cores (b >= 8)

// A workgroup of four waves owns 16 output rows; wave w takes the groups
// g = w, w + 4, ...  Lane l holds row l & 15 of the 16-row tile and the
// 16-byte chunk l >> 4 of each group (32 channels) - exactly the A operand of
// v_mfma_f32_16x16x32_f16 for four k-steps: the unscaled pairs feed steps 0
// and 2, the pairs that carry 16 x code feed steps 1 and 3 into a second
// accumulator that is divided by 16 before the group scale is applied.  The B
// operand (activations, batch column l & 15) is read from memory in the same
// channel order.  Partial sums of the four waves meet in LDS.
template <int NBT>
__global__ __launch_bounds__(256) void qgemm_int4o_mfma(Int4oArgs a, int b) {
    __shared__ float red[4][NBT][16][17];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int m = lane & 15;           // row within the tile (A) / batch column (B)
    const int c = lane >> 4;           // 32-channel chunk of the group / k-block
    const int row = blockIdx.x * 16 + m;
    const int N4 = (a.N + 3) & ~3;
    const bool row_ok = row < N4;
    const int CPR = a.G4 * 4;
    const uint4* wrow = a.codes + (int64_t)row * CPR;
    const int quad0 = blockIdx.x * 4;  // first quad of the tile

    f4 acc[NBT];
#pragma unroll
    for (int t = 0; t < NBT; ++t) acc[t] = (f4){0.f, 0.f, 0.f, 0.f};

    for (int g = wave; g < a.G4; g += 4) {
        uint4 w = row_ok ? gload_nt(wrow + 4 * g + c) : make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
        const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
        const uint32_t bias = bias_reg();
        Int4Pairs p[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) p[d] = int4_pairs(wd[d], bias);
        // A operands of the four k-steps (8 fp16 each)
        h8 A[4];
#pragma unroll
        for (int P = 0; P < 2; ++P) {
            const Int4Pairs& e0 = p[2 * P];
            const Int4Pairs& e1 = p[2 * P + 1];
            A[2 * P + 0] = (h8){e0.lo0[0], e0.lo0[1], e0.lo1[0], e0.lo1[1], e1.lo0[0], e1.lo0[1], e1.lo1[0], e1.lo1[1]};
            A[2 * P + 1] = (h8){e0.hi0[0], e0.hi0[1], e0.hi1[0], e0.hi1[1], e1.hi0[0], e1.hi0[1], e1.hi1[0], e1.hi1[1]};
        }
        // per-row scales of this group for the four D rows this lane holds
        float s[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = 4 * c + i;      // D row held by this lane
            const int q = quad0 + (rr >> 2);
            s[i] = (q * 4 < N4) ? h_to_f(*gptr(reinterpret_cast<const uint16_t*>(a.scales) + ((int64_t)q * a.G4 + g) * 4 + (rr & 3))) : 0.0f;
        }
#pragma unroll
        for (int t = 0; t < NBT; ++t) {
            const int col = t * 16 + m;    // batch column of the B operand
            h8 Bv[4];
            if (col < b) {
                const gx_ptr xs = (gx_ptr)(a.xp + (int64_t)col * a.xp_len + 128 * g + 32 * c);
#pragma unroll
                for (int j = 0; j < 4; ++j) Bv[j] = __builtin_bit_cast(h8, load_x16(xs + 8 * j));
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) Bv[j] = (h8){0, 0, 0, 0, 0, 0, 0, 0};
            }
            f4 lo = (f4){0.f, 0.f, 0.f, 0.f}, hi = (f4){0.f, 0.f, 0.f, 0.f};
            lo = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[0], Bv[0], lo, 0, 0, 0);
            hi = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[1], Bv[1], hi, 0, 0, 0);
            lo = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[2], Bv[2], lo, 0, 0, 0);
            hi = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[3], Bv[3], hi, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][i] = fmaf(s[i], fmaf(hi[i], 0.0625f, lo[i]), acc[t][i]);
        }
    }

    // FP16 outlier columns, 32 per k-step, split over the waves
    const uint16_t* xo_base = a.xp + 128 * a.G4;
    const int n_o8 = a.no8 * 8;
    for (int st = wave; st * 32 < n_o8; st += 4) {
        const int col0 = 32 * st + 8 * c;
        h8 Av = (h8){0, 0, 0, 0, 0, 0, 0, 0};
        if (row_ok && col0 < n_o8)
            Av = __builtin_bit_cast(h8, gload_u4(a.wout + (int64_t)row * a.no8 + (col0 >> 3)));
#pragma unroll
        for (int t = 0; t < NBT; ++t) {
            const int bc = t * 16 + m;
            h8 Bv = (h8){0, 0, 0, 0, 0, 0, 0, 0};
            if (bc < b && col0 < n_o8)
                Bv = __builtin_bit_cast(h8, load_x16((gx_ptr)(xo_base + (int64_t)bc * a.xp_len + col0)));
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Av, Bv, acc[t], 0, 0, 0);
        }
    }

#pragma unroll
    for (int t = 0; t < NBT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][t][4 * c + i][m] = acc[t][i];
    __syncthreads();
    for (int e = threadIdx.x; e < NBT * 256; e += 256) {
        const int t = e >> 8, rr = (e >> 4) & 15, col = e & 15;
        const int bc = t * 16 + col;
        const int n = blockIdx.x * 16 + rr;
        if (bc < b && n < a.N) {
            float v = red[0][t][rr][col] + red[1][t][rr][col] + red[2][t][rr][col] + red[3][t][rr][col];
            *gptr(a.y + (int64_t)bc * a.ldy + n) = f_to_h(v);
        }
    }
}

// Launch a kernel; with timing events set, through hipExtLaunchKernel so the
// events take the dispatch's own start and end timestamps.
template <class K, class... A>
hipError_t launch_kernel(K kernel, dim3 grid, dim3 block, size_t shmem, hipStream_t s, A... args) {
    void* argv[] = {(void*)&args...};
    if (woq::g_ev_start)
        return hipExtLaunchKernel((const void*)kernel, grid, block, argv, shmem, s, woq::g_ev_start, woq::g_ev_stop, 0);
    return hipLaunchKernel((const void*)kernel, grid, block, argv, shmem, s);
}

int launch_status(hipError_t e) {
    if (e != hipSuccess) {
        woq::set_hip_error((int)e);
        return WOQ_EHIP;
    }
    return WOQ_OK;
}

template <int B>
hipError_t launch_int4o_valu(const Int4oArgs& a, int quads, hipStream_t s) {
    return launch_kernel(qgemv_int4o_valu<B>, dim3(quads), dim3(64), 0, s, a);
}

template <int B>
hipError_t launch_int4o_gx(const Int4oGxArgs& a, hipStream_t s) {
    const int quads = (int)woq::ceil_div(a.p.N, 4);
    const int grid = (int)woq::ceil_div(quads, (int64_t)GX_WAVES * a.qpw);
    const size_t lds = (size_t)B * a.p.xp_len * sizeof(uint16_t);
    return launch_kernel(qgemv_int4o_gx<B>, dim3(grid), dim3(GX_THREADS), lds, s, a);
}

template <int B>
hipError_t launch_int8_valu(const Int8Args& a, int quads, hipStream_t s) {
    return launch_kernel(qgemv_int8_valu<B>, dim3(quads), dim3(64), 0, s, a);
}

template <int NBT>
hipError_t launch_int4o_mfma(const Int4oArgs& a, int b, hipStream_t s) {
    const int tiles = (int)woq::ceil_div(woq::round_up(a.N, 4), 16);
    return launch_kernel(qgemm_int4o_mfma<NBT>, dim3(tiles), dim3(256), 0, s, a, b);
}

int check_int4o_w(const woq_int4o_w* w) {
    if (!w || w->N < 0 || !woq::int4o_geom_valid(&w->geom)) return WOQ_EINVAL;
    if (w->N > 0 && ((w->geom.G4 && (!w->codes || !w->scales)) || (w->geom.n_out8 && !w->w_out))) return WOQ_EINVAL;
    if (!woq::aligned16(w->codes) || !woq::aligned16(w->w_out) || (((uintptr_t)w->scales) & 7u)) return WOQ_EALIGN;
    if (w->N > (int64_t)INT32_MAX - 64 || w->geom.xp_len > (int64_t)INT32_MAX / 64) return WOQ_EUNSUPPORTED;
    return WOQ_OK;
}

Int4oArgs make_int4o_args(const woq_int4o_w* w, const uint16_t* xp, uint16_t* y, int64_t ldy) {
    Int4oArgs a;
    a.codes = reinterpret_cast<const uint4*>(w->codes);
    a.scales = reinterpret_cast<const uint2*>(w->scales);
    a.wout = reinterpret_cast<const uint4*>(w->w_out);
    a.xp = xp;
    a.y = y;
    a.N = (int)w->N;
    a.G4 = (int)w->geom.G4;
    a.no8 = (int)(w->geom.n_out8 / 8);
    a.xp_len = (int)w->geom.xp_len;
    a.ldy = (int)ldy;
    return a;
}

int int4o_common_checks(const woq_int4o_w* w, const uint16_t* xp, int64_t b, uint16_t* y, int64_t ldy) {
    int st = check_int4o_w(w);
    if (st) return st;
    if (b < 0 || b > 64 || ldy < w->N || ldy > INT32_MAX) return WOQ_EINVAL;
    if (b > 0 && w->N > 0 && (!xp || !y)) return WOQ_EINVAL;
    if (!woq::aligned16(xp) || ((uintptr_t)y & 1u)) return WOQ_EALIGN;
    return WOQ_OK;
}

}  // namespace

extern "C" {

int woq_permute_x(const uint16_t* x, int64_t ldx, const int32_t* perm, int64_t b, const woq_int4o_geom* g,
                  uint16_t* xp, void* stream) {
    if (!woq::int4o_geom_valid(g) || b < 0 || ldx < g->K) return WOQ_EINVAL;
    if (b == 0) return WOQ_OK;
    if (!x || !perm || !xp) return WOQ_EINVAL;
    if (!woq::aligned16(xp) || ((uintptr_t)x & 1u) || ((uintptr_t)perm & 3u)) return WOQ_EALIGN;
    if (b > 65535 || g->xp_len > INT32_MAX) return WOQ_EUNSUPPORTED;
    const int threads = 256;
    int blocks = (int)std::min<int64_t>(woq::ceil_div(g->xp_len, threads), 1024);
    hipLaunchKernelGGL(permute_x_kernel, dim3(blocks, (unsigned)b), dim3(threads), 0, (hipStream_t)stream, x, ldx,
                       perm, (int)g->K, (int)g->K_bg, (int)g->n_out, (int)(128 * g->G4), (int)g->xp_len, xp);
    return launch_status(hipGetLastError());
}

int woq_qgemv_int4o(const woq_int4o_w* w, const uint16_t* xp, int64_t b, uint16_t* y, int64_t ldy, void* stream) {
    int st = int4o_common_checks(w, xp, b, y, ldy);
    if (st) return st;
    if (b == 0 || w->N == 0) return WOQ_OK;
    if (b >= 8) return woq_qgemm_int4o(w, xp, b, y, ldy, stream);
    Int4oArgs a = make_int4o_args(w, xp, y, ldy);
    const int quads = (int)woq::ceil_div(w->N, 4);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    switch (b) {
        case 1: e = launch_int4o_valu<1>(a, quads, s); break;
        case 2: e = launch_int4o_valu<2>(a, quads, s); break;
        case 3: e = launch_int4o_valu<3>(a, quads, s); break;
        case 4: e = launch_int4o_valu<4>(a, quads, s); break;
        case 5: e = launch_int4o_valu<5>(a, quads, s); break;
        case 6: e = launch_int4o_valu<6>(a, quads, s); break;
        default: e = launch_int4o_valu<7>(a, quads, s); break;
    }
    return launch_status(e);
}

int woq_qgemv_int4o_x(const woq_int4o_w* w, const uint16_t* x, int64_t ldx, const uint16_t* pos, int64_t b,
                      uint16_t* y, int64_t ldy, void* stream) {
    int st = check_int4o_w(w);
    if (st) return st;
    const woq_int4o_geom& g = w->geom;
    if (b < 0 || ldx < g.K || ldy < w->N || ldx > INT32_MAX || ldy > INT32_MAX) return WOQ_EINVAL;
    if (b == 0 || w->N == 0) return WOQ_OK;
    if (!x || !pos || !y) return WOQ_EINVAL;
    if (!woq::aligned16(x) || !woq::aligned16(pos) || (ldx & 7) || ((uintptr_t)y & 1u)) return WOQ_EALIGN;
    if (!woq_qgemv_int4o_x_supported(&g, b)) return WOQ_EUNSUPPORTED;
    Int4oGxArgs a;
    a.p = make_int4o_args(w, nullptr, y, ldy);
    a.x = x;
    a.pos = pos;
    a.K = (int)g.K;
    a.K_bg = (int)g.K_bg;
    a.n_out = (int)g.n_out;
    a.ldx = (int)ldx;
    // one quad per wave: more quads per workgroup would stage the activations
    // fewer times but leaves fewer waves to keep loads in flight, which costs
    // more (measured on the 70B-shaped products)
    a.qpw = 1;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    switch (b) {
        case 1: e = launch_int4o_gx<1>(a, s); break;
        case 2: e = launch_int4o_gx<2>(a, s); break;
        case 3: e = launch_int4o_gx<3>(a, s); break;
        case 4: e = launch_int4o_gx<4>(a, s); break;
        case 5: e = launch_int4o_gx<5>(a, s); break;
        case 6: e = launch_int4o_gx<6>(a, s); break;
        default: e = launch_int4o_gx<7>(a, s); break;
    }
    return launch_status(e);
}

int woq_qgemv_int4o_x_supported(const woq_int4o_geom* g, int64_t b) {
    if (!g || b < 1 || b > 7) return 0;
    return g->xp_len <= 65535 && b * g->xp_len * 2 <= GX_LDS_BYTES;
}

int woq_qgemm_int4o(const woq_int4o_w* w, const uint16_t* xp, int64_t b, uint16_t* y, int64_t ldy, void* stream) {
    int st = int4o_common_checks(w, xp, b, y, ldy);
    if (st) return st;
    if (b == 0 || w->N == 0) return WOQ_OK;
    Int4oArgs a = make_int4o_args(w, xp, y, ldy);
    hipStream_t s = (hipStream_t)stream;
    const int nbt = (int)woq::ceil_div(b, 16);
    hipError_t e;
    switch (nbt) {
        case 1: e = launch_int4o_mfma<1>(a, (int)b, s); break;
        case 2: e = launch_int4o_mfma<2>(a, (int)b, s); break;
        case 3: e = launch_int4o_mfma<3>(a, (int)b, s); break;
        default: e = launch_int4o_mfma<4>(a, (int)b, s); break;
    }
    return launch_status(e);
}

int woq_qgemv_int8(const woq_int8_w* w, const uint16_t* x, int64_t ldx, int64_t b, uint16_t* y, int64_t ldy,
                   void* stream) {
    if (!w || w->N < 0 || w->K < 1 || b < 0 || b > 8 || ldx < w->K || ldy < w->N) return WOQ_EINVAL;
    if (w->nseg < 1 || w->nseg > WOQ_MAX_SEGMENTS || w->seg_end[w->nseg - 1] != w->N) return WOQ_EINVAL;
    for (int i = 0; i < w->nseg; ++i) {
        int64_t lo = i ? w->seg_end[i - 1] : 0;
        if (w->seg_end[i] < lo) return WOQ_EINVAL;
    }
    if (b == 0 || w->N == 0) return WOQ_OK;
    if (!w->codes || !x || !y) return WOQ_EINVAL;
    if (!woq::aligned16(w->codes) || !woq::aligned16(x) || (ldx & 7) || ((uintptr_t)y & 1u)) return WOQ_EALIGN;
    if (w->N > (int64_t)INT32_MAX - 64 || w->K > (int64_t)INT32_MAX - 64 || ldx > INT32_MAX || ldy > INT32_MAX)
        return WOQ_EUNSUPPORTED;
    Int8Args a;
    a.codes = reinterpret_cast<const uint4*>(w->codes);
    a.x = x;
    a.y = y;
    a.N = (int)w->N;
    a.K = (int)w->K;
    a.CPR = (int)(woq::round_up(w->K, 64) / 16);
    a.ldx = (int)ldx;
    a.ldy = (int)ldy;
    a.nseg = w->nseg;
    for (int i = 0; i < WOQ_MAX_SEGMENTS; ++i) {
        a.seg_end[i] = i < w->nseg ? (int)w->seg_end[i] : (int)w->N;
        a.seg_scale[i] = i < w->nseg ? w->seg_scale[i] : 0.0f;
    }
    const int quads = (int)woq::ceil_div(w->N, 4);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    switch (b) {
        case 1: e = launch_int8_valu<1>(a, quads, s); break;
        case 2: e = launch_int8_valu<2>(a, quads, s); break;
        case 3: e = launch_int8_valu<3>(a, quads, s); break;
        case 4: e = launch_int8_valu<4>(a, quads, s); break;
        case 5: e = launch_int8_valu<5>(a, quads, s); break;
        case 6: e = launch_int8_valu<6>(a, quads, s); break;
        case 7: e = launch_int8_valu<7>(a, quads, s); break;
        default: e = launch_int8_valu<8>(a, quads, s); break;
    }
    return launch_status(e);
}

}  // extern "C"
