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

#include "woq_gemv.h"
#include "woq_internal.h"

#include <hip/hip_ext.h>

#include <atomic>
#include <mutex>

namespace woq {
static thread_local int g_last_hip_error = 0;
// Record a failing HIP call's error for woq_last_hip_error and clear the HIP
// runtime's own last-error state: the failure is reported through the
// library's status code, and a pending runtime error would otherwise be
// picked up by the caller's next, unrelated, error check.
void set_hip_error(int code) {
    g_last_hip_error = code;
    (void)hipGetLastError();
}
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

// ------------------------------------------------------ streaming-read rate

// Four 16-byte non-temporal loads per lane, all in flight at once; the grid
// covers the buffer in one pass (a probe sweep of grid and block shapes found
// this among the fastest read patterns on MI355X).  The data is folded into
// one word that is stored only if it equals an arbitrary constant: the store
// keeps the loads alive; nothing reads the sink.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += 4 * stride) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = gload_nt(p + (i + u * stride < n16 ? i + u * stride : i));
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) *gptr(sink) = acc;
}

// ------------------------------------------------- INT8 vocabulary lookup

struct EmbedArgs {
    const uint4* codes;     // INT8 device layout, row-major [V4][Kd] offset-binary bytes
    const int32_t* ids;     // [b]
    uint16_t* y;            // [b][ldy]
    int V, K, CPR, ldy;     // CPR = Kd / 16
    int nseg;
    int seg_end[WOQ_MAX_SEGMENTS];
    float seg_scale[WOQ_MAX_SEGMENTS];
};

// One token per blockIdx.y; each lane expands 16 codes of the row.  The value
// is the code times the scale rounded to fp32 and then to fp16, both to
// nearest even.  The fp32 product is pinned in a register before the
// narrowing: otherwise the compiler fuses the multiply and the narrowing into
// one mixed-precision FMA that rounds once, straight to fp16, which differs
// from the two roundings where the fp32 product lands on an fp16 tie.
__global__ __launch_bounds__(256) void embed_int8_kernel(EmbedArgs a) {
    const int r = blockIdx.y;
    const int c = blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= a.CPR || 16 * c >= a.K) return;
    const int t = *gptr(a.ids + r);
    const bool valid = (unsigned)t < (unsigned)a.V;
    float s = 0.0f;
    if (valid) {
        int i = 0;
        while (i + 1 < a.nseg && t >= a.seg_end[i]) ++i;
        s = a.seg_scale[i];
    }
    uint4 w = make_uint4(0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u);   // code 0
    if (valid) w = gload_u4(a.codes + (int64_t)t * a.CPR + c);
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    uint32_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t word = wd[j >> 1];
        const int sh = 16 * (j & 1);
        float lo = (float)((int)((word >> sh) & 0xFFu) - 128) * s;
        float hi = (float)((int)((word >> (sh + 8)) & 0xFFu) - 128) * s;
        asm volatile("" : "+v"(lo), "+v"(hi));
        h[j] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
    }
    uint16_t* yr = a.y + (int64_t)r * a.ldy + 16 * c;
    if (16 * c + 16 <= a.K) {
        uint4* d = reinterpret_cast<uint4*>(yr);
        gstore_u4(d, make_uint4(h[0], h[1], h[2], h[3]));
        gstore_u4(d + 1, make_uint4(h[4], h[5], h[6], h[7]));
    } else {
        for (int j = 0; j < 16 && 16 * c + j < a.K; ++j) *gptr(yr + j) = (uint16_t)(h[j >> 1] >> (16 * (j & 1)));
    }
}

// ---------------------------------------------------- INT4O, vector ALU (b <= 4)

struct Int4oArgs {
    const uint4* codes;     // [tiles][G4][4 chunks][16 rows] x 16 bytes
    const uint16_t* scales; // [tiles][G4][16] fp16
    const uint4* wout;      // [tiles][no8][16] chunks of 8 fp16
    const uint16_t* xp;     // [b][xp_len] permuted, split activations
    uint16_t* y;            // [b][ldy]
    int N, G4, no8, xp_len, ldy;
    // split of the groups over blockIdx.y (matrix-core kernel): 0, or the
    // groups per split; split s writes its fp32 partial sums to
    // part[s][b][N] instead of y, and only split 0 adds the outlier columns
    int gsplit = 0;
    float* part = nullptr;
};

// Activations in their natural channel order and the position of every
// channel in the permuted row (the permutation folded into the product).
struct GatherArgs {
    const uint16_t* x;      // [b][ldx]
    const uint16_t* pos;    // [round_up(K, 8)], 0xFFFF: no position
    int K, K_bg, n_out, ldx;
};

// Groups of weights in flight per wave: six at b = 1, eight above.  A
// shallower window lets the activation row arrive sooner behind the weight
// loads issued with it, and at b = 1 that outweighs the shorter lead of the
// weight stream: measured on MI355X over whole stacks, six against eight
// took the 70B-shaped layer from 85.0 to 82.9 us and the 3B-shaped one from
// 22.5 to 21.6 us (seven and mixed depths fell in between).
template <int B>
constexpr int tile_window() { return B == 1 ? 6 : 8; }

// Write 8 channels (one 16-byte chunk per batch row) to their positions in
// the staged row; positions outside the row (table padding) are skipped.
template <int B>
__device__ __forceinline__ void scatter8(uint16_t* xs, int xp_len, const uint4 (&xv)[B], uint4 pv) {
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

// Dword i of the result is dword (i + r) & 3 of v (r in 0..3).
__device__ __forceinline__ uint4 rot_dwords(uint4 v, int r) {
    const bool r2 = (r & 2) != 0, r1 = (r & 1) != 0;
    const uint32_t t0 = r2 ? v.z : v.x, t1 = r2 ? v.w : v.y, t2 = r2 ? v.x : v.z, t3 = r2 ? v.y : v.w;
    return make_uint4(r1 ? t1 : t0, r1 ? t2 : t1, r1 ? t3 : t2, r1 ? t0 : t3);
}

// scatter8 for a piece whose eight positions all lie in the row (every piece
// of a position table but the last when K is not a multiple of 8), without
// branches.  Lanes rotate their piece by r dwords first: with 16-byte pieces
// on consecutive lanes, the j-th write of every lane would otherwise hit only
// eight of the 32 LDS banks; rotating by (lane / 8) % 4 spreads it over all.
// Measured on MI355X: the scatter of the 70B-shaped q|k|v product's row from
// 1.3 to 1.0 us per wave (median), the 70B-shaped step at b = 1 1.3% and the
// 3B-shaped step 1.9% faster.
template <int B>
__device__ __forceinline__ void scatter8_full(uint16_t* xs, int xp_len, const uint4 (&xv)[B], uint4 pv, int r) {
    const uint4 pr = rot_dwords(pv, r);
    const uint32_t pw[4] = {pr.x, pr.y, pr.z, pr.w};
    uint32_t xw[B][4];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const uint4 t = rot_dwords(xv[b], r);
        xw[b][0] = t.x; xw[b][1] = t.y; xw[b][2] = t.z; xw[b][3] = t.w;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int p = (int)((pw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
#pragma unroll
        for (int b = 0; b < B; ++b) xs[b * xp_len + p] = (uint16_t)(xw[b][j >> 1] >> (16 * (j & 1)));
    }
}

// A workgroup of T x S waves owns T tiles of 16 rows; the S waves of a tile
// take the groups g = s, s + S, ... of every row.  Lane l holds row l & 15 of
// its tile and chunk c = l >> 4 (32 channels) of each of its groups, so a
// wave's weight load is one contiguous kilobyte (a tile's group block), and
// the 16 lanes of a chunk read the same activations (an LDS broadcast).  The
// activation rows are staged in LDS once per workgroup - copied from the
// permuted row, or (GATHER) scattered from the natural-order row through the
// channel-position table - while the first window of weight groups is
// already in flight.  Weights and scales stream through a window of
// tile_window<B>() register slots; every window but the last refills each slot
// right after using it, unconditionally (past the last group the refill
// rereads it), so every wait on a slot counts loads exactly.  Lane sums meet
// over the four chunks with cross-lane shuffles and over the S waves in LDS,
// in a fixed order.
template <int B, int T, int S, bool GATHER>
__global__ __launch_bounds__(64 * T * S) void qgemv_int4o_tile(Int4oArgs a, GatherArgs ga) {
    extern __shared__ __align__(16) uint16_t xs[];   // [B][xp_len], then float corr[B][4 * G4]
    __shared__ float red[S > 1 ? T * S : 1][B][16];
    constexpr int W = T * S, NT = 64 * W, P = tile_window<B>();
    constexpr int SC = 4;                            // staged pieces per thread issued before the weights
    // the wave index is uniform across the wave: read it into a scalar
    // register, so that everything derived from it (the tile, the groups, the
    // weight and scale addresses of every refill) is scalar arithmetic
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int tile = wave / S, s = wave % S;
    const int m = lane & 15, c = lane >> 4;
    const int tiles = (a.N + 15) >> 4;
    const int t16 = blockIdx.x * T + tile;
    const bool tile_ok = t16 < tiles;
    const int tb = tile_ok ? t16 : 0;
    const int G4 = a.G4, xp_len = a.xp_len, bg_len = 128 * G4;

    // 1. activation loads (16-byte pieces; unconditional, out-of-range pieces reread piece 0)
    uint4 pv[SC];
    uint4 xv[SC][GATHER ? B : 1];
    const int npieces = GATHER ? (ga.K + 7) >> 3 : B * xp_len / 8;
    const int ldx16 = GATHER ? ga.ldx >> 3 : 0;
#pragma unroll
    for (int i = 0; i < SC; ++i) {
        const int p = tid + i * NT;
        const int pp = p < npieces ? p : 0;
        if (GATHER) {
            pv[i] = as_uint4(((const g_u32x4*)ga.pos)[pp]);
#pragma unroll
            for (int b = 0; b < B; ++b) xv[i][b] = as_uint4(((const g_u32x4*)ga.x)[b * ldx16 + pp]);
        } else {
            xv[i][0] = as_uint4(((const g_u32x4*)a.xp)[pp]);
        }
    }

    // 2. weight window: this wave's groups s, s + S, ... (J of them), and
    // the first outlier chunk.  Every load is issued unconditionally (a wave
    // without groups rereads its tile's group 0; with no groups or no
    // outliers at all, the loads read the start of the activation row and
    // are ignored): a load skipped on some path makes the compiler count
    // every later wait as if it had not been issued, and the activation
    // staging would then wait for the whole window.
    const int J = G4 > s ? (G4 - 1 - s) / S + 1 : 0;
    const uint4* dummy = reinterpret_cast<const uint4*>(GATHER ? ga.x : a.xp);
    // weight and scale addresses: a scalar base per (tile, group) plus a
    // 32-bit per-lane byte offset (lane (m, c): 16 bytes of the 1 KB block,
    // and the 16-bit scale of row m), so a refill costs no vector address
    // arithmetic (measured on MI355X: the 70B-shaped step at b = 1 from about
    // 90.8 to 85.8 us per layer, with the plans below and the biased-sum seed
    // of int4o_row_chunk; the 3B-shaped step 24.2 -> 23.7 us per layer)
    const char* wtile = reinterpret_cast<const char*>(G4 > 0 ? a.codes + (int64_t)tb * G4 * 64 : dummy);
    const char* stile = reinterpret_cast<const char*>(G4 > 0 ? a.scales + (int64_t)tb * G4 * 16 : (const uint16_t*)dummy);
    const uint32_t woff = G4 > 0 ? (uint32_t)(c * 16 + m) * 16u : 0u;
    const uint32_t soff = G4 > 0 ? (uint32_t)m * 2u : 0u;
    auto wload = [&](int g) {
        return gload_nt(reinterpret_cast<const uint4*>(wtile + (size_t)(uint32_t)g * 1024u + woff));
    };
    auto sload = [&](int g) {
        return (uint32_t)*gptr(reinterpret_cast<const uint16_t*>(stile + (size_t)(uint32_t)g * 32u + soff));
    };
    uint4 wq[P];
    uint32_t sq[P];
#pragma unroll
    for (int u = 0; u < P; ++u) {
        const int g = G4 > 0 ? (J > 0 ? s + S * (u < J ? u : J - 1) : 0) : 0;
        wq[u] = wload(g);
        sq[u] = sload(g);
    }
    const uint4* ob = a.wout + (int64_t)tb * a.no8 * 16 + m;
    const int i80 = 4 * s + c;
    const uint4 wo0 = gload_u4(a.no8 > 0 ? ob + (int64_t)(i80 < a.no8 ? i80 : 0) * 16 : dummy);
    // a wave with a second outlier step (more than 4 S chunks of outlier
    // columns, e.g. 288 columns over eight waves) loads it here too, so that
    // no wave ends on a memory round trip; the load is unconditional (a wave
    // without a second step rereads its first chunk, a line already in
    // flight), since a load on one path only would make the compiler wait for
    // every load in flight where the paths join
    const int i81 = 4 * (s + S) + c;
    const uint4 wo1 = gload_u4(a.no8 > 0 ? ob + (int64_t)(i81 < a.no8 ? i81 : (i80 < a.no8 ? i80 : 0)) * 16 : dummy);

    // 3. activations into LDS
#pragma unroll
    for (int i = 0; i < SC; ++i) {
        const int p = tid + i * NT;
        if (p < npieces) {
            if (GATHER) {
                uint4 x1[B];
#pragma unroll
                for (int b = 0; b < B; ++b) x1[b] = xv[i][b];
                if (p == npieces - 1 && (ga.K & 7)) scatter8<B>(xs, xp_len, x1, pv[i]);
                else scatter8_full<B>(xs, xp_len, x1, pv[i], (lane >> 3) & 3);
            } else {
                *(__attribute__((address_space(3))) u32x4*)&xs[8 * p] =
                    (u32x4){xv[i][0].x, xv[i][0].y, xv[i][0].z, xv[i][0].w};
            }
        }
    }
    for (int p = tid + SC * NT; p < npieces; p += NT) {
        if (GATHER) {
            uint4 x1[B];
            const uint4 p1 = as_uint4(((const g_u32x4*)ga.pos)[p]);
#pragma unroll
            for (int b = 0; b < B; ++b) x1[b] = as_uint4(((const g_u32x4*)ga.x)[b * ldx16 + p]);
            if (p == npieces - 1 && (ga.K & 7)) scatter8<B>(xs, xp_len, x1, p1);
            else scatter8_full<B>(xs, xp_len, x1, p1, (lane >> 3) & 3);
        } else {
            const uint4 v = as_uint4(((const g_u32x4*)a.xp)[p]);
            *(__attribute__((address_space(3))) u32x4*)&xs[8 * p] = (u32x4){v.x, v.y, v.z, v.w};
        }
    }
    if (GATHER) {
        // padding of the permuted row: [K_bg, bg_len) and [bg_len + n_out, xp_len)
        for (int k = ga.K_bg + tid; k < bg_len; k += NT)
#pragma unroll
            for (int b = 0; b < B; ++b) xs[b * xp_len + k] = 0;
        for (int k = bg_len + ga.n_out + tid; k < xp_len; k += NT)
#pragma unroll
            for (int b = 0; b < B; ++b) xs[b * xp_len + k] = 0;
    }
    lds_barrier();

    // 4. bias correction of every 32-channel background chunk, per batch row
    const lx_ptr xl = (lx_ptr)xs;
    float* corr = reinterpret_cast<float*>(xs + B * xp_len);
    const int nq = 4 * G4;
    for (int e = tid; e < B * nq; e += NT) {
        const int b = e / nq, q = e - b * nq;
        uint4 xq[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) xq[k] = load_x16(xl + b * xp_len + 32 * q + 8 * k);
        corr[e] = -activation_chunk_correction(xq);     // negated: it seeds the low-nibble sums
    }
    lds_barrier();

    // 5. background groups.  A slot is consumed before its refill is issued,
    // so the refill can land in the same registers: with the old value still
    // live, the compiler moves refilled slots back at the loop latch, which
    // waits for every load in flight once per window.  The last window (the
    // only one for rows that fit in one) takes no refills.
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.0f;
    const uint32_t bias = bias_reg();
    auto consume = [&](int j, uint4 w, uint32_t sq1) {
        const int g = s + S * j;
        // the scale word is unpacked only here, after the wait for its slot
        asm volatile("" : "+v"(sq1));
        const float sc = h_to_f((uint16_t)sq1);
        uint4 xg[B][4];
        float cg[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
#pragma unroll
            for (int q = 0; q < 4; ++q) xg[b][q] = load_x16(xl + b * xp_len + 128 * g + 32 * c + 8 * q);
            cg[b] = corr[b * nq + 4 * g + c];
        }
        int4o_row_chunk<B>(w, sc, xg, cg, acc, bias);
    };
    int j0 = 0;
    for (; j0 + P < J; j0 += P) {
#pragma unroll
        for (int u = 0; u < P; ++u) {
            const int j = j0 + u;
            consume(j, wq[u], sq[u]);
            const int gn = s + S * (j + P < J ? j + P : J - 1);
            wq[u] = wload(gn);
            sq[u] = sload(gn);
        }
    }
#pragma unroll
    for (int u = 0; u < P; ++u)
        if (j0 + u < J) consume(j0 + u, wq[u], sq[u]);

    // 6. FP16 outlier columns: step st covers outlier chunks 4 st .. 4 st + 3
    // (lane chunk c); the chunks of the first two steps were loaded with the
    // window
    for (int st = s; 32 * st < 8 * a.no8; st += S) {
        const int i8 = 4 * st + c;
        const bool in = i8 < a.no8;
        const uint4 wo = st == s ? wo0 : st == s + S ? wo1 : gload_u4(ob + (int64_t)(in ? i8 : 0) * 16);
        if (in) {
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const uint4 xo = load_x16(xl + b * xp_len + bg_len + 8 * i8);
                float v = acc[b];
                v = dot2(as_h2(wo.x), as_h2(xo.x), v);
                v = dot2(as_h2(wo.y), as_h2(xo.y), v);
                v = dot2(as_h2(wo.z), as_h2(xo.z), v);
                v = dot2(as_h2(wo.w), as_h2(xo.w), v);
                acc[b] = v;
            }
        }
    }

    // 7. sums over the four chunk lanes, then over the S waves of the tile
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = sum_over_chunks(acc[b]);
    if (S > 1) {
        if (c == 0)
#pragma unroll
            for (int b = 0; b < B; ++b) red[wave][b][m] = acc[b];
        __syncthreads();
        if (s == 0 && c == 0)
#pragma unroll
            for (int b = 0; b < B; ++b) {
                float v = acc[b];
                for (int p = 1; p < S; ++p) v += red[wave + p][b][m];
                acc[b] = v;
            }
    }
    if (s == 0 && c == 0 && tile_ok) {
        const int n = t16 * 16 + m;
        if (n < a.N)
#pragma unroll
            for (int b = 0; b < B; ++b) *gptr(a.y + (int64_t)b * a.ldy + n) = f_to_h(acc[b]);
    }
}

// --------------------------------------------------------- INT8, batch <= 8

// Which INT8 kernel serves a product of N rows at batch b (measured on
// MI355X over the 9B-shaped products): the vector kernel streams the
// row-major codes at up to 5 TB/s but re-reads each activation chunk from L1
// for every four rows and spends 2 dot2 per 4 weights per batch row, so its
// time grows with b; the matrix-core kernel's time does not grow with b but
// its wave loads cover 16 rows x 64 bytes, which streams slower.  The matrix
// cores win on wide products from b = 4 (9B layer at b = 4, gate|up on the
// matrix cores: 77.3 -> 74.1 us; at b = 3 the two are even) and on mid-size
// ones from b = 7; narrow ones stay on the vector ALU.
inline bool int8_use_mfma(int64_t N, int64_t b) {
    const int64_t tiles = (N + 15) / 16;
    return (tiles >= 1024 && b >= 4) || (tiles >= 512 && b >= 7);
}

struct Int8Args {
    const uint4* codes;     // [N4][Kd/16] chunks of 16 bytes
    const uint16_t* x;      // [b][ldx]
    uint16_t* y;            // [b][ldy]
    int N, K, CPR, ldx, ldy, nseg;
    int seg_end[WOQ_MAX_SEGMENTS];
    float seg_scale[WOQ_MAX_SEGMENTS];
};

// One quad of four rows per wave; lane l takes the 16-byte chunks
// l, l + 64, ... of each row.  The full chunks stream through two register
// buffers: the loads of chunk i + 1 are in flight while chunk i is consumed,
// and a buffer is refilled only after it has been consumed, so no register
// moves (and no waits for loads still in flight) sit at the loop latch.
// Every load in the loop is unconditional: a lane past the last full chunk
// rereads it and multiplies it by zero activations.  The chunk that holds the
// end of a row not a multiple of 16 long is read element by element, by the
// lane it falls to, after the loop.
template <int B>
__global__ __launch_bounds__(64) void qgemv_int8_valu(Int8Args a) {
    const int lane = threadIdx.x;
    const int quad = blockIdx.x;
    const uint4* w0 = a.codes + (int64_t)quad * 4 * a.CPR;
    const int nfull = a.K >> 4;            // chunks whose 16 channels are all real
    const int iters = (nfull + 63) >> 6;   // the same for every lane
    float acc[4][B];
    float sx[B];
    zero_acc(acc);
#pragma unroll
    for (int b = 0; b < B; ++b) sx[b] = 0.0f;
    struct Buf {
        uint4 w[4];
        uint4 x[B][2];
    };
    auto load = [&](Buf& d, int i) {
        const int c0 = lane + 64 * i;
        const int cc = c0 < nfull ? c0 : nfull - 1;
#pragma unroll
        for (int r = 0; r < 4; ++r) d.w[r] = gload_nt(w0 + r * a.CPR + cc);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const gx_ptr xs = (gx_ptr)(a.x + (int64_t)b * a.ldx + 16 * cc);
            d.x[b][0] = load_x16(xs);
            d.x[b][1] = load_x16(xs + 8);
        }
    };
    auto consume = [&](const Buf& d, int i) {
        const bool real = lane + 64 * i < nfull;
        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
        uint4 xv[B][2];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            xv[b][0] = real ? d.x[b][0] : z;
            xv[b][1] = real ? d.x[b][1] : z;
        }
        int8_chunk<B>(d.w, xv, acc, sx);
    };
    // the scheduling barriers keep each buffer's loads ahead of the other
    // buffer's waits (the scheduler would otherwise sink them below them)
    if (iters > 0) {
        Buf p, q;
        load(p, 0);
        int i = 0;
        for (; i + 2 < iters; i += 2) {
            load(q, i + 1);
            __builtin_amdgcn_sched_barrier(0);
            consume(p, i);
            load(p, i + 2);
            __builtin_amdgcn_sched_barrier(0);
            consume(q, i + 1);
        }
        if (iters - i == 2) {
            load(q, i + 1);
            __builtin_amdgcn_sched_barrier(0);
            consume(p, i);
            consume(q, i + 1);
        } else {
            consume(p, i);
        }
    }
    if (nfull * 16 < a.K && lane == (nfull & 63)) {
        uint4 w[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = gload_nt(w0 + r * a.CPR + nfull);
        uint4 xv[B][2];
        const int k0 = 16 * nfull;
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
        int8_chunk<B>(w, xv, acc, sx);
    }
    int8_unbias<B>(acc, sx);
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

// y[r][n] = fp16(sum over s of part[s][r][n]), s in order: the split-K
// partial sums of the matrix-core kernel, added in a fixed order.
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ part, int splits, int b, int N,
                                                            uint16_t* __restrict__ y, int ldy) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)b * N) return;
    const int r = (int)(i / N), n = (int)(i % N);
    float v = *gptr(part + i);
    for (int q = 1; q < splits; ++q) v += *gptr(part + (int64_t)q * b * N + i);
    *gptr(y + (int64_t)r * ldy + n) = f_to_h(v);
}

// ------------------------------------------------ INT8, matrix cores (b >= 3)

// A workgroup of T x S waves owns T tiles of 16 output rows of the row-major
// INT8 layout; the S waves of a tile split the 64-channel groups of every K
// chunk (CH groups) between them.  Lane l loads the 16-byte piece l >> 4 of
// group g of row l & 15 (channels 64g + 16(l >> 4) .. + 15); its first and
// last 8 codes are the A operands of two v_mfma_f32_16x16x32_f16 steps whose
// k slots 8(l >> 4) .. + 7 stand for those channels, and the B operands (batch
// column l & 15) read the same channels from the activations staged in LDS.
// The per-tensor (per-segment) scale multiplies the fp32 sum once, at the end.
// Activations are staged per K chunk (all b columns) once for the T tiles, two
// chunks ahead of use through registers, as in the INT4O matrix-core kernel.
template <int T, int S>
__global__ __launch_bounds__(64 * T * S) void qgemm_int8_mfma(Int8Args a, int b) {
    constexpr int W = T * S;
    constexpr int CH = S > 8 ? S : 8;                 // 64-channel groups per chunk
    constexpr int KC = CH / S;                        // groups per wave per chunk
    constexpr int P = 8;                              // weight window (groups)
    static_assert(P % KC == 0, "window must hold whole chunks");
    constexpr int UNR = P / KC < 2 ? 2 : P / KC;
    static_assert(UNR % 2 == 0 && UNR % (P / KC) == 0, "unroll");
    constexpr int COLS = 16;                          // batch columns of the B operand
    constexpr int XS = CH * 64 + 8;                   // LDS column stride (fp16), padded against bank conflicts
    constexpr int PPC = CH * 8;                       // 16-byte pieces of one column per chunk
    constexpr int NPT = (COLS * PPC + 64 * W - 1) / (64 * W);
    constexpr int RED = 4 * W * 16 * 17;
    constexpr int XSB = 2 * 2 * COLS * XS;
    __shared__ __align__(16) uint16_t lds[(XSB > RED ? XSB : RED) / 2];
    uint16_t (*xs)[COLS][XS] = reinterpret_cast<uint16_t (*)[COLS][XS]>(lds);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int tile = wave / S, s = wave % S;
    const int m = lane & 15;
    const int c = lane >> 4;
    const int tiles = (a.N + 15) >> 4;
    const int t16 = blockIdx.x * T + tile;
    const bool tile_ok = t16 < tiles;
    const int n4 = (a.N + 3) & ~3;                    // rows of the layout
    const int row = tile_ok && t16 * 16 + m < n4 ? t16 * 16 + m : 0;
    const int G = a.CPR / 4;                          // 64-channel groups per row (Kd / 64)
    const int nchunks = (G + CH - 1) / CH;

    f4 acc = (f4){0.f, 0.f, 0.f, 0.f};
    for (int e = tid; e < 2 * COLS * XS; e += 64 * W) {
        const int col = (e / XS) % COLS;
        if (col >= b) lds[e] = 0;
    }

    // staging: piece p of chunk k -> column p / PPC, channels 8 (p % PPC) of the chunk
    uint4 stg[2][NPT];
    auto stage_load = [&](uint4 (&r)[NPT], int k) {
        const int kk = k < nchunks ? k : 0;
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const int p = tid + i * 64 * W;
            const int col = p / PPC, ch = kk * CH * 64 + 8 * (p % PPC);
            const bool ok = col < b && ch < a.K;
            r[i] = load_x16((gx_ptr)(a.x + (ok ? (int64_t)col * a.ldx + ch : 0)));
        }
    };
    // pieces past the row (or past the batch) are zeroed here, when they are
    // stored, so that no load is waited for as soon as it is issued
    auto stage_store = [&](const uint4 (&r)[NPT], int buf, int k) {
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const int p = tid + i * 64 * W;
            const int col = p / PPC, off = p % PPC, ch = k * CH * 64 + 8 * off;
            if (col < b) {
                uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (ch + 2 * j >= a.K) w[j] = 0;
                    else if (ch + 2 * j + 1 >= a.K) w[j] &= 0xFFFFu;
                }
                *(__attribute__((address_space(3))) u32x4*)&xs[buf][col][8 * off] = (u32x4){w[0], w[1], w[2], w[3]};
            }
        }
    };

    // this wave's groups: in chunk k, k*CH + s*KC + kk (kk < KC); j counts them
    const int full = G / CH, rem = G - full * CH;
    const int J = full * KC + min(max(rem - s * KC, 0), KC);
    auto group_of = [&](int j) { return (j / KC) * CH + s * KC + (j % KC); };
    const uint4* wld = a.codes + (int64_t)row * a.CPR + c;

    // Loads are unconditional and go out in the order the loop keeps them in
    // (chunk c issues the activation loads of chunk c + 2, then the window
    // slots of chunk c + WC; the prologue plays chunks -WC .. -1), so every
    // wait counts loads exactly and the window runs ahead across chunks.
    // Without groups (K = 0 is refused by the entry points, so never) the
    // window would reread row 0's first chunk.
    constexpr int WC = P / KC;
    uint4 wq[P];
#pragma unroll
    for (int c2 = 0; c2 < 2 - WC; ++c2) {
        stage_load(stg[c2], c2);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int cp = -WC; cp < 0; ++cp) {
        if (cp + 2 >= 0) {
            stage_load(stg[(cp + 2) & 1], cp + 2);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
            const int j = (cp + WC) * KC + kk;
            wq[j] = gload_nt(wld + 4 * (j < J ? group_of(j) : 0));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (nchunks > 0) stage_store(stg[0], 0, 0);
    lds_barrier();
    // one chunk; a slot is refilled after its products, into the same registers
    auto chunk = [&](int k, int cb) {
        stage_load(stg[cb & 1], k + 2);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
            const int u = (cb * KC + kk) % P;
            const int j = k * KC + kk;
            const bool gv = k * CH + s * KC + kk < G;
            const uint4 w = wq[u];
            h2 p0, p1, p2, p3, p4, p5, p6, p7;
            int8_pairs(w.x, p0, p1);
            int8_pairs(w.y, p2, p3);
            int8_pairs(w.z, p4, p5);
            int8_pairs(w.w, p6, p7);
            const h8 A0 = (h8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
            const h8 A1 = (h8){p4[0], p4[1], p5[0], p5[1], p6[0], p6[1], p7[0], p7[1]};
            const int gl = s * KC + kk;
            const lx_ptr xb = (lx_ptr)&xs[cb & 1][m][64 * gl + 16 * c];
            const h8 B0 = __builtin_bit_cast(h8, load_x16(xb));
            const h8 B1 = __builtin_bit_cast(h8, load_x16(xb + 8));
            if (gv) {
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, B0, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, B1, acc, 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            wq[u] = gload_nt(wld + 4 * (j + P < J ? group_of(j + P) : 0));
            __builtin_amdgcn_sched_barrier(0);
        }
        if (k + 1 < nchunks) stage_store(stg[(cb + 1) & 1], (cb + 1) & 1, k + 1);
        lds_barrier();
    };
    const int whole = nchunks / UNR;
    for (int it = 0; it < whole; ++it) {
#pragma unroll
        for (int cb = 0; cb < UNR; ++cb) chunk(it * UNR + cb, cb);
    }
    const int rest = nchunks - whole * UNR;
#pragma unroll
    for (int cb = 0; cb < UNR - 1; ++cb)
        if (cb < rest) chunk(whole * UNR + cb, cb);

    // lane (c, m) holds rows 4c .. 4c + 3 of the tile, batch column m
    if (S > 1) {
        typedef float RedTile[16][17];
        RedTile* red = reinterpret_cast<RedTile*>(lds);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][4 * c + i][m] = acc[i];
        __syncthreads();
        if (s == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = acc[i];
                for (int p = 1; p < S; ++p) v += red[wave + p][4 * c + i][m];
                acc[i] = v;
            }
        }
    }
    if (s == 0 && tile_ok && m < b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = t16 * 16 + 4 * c + i;
            if (n < a.N) {
                float sc = a.seg_scale[a.nseg - 1];
                for (int q = a.nseg - 1; q >= 0; --q)
                    if (n < a.seg_end[q]) sc = a.seg_scale[q];
                *gptr(a.y + (int64_t)m * a.ldy + n) = f_to_h(acc[i] * sc);
            }
        }
    }
}

// ------------------------------------------------ INT4O, matrix cores (b >= 8)

// Column stride (fp16) of the whole-row staging of the matrix-core kernel: the
// row rounded up to 128 channels plus 8, so that consecutive columns start 16
// bytes apart modulo 256 bytes, as the padded chunk buffers of the staged form
// do (fewer LDS bank conflicts on the B-operand reads).
__host__ __device__ inline int int4o_whole_stride(int xp_len) { return ((xp_len + 127) & ~127) + 8; }

// A workgroup of T x S waves owns T tiles of 16 output rows; the S waves of a
// tile split the groups of every K chunk (CH groups) between them.  Lane l
// holds row l & 15 of its tile and the 16-byte chunk l >> 4 of each group (32
// channels) - exactly the A operand of v_mfma_f32_16x16x32_f16 for four
// k-steps: the unscaled pairs feed steps 0 and 2, the pairs that carry
// 16 x code feed steps 1 and 3 into a second accumulator that is divided by
// 16 before the group scale is applied.
//
// The B operand (activations, batch column l & 15) is read from LDS.  The
// workgroup stages each K chunk of the permuted activations (all b columns)
// once for its T tiles, two chunks ahead of use: the loads of chunk k + 2 are
// issued when chunk k starts, held in registers, and written to LDS at the end
// of chunk k + 1, so they return in the shadow of the weight stream instead of
// stalling it.  Each wave streams its weights and scales through a window of
// P register slots that runs ahead across chunk boundaries.  Every load is
// unconditional (clamped to a valid address, results unused), so the number
// of loads in flight is the same on every path and each wait is exact.
// Partial sums of the S waves of a tile meet in LDS.
//
// WHOLE (8 staged columns only): the permutation is folded in instead.  The
// workgroup gathers the whole permuted row of all 8 columns into LDS once,
// scattered from the natural-order activations ga.x through the
// channel-position table ga.pos (as the vector kernel does) while its first
// weight window is in flight; the chunk loop then runs without staging or
// barriers, and lanes of batch columns 8..15 read columns 0..7 again (their
// outputs are never stored; the MFMA columns are independent).  Groups, their
// order per wave, the matrix-core steps and the reductions are those of the
// staged form, so both give the same bits.
//
// BIAS (plans of one wave per tile group and two tiles per wave, 16 or more
// staged columns): the code pairs enter the matrix cores with their exponent
// bias (code + 1032, 16 code + 1152) instead of having it subtracted, as in
// the vector kernel, and the low-nibble accumulator of each group starts from
// minus the group's correction 1032 (sum of the activations over the group's
// low-nibble channels) + 72 (sum over the high-nibble ones), which the staging
// computes per group and batch column from the pieces it writes (four dot2
// per piece and a fixed-order sum over the 16 lanes that hold a group).  The
// products stay exact; the cancellation costs about 1e-5 of a group's
// magnitude in fp32.
template <int NBT, int T, int S, int RB, bool HALF, bool WHOLE = false>
__global__ __launch_bounds__(64 * T * S) void qgemm_int4o_mfma(Int4oArgs a, int b, GatherArgs ga) {
    static_assert(!HALF || NBT == 1, "half-width staging is for one column tile");
    static_assert(!WHOLE || HALF, "the whole-row form stages 8 columns");
    constexpr bool BIAS = !HALF && !WHOLE && S == 1 && RB == 2;
    constexpr int W = T * S;
    // groups per chunk: with the K split, chunks of 8 groups halve the
    // barriers per group (measured faster on MI355X); wide batches are bound
    // by the LDS the staged columns need; with 8 staged columns (b <= 8) the
    // same LDS holds chunks of 16 groups
    constexpr int CHB = NBT == 1 ? (S >= 2 ? (HALF ? 16 : 8) : 4) : NBT == 2 ? 4 : 2;
    constexpr int CH = S > CHB ? S : CHB;             // groups per chunk
    constexpr int KC = CH / S;                        // groups per wave per chunk
    // weight window (groups, whole chunks): as in the vector kernel a
    // shallower window lets the staged activations arrive sooner.  Where
    // whole chunks allow it, four groups for one column tile and two for two
    // (measured on MI355X over the 70B-shaped layer: 122.3 -> 120.2 us at
    // b = 8, 117.5 -> 115.9 us at b = 4, 132.7 -> 128.6 us at b = 16 with
    // four instead of eight; 176.2 -> 174.5 us at b = 32 with two instead of
    // four); otherwise eight for one column tile, four for more
    constexpr int P = NBT == 1 ? (4 % KC == 0 ? 4 : 8) : (NBT == 2 && 2 % KC == 0 ? 2 : 4);
    static_assert(P % KC == 0, "window must hold whole chunks");
    constexpr int UNR = P / KC < 2 ? 2 : P / KC;      // chunks per unrolled loop body (even)
    static_assert(UNR % 2 == 0 && UNR % (P / KC) == 0, "unroll");
    constexpr int COLS = HALF ? 8 : 16 * NBT;         // staged batch columns (the B operand has 16 * NBT)
    constexpr int XS = CH * 128 + 8;                  // LDS column stride (fp16), padded against bank conflicts
    constexpr int PPC = CH * 16;                      // 16-byte pieces of one column per chunk
    constexpr int NPT = (COLS * PPC + 64 * W - 1) / (64 * W);   // staged pieces per thread (b = COLS)
    constexpr int RED = 4 * W * RB * NBT * 16 * 17;
    // with HALF, lanes of batch columns 8..15 read an extra column that
    // holds zeros for the whole kernel (no branch, no register clears)
    constexpr int XCOLS = HALF ? COLS + 1 : COLS;
    constexpr int XSB = 2 * 2 * XCOLS * XS;
    __shared__ __align__(16) uint16_t lds[WHOLE ? 8 : (XSB > RED ? XSB : RED) / 2];
    uint16_t (*xs)[XCOLS][XS] = reinterpret_cast<uint16_t (*)[XCOLS][XS]>(lds);
    // BIAS: minus the correction of each group of the staged chunk, per column
    __shared__ float ncorr[BIAS ? 2 * CH * COLS : 1];
    // WHOLE: the permuted rows of the 8 staged columns, [8][XW] fp16 (dynamic LDS)
    extern __shared__ __align__(16) uint16_t xw[];
    const int XW = int4o_whole_stride(a.xp_len);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int tile = wave / S, s = wave % S;
    const int m = lane & 15;           // row within the tile (A) / batch column (B)
    const int c = lane >> 4;           // 32-channel chunk of the group / k-block
    const int tiles = (a.N + 15) >> 4;
    // this wave's RB tiles (register blocking: every staged activation read
    // from LDS feeds RB tiles' matrix-core steps)
    const int t16 = (blockIdx.x * T + tile) * RB;
    bool tile_ok[RB];
    int tb[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        tile_ok[r] = t16 + r < tiles;
        tb[r] = tile_ok[r] ? t16 + r : 0;
    }
    const int split = blockIdx.y;
    const int G4s = a.G4;                             // groups per tile row in memory
    const int gbeg = a.gsplit ? split * a.gsplit : 0; // first group of this launch's K range
    const int G4 = a.gsplit ? max(0, min(a.gsplit, G4s - gbeg)) : G4s;
    const int xp_len = a.xp_len;
    const int nchunks = (G4 + CH - 1) / CH;
    const int bgl = 128 * G4;
    const uint16_t* xpb = a.xp + 128 * gbeg;          // this K range's activations

    f4 acc[RB][NBT];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < NBT; ++t) acc[r][t] = (f4){0.f, 0.f, 0.f, 0.f};

    // columns b .. XCOLS-1 of both buffers hold zeros for the whole kernel
    if constexpr (!WHOLE)
        for (int e = tid; e < 2 * XCOLS * XS; e += 64 * W) {
            const int col = (e / XS) % XCOLS;
            if (col >= b) lds[e] = 0;
        }

    // staging: piece p of chunk k -> column p / PPC, channels 8 (p % PPC) of the chunk
    uint4 stg[2][NPT];
    auto stage_load = [&](uint4 (&r)[NPT], int k) {
        const int kk = k < nchunks ? k : 0;
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const int p = tid + i * 64 * W;
            const int col = p / PPC, ch = kk * CH * 128 + 8 * (p % PPC);
            const bool ok = col < b && ch < bgl;
            r[i] = load_x16((gx_ptr)(ok ? xpb + (int64_t)col * xp_len + ch : a.xp));
        }
    };
    auto stage_store = [&](const uint4 (&r)[NPT], int buf, int k) {
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const int p = tid + i * 64 * W;
            const int col = p / PPC, off = p % PPC;
            if (col < b) {
                const bool ok = k * CH * 128 + 8 * off < bgl;   // past the last group: zeros
                *(__attribute__((address_space(3))) u32x4*)&xs[buf][col][8 * off] =
                    ok ? (u32x4){r[i].x, r[i].y, r[i].z, r[i].w} : (u32x4){0u, 0u, 0u, 0u};
            }
        }
        if constexpr (BIAS) {
            // the 16 pieces of a (group, column) sit on the 16 lanes of one
            // row (PPC and the thread count are multiples of 16); pieces of
            // even index within their group meet low-nibble codes (weight
            // 1032), odd ones high-nibble codes (72)
#pragma unroll
            for (int i = 0; i < NPT; ++i) {
                const int p = tid + i * 64 * W;
                const int col = p / PPC, off = p % PPC;
                const bool ok = col < b && k * CH * 128 + 8 * off < bgl;
                const h2 wt = as_h2((off & 1) ? 0x54805480u : 0x64086408u);
                float v = dot2(as_h2(r[i].x), wt, 0.0f);
                v = dot2(as_h2(r[i].y), wt, v);
                v = dot2(as_h2(r[i].z), wt, v);
                v = dot2(as_h2(r[i].w), wt, v);
                v = row16_sum(ok ? v : 0.0f);
                if ((lane & 15) == 0 && col < COLS) ncorr[(buf * CH + (off >> 4)) * COLS + col] = -v;
            }
        }
    };

    // this wave's groups: in chunk k, k*CH + s*KC + kk (kk < KC); j counts them
    const int full = G4 / CH, rem = G4 - full * CH;
    const int J = full * KC + min(max(rem - s * KC, 0), KC);
    auto group_of = [&](int j) { return (j / KC) * CH + s * KC + (j % KC); };
    // tile layout: lane (m, c) reads 16 bytes of the tile's 1 KB block of group g,
    // and the scales of D rows 4c .. 4c + 3 (8 contiguous bytes)
    // a scalar base per tile and group plus a 32-bit per-lane byte offset,
    // with the wave index in a scalar register: no vector address arithmetic
    // per refill (with the zero column below, the 70B-shaped step at b = 4
    // went from 119 to 115 us per layer and at b = 8 from 123 to 120 us; no
    // change at b = 32)
    const char* wtb[RB];
    const char* stb[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        wtb[r] = reinterpret_cast<const char*>(a.codes + ((int64_t)tb[r] * G4s + gbeg) * 64);
        stb[r] = reinterpret_cast<const char*>(a.scales + ((int64_t)tb[r] * G4s + gbeg) * 16);
    }
    uint32_t woff = (uint32_t)(c * 16 + m) * 16u, soff = (uint32_t)c * 8u;

    // Every load below is unconditional, so each wait counts loads exactly
    // and the weight window keeps running ahead across chunk boundaries (a
    // load skipped on some path makes the compiler count every later wait as
    // if it had not been issued, which drained the window at each chunk).
    // Without groups (an empty K range) the loads read the activation row.
    if (nchunks == 0) {
#pragma unroll
        for (int r = 0; r < RB; ++r) wtb[r] = stb[r] = reinterpret_cast<const char*>(a.xp);
        woff = soff = 0;
    }
    auto wload = [&](int r, int g) {
        return gload_nt(reinterpret_cast<const uint4*>(wtb[r] + (size_t)(uint32_t)g * 1024u + woff));
    };
    auto sload = [&](int r, int g) {
        return gload_u2(reinterpret_cast<const uint2*>(stb[r] + (size_t)(uint32_t)g * 32u + soff));
    };
    // The loads go out in the order the loop keeps them in: chunk c issues
    // the activation loads of chunk c + 2 and then the window slots of chunk
    // c + WC, so the prologue plays chunks -WC .. -1.  The wait counts at the
    // loop head then hold for the first pass and for later ones alike.  The
    // scheduling barriers keep the compiler from reordering the loads.
    constexpr int WC = P / KC;                        // chunks the window spans
    uint4 wq[P][RB];
    uint2 sc[P][RB];
    // WHOLE: the first pieces of the row (a channel-position piece and the 8
    // columns' activations for it) go out before the weight window
    constexpr int SCW = WHOLE ? (W >= 16 ? 1 : 2) : 1;
    const int npieces = (ga.K + 7) >> 3;
    const int ldx16 = ga.ldx >> 3;
    uint4 pvw[SCW], xvw[SCW][WHOLE ? 8 : 1];
    if constexpr (WHOLE) {
#pragma unroll
        for (int i = 0; i < SCW; ++i) {
            const int p = tid + i * 64 * W;
            const int pp = p < npieces ? p : 0;
            pvw[i] = as_uint4(((const g_u32x4*)ga.pos)[pp]);
#pragma unroll
            for (int c8 = 0; c8 < 8; ++c8)
                xvw[i][c8] = as_uint4(((const g_u32x4*)ga.x)[(c8 < b ? c8 : 0) * ldx16 + pp]);
        }
        __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
        for (int c2 = 0; c2 < 2 - WC; ++c2) {
            stage_load(stg[c2], c2);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int cp = -WC; cp < 0; ++cp) {
        if (!WHOLE && cp + 2 >= 0) {
            stage_load(stg[(cp + 2) & 1], cp + 2);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
            const int j = (cp + WC) * KC + kk;
            const int g = j < J ? group_of(j) : 0;
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                wq[j][r] = wload(r, g);
                sc[j][r] = sload(r, g);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if constexpr (WHOLE) {
        // scatter the row (columns b..7 hold copies of column 0, never used)
        // into its permuted positions; then zero the padding of the permuted
        // row: [K_bg, 128 G4) and [128 G4 + n_out, xp_len)
#pragma unroll
        for (int i = 0; i < SCW; ++i) {
            const int p = tid + i * 64 * W;
            if (p < npieces) {
                if (p == npieces - 1 && (ga.K & 7)) scatter8<8>(xw, XW, xvw[i], pvw[i]);
                else scatter8_full<8>(xw, XW, xvw[i], pvw[i], (lane >> 3) & 3);
            }
        }
        for (int p = tid + SCW * 64 * W; p < npieces; p += 64 * W) {
            uint4 x1[8];
            const uint4 p1 = as_uint4(((const g_u32x4*)ga.pos)[p]);
#pragma unroll
            for (int c8 = 0; c8 < 8; ++c8) x1[c8] = as_uint4(((const g_u32x4*)ga.x)[(c8 < b ? c8 : 0) * ldx16 + p]);
            if (p == npieces - 1 && (ga.K & 7)) scatter8<8>(xw, XW, x1, p1);
            else scatter8_full<8>(xw, XW, x1, p1, (lane >> 3) & 3);
        }
        for (int k = ga.K_bg + tid; k < bgl; k += 64 * W)
#pragma unroll
            for (int c8 = 0; c8 < 8; ++c8) xw[c8 * XW + k] = 0;
        for (int k = bgl + ga.n_out + tid; k < xp_len; k += 64 * W)
#pragma unroll
            for (int c8 = 0; c8 < 8; ++c8) xw[c8 * XW + k] = 0;
    } else {
        if (nchunks > 0) stage_store(stg[0], 0, 0);
    }
    lds_barrier();
    const uint32_t bias = bias_reg();
    // one chunk: stage the loads of chunk k + 2, consume this wave's KC groups
    // (a slot is refilled only after its group's products, so the refill
    // lands in the same registers), write chunk k + 1 to the other buffer
    auto chunk = [&](int k, int cb) {
        if constexpr (!WHOLE) {
            stage_load(stg[cb & 1], k + 2);      // chunk k's registers are free again
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
            const int u = (cb * KC + kk) % P;
            const int j = k * KC + kk;
            const int g = k * CH + s * KC + kk;
            const bool gv = g < G4;
            h8 A[RB][4];
            float sf[RB][4];
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const uint32_t wd[4] = {wq[u][r].x, wq[u][r].y, wq[u][r].z, wq[u][r].w};
                uint32_t s0 = sc[u][r].x, s1 = sc[u][r].y;
                asm volatile("" : "+v"(s0), "+v"(s1));   // unpacked here, after the slot's wait
                sf[r][0] = h_to_f((uint16_t)(s0 & 0xFFFF));
                sf[r][1] = h_to_f((uint16_t)(s0 >> 16));
                sf[r][2] = h_to_f((uint16_t)(s1 & 0xFFFF));
                sf[r][3] = h_to_f((uint16_t)(s1 >> 16));
                Int4Pairs pr[4];
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    if constexpr (BIAS) {
                        // biased pairs (the correction seeds the low-nibble sum)
                        const uint32_t sh = wd[d] >> 8;
                        pr[d].lo0 = as_h2((wd[d] & 0x000F000Fu) | bias);
                        pr[d].lo1 = as_h2((sh & 0x000F000Fu) | bias);
                        pr[d].hi0 = as_h2((wd[d] & 0x00F000F0u) | bias);
                        pr[d].hi1 = as_h2((sh & 0x00F000F0u) | bias);
                    } else {
                        pr[d] = int4_pairs(wd[d], bias);
                    }
                }
#pragma unroll
                for (int Pp = 0; Pp < 2; ++Pp) {
                    const Int4Pairs& e0 = pr[2 * Pp];
                    const Int4Pairs& e1 = pr[2 * Pp + 1];
                    A[r][2 * Pp + 0] = (h8){e0.lo0[0], e0.lo0[1], e0.lo1[0], e0.lo1[1],
                                            e1.lo0[0], e1.lo0[1], e1.lo1[0], e1.lo1[1]};
                    A[r][2 * Pp + 1] = (h8){e0.hi0[0], e0.hi0[1], e0.hi1[0], e0.hi1[1],
                                            e1.hi0[0], e1.hi0[1], e1.hi1[0], e1.hi1[1]};
                }
            }
            const int gl = s * KC + kk;  // group within the chunk
#pragma unroll
            for (int t = 0; t < NBT; ++t) {
                h8 Bv[4];
                {
                    const int col = HALF ? (m < COLS ? m : COLS) : 16 * t + m;
                    const lx_ptr xb = WHOLE ? (lx_ptr)&xw[(m & 7) * XW + 128 * (gv ? g : 0) + 32 * c]
                                            : (lx_ptr)&xs[cb & 1][col][128 * gl + 32 * c];
#pragma unroll
                    for (int q = 0; q < 4; ++q) Bv[q] = __builtin_bit_cast(h8, load_x16(xb + 8 * q));
                }
                f4 seed = (f4){0.f, 0.f, 0.f, 0.f};
                if constexpr (BIAS) {
                    const float nc = ncorr[((cb & 1) * CH + gl) * COLS + 16 * t + m];
                    seed = (f4){nc, nc, nc, nc};
                }
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    f4 lo = seed, hi = (f4){0.f, 0.f, 0.f, 0.f};
                    lo = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[r][0], Bv[0], lo, 0, 0, 0);
                    hi = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[r][1], Bv[1], hi, 0, 0, 0);
                    lo = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[r][2], Bv[2], lo, 0, 0, 0);
                    hi = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[r][3], Bv[3], hi, 0, 0, 0);
                    if (gv)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            acc[r][t][i] = fmaf(sf[r][i], fmaf(hi[i], 0.0625f, lo[i]), acc[r][t][i]);
                }
            }
            const int gn = j + P < J ? group_of(j + P) : 0;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                wq[u][r] = wload(r, gn);
                sc[u][r] = sload(r, gn);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // chunk k + 1 (loaded during chunk k - 1) into the other buffer, last read in chunk k - 1
        if constexpr (!WHOLE) {
            if (k + 1 < nchunks) stage_store(stg[(cb + 1) & 1], (cb + 1) & 1, k + 1);
            lds_barrier();
        }
    };
    // whole unrolled bodies first (k & 1 == cb & 1 and the slots of chunk k
    // are fixed by cb), then the last nchunks % UNR chunks
    const int whole = nchunks / UNR;
    for (int it = 0; it < whole; ++it) {
#pragma unroll
        for (int cb = 0; cb < UNR; ++cb) chunk(it * UNR + cb, cb);
    }
    const int rest = nchunks - whole * UNR;
#pragma unroll
    for (int cb = 0; cb < UNR - 1; ++cb)
        if (cb < rest) chunk(whole * UNR + cb, cb);

    // FP16 outlier columns, 32 per k-step, split over the S waves of the tile;
    // up to four k-steps' loads in flight at once
    const uint16_t* xo_base = a.xp + 128 * G4s;
    const int n_o8 = split == 0 ? a.no8 * 8 : 0;
    for (int st0 = s; st0 * 32 < n_o8; st0 += 4 * S) {
        h8 Av[RB][4], Bo[4][NBT];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int col0 = 32 * (st0 + q * S) + 8 * c;
            const bool in = col0 < n_o8;
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                Av[r][q] = __builtin_bit_cast(
                    h8, gload_u4(a.wout + ((int64_t)tb[r] * a.no8 + (in ? col0 >> 3 : 0)) * 16 + m));
                if (!in) Av[r][q] = (h8){0, 0, 0, 0, 0, 0, 0, 0};
            }
#pragma unroll
            for (int t = 0; t < NBT; ++t) {
                const int bc = t * 16 + m;
                const bool okb = bc < b && in;
                if constexpr (WHOLE)
                    Bo[q][t] = __builtin_bit_cast(h8, load_x16((lx_ptr)&xw[(m & 7) * XW + bgl + (in ? col0 : 0)]));
                else
                    Bo[q][t] = __builtin_bit_cast(
                        h8, load_x16((gx_ptr)(xo_base + (okb ? (int64_t)bc * xp_len + col0 : 0))));
                if (!okb) Bo[q][t] = (h8){0, 0, 0, 0, 0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int t = 0; t < NBT; ++t)
                    acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Av[r][q], Bo[q][t], acc[r][t], 0, 0, 0);
    }

    // lane (c, m) holds rows 4c .. 4c + 3 of the tile, batch column 16t + m
    if (S > 1) {
        typedef float RedTile[RB][NBT][16][17];
        RedTile* red = reinterpret_cast<RedTile*>(WHOLE ? xw : lds);
        __syncthreads();                               // the staging buffers are dead
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int t = 0; t < NBT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) red[wave][r][t][4 * c + i][m] = acc[r][t][i];
        __syncthreads();
        if (s == 0) {
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int t = 0; t < NBT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float v = acc[r][t][i];
                        for (int p = 1; p < S; ++p) v += red[wave + p][r][t][4 * c + i][m];
                        acc[r][t][i] = v;
                    }
        }
    }
    if (s == 0) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            if (!tile_ok[r]) continue;
            const int trow0 = (t16 + r) * 16;
#pragma unroll
            for (int t = 0; t < NBT; ++t) {
                const int bc = t * 16 + m;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n = trow0 + 4 * c + i;
                    if (bc < b && n < a.N) {
                        if (a.part) *gptr(a.part + ((int64_t)split * b + bc) * a.N + n) = acc[r][t][i];
                        else *gptr(a.y + (int64_t)bc * a.ldy + n) = f_to_h(acc[r][t][i]);
                    }
                }
            }
        }
    }
}

// Launch a kernel; with timing events set (set_launch_events), through
// hipExtLaunchKernel so the events take dispatch timestamps: the first launch
// after the events were set records the start event at its own start (and
// clears it), every launch records the stop event at its end, so a sequence of
// launches (permutation, product, reduction) is bracketed as a whole.
template <class K, class... A>
hipError_t launch_kernel(K kernel, dim3 grid, dim3 block, size_t shmem, hipStream_t s, A... args) {
    void* argv[] = {(void*)&args...};
    if (woq::g_ev_start || woq::g_ev_stop) {
        hipEvent_t start = woq::g_ev_start;
        woq::g_ev_start = nullptr;
        return hipExtLaunchKernel((const void*)kernel, grid, block, argv, shmem, s, start, woq::g_ev_stop, 0);
    }
    return hipLaunchKernel((const void*)kernel, grid, block, argv, shmem, s);
}

int launch_status(hipError_t e) {
    if (e != hipSuccess) {
        woq::set_hip_error((int)e);
        return WOQ_EHIP;
    }
    return WOQ_OK;
}

int compute_units();

// Tiles per workgroup and waves per tile of the vector kernel (measured on
// MI355X over the 3B- and 70B-shaped products): narrow products split each
// tile's groups over four waves so that enough loads are in flight on every
// compute unit; from 1024 tiles on, two tiles share a workgroup (one staged
// copy of the activations) and each tile takes two waves.
template <int B, int T, int S, bool GATHER>
hipError_t launch_int4o_plan(const Int4oArgs& a, const GatherArgs& ga, size_t lds, hipStream_t s) {
    const int tiles = (int)woq::ceil_div(a.N, 16);
    return launch_kernel(qgemv_int4o_tile<B, T, S, GATHER>, dim3((unsigned)woq::ceil_div(tiles, T)), dim3(64 * T * S),
                         lds, s, a, ga);
}

template <int B, bool GATHER>
hipError_t launch_int4o_tile(const Int4oArgs& a, const GatherArgs& ga, hipStream_t s) {
    const int tiles = (int)woq::ceil_div(a.N, 16);
    const size_t lds = (size_t)woq::int4o_valu_lds_bytes(a.xp_len, 4 * (int64_t)a.G4, B);
    // plans from whole-stack sweeps on MI355X: rows of 128 groups or more on
    // 512 tiles or more (70B down) run two tiles of eight waves per workgroup
    // (70B down 23.1 -> 22.3 us); 1024 tiles or more (3B and 70B gate|up, the
    // 128256-row heads) two tiles of two waves, one staged copy of the
    // activations for both (70B gate|up 40.8 -> 40.1 us)
    if (a.G4 >= 128 && tiles >= 512) return launch_int4o_plan<B, 2, 8, GATHER>(a, ga, lds, s);
    if constexpr (B == 1) {
        // b = 1: long rows on few tiles one tile of eight waves, so every SIMD
        // streams.  Otherwise one tile of four waves per workgroup, unless
        // that leaves some compute units a workgroup more than others: then
        // two tiles of two waves, or three of four, so that every compute unit
        // runs at most one workgroup (70B q|k|v, 640 tiles: 10.9 -> 10.4 us
        // with three tiles; 3B q|k|v, 320 tiles: 5.6 -> 5.2 us with two; 70B
        // o, 512 tiles, and 3B o, 192, stay at one).  3B down (192 tiles of 64
        // groups) measured 6.4 -> 6.0 us with four waves instead of eight.
        if (a.G4 >= 128) return launch_int4o_plan<B, 1, 8, GATHER>(a, ga, lds, s);
        if (tiles >= 1024) return launch_int4o_plan<B, 2, 2, GATHER>(a, ga, lds, s);
        const int cus = compute_units();
        if (tiles > cus && tiles % cus != 0) {
            if (tiles <= 2 * cus) return launch_int4o_plan<B, 2, 2, GATHER>(a, ga, lds, s);
            if (tiles <= 3 * cus) return launch_int4o_plan<B, 3, 4, GATHER>(a, ga, lds, s);
        }
        return launch_int4o_plan<B, 1, 4, GATHER>(a, ga, lds, s);
    } else {
        // b = 2..4: long rows on few tiles one tile of eight waves, 1024
        // tiles or more two tiles of two waves, the rest one tile of four
        if (a.G4 >= 48 && (tiles < 256 || a.G4 >= 128)) return launch_int4o_plan<B, 1, 8, GATHER>(a, ga, lds, s);
        if (tiles >= 1024) return launch_int4o_plan<B, 2, 2, GATHER>(a, ga, lds, s);
        return launch_int4o_plan<B, 1, 4, GATHER>(a, ga, lds, s);
    }
}

template <bool GATHER>
hipError_t launch_int4o_tile_b(const Int4oArgs& a, const GatherArgs& ga, int64_t b, hipStream_t s) {
    switch (b) {
        case 1: return launch_int4o_tile<1, GATHER>(a, ga, s);
        case 2: return launch_int4o_tile<2, GATHER>(a, ga, s);
        case 3: return launch_int4o_tile<3, GATHER>(a, ga, s);
        default: return launch_int4o_tile<4, GATHER>(a, ga, s);
    }
}

template <int B>
hipError_t launch_int8_valu(const Int8Args& a, int quads, hipStream_t s) {
    return launch_kernel(qgemv_int8_valu<B>, dim3(quads), dim3(64), 0, s, a);
}

// Compute units of the current device, read once per device.
int compute_units() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// The widest matrix-core plans put eight tiles (each of rb tiles per wave) in
// a workgroup.  Where that grid leaves compute units idle and seven tiles
// still give at most one workgroup per compute unit, seven spread the same
// rows over more of them.  Measured on MI355X: the 70B gate|up product
// (3584 tiles, two per wave) goes from 224 to 256 workgroups and the 70B
// step at b = 8 from 9.92 to 9.80 ms (unchanged at b = 32); the 9B INT8
// gate|up (1792 tiles) likewise, and the 9B step at b = 8 from 2.860 to
// 2.790 ms.
bool seven_tiles_fill(int tiles, int rb) {
    const int cus = compute_units();
    return woq::ceil_div(tiles, 8 * rb) < cus && woq::ceil_div(tiles, 7 * rb) <= cus;
}

template <int T, int S>
hipError_t launch_int8_mfma_ts(const Int8Args& a, int b, hipStream_t s) {
    const int tiles = (int)woq::ceil_div(a.N, 16);
    return launch_kernel(qgemm_int8_mfma<T, S>, dim3((unsigned)woq::ceil_div(tiles, T)), dim3(64 * T * S), 0, s, a,
                         b);
}

hipError_t launch_int8_mfma(const Int8Args& a, int b, hipStream_t s) {
    const int tiles = (int)woq::ceil_div(a.N, 16);
    if (tiles >= 1024) {
        if (seven_tiles_fill(tiles, 1)) return launch_int8_mfma_ts<7, 1>(a, b, s);
        return launch_int8_mfma_ts<8, 1>(a, b, s);
    }
    return launch_int8_mfma_ts<2, 4>(a, b, s);
}

// Dynamic LDS of the whole-row form: the 8 staged columns of the permuted row.
size_t int4o_whole_lds_bytes(int64_t xp_len) { return (size_t)16 * int4o_whole_stride((int)xp_len); }

// Allow a kernel the dynamic LDS it is launched with (above the default
// limit), once per kernel and size.
template <class K>
void allow_dynamic_lds(K kernel, size_t bytes) {
    static std::atomic<size_t> allowed{0};
    if (bytes <= allowed.load(std::memory_order_relaxed)) return;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)bytes) == hipSuccess)
        allowed.store(bytes, std::memory_order_relaxed);
}

template <int NBT, int T, int S, int RB = 1>
hipError_t launch_int4o_mfma_ts(const Int4oArgs& a, int b, int tiles, hipStream_t s, int splits = 1,
                                const GatherArgs* ga = nullptr) {
    const GatherArgs none = {};
    const dim3 grid((unsigned)woq::ceil_div(tiles, T * RB), (unsigned)splits), block(64 * T * S);
    // up to 8 batch columns on long rows: stage 8 columns only, in chunks of
    // 16 groups (70B down at b = 8: 42.6 -> 37.5 us; on rows of 24 groups the
    // longer chunks were slower), or (ga) the whole row, gathered through the
    // channel positions
    if constexpr (NBT == 1) {
        if (b <= 8 && a.G4 >= 64) {
            if (ga) {
                const size_t lds = int4o_whole_lds_bytes(a.xp_len);
                allow_dynamic_lds(qgemm_int4o_mfma<NBT, T, S, RB, true, true>, lds);
                return launch_kernel(qgemm_int4o_mfma<NBT, T, S, RB, true, true>, grid, block, lds, s, a, b, *ga);
            }
            return launch_kernel(qgemm_int4o_mfma<NBT, T, S, RB, true>, grid, block, 0, s, a, b, none);
        }
    }
    return launch_kernel(qgemm_int4o_mfma<NBT, T, S, RB, false>, grid, block, 0, s, a, b, none);
}

// Tiles per workgroup (T), waves per tile (S) and tiles per wave (RB) of the
// matrix-core kernel, measured on MI355X over the 3B- and 70B-shaped
// products: the widest products give each wave two whole tiles (each
// activation fragment read from LDS feeds both, which halves the LDS reads
// and the staged activation traffic per weight byte: 70B gate|up 59 -> 51 us
// at b = 8 and 88 -> 67 us at b = 32) and share the staged activations among
// eight waves; narrower ones split K over more waves so that every compute
// unit has loads in flight (there, two tiles per wave were slower).
// (the whole-row form, ga, takes the same plans: int4o_half_grid mirrors
// the choice for 8 staged columns)
template <int NBT>
hipError_t launch_int4o_mfma(const Int4oArgs& a, int b, hipStream_t s, const GatherArgs* ga = nullptr) {
    const int tiles = (int)woq::ceil_div(a.N, 16);
    if (tiles >= 2048) {
        constexpr int RB = NBT <= 2 ? 2 : 1;
        if (seven_tiles_fill(tiles, RB)) return launch_int4o_mfma_ts<NBT, 7, 1, RB>(a, b, tiles, s, 1, ga);
        return launch_int4o_mfma_ts<NBT, 8, 1, RB>(a, b, tiles, s, 1, ga);
    }
    if constexpr (NBT >= 3) {
        return launch_int4o_mfma_ts<NBT, 2, 2>(a, b, tiles, s);
    } else {
        // on rows of 64 groups or more these products are bound by the loads
        // in flight per compute unit: one workgroup per compute unit, as many
        // waves as fit, and the fewest tiles per workgroup that still place
        // every tile in one round (two tiles of eight waves, three of four,
        // else four of four; measured on MI355X against the one plan of
        // earlier builds: 70B o 18.0 -> 17.5 us at b = 8, 17.4 -> 16.7 us at
        // b = 4 and 24.3 -> 23.3 us at b = 32, 70B q|k|v 20.6 -> 19.6, 19.8
        // -> 19.0 and 29.6 -> 25.8 us; deeper weight windows, longer chunks
        // and the other plans of 4-16 waves were slower)
        if (tiles >= 256 && a.G4 >= 64) {
            const int per = (int)woq::ceil_div(tiles, compute_units());
            if (per <= 2) return launch_int4o_mfma_ts<NBT, 2, 8>(a, b, tiles, s, 1, ga);
            if (per == 3) return launch_int4o_mfma_ts<NBT, 3, 4>(a, b, tiles, s, 1, ga);
            return launch_int4o_mfma_ts<NBT, 4, 4>(a, b, tiles, s, 1, ga);
        }
        if (tiles >= 640) return launch_int4o_mfma_ts<NBT, 4, 2>(a, b, tiles, s, 1, ga);
        if (tiles >= 256) return launch_int4o_mfma_ts<NBT, 2, 4>(a, b, tiles, s, 1, ga);
        return launch_int4o_mfma_ts<NBT, 1, 8>(a, b, tiles, s, 1, ga);
    }
}

// Workgroups of launch_int4o_mfma<1> on rows of 64 groups or more at b <= 8
// (the plans above, 8 staged columns).
int int4o_half_grid(int tiles) {
    if (tiles >= 2048) return (int)woq::ceil_div(tiles, (seven_tiles_fill(tiles, 2) ? 7 : 8) * 2);
    if (tiles >= 256) {
        const int per = (int)woq::ceil_div(tiles, compute_units());
        return (int)woq::ceil_div(tiles, per <= 2 ? 2 : per == 3 ? 3 : 4);
    }
    return tiles;
}

// LDS per workgroup of the current device, read once per device.
int lds_per_block() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 65536;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || n < 1)
            n = 65536;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Split-K launches: each workgroup covers more rows (fewer workgroups along
// N, so fewer re-reads of the staged activations) and blockIdx.y picks the K
// range.
template <int NBT>
hipError_t launch_int4o_mfma_split_nbt(const Int4oArgs& a, int b, int splits, hipStream_t s) {
    const int tiles = (int)woq::ceil_div(a.N, 16);
    if constexpr (NBT == 2) return launch_int4o_mfma_ts<NBT, 8, 1, 2>(a, b, tiles, s, splits);
    return launch_int4o_mfma_ts<NBT, 8, 1, 1>(a, b, tiles, s, splits);
}

hipError_t launch_int4o_mfma_split(const Int4oArgs& a, int b, int splits, hipStream_t s) {
    switch ((b + 15) / 16) {
        case 1: return launch_int4o_mfma_split_nbt<1>(a, b, splits, s);
        case 2: return launch_int4o_mfma_split_nbt<2>(a, b, splits, s);
        case 3: return launch_int4o_mfma_split_nbt<3>(a, b, splits, s);
        default: return launch_int4o_mfma_split_nbt<4>(a, b, splits, s);
    }
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
    a.scales = reinterpret_cast<const uint16_t*>(w->scales);
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
    return launch_status(launch_kernel(permute_x_kernel, dim3(blocks, (unsigned)b), dim3(threads), 0,
                                       (hipStream_t)stream, x, ldx, perm, (int)g->K, (int)g->K_bg, (int)g->n_out,
                                       (int)(128 * g->G4), (int)g->xp_len, xp));
}

int woq_qgemv_int4o(const woq_int4o_w* w, const uint16_t* xp, int64_t b, uint16_t* y, int64_t ldy, void* stream) {
    int st = int4o_common_checks(w, xp, b, y, ldy);
    if (st) return st;
    if (b == 0 || w->N == 0) return WOQ_OK;
    if (!woq::int4o_use_valu(w->N, w->geom, b)) return woq_qgemm_int4o(w, xp, b, y, ldy, stream);
    Int4oArgs a = make_int4o_args(w, xp, y, ldy);
    GatherArgs ga = {};
    return launch_status(launch_int4o_tile_b<false>(a, ga, b, (hipStream_t)stream));
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
    Int4oArgs a = make_int4o_args(w, nullptr, y, ldy);
    GatherArgs ga;
    ga.x = x;
    ga.pos = pos;
    ga.K = (int)g.K;
    ga.K_bg = (int)g.K_bg;
    ga.n_out = (int)g.n_out;
    ga.ldx = (int)ldx;
    return launch_status(launch_int4o_tile_b<true>(a, ga, b, (hipStream_t)stream));
}

int woq_qgemv_int4o_x_supported(const woq_int4o_geom* g, int64_t b) {
    if (!g || b < 1 || b > 4) return 0;
    return g->xp_len <= 65535 && woq::int4o_valu_lds_bytes(g->xp_len, 4 * g->G4, b) <= woq::INT4O_VALU_LDS_BYTES;
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

int woq_qgemm_int4o_x_supported(const woq_int4o_geom* g, int64_t N, int64_t b) {
    if (!g || b < 1 || b > 8 || N < 1 || N > (int64_t)INT32_MAX - 64 || g->G4 < 64 || g->xp_len > 65535) return 0;
    if (int4o_whole_lds_bytes(g->xp_len) + 64 > (size_t)lds_per_block()) return 0;
    // one workgroup per compute unit (the LDS allows no more), in one round
    return int4o_half_grid((int)woq::ceil_div(N, 16)) <= compute_units();
}

int woq_qgemm_int4o_x(const woq_int4o_w* w, const uint16_t* x, int64_t ldx, const uint16_t* pos, int64_t b,
                      uint16_t* y, int64_t ldy, void* stream) {
    int st = check_int4o_w(w);
    if (st) return st;
    const woq_int4o_geom& g = w->geom;
    if (b < 0 || ldx < g.K || ldy < w->N || ldx > INT32_MAX || ldy > INT32_MAX) return WOQ_EINVAL;
    if (b == 0 || w->N == 0) return WOQ_OK;
    if (!x || !pos || !y) return WOQ_EINVAL;
    if (!woq::aligned16(x) || !woq::aligned16(pos) || (ldx & 7) || ((uintptr_t)y & 1u)) return WOQ_EALIGN;
    if (!woq_qgemm_int4o_x_supported(&g, w->N, b)) return WOQ_EUNSUPPORTED;
    // a.xp = x: the kernel's clamped, unused loads need a valid address
    Int4oArgs a = make_int4o_args(w, x, y, ldy);
    GatherArgs ga;
    ga.x = x;
    ga.pos = pos;
    ga.K = (int)g.K;
    ga.K_bg = (int)g.K_bg;
    ga.n_out = (int)g.n_out;
    ga.ldx = (int)ldx;
    return launch_status(launch_int4o_mfma<1>(a, (int)b, (hipStream_t)stream, &ga));
}

int64_t woq_qgemm_int4o_splitk_workspace(int64_t N, int64_t b, int32_t splits) {
    if (N < 0 || b < 0 || splits < 1) return -1;
    return (int64_t)splits * b * N * (int64_t)sizeof(float);
}

int woq_qgemm_int4o_splitk(const woq_int4o_w* w, const uint16_t* xp, int64_t b, uint16_t* y, int64_t ldy,
                           int32_t splits, float* workspace, int64_t workspace_bytes, void* stream) {
    int st = int4o_common_checks(w, xp, b, y, ldy);
    if (st) return st;
    if (splits < 1 || splits > 16) return WOQ_EINVAL;
    if (b == 0 || w->N == 0) return WOQ_OK;
    if (!workspace || workspace_bytes < woq_qgemm_int4o_splitk_workspace(w->N, b, splits)) return WOQ_EINVAL;
    if (!woq::aligned16(workspace)) return WOQ_EALIGN;
    if ((int64_t)splits * b * w->N > INT32_MAX) return WOQ_EUNSUPPORTED;
    Int4oArgs a = make_int4o_args(w, xp, y, ldy);
    a.gsplit = (int)woq::ceil_div(w->geom.G4, splits);
    a.part = workspace;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_int4o_mfma_split(a, (int)b, splits, s);
    if (e == hipSuccess) {
        const int64_t n = b * w->N;
        e = launch_kernel(reduce_splits_kernel, dim3((unsigned)woq::ceil_div(n, 256)), dim3(256), 0, s,
                          (const float*)workspace, (int)splits, (int)b, (int)w->N, y, (int)ldy);
    }
    return launch_status(e);
}

int woq_stream_read(const void* buf, int64_t bytes, void* stream) {
    if (bytes < 0 || (bytes & 15)) return WOQ_EINVAL;
    if (bytes == 0) return WOQ_OK;
    if (!buf) return WOQ_EINVAL;
    if (!woq::aligned16(buf)) return WOQ_EALIGN;
    // one scratch word per device for the kernel's never-taken store
    static std::mutex mu;
    static uint32_t* sinks[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= 64) {
        woq::set_hip_error((int)e);
        return WOQ_EHIP;
    }
    uint32_t* sink;
    {
        std::lock_guard<std::mutex> lock(mu);
        if (!sinks[dev]) {
            e = hipMalloc((void**)&sinks[dev], sizeof(uint32_t));
            if (e != hipSuccess) {
                sinks[dev] = nullptr;
                woq::set_hip_error((int)e);
                return WOQ_ENOMEM;
            }
        }
        sink = sinks[dev];
    }
    const int64_t n16 = bytes / 16;
    const int64_t blocks = woq::ceil_div(n16, 256 * 4);
    if (blocks > INT32_MAX) return WOQ_EUNSUPPORTED;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       (const uint4*)buf, n16, sink);
    return launch_status(hipGetLastError());
}

int woq_embed_int8(const woq_int8_w* w, const int32_t* ids, int64_t b, uint16_t* y, int64_t ldy, void* stream) {
    if (!w || w->N < 0 || w->K < 1 || b < 0 || ldy < w->K) return WOQ_EINVAL;
    if (w->nseg < 1 || w->nseg > WOQ_MAX_SEGMENTS || w->seg_end[w->nseg - 1] != w->N) return WOQ_EINVAL;
    for (int i = 0; i < w->nseg; ++i) {
        int64_t lo = i ? w->seg_end[i - 1] : 0;
        if (w->seg_end[i] < lo) return WOQ_EINVAL;
    }
    if (b == 0) return WOQ_OK;
    if (!ids || !y || (w->N > 0 && !w->codes)) return WOQ_EINVAL;
    if ((w->N > 0 && !woq::aligned16(w->codes)) || ((uintptr_t)ids & 3u) || !woq::aligned16(y) || (ldy & 7))
        return WOQ_EALIGN;
    if (b > 65535 || w->N > (int64_t)INT32_MAX - 64 || w->K > (int64_t)INT32_MAX - 64 || ldy > INT32_MAX)
        return WOQ_EUNSUPPORTED;
    EmbedArgs a;
    a.codes = reinterpret_cast<const uint4*>(w->codes);
    a.ids = ids;
    a.y = y;
    a.V = (int)w->N;
    a.K = (int)w->K;
    a.CPR = (int)(woq::round_up(w->K, 64) / 16);
    a.ldy = (int)ldy;
    a.nseg = w->nseg;
    for (int i = 0; i < WOQ_MAX_SEGMENTS; ++i) {
        a.seg_end[i] = i < w->nseg ? (int)w->seg_end[i] : (int)w->N;
        a.seg_scale[i] = i < w->nseg ? w->seg_scale[i] : 0.0f;
    }
    const int threads = 256;
    const int blocks = (int)woq::ceil_div(woq::ceil_div(w->K, 16), threads);
    hipLaunchKernelGGL(embed_int8_kernel, dim3(blocks, (unsigned)b), dim3(threads), 0, (hipStream_t)stream, a);
    return launch_status(hipGetLastError());
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
    if (int8_use_mfma(w->N, b)) return launch_status(launch_int8_mfma(a, (int)b, s));
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
