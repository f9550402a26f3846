// Device building blocks shared by the single-launch kernels and the
// persistent stack kernel: the per-quad dequantise-and-dot loops.
//
// A "quad" is four consecutive output rows handled by one wave.  Lane l owns
// the 16-byte chunks l, l + 64, ... of each of the four rows (a chunk is 32
// INT4O background channels, or 16 INT8 channels), so every wave-wide weight
// load is one contiguous kilobyte of a row.  Codes become exact fp16 numbers
// with the exponent-bias trick (an offset-binary code u in the low mantissa
// bits of 0x6400 is 1024 + u) and are multiplied with v_dot2_f32_f16 (exact
// fp16 products, fp32 accumulation).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace woqk {

typedef _Float16 f16;
typedef f16 h2 __attribute__((ext_vector_type(2)));
typedef f16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ float h_to_f(uint16_t v) { return (float)__builtin_bit_cast(f16, v); }
__device__ __forceinline__ uint16_t f_to_h(float v) { return __builtin_bit_cast(uint16_t, (f16)v); }
__device__ __forceinline__ float dot2(h2 a, h2 b, float c) { return __builtin_amdgcn_fdot2(a, b, c, false); }

// Streamed 16-byte load: weight bytes are read exactly once, so they are
// marked non-temporal and do not push the shared activations out of cache.
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
    u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// fp16 pairs from an INT4O device dword (layout: see woq_layout_int4o):
// lo0/lo1 are channels (4e, 4e+1) and (4e+2, 4e+3) of the half-chunk, hi0/hi1
// are channels (8+4e, 9+4e) and (10+4e, 11+4e) and carry 16 x code.
struct Int4Pairs {
    h2 lo0, lo1, hi0, hi1;
};
__device__ __forceinline__ Int4Pairs int4_pairs(uint32_t w) {
    const h2 off_lo = {(f16)1032.0f, (f16)1032.0f};   // 1024 + 8
    const h2 off_hi = {(f16)1152.0f, (f16)1152.0f};   // 1024 + 16 * 8
    uint32_t s = w >> 8;
    Int4Pairs p;
    p.lo0 = as_h2((w & 0x000F000Fu) | 0x64006400u) - off_lo;
    p.lo1 = as_h2((s & 0x000F000Fu) | 0x64006400u) - off_lo;
    p.hi0 = as_h2((w & 0x00F000F0u) | 0x64006400u) - off_hi;
    p.hi1 = as_h2((s & 0x00F000F0u) | 0x64006400u) - off_hi;
    return p;
}

// fp16 pairs (channels 0,1 and 2,3) of an INT8 device dword (code + 128).
__device__ __forceinline__ void int8_pairs(uint32_t w, h2& a, h2& b) {
    const h2 off = {(f16)1152.0f, (f16)1152.0f};      // 1024 + 128
    a = as_h2(__builtin_amdgcn_perm(w, 0x64646464u, 0x00050004u)) - off;
    b = as_h2(__builtin_amdgcn_perm(w, 0x64646464u, 0x00070006u)) - off;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

template <int B>
__device__ __forceinline__ void zero_acc(float (&acc)[4][B]) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;
}

// Dot products of one INT4O chunk (four rows, 32 channels) with B activation
// rows; x points at channel 32 * cc of activation row 0, rows xs apart.
template <int B>
__device__ __forceinline__ void int4o_chunk(const uint4 (&w)[4], uint2 sc, const uint16_t* x, int xs,
                                            float (&acc)[4][B]) {
    uint4 xv[B][4];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const uint4* p = reinterpret_cast<const uint4*>(x + b * xs);
#pragma unroll
        for (int j = 0; j < 4; ++j) xv[b][j] = p[j];
    }
    const float s[4] = {h_to_f((uint16_t)(sc.x & 0xFFFF)), h_to_f((uint16_t)(sc.x >> 16)),
                        h_to_f((uint16_t)(sc.y & 0xFFFF)), h_to_f((uint16_t)(sc.y >> 16))};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t wd[4] = {w[r].x, w[r].y, w[r].z, w[r].w};
        Int4Pairs p[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) p[d] = int4_pairs(wd[d]);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const uint32_t xw[16] = {xv[b][0].x, xv[b][0].y, xv[b][0].z, xv[b][0].w,
                                     xv[b][1].x, xv[b][1].y, xv[b][1].z, xv[b][1].w,
                                     xv[b][2].x, xv[b][2].y, xv[b][2].z, xv[b][2].w,
                                     xv[b][3].x, xv[b][3].y, xv[b][3].z, xv[b][3].w};
            float lo = 0.0f, hi = 0.0f;
#pragma unroll
            for (int P = 0; P < 2; ++P) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const Int4Pairs& q = p[2 * P + e];
                    lo = dot2(q.lo0, as_h2(xw[8 * P + 2 * e + 0]), lo);
                    lo = dot2(q.lo1, as_h2(xw[8 * P + 2 * e + 1]), lo);
                    hi = dot2(q.hi0, as_h2(xw[8 * P + 4 + 2 * e + 0]), hi);
                    hi = dot2(q.hi1, as_h2(xw[8 * P + 4 + 2 * e + 1]), hi);
                }
            }
            acc[r][b] = fmaf(s[r], fmaf(hi, 0.0625f, lo), acc[r][b]);
        }
    }
}

// One quad of an INT4O linear: codes w0 = the quad's first row ([4][CPR]
// chunks), sc = the quad's scales ([G4] x 4 fp16), xp = permuted activations
// (row stride xs, background then outliers at 128 * G4), wo = the quad's
// outlier columns ([4][no8] chunks of 8 fp16).
template <int B>
__device__ __forceinline__ void int4o_quad(const uint4* __restrict__ w0, int CPR, const uint2* __restrict__ sc,
                                           const uint4* __restrict__ wo, int no8, const uint16_t* xp, int xs,
                                           int bg_len, int lane, float (&acc)[4][B]) {
    zero_acc(acc);
#pragma unroll 2
    for (int cc = lane; cc < CPR; cc += 64) {
        uint4 w[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = load_stream(w0 + r * CPR + cc);
        int4o_chunk<B>(w, sc[cc >> 2], xp + 32 * cc, xs, acc);
    }
    const uint16_t* xo = xp + bg_len;
    for (int oc = lane; oc < no8; oc += 64) {
        uint4 o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = wo[r * no8 + oc];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const uint4 xv = *reinterpret_cast<const uint4*>(xo + b * xs + 8 * oc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float t = acc[r][b];
                t = dot2(as_h2(o[r].x), as_h2(xv.x), t);
                t = dot2(as_h2(o[r].y), as_h2(xv.y), t);
                t = dot2(as_h2(o[r].z), as_h2(xv.z), t);
                t = dot2(as_h2(o[r].w), as_h2(xv.w), t);
                acc[r][b] = t;
            }
        }
    }
}

// Dot products of one INT8 chunk (four rows, 16 channels) with B activation rows.
template <int B>
__device__ __forceinline__ void int8_chunk(const uint4 (&w)[4], const uint4 (&xv)[B][2], float (&acc)[4][B]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t wd[4] = {w[r].x, w[r].y, w[r].z, w[r].w};
        h2 q[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) int8_pairs(wd[d], q[2 * d], q[2 * d + 1]);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const uint32_t xw[8] = {xv[b][0].x, xv[b][0].y, xv[b][0].z, xv[b][0].w,
                                    xv[b][1].x, xv[b][1].y, xv[b][1].z, xv[b][1].w};
            float t = acc[r][b];
#pragma unroll
            for (int j = 0; j < 8; ++j) t = dot2(q[j], as_h2(xw[j]), t);
            acc[r][b] = t;
        }
    }
}

// One quad of an INT8 linear whose activations are zero-padded to a whole
// number of chunks (row stride xs), e.g. staged in LDS.
template <int B>
__device__ __forceinline__ void int8_quad_padded(const uint4* __restrict__ w0, int CPR, int nchunks, const uint16_t* x,
                                                 int xs, int lane, float (&acc)[4][B]) {
    zero_acc(acc);
#pragma unroll 2
    for (int cc = lane; cc < nchunks; cc += 64) {
        uint4 w[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = load_stream(w0 + r * CPR + cc);
        uint4 xv[B][2];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const uint4* p = reinterpret_cast<const uint4*>(x + b * xs + 16 * cc);
            xv[b][0] = p[0];
            xv[b][1] = p[1];
        }
        int8_chunk<B>(w, xv, acc);
    }
}

// Reduce a quad's accumulators over the wave; lane r * B + b returns the sum
// for row r, batch row b (other lanes return 0).
template <int B>
__device__ __forceinline__ float quad_reduce(float (&acc)[4][B], int lane) {
    float out = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) {
            float v = wave_sum(acc[r][b]);
            if (lane == r * B + b) out = v;
        }
    return out;
}

}  // namespace woqk
