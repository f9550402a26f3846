// Device building blocks shared by the product kernels: code unpacking,
// the dequantise-and-dot inner loops and the cross-lane reductions.
//
// Codes become exact fp16 numbers with the exponent-bias ("magic number")
// conversion that published weight-only INT4/INT8 GEMM kernels use (e.g.
// Kim et al., 2022, "Who Says Elephants Can't Run: Bringing Large Scale MoE
// Models into Cloud Scale Production", arXiv:2211.10017): an offset-binary
// code u placed in the low mantissa bits of the fp16 number 1024 (bits
// 0x6400) reads as 1024 + u, so one AND-OR per pair of codes gives two fp16
// values; the offset is removed by one subtraction, or (INT4O vector kernel,
// INT8 at b <= 2) once per chunk from the sum instead.  Products use
// v_dot2_f32_f16 (exact fp16 products, fp32 accumulation) or the fp16 matrix
// cores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace woqk {

typedef _Float16 f16;
typedef f16 h2 __attribute__((ext_vector_type(2)));
typedef f16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Address-space-qualified pointers.  Loads through generic pointers become
// FLAT instructions, which count against the LDS wait counter as well and so
// serialise LDS waits behind every outstanding weight load.
typedef __attribute__((address_space(1))) const u32x4 g_u32x4;
typedef __attribute__((address_space(1))) const u32x2 g_u32x2;
typedef __attribute__((address_space(3))) const u32x4 l_u32x4;
typedef __attribute__((address_space(1))) const uint16_t* gx_ptr;   // activations in global memory
typedef __attribute__((address_space(3))) const uint16_t* lx_ptr;   // activations staged in LDS

// The same pointer in the global address space (for loads and stores that
// must not become FLAT instructions).
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gptr(T* p) {
    return (__attribute__((address_space(1))) T*)p;
}

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ float h_to_f(uint16_t v) { return (float)__builtin_bit_cast(f16, v); }
__device__ __forceinline__ uint16_t f_to_h(float v) { return __builtin_bit_cast(uint16_t, (f16)v); }
__device__ __forceinline__ float dot2(h2 a, h2 b, float c) { return __builtin_amdgcn_fdot2(a, b, c, false); }

__device__ __forceinline__ uint4 as_uint4(u32x4 v) { return make_uint4(v[0], v[1], v[2], v[3]); }

// 16 bytes of activations (8 fp16), 16-byte aligned.
__device__ __forceinline__ uint4 load_x16(gx_ptr p) { return as_uint4(*(g_u32x4*)p); }
__device__ __forceinline__ uint4 load_x16(lx_ptr p) { return as_uint4(*(l_u32x4*)p); }
// 16 and 8 bytes from global memory (cached).
__device__ __forceinline__ uint4 gload_u4(const uint4* p) { return as_uint4(*(g_u32x4*)p); }
__device__ __forceinline__ uint2 gload_u2(const uint2* p) {
    u32x2 v = *(g_u32x2*)p;
    return make_uint2(v[0], v[1]);
}

// 16-byte global store, 16-byte aligned.
__device__ __forceinline__ void gstore_u4(uint4* p, uint4 v) {
    *(__attribute__((address_space(1))) u32x4*)p = u32x4{v.x, v.y, v.z, v.w};
}

// Streamed 16-byte weight load: weight bytes are read exactly once, so they
// are marked non-temporal and do not push the shared activations out of cache.
__device__ __forceinline__ uint4 gload_nt(const uint4* p) {
    return as_uint4(__builtin_nontemporal_load((g_u32x4*)p));
}

// The fp16 exponent bias 0x64006400 is kept in a VGPR: VOP3 instructions on
// this target take no literal operands, and with the bias in a register each
// pair costs a single v_and_or_b32 (mask from an SGPR) instead of an and + or.
__device__ __forceinline__ uint32_t bias_reg() {
    uint32_t v = 0x64006400u;
    asm volatile("" : "+v"(v));
    return v;
}

// fp16 pairs from an INT4O device dword (layout: see woq_layout_int4o):
// lo0/lo1 are channels (4e, 4e+1) and (4e+2, 4e+3) of the half-chunk, hi0/hi1
// are channels (8+4e, 9+4e) and (10+4e, 11+4e) and carry 16 x code.
struct Int4Pairs {
    h2 lo0, lo1, hi0, hi1;
};
__device__ __forceinline__ Int4Pairs int4_pairs(uint32_t w, uint32_t bias) {
    const h2 off_lo = {(f16)1032.0f, (f16)1032.0f};   // 1024 + 8
    const h2 off_hi = {(f16)1152.0f, (f16)1152.0f};   // 1024 + 16 * 8
    uint32_t s = w >> 8;
    Int4Pairs p;
    p.lo0 = as_h2((w & 0x000F000Fu) | bias) - off_lo;
    p.lo1 = as_h2((s & 0x000F000Fu) | bias) - off_lo;
    p.hi0 = as_h2((w & 0x00F000F0u) | bias) - off_hi;
    p.hi1 = as_h2((s & 0x00F000F0u) | bias) - off_hi;
    return p;
}

// fp16 pairs (channels 0,1 and 2,3) of an INT8 device dword (code + 128).
__device__ __forceinline__ void int8_pairs(uint32_t w, h2& a, h2& b) {
    const h2 off = {(f16)1152.0f, (f16)1152.0f};      // 1024 + 128
    a = as_h2(__builtin_amdgcn_perm(w, 0x64646464u, 0x00050004u)) - off;
    b = as_h2(__builtin_amdgcn_perm(w, 0x64646464u, 0x00070006u)) - off;
}

template <int B>
__device__ __forceinline__ void zero_acc(float (&acc)[4][B]) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;
}

// Dot products of one INT4O chunk of one row (32 background channels of one
// group) with B activation rows (the same 32 channels, fp16), on the biased
// fp16 values the masks produce: low-nibble pairs hold code + 1032 and
// high-nibble pairs 16 code + 1152, so the chunk's sum of code * x is
// lo + hi / 16 - corr, with corr = 1032 (sum of x over the low-nibble
// channels) + 72 (sum of x over the high-nibble channels), computed once per
// chunk and batch row (activation_chunk_correction); ncorr = -corr is passed
// in and seeds the low-nibble sum, which saves a subtraction and a register
// clear per chunk.  bias holds 0x64006400 in a vector register.  Skipping the bias
// subtraction saves one packed add per weight pair; products stay exact and
// the cancellation costs about 1e-5 of the chunk's magnitude in fp32.  The
// group scale s multiplies the chunk's sum.
template <int B>
__device__ __forceinline__ void int4o_row_chunk(uint4 w, float s, const uint4 (&xv)[B][4], const float (&ncorr)[B],
                                                float (&acc)[B], uint32_t bias) {
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    h2 lo0[4], lo1[4], hi0[4], hi1[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t sh = wd[d] >> 8;
        lo0[d] = as_h2((wd[d] & 0x000F000Fu) | bias);
        lo1[d] = as_h2((sh & 0x000F000Fu) | bias);
        hi0[d] = as_h2((wd[d] & 0x00F000F0u) | bias);
        hi1[d] = as_h2((sh & 0x00F000F0u) | bias);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const uint32_t xw[16] = {xv[b][0].x, xv[b][0].y, xv[b][0].z, xv[b][0].w,
                                 xv[b][1].x, xv[b][1].y, xv[b][1].z, xv[b][1].w,
                                 xv[b][2].x, xv[b][2].y, xv[b][2].z, xv[b][2].w,
                                 xv[b][3].x, xv[b][3].y, xv[b][3].z, xv[b][3].w};
        float lo = ncorr[b], hi = 0.0f;
#pragma unroll
        for (int P = 0; P < 2; ++P) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int d = 2 * P + e;
                lo = dot2(lo0[d], as_h2(xw[8 * P + 2 * e + 0]), lo);
                lo = dot2(lo1[d], as_h2(xw[8 * P + 2 * e + 1]), lo);
                hi = dot2(hi0[d], as_h2(xw[8 * P + 4 + 2 * e + 0]), hi);
                hi = dot2(hi1[d], as_h2(xw[8 * P + 4 + 2 * e + 1]), hi);
            }
        }
        acc[b] = fmaf(s, fmaf(hi, 0.0625f, lo), acc[b]);
    }
}

// The bias correction of one 32-channel background chunk of activations (see
// int4o_row_chunk): channels 0-7 and 16-23 meet low-nibble codes, 8-15 and
// 24-31 high-nibble codes.
__device__ __forceinline__ float activation_chunk_correction(const uint4 (&xv)[4]) {
    const h2 one = {(f16)1.0f, (f16)1.0f};
    float sl = 0.0f, sh = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t xw[4] = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
        float t = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) t = dot2(as_h2(xw[j]), one, t);
        if (q & 1) sh += t;
        else sl += t;
    }
    return 1032.0f * sl + 72.0f * sh;
}

// INT8 products at b <= 2 run on the biased code values (code + 1152 as
// fp16, one v_perm per pair and no subtraction); each lane also sums the
// activations it multiplies, and int8_unbias removes 1152 times that sum once,
// before the wave reduction.  The products stay exact; the cancellation costs
// about 1e-5 of a lane's partial sum in fp32.  From b = 3 on, the dot
// products per batch row outnumber the subtractions they save.
template <int B>
constexpr bool int8_biased() { return B <= 2; }

// fp16 pairs (channels 0,1 and 2,3) of an INT8 device dword, biased: code + 1152.
__device__ __forceinline__ void int8_pairs_biased(uint32_t w, h2& a, h2& b) {
    a = as_h2(__builtin_amdgcn_perm(w, 0x64646464u, 0x00050004u));
    b = as_h2(__builtin_amdgcn_perm(w, 0x64646464u, 0x00070006u));
}

// Dot products of one INT8 chunk (four rows, 16 channels) with B activation
// rows; sx[b] accumulates the activations' sum where the codes stay biased.
template <int B>
__device__ __forceinline__ void int8_chunk(const uint4 (&w)[4], const uint4 (&xv)[B][2], float (&acc)[4][B],
                                           float (&sx)[B]) {
    constexpr bool BIASED = int8_biased<B>();
    if constexpr (BIASED) {
        const h2 one = {(f16)1.0f, (f16)1.0f};
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const uint32_t xw[8] = {xv[b][0].x, xv[b][0].y, xv[b][0].z, xv[b][0].w,
                                    xv[b][1].x, xv[b][1].y, xv[b][1].z, xv[b][1].w};
            float t = sx[b];
#pragma unroll
            for (int j = 0; j < 8; ++j) t = dot2(as_h2(xw[j]), one, t);
            sx[b] = t;
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t wd[4] = {w[r].x, w[r].y, w[r].z, w[r].w};
        h2 q[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            if constexpr (BIASED) int8_pairs_biased(wd[d], q[2 * d], q[2 * d + 1]);
            else int8_pairs(wd[d], q[2 * d], q[2 * d + 1]);
        }
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

// Remove the bias of int8_chunk's biased products (before the reduction) and
// clear the activation sums.
template <int B>
__device__ __forceinline__ void int8_unbias(float (&acc)[4][B], float (&sx)[B]) {
    if constexpr (int8_biased<B>()) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] = fmaf(-1152.0f, sx[b], acc[r][b]);
#pragma unroll
        for (int b = 0; b < B; ++b) sx[b] = 0.0f;
    }
}

// Sum of v over the 64 lanes of the wave, returned to every lane.  Within each
// 16-lane row: DPP exchanges with lane ^ 1, lane ^ 2, the mirrored lane of the
// 8-lane half row and of the row; the four row sums are then read with
// v_readlane.  No LDS round trips, so the dependent chain is a few cycles long.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// Sum of v over the 16 lanes of its row, returned to every lane of the row,
// in a fixed order (the first four exchanges of wave_sum_dpp).
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_move<0xB1>(v);
    v += dpp_move<0x4E>(v);
    v += dpp_move<0x141>(v);
    v += dpp_move<0x140>(v);
    return v;
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += dpp_move<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
    v += dpp_move<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
    v += dpp_move<0x141>(v);   // row_half_mirror
    v += dpp_move<0x140>(v);   // row_mirror
    const int iv = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 48));
    return (r0 + r1) + (r2 + r3);
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
            const float v = wave_sum_dpp(acc[r][b]);
            if (lane == r * B + b) out = v;
        }
    return out;
}

// Workgroup control barrier that waits only for this wave's LDS and scalar
// memory operations, not for its outstanding vector loads and stores.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
}

// Sum of v over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 32-channel
// chunks of a group that lanes c = l >> 4 hold for row l & 15).
__device__ __forceinline__ float sum_over_chunks(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

}  // namespace woqk
