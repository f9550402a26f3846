// On-device encoders: the INT8 per-tensor and the outlier-aware INT4 encodings
// of the host functions (woq_quantize_int8, woq_quantize_int4o + the device
// layouts), computed by the GPU from fp32 weights already in device memory and
// written straight into the kernels' device layouts, bit for bit the same.
//
// Exactness: the scale divisions (max / 127, max / 7) and the code divisions
// (W / scale) are IEEE fp32 divisions (HIP's default, correctly rounded fp32
// division), rounding is v_rndne_f32 (half to even), the fp16 scale is an RNE
// fp32 -> fp16 conversion, and maxima are order-independent; so the result
// does not depend on how the work is split.
#include <hip/hip_runtime.h>

#include "woq_gemv.h"
#include "woq_internal.h"

namespace {

using namespace woqk;

// |w| as an unsigned bit pattern: for non-negative floats the patterns order
// like the values, and infinities and NaNs order above every finite value.
__device__ __forceinline__ uint32_t abs_bits(float w) { return __float_as_uint(w) & 0x7FFFFFFFu; }
constexpr uint32_t NONFINITE_BITS = 0x7F800000u;

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) *gptr(p + i) = v;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, m));
    return v;
}

// Pass 1 of INT8: max |W| over the whole tensor into *acc (as bits).
__global__ __launch_bounds__(256) void absmax_kernel(const float* __restrict__ W, int64_t n,
                                                     uint32_t* __restrict__ acc) {
    uint32_t m = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        m = max(m, abs_bits(*gptr(W + i)));
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0 && m) atomicMax(acc, m);
}

// Pass 2 of INT8: codes into the device layout, one dword (4 columns) per lane.
// Every lane derives the scale from the maximum itself.
__global__ __launch_bounds__(256) void quantize_int8_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                                            int64_t Kd, int64_t n_dwords,
                                                            const uint32_t* __restrict__ maxbits,
                                                            uint32_t* __restrict__ dev) {
    const uint32_t mb = *gptr(maxbits);
    const float s = mb >= NONFINITE_BITS ? 0.0f : __uint_as_float(mb) / 127.0f;
    const int64_t dpr = Kd / 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < n_dwords; d += stride) {
        const int64_t n = d / dpr, k0 = 4 * (d % dpr);
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int q = 0;
            if (n < N && k0 + j < K && s != 0.0f) {
                float t = rintf(*gptr(W + n * K + k0 + j) / s);
                q = (int)fminf(fmaxf(t, -127.0f), 127.0f);
            }
            word |= (uint32_t)(q + 128) << (8 * j);
        }
        *gptr(dev + d) = word;
    }
}

// Pass 3 of INT8: the scale (NaN, with status WOQ_ERANGE, for a non-finite weight).
__global__ void finish_int8_kernel(uint32_t* maxbits_then_scale, int32_t* status) {
    const uint32_t mb = *gptr(maxbits_then_scale);
    float s;
    if (mb >= NONFINITE_BITS) {
        s = __uint_as_float(0x7FC00000u);
        *gptr(status) = WOQ_ERANGE;
    } else {
        s = __uint_as_float(mb) / 127.0f;
    }
    *gptr(reinterpret_cast<float*>(maxbits_then_scale)) = s;
}

struct Int4oPrepArgs {
    const float* W;          // [N][K] fp32
    const int32_t* perm;     // [K]
    uint32_t* codes;         // device layout, as dwords
    uint16_t* scales;        // device layout
    int32_t* status;
    int64_t N, K;
    int K_bg, G4, N16;
};

// Nibble position of channel t (0..15) of a 16-channel half inside its dword:
// t = 4e + i (i = 0..3) -> dword e, positions 0, 4, 2, 6; t = 8 + 4e + i ->
// dword e, positions 1, 5, 3, 7.
__device__ __forceinline__ int nibble_pos(int t) {
    const int i = t & 3;
    return ((i & 1) << 2) | ((i >> 1) << 1) | ((t >> 3) & 1);
}

// One wave per (row r, group g) of the padded layout; lane l holds background
// channels 128g + 2l and 128g + 2l + 1.
__global__ __launch_bounds__(64) void quantize_int4o_kernel(Int4oPrepArgs a) {
    const int64_t blk = blockIdx.x;
    const int g = (int)(blk % a.G4);
    const int64_t r = blk / a.G4;
    const int l = threadIdx.x;
    float w[2] = {0.0f, 0.0f};
    bool bad = false;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int kb = 128 * g + 2 * l + u;
        if (r < a.N && kb < a.K_bg) {
            const int src = *gptr(a.perm + kb);
            if ((unsigned)src < (unsigned)a.K) w[u] = *gptr(a.W + r * a.K + src);
            else bad = true;    // not a permutation of [0, K)
        }
    }
    const uint32_t mb = wave_max(max(abs_bits(w[0]), abs_bits(w[1])));
    const float s16f = __uint_as_float(mb) / 7.0f;
    const _Float16 s16 = (_Float16)s16f;
    const float s = (float)s16;
    if (l == 0 && (mb >= NONFINITE_BITS || !(s <= 65504.0f))) *gptr(a.status) = WOQ_ERANGE;
    if (bad) *gptr(a.status) = WOQ_EINVAL;
    uint32_t pair = 0;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        int q = 0;
        if (s != 0.0f && mb < NONFINITE_BITS) {
            float t = rintf(w[u] / s);
            q = (int)fminf(fmaxf(t, -7.0f), 7.0f);
        }
        pair |= (uint32_t)(q + 8) << (4 * u);
    }
    // lane L < 16 builds dword L of the group: chunk c = L / 4, half P and
    // dword e inside it; its 8 channels come from the lanes that hold them
    const int L = l & 15;
    const int c = L >> 2, P = (L >> 1) & 1, e = L & 1;
    uint32_t word = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 8 * h + 4 * e + i;
            const int ch = 32 * c + 16 * P + t;
            const uint32_t v = (uint32_t)__shfl((int)pair, ch >> 1);
            const uint32_t code = (ch & 1) ? (v >> 4) & 15u : v & 15u;
            word |= code << (4 * nibble_pos(t));
        }
    }
    const int64_t tile = r >> 4, row = r & 15;
    if (l < 16) {
        const int64_t byte = ((tile * a.G4 + g) * 4 + c) * 256 + row * 16 + 4 * (2 * P + e);
        *gptr(a.codes + byte / 4) = word;
    }
    if (l == 0) *gptr(a.scales + (tile * a.G4 + g) * 16 + row) = (r < a.N) ? __builtin_bit_cast(uint16_t, s16) : 0;
}

// Outlier weights, fp16(W[r, perm[K_bg + i]]), into the device layout; one
// lane per (row, outlier slot) of the padded layout.
__global__ __launch_bounds__(256) void outliers_int4o_kernel(const float* __restrict__ W,
                                                             const int32_t* __restrict__ perm, int64_t N, int64_t K,
                                                             int K_bg, int n_out, int no8, int64_t total,
                                                             uint16_t* __restrict__ wout, int32_t* status) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const int64_t r = idx / (8 * no8);
    const int i = (int)(idx % (8 * no8));
    uint16_t v = 0;
    if (r < N && i < n_out) {
        const int src = *gptr(perm + K_bg + i);
        if ((unsigned)src < (unsigned)K) {
            const float x = *gptr(W + r * K + src);
            if (abs_bits(x) >= NONFINITE_BITS) *gptr(status) = WOQ_ERANGE;
            v = __builtin_bit_cast(uint16_t, (_Float16)x);
        } else {
            *gptr(status) = WOQ_EINVAL;
        }
    }
    const int64_t tile = r >> 4, row = r & 15;
    *gptr(wout + (((tile * no8 + i / 8) * 16 + row) * 8 + i % 8)) = v;
}

int launch_status(hipError_t e) {
    if (e == hipSuccess) return WOQ_OK;
    woq::set_hip_error((int)e);
    return WOQ_EHIP;
}

}  // namespace

extern "C" {

int woq_quantize_int8_dev(const float* W, int64_t N, int64_t K, uint8_t* dev, float* scale, int32_t* status,
                          void* stream) {
    if (N < 1 || K < 1 || !W || !dev || !scale || !status) return WOQ_EINVAL;
    if (((uintptr_t)W & 3u) || !woq::aligned16(dev) || ((uintptr_t)scale & 3u) || ((uintptr_t)status & 3u))
        return WOQ_EALIGN;
    if (N > ((int64_t)1 << 40) / K) return WOQ_EUNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    const int64_t n_dwords = woq_int8_dev_bytes(N, K) / 4;
    uint32_t* acc = reinterpret_cast<uint32_t*>(scale);
    hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(64), 0, s, acc, 0u, 1);
    hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(64), 0, s, reinterpret_cast<uint32_t*>(status), 0u, 1);
    const int64_t n = N * K;
    const int blocks = (int)std::min<int64_t>(woq::ceil_div(n, 256 * 8), 4096);
    hipLaunchKernelGGL(absmax_kernel, dim3(blocks), dim3(256), 0, s, W, n, acc);
    const int qblocks = (int)std::min<int64_t>(woq::ceil_div(n_dwords, 256), 16384);
    hipLaunchKernelGGL(quantize_int8_kernel, dim3(qblocks), dim3(256), 0, s, W, N, K, woq::round_up(K, 64), n_dwords,
                       (const uint32_t*)acc, reinterpret_cast<uint32_t*>(dev));
    hipLaunchKernelGGL(finish_int8_kernel, dim3(1), dim3(1), 0, s, acc, status);
    return launch_status(hipGetLastError());
}

int woq_quantize_int4o_dev(const float* W, int64_t N, const int32_t* perm, const woq_int4o_geom* g,
                           uint8_t* dev_codes, uint16_t* dev_scales, uint16_t* dev_wout, int32_t* status,
                           void* stream) {
    if (!woq::int4o_geom_valid(g) || N < 1 || !W || !perm || !status) return WOQ_EINVAL;
    // with every channel an outlier there is no background (no codes, no scales)
    if ((g->G4 > 0 && (!dev_codes || !dev_scales)) || (g->n_out8 > 0 && !dev_wout)) return WOQ_EINVAL;
    if (((uintptr_t)W & 3u) || ((uintptr_t)perm & 3u) || (dev_codes && !woq::aligned16(dev_codes)) ||
        (dev_scales && !woq::aligned16(dev_scales)) || (dev_wout && !woq::aligned16(dev_wout)) ||
        ((uintptr_t)status & 3u))
        return WOQ_EALIGN;
    const int64_t N16 = woq::round_up(N, 16);
    if (N16 * g->G4 > INT32_MAX || N > ((int64_t)1 << 40) / g->K || N16 > INT32_MAX) return WOQ_EUNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(64), 0, s, reinterpret_cast<uint32_t*>(status), 0u, 1);
    Int4oPrepArgs a;
    a.W = W;
    a.perm = perm;
    a.codes = reinterpret_cast<uint32_t*>(dev_codes);
    a.scales = dev_scales;
    a.status = status;
    a.N = N;
    a.K = g->K;
    a.K_bg = (int)g->K_bg;
    a.G4 = (int)g->G4;
    a.N16 = (int)N16;
    if (g->G4 > 0) hipLaunchKernelGGL(quantize_int4o_kernel, dim3((unsigned)(N16 * g->G4)), dim3(64), 0, s, a);
    if (g->n_out8 > 0) {
        const int64_t total = N16 * g->n_out8;
        hipLaunchKernelGGL(outliers_int4o_kernel, dim3((unsigned)woq::ceil_div(total, 256)), dim3(256), 0, s, W, perm,
                           N, g->K, (int)g->K_bg, (int)g->n_out, (int)(g->n_out8 / 8), total, dev_wout, status);
    }
    return launch_status(hipGetLastError());
}

}  // extern "C"
